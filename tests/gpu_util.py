"""Helpers for the GPU tests: move seeded host inputs to the device, call the
library through its binding, compare with the oracle."""

import numpy as np

import workloads as wl


def dev():
    import torch

    return torch.device("cuda:0")


def to_dev_bf16(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev()).view(torch.bfloat16)


def to_dev_i32(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def bf16_to_f32(t):
    """Device bf16 tensor -> host float32 numpy (exact)."""
    return t.float().cpu().numpy()


def run_gpu(case, q, kp, vp, max_context_len=None, tables=None, lens=None):
    import torch

    import paged_kv_cache_280_amd as pkv

    tables = case.block_tables if tables is None else tables
    lens = case.context_lens if lens is None else lens
    if max_context_len is None:
        max_context_len = int(np.max(lens)) if len(lens) else 0
    out = pkv.paged_attn_decode(to_dev_bf16(q), to_dev_bf16(kp), to_dev_bf16(vp),
                                to_dev_i32(tables), to_dev_i32(lens), case.block_size,
                                case.scale, max_context_len=max_context_len)
    torch.cuda.synchronize()
    return out


def errors(got, ref):
    d = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    rel = np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30)
    return float(d.max()), float(d.mean()), float(rel)


def assert_parity(got, ref, label=""):
    assert np.isfinite(got).all(), "non-finite output " + label
    mx, mean, rel = errors(got, ref)
    print("parity %s: max_abs=%.3g mean_abs=%.3g rel_rms=%.3g" % (label, mx, mean, rel), flush=True)
    assert mx <= 1e-2 and mean <= 1e-3, label
