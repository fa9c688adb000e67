"""GPU decode with append (paged_attn_decode_append and its fp8 form) against the
oracle's kv_append followed by its decode: outputs within the parity gate, pools
byte for byte.  Lengths cover every offset of the newest position in its block
and tile, sequences whose only position is the new one, empty sequences, long
contexts split over many workers, and the pair-mode launch of short batches."""

import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import assert_parity, bf16_to_f32, to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu


def _u16(t):
    import torch

    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _u8(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _run_bf16(case, lens):
    import torch

    import paged_kv_cache_280_amd as pkv

    rng = np.random.default_rng(case.seed + 1)
    S, H, D, B = case.num_seqs, case.num_kv_heads, case.head_dim, case.block_size
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    kn = wl.randn_bf16(rng, (S, H, D))
    vn = wl.randn_bf16(rng, (S, H, D))
    kd, vd = to_dev_bf16(kp), to_dev_bf16(vp)
    out = pkv.paged_attn_decode_append(to_dev_bf16(q), to_dev_bf16(kn), to_dev_bf16(vn), kd, vd,
                                       to_dev_i32(case.block_tables), to_dev_i32(lens), B,
                                       case.scale, max_context_len=int(lens.max()))
    torch.cuda.synchronize()
    seq = np.array([s for s in range(S) if lens[s] >= 1], np.int32)
    pos = (lens[seq] - 1).astype(np.int32)
    oracle.kv_append(kn[seq], vn[seq], kp, vp, case.block_tables, seq, pos, B)
    ref = oracle.paged_decode(q, kp, vp, case.block_tables, lens, B, case.scale, H)
    return bf16_to_f32(out), ref, kd, vd, kp, vp, vn


LENS = [1, 2, 15, 16, 17, 31, 32, 33, 0, 100, 257, 700]


@pytest.mark.parametrize("D,B,G", [(128, 16, 4), (64, 8, 1), (128, 32, 8), (64, 16, 16)])
def test_decode_append_matches_append_then_decode(D, B, G):
    H = 2 if G < 16 else 1
    lens = np.array(LENS, np.int32)
    case = wl.case_random(D + B + G, len(lens), H * G, H, D, B, lens)
    got, ref, kd, vd, kp, vp, vn = _run_bf16(case, lens)
    assert np.array_equal(_u16(kd), kp) and np.array_equal(_u16(vd), vp), "pools after the call"
    assert not got[lens == 0].any()
    for s in np.nonzero(lens == 1)[0]:     # softmax over one position: the value itself
        want = wl.f32_from_bf16(np.repeat(vn[s], G, axis=0))
        assert np.array_equal(got[s], want)
    assert_parity(got, ref, "decode+append D=%d B=%d G=%d" % (D, B, G))


def test_decode_append_long_contexts_split_over_workers():
    lens = np.array([20000, 16385, 9001, 1, 4096], np.int32)
    case = wl.case_random(5, len(lens), 32, 8, 128, 16, lens)
    got, ref, kd, vd, kp, vp, _ = _run_bf16(case, lens)
    assert np.array_equal(_u16(kd), kp) and np.array_equal(_u16(vd), vp)
    assert_parity(got, ref, "decode+append long")


def test_decode_append_equals_separate_append_and_decode_on_the_gpu():
    """Against kv_append + paged_attn_decode on the GPU: the pools are identical and
    the outputs agree to rounding (the newest weight is formed on the vector units)."""
    import torch

    import paged_kv_cache_280_amd as pkv

    lens = np.array([300, 17, 1, 48, 1000, 5], np.int32)
    case = wl.case_random(9, len(lens), 16, 4, 128, 16, lens)
    rng = np.random.default_rng(4)
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    kn = wl.randn_bf16(rng, (len(lens), 4, 128))
    vn = wl.randn_bf16(rng, (len(lens), 4, 128))
    tabs, ld = to_dev_i32(case.block_tables), to_dev_i32(lens)
    k1, v1 = to_dev_bf16(kp), to_dev_bf16(vp)
    fused = pkv.paged_attn_decode_append(to_dev_bf16(q), to_dev_bf16(kn), to_dev_bf16(vn), k1, v1,
                                         tabs, ld, 16, case.scale, max_context_len=1000)
    k2, v2 = to_dev_bf16(kp), to_dev_bf16(vp)
    pkv.kv_append(to_dev_bf16(kn), to_dev_bf16(vn), k2, v2, tabs,
                  to_dev_i32(np.arange(len(lens), dtype=np.int32)), to_dev_i32(lens - 1), 16)
    sep = pkv.paged_attn_decode(to_dev_bf16(q), k2, v2, tabs, ld, 16, case.scale,
                                max_context_len=1000)
    torch.cuda.synchronize()
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    diff = (fused.float() - sep.float()).abs().max().item()
    assert diff <= 2e-2, diff


@pytest.mark.parametrize("D,B", [(128, 16), (64, 8), (128, 32)])
def test_decode_append_over_fp8_pools(D, B):
    import torch

    import paged_kv_cache_280_amd as pkv

    H, G = 2, 4
    lens = np.array(LENS + [5000], np.int32)
    case = wl.case_random(D + B + 3, len(lens), H * G, H, D, B, lens)
    ks, vs = 0.047, 0.031
    kp8, vp8 = wl.host_pools_fp8(case, ks, vs)
    rng = np.random.default_rng(D + B)
    S = len(lens)
    q = wl.host_q(case)
    kn = wl.randn_bf16(rng, (S, H, D))
    vn = wl.randn_bf16(rng, (S, H, D))
    kd, vd = _u8(kp8), _u8(vp8)
    out = pkv.paged_attn_decode_append(to_dev_bf16(q), to_dev_bf16(kn), to_dev_bf16(vn), kd, vd,
                                       to_dev_i32(case.block_tables), to_dev_i32(lens), B,
                                       case.scale, max_context_len=int(lens.max()), k_scale=ks,
                                       v_scale=vs)
    torch.cuda.synchronize()
    seq = np.array([s for s in range(S) if lens[s] >= 1], np.int32)
    oracle.kv_append_fp8(kn[seq], vn[seq], kp8, vp8, case.block_tables, seq,
                         (lens[seq] - 1).astype(np.int32), B, ks, vs)
    assert np.array_equal(kd.cpu().numpy(), kp8) and np.array_equal(vd.cpu().numpy(), vp8)
    ref = oracle.paged_decode_fp8(q, kp8, vp8, case.block_tables, lens, B, case.scale, ks, vs, H)
    got = bf16_to_f32(out)
    assert not got[lens == 0].any()
    assert_parity(got, ref, "fp8 decode+append D=%d B=%d" % (D, B))


def test_decode_append_in_pair_mode():
    """The pages' 100-token request with one more token: a batch short enough for the
    one-worker-per-pair launch."""
    case = wl.case_tiny(0)
    lens = case.context_lens.copy()
    got, ref, kd, vd, kp, vp, _ = _run_bf16(case, lens)
    assert np.array_equal(_u16(kd), kp) and np.array_equal(_u16(vd), vp)
    assert_parity(got, ref, "decode+append tiny")


def test_decode_append_with_more_pairs_than_workers():
    """1,600 (sequence, KV head) pairs: the call appends first and then decodes, and
    the outputs equal kv_append + paged_attn_decode on the GPU bit for bit."""
    import torch

    import paged_kv_cache_280_amd as pkv

    rng = np.random.default_rng(12)
    S, Hq, Hkv, D, B = 200, 64, 8, 128, 16
    lens = rng.integers(1, 600, S).astype(np.int32)
    lens[:3] = [1, 16, 17]
    case = wl.case_random(44, S, Hq, Hkv, D, B, lens)
    got, ref, kd, vd, kp, vp, _ = _run_bf16(case, lens)
    assert np.array_equal(_u16(kd), kp) and np.array_equal(_u16(vd), vp)
    assert_parity(got, ref, "decode+append, 1600 pairs")
    q = wl.host_q(case)
    kp0, vp0 = wl.host_pools(case)
    k2, v2 = to_dev_bf16(kp0), to_dev_bf16(vp0)
    tabs, ld = to_dev_i32(case.block_tables), to_dev_i32(lens)
    rng2 = np.random.default_rng(case.seed + 1)
    kn = wl.randn_bf16(rng2, (S, Hkv, D))
    vn = wl.randn_bf16(rng2, (S, Hkv, D))
    pkv.kv_append(to_dev_bf16(kn), to_dev_bf16(vn), k2, v2, tabs,
                  to_dev_i32(np.arange(S, dtype=np.int32)), to_dev_i32(lens - 1), B)
    sep = pkv.paged_attn_decode(to_dev_bf16(q), k2, v2, tabs, ld, B, case.scale,
                                max_context_len=int(lens.max()))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_f32(sep).view(np.uint32), got.view(np.uint32))


def _bad_entry_case(seed, lens, Hq=16, Hkv=4):
    """A batch whose tables name blocks outside the pool for some sequences'
    newest positions (and the only block of a one-position sequence)."""
    lens = np.asarray(lens, np.int32)
    case = wl.case_random(seed, len(lens), Hq, Hkv, 128, 16, lens)
    tables = case.block_tables.copy()
    NB = case.num_blocks
    bad = {1: NB + 5, 2: -3, 4: NB}
    for s, b in bad.items():
        tables[s, (int(lens[s]) - 1) // 16] = b
    return case, tables, sorted(bad)


@pytest.mark.parametrize("fp8", [False, True])
def test_a_table_entry_outside_the_pool_is_never_written(fp8):
    """Decode with append where some newest positions map to no block of the pool:
    the fused call writes nothing for them, exactly as kv_append skips such tokens,
    so the pools after the fused call, after kv_append + decode on the GPU and after
    the oracle's append are the same bytes; the other sequences' outputs stay at
    parity."""
    import torch

    import paged_kv_cache_280_amd as pkv

    lens = [300, 17, 1, 48, 1000, 5, 1, 33]
    case, tables, bad = _bad_entry_case(14, lens)
    lens = case.context_lens
    S, H, D, B = case.num_seqs, case.num_kv_heads, case.head_dim, case.block_size
    rng = np.random.default_rng(15)
    q = wl.host_q(case)
    kn = wl.randn_bf16(rng, (S, H, D))
    vn = wl.randn_bf16(rng, (S, H, D))
    ks = vs = 0.05
    if fp8:
        kp, vp = wl.host_pools_fp8(case, ks, vs)
        dev = _u8
        sc = dict(k_scale=ks, v_scale=vs)
    else:
        kp, vp = wl.host_pools(case)
        dev = to_dev_bf16
        sc = {}
    tabs, ld = to_dev_i32(tables), to_dev_i32(lens)
    qd, knd, vnd = to_dev_bf16(q), to_dev_bf16(kn), to_dev_bf16(vn)
    k1, v1 = dev(kp), dev(vp)
    print("bad entries fused fp8=%s" % fp8, flush=True)
    fused = pkv.paged_attn_decode_append(qd, knd, vnd, k1, v1, tabs, ld, B, case.scale,
                                         max_context_len=int(lens.max()), **sc)
    k2, v2 = dev(kp), dev(vp)
    seq_d = to_dev_i32(np.arange(S, dtype=np.int32))
    if fp8:
        pkv.kv_append_fp8(knd, vnd, k2, v2, tabs, seq_d, to_dev_i32(lens - 1), B, ks, vs)
        sep = pkv.paged_attn_decode_fp8(qd, k2, v2, tabs, ld, B, case.scale, ks, vs,
                                        max_context_len=int(lens.max()))
    else:
        pkv.kv_append(knd, vnd, k2, v2, tabs, seq_d, to_dev_i32(lens - 1), B)
        sep = pkv.paged_attn_decode(qd, k2, v2, tabs, ld, B, case.scale,
                                    max_context_len=int(lens.max()))
    torch.cuda.synchronize()
    seq = np.arange(S, dtype=np.int32)
    if fp8:
        oracle.kv_append_fp8(kn, vn, kp, vp, tables, seq, (lens - 1).astype(np.int32), B, ks, vs)
    else:
        oracle.kv_append(kn, vn, kp, vp, tables, seq, (lens - 1).astype(np.int32), B)
    host = (lambda t: t.cpu().numpy()) if fp8 else _u16
    for a, b, want in ((k1, k2, kp), (v1, v2, vp)):
        assert np.array_equal(host(a), want) and np.array_equal(host(b), want)
    good = np.array([s for s in range(S) if s not in bad])
    if fp8:
        ref = oracle.paged_decode_fp8(q[good], kp, vp, tables[good], lens[good], B, case.scale,
                                      ks, vs, H)
    else:
        ref = oracle.paged_decode(q[good], kp, vp, tables[good], lens[good], B, case.scale, H)
    assert_parity(bf16_to_f32(fused)[good], ref, "fused, good sequences")
    assert_parity(bf16_to_f32(sep)[good], ref, "separate, good sequences")


def test_a_table_entry_outside_the_pool_with_more_pairs_than_workers():
    """The two-launch form (append kernel, then decode) with broken entries: the
    pools and every output (the broken sequences' too) equal kv_append followed by
    paged_attn_decode bit for bit."""
    import torch

    import paged_kv_cache_280_amd as pkv

    rng = np.random.default_rng(16)
    lens = rng.integers(1, 600, 200).astype(np.int32)
    lens[:3] = [1, 16, 17]
    case, tables, bad = _bad_entry_case(45, lens, Hq=64, Hkv=8)
    S, H, D, B = case.num_seqs, case.num_kv_heads, case.head_dim, case.block_size
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    kn = wl.randn_bf16(rng, (S, H, D))
    vn = wl.randn_bf16(rng, (S, H, D))
    tabs, ld = to_dev_i32(tables), to_dev_i32(lens)
    qd, knd, vnd = to_dev_bf16(q), to_dev_bf16(kn), to_dev_bf16(vn)
    k1, v1 = to_dev_bf16(kp), to_dev_bf16(vp)
    print("bad entries two-launch", flush=True)
    got = pkv.paged_attn_decode_append(qd, knd, vnd, k1, v1, tabs, ld, B, case.scale,
                                       max_context_len=int(lens.max()))
    k2, v2 = to_dev_bf16(kp), to_dev_bf16(vp)
    pkv.kv_append(knd, vnd, k2, v2, tabs, to_dev_i32(np.arange(S, dtype=np.int32)),
                  to_dev_i32(lens - 1), B)
    sep = pkv.paged_attn_decode(qd, k2, v2, tabs, ld, B, case.scale,
                                max_context_len=int(lens.max()))
    torch.cuda.synchronize()
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    assert torch.equal(got.view(torch.int16), sep.view(torch.int16))
    oracle.kv_append(kn, vn, kp, vp, tables, np.arange(S, dtype=np.int32),
                     (lens - 1).astype(np.int32), B)
    assert np.array_equal(_u16(k1), kp) and np.array_equal(_u16(v1), vp)
