"""The library's calls captured in a HIP graph (through torch's CUDA-graph API)
and replayed several times, with new inputs written into the captured buffers and
eager work between replays: every replay must match the oracle (the workspace and
the merge's descriptors are rewritten by each replay, never carried over)."""

import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import assert_parity, bf16_to_f32

pytestmark = pytest.mark.gpu


def test_append_and_decode_replayed_from_a_graph():
    import torch

    import paged_kv_cache_280_amd as pkv

    dev = torch.device("cuda:0")
    case = wl.case_chat(seed=5, num_seqs=12)
    S, Hq, H, D, B = case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size
    kp, vp = wl.host_pools(case)
    kd = torch.from_numpy(kp.view(np.int16)).to(dev).view(torch.bfloat16)
    vd = torch.from_numpy(vp.view(np.int16)).to(dev).view(torch.bfloat16)
    tabs = torch.from_numpy(case.block_tables).to(dev)
    lens = torch.from_numpy(case.context_lens).to(dev)
    q = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(q)
    kn = torch.empty((S, H, D), dtype=torch.bfloat16, device=dev)
    vn = torch.empty_like(kn)
    seq = torch.arange(S, dtype=torch.int32, device=dev)
    pos = (lens - 1).to(torch.int32)        # each step rewrites the newest position
    mx = int(case.context_lens.max())
    ws = pkv.new_workspace(S, Hq, H, D, B, mx, dev)

    def step():
        pkv.kv_append(kn, vn, kd, vd, tabs, seq, pos, B)
        pkv.paged_attn_decode(q, kd, vd, tabs, lens, B, case.scale, out, workspace=ws,
                              max_context_len=mx)

    rng = np.random.default_rng(0)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()                               # warm-up on a side stream, as capture requires
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for replay in range(4):
        qh = wl.randn_bf16(rng, (S, Hq, D))
        knh, vnh = wl.randn_bf16(rng, (S, H, D)), wl.randn_bf16(rng, (S, H, D))
        q.copy_(torch.from_numpy(qh.view(np.int16)).to(dev).view(torch.bfloat16))
        kn.copy_(torch.from_numpy(knh.view(np.int16)).to(dev).view(torch.bfloat16))
        vn.copy_(torch.from_numpy(vnh.view(np.int16)).to(dev).view(torch.bfloat16))
        out.fill_(float("nan"))              # eager work between replays
        ws.fill_(0xA5)
        graph.replay()
        torch.cuda.synchronize()
        oracle.kv_append(knh, vnh, kp, vp, case.block_tables, np.arange(S, dtype=np.int32),
                         (case.context_lens - 1).astype(np.int32), B)
        assert np.array_equal(kd.view(torch.int16).cpu().numpy().view(np.uint16), kp)
        ref = oracle.paged_decode(qh, kp, vp, case.block_tables, case.context_lens, B,
                                  case.scale, H)
        assert_parity(bf16_to_f32(out), ref, "graph replay %d" % replay)


def test_copy_blocks_replayed_from_a_graph():
    import torch

    import paged_kv_cache_280_amd as pkv

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(1)
    nb, H, D, B = 40, 4, 128, 16
    k = rng.integers(0, 65536, size=wl.k_pool_shape(nb, H, D, B), dtype=np.uint16)
    v = rng.integers(0, 65536, size=wl.v_pool_shape(nb, H, D, B), dtype=np.uint16)
    kd = torch.from_numpy(k.view(np.int16)).to(dev)
    vd = torch.from_numpy(v.view(np.int16)).to(dev)
    p0 = np.arange(10, dtype=np.int32).reshape(5, 2)
    pairs = torch.from_numpy(p0).to(dev)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        pkv.copy_blocks([kd], [vd], pairs)   # warm-up: a real copy, mirrored on the host
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    oracle.copy_blocks([k], [v], p0)
    with torch.cuda.graph(graph):
        pkv.copy_blocks([kd], [vd], pairs)
    for replay in range(3):
        ids = rng.permutation(nb)
        p = np.stack([ids[:5], ids[5:10]], axis=1).astype(np.int32)
        pairs.copy_(torch.from_numpy(p).to(dev))
        graph.replay()
        torch.cuda.synchronize()
        oracle.copy_blocks([k], [v], p)
        assert np.array_equal(kd.cpu().numpy().view(np.uint16), k)
        assert np.array_equal(vd.cpu().numpy().view(np.uint16), v)


def test_multi_token_chunk_waves_replayed_from_a_graph():
    """A 40-token multi-token call (a launch of four chunk waves, then one) captured
    once and replayed with new queries and eager work between replays."""
    import torch

    import paged_kv_cache_280_amd as pkv

    dev = torch.device("cuda:0")
    S, Hq, H, D, B, Q = 6, 32, 8, 128, 16, 40
    lens = np.array([3000, 2600, 40, 41, 900, 2048], np.int32)
    case = wl.case_random(123, S, Hq, H, D, B, lens)
    kp, vp = wl.host_pools(case, poison=False)
    kd = torch.from_numpy(kp.view(np.int16)).to(dev).view(torch.bfloat16)
    vd = torch.from_numpy(vp.view(np.int16)).to(dev).view(torch.bfloat16)
    tabs = torch.from_numpy(case.block_tables).to(dev)
    ld = torch.from_numpy(lens).to(dev)
    qlens = np.minimum(np.full(S, Q, np.int32), lens)
    qld = torch.from_numpy(qlens).to(dev)
    q = torch.empty((S, Q, Hq, D), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(q)
    mx = int(lens.max())
    ws = pkv.new_multi_workspace(S, Hq, H, D, B, mx, Q, dev)

    def step():
        pkv.paged_attn_multi(q, kd, vd, tabs, ld, qld, B, case.scale, out, max_context_len=mx,
                             workspace=ws)

    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    rng = np.random.default_rng(5)
    for replay in range(3):
        qh = wl.randn_bf16(rng, (S, Q, Hq, D))
        q.copy_(torch.from_numpy(qh.view(np.int16)).to(dev).view(torch.bfloat16))
        out.fill_(float("nan"))
        ws.fill_(0xA5)
        graph.replay()
        torch.cuda.synchronize()
        ref = oracle.paged_attn_multi(qh, kp, vp, case.block_tables, lens, qlens, B, case.scale, H)
        assert_parity(bf16_to_f32(out), ref, "multi graph replay %d" % replay)
