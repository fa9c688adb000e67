"""GPU multi-token paged attention (causal, several query tokens per sequence)
against the oracle: one and two MFMA column tiles, several runs of query tokens
per call, empty and partial query sets, sequences whose whole context is the
query, and equality with decode at one token."""

import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import assert_parity, bf16_to_f32, to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu


def _q_with_nan_padding(rng, S, Q, Hq, D, qlens):
    """q rows past a sequence's query tokens are NaN: the kernel must not read them."""
    q = wl.randn_bf16(rng, (S, Q, Hq, D))
    for s, T in enumerate(qlens):
        q[s, T:] = wl.BF16_NAN
    return q


def _run(case, q, kp, vp, qlens, max_context_len=None):
    import torch

    import paged_kv_cache_280_amd as pkv

    lens = case.context_lens
    if max_context_len is None:
        max_context_len = int(lens.max()) if len(lens) else 0
    out = pkv.paged_attn_multi(to_dev_bf16(q), to_dev_bf16(kp), to_dev_bf16(vp),
                               to_dev_i32(case.block_tables), to_dev_i32(lens),
                               to_dev_i32(qlens), case.block_size, case.scale,
                               max_context_len=max_context_len)
    torch.cuda.synchronize()
    return bf16_to_f32(out)


# (head_dim, block_size, q heads, kv heads, max query tokens): one column tile,
# two column tiles, several runs of tokens per call, groups of 1 .. 16
SHAPES = [
    (128, 16, 32, 8, 4),     # 16 rows, one run
    (128, 16, 32, 8, 8),     # 32 rows: two column tiles
    (128, 16, 32, 8, 13),    # runs of 8 and 5 tokens
    (64, 8, 8, 8, 40),       # group 1: runs of 32 and 8 tokens
    (128, 32, 16, 2, 3),     # group 8: 24 rows
    (128, 16, 16, 1, 3),     # group 16: runs of 2 and 1 tokens
    (64, 32, 4, 2, 6),       # group 2: 12 rows
    (128, 16, 32, 8, 24),    # three chunks of 8: a launch of four chunk waves, one empty
    (128, 32, 32, 8, 36),    # five chunks: four chunk waves, then one (the last of 4 tokens)
    (64, 16, 16, 4, 64),     # eight chunks of 8: two launches of four chunk waves
]


@pytest.mark.parametrize("long_ctx", [False, True])
@pytest.mark.parametrize("D,B,Hq,Hkv,Q", SHAPES)
def test_multi_matches_the_oracle(D, B, Hq, Hkv, Q, long_ctx):
    """Contexts up to 2,000 positions (16-row chunks), and with one of 2,600
    positions (32-row chunks)."""
    rng = np.random.default_rng(D * 7 + B * 3 + Hq + Q + long_ctx)
    lens = np.array([Q + 3, 5 * B + 1, Q, 0, 40, 700, 2600 if long_ctx else 2000], np.int32)
    qlens = np.array([Q, 1, Q, 0, min(7, Q), Q // 2, Q - 1], np.int32)
    qlens = np.minimum(qlens, lens)
    case = wl.case_random(D + Q, len(lens), Hq, Hkv, D, B, lens)
    kp, vp = wl.host_pools(case)
    q = _q_with_nan_padding(rng, len(lens), Q, Hq, D, qlens)
    got = _run(case, q, kp, vp, qlens)
    ref = oracle.paged_attn_multi(q, kp, vp, case.block_tables, lens, qlens, B, case.scale, Hkv)
    for s, T in enumerate(qlens):
        assert not got[s, T:].any(), "rows past the query tokens must be zero (seq %d)" % s
    assert_parity(got, ref, "multi D=%d B=%d G=%d Q=%d long=%d" % (D, B, Hq // Hkv, Q, long_ctx))


@pytest.mark.parametrize("B", [8, 16, 32])
def test_multi_with_one_token_is_decode_bit_for_bit(B):
    import torch

    import paged_kv_cache_280_amd as pkv

    case = wl.case_chat(seed=B, num_seqs=24, block_size=B)
    kp, vp = wl.host_pools(case)
    q = wl.host_q(case)
    S = case.num_seqs
    args = (to_dev_bf16(kp), to_dev_bf16(vp), to_dev_i32(case.block_tables),
            to_dev_i32(case.context_lens))
    mx = int(case.context_lens.max())
    dec = pkv.paged_attn_decode(to_dev_bf16(q), *args, B, case.scale, max_context_len=mx)
    multi = pkv.paged_attn_multi(to_dev_bf16(q[:, None]), *args, to_dev_i32(np.ones(S, np.int32)),
                                 B, case.scale, max_context_len=mx)
    torch.cuda.synchronize()
    assert torch.equal(dec.view(torch.int16), multi[:, 0].contiguous().view(torch.int16))


def test_multi_with_no_query_tokens():
    import torch

    import paged_kv_cache_280_amd as pkv

    case = wl.case_random(11, 3, 8, 2, 128, 16, [50, 0, 17])
    kp, vp = wl.host_pools(case)
    args = (to_dev_bf16(kp), to_dev_bf16(vp), to_dev_i32(case.block_tables),
            to_dev_i32(case.context_lens))
    # every query set empty: all rows zero (the output starts as NaN)
    out = torch.full((3, 5, 8, 128), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    pkv.paged_attn_multi(torch.zeros_like(out), *args, to_dev_i32(np.zeros(3, np.int32)), 16,
                         case.scale, out=out, max_context_len=50)
    torch.cuda.synchronize()
    assert not out.float().abs().sum().item() and not out.isnan().any().item()
    # max_query_len = 0 is a no-op
    empty = torch.zeros((3, 0, 8, 128), dtype=torch.bfloat16, device="cuda:0")
    pkv.paged_attn_multi(empty, *args, to_dev_i32(np.zeros(3, np.int32)), 16, case.scale,
                         max_context_len=50)
    torch.cuda.synchronize()


def test_multi_prefill_chunks_add_up_to_whole_prefill():
    """Prefill of a 300-token prompt in chunks of 64 (each chunk's K/V appended
    before its attention) gives the same rows as the oracle's single pass over
    all 300 query tokens."""
    import torch

    import paged_kv_cache_280_amd as pkv

    rng = np.random.default_rng(3)
    L, chunk, Hq, Hkv, D, B = 300, 64, 32, 8, 128, 16
    case = wl.case_random(5, 1, Hq, Hkv, D, B, [L])
    kp, vp = wl.host_pools(case)
    q_all = wl.randn_bf16(rng, (1, L, Hq, D))
    ref = oracle.paged_attn_multi(q_all, kp, vp, case.block_tables, case.context_lens,
                                  np.array([L], np.int32), B, case.scale, Hkv)
    kd, vd, td = to_dev_bf16(kp), to_dev_bf16(vp), to_dev_i32(case.block_tables)
    rows = []
    for start in range(0, L, chunk):
        T = min(chunk, L - start)
        q = np.ascontiguousarray(q_all[:, start:start + T])
        out = pkv.paged_attn_multi(to_dev_bf16(q), kd, vd, td,
                                   to_dev_i32(np.array([start + T], np.int32)),
                                   to_dev_i32(np.array([T], np.int32)), B, case.scale,
                                   max_context_len=start + T)
        torch.cuda.synchronize()
        rows.append(bf16_to_f32(out))
    assert_parity(np.concatenate(rows, axis=1), ref, "chunked prefill 300/64")


@pytest.mark.parametrize("Q", [4, 16, 24])
def test_multi_verify_at_long_context_sampled(Q):
    """Speculative verification at the long-context size: 8 sequences x 16,000
    positions, Q query tokens each (the last Q positions; 16 and 24 run as two and
    three chunk waves per slot over pairs split across many slots), one layer's
    pools; every output is checked against the oracle."""
    case = wl.case_long(seed=1, num_layers=1)
    rng = np.random.default_rng(8)
    kp, vp = wl.host_pools(case, poison=False)
    S = case.num_seqs
    qlens = np.full(S, Q, np.int32)
    q = wl.randn_bf16(rng, (S, Q, case.num_q_heads, case.head_dim))
    got = _run(case, q, kp, vp, qlens)
    ref = oracle.paged_attn_multi(q, kp, vp, case.block_tables, case.context_lens, qlens,
                                  case.block_size, case.scale, case.num_kv_heads)
    assert_parity(got, ref, "verify 8x16000 Q=%d" % Q)


def test_multi_chunk_waves_give_the_same_bits_on_every_call():
    """Split pairs over chunk waves (16 and 32 query tokens, 8 x 3,000 positions):
    the merge folds each pair's records in a fixed order, so repeated calls agree
    bit for bit."""
    rng = np.random.default_rng(77)
    lens = np.full(8, 3000, np.int32)
    case = wl.case_random(77, 8, 32, 8, 128, 16, lens)
    kp, vp = wl.host_pools(case, poison=False)
    for Q in (16, 32):
        qlens = np.full(8, Q, np.int32)
        q = wl.randn_bf16(rng, (8, Q, 32, 128))
        first = _run(case, q, kp, vp, qlens)
        for _ in range(2):
            assert np.array_equal(_run(case, q, kp, vp, qlens).view(np.uint32),
                                  first.view(np.uint32)), "Q=%d" % Q
        ref = oracle.paged_attn_multi(q, kp, vp, case.block_tables, lens, qlens, 16, case.scale, 8)
        assert_parity(first, ref, "repeat Q=%d" % Q)


@pytest.mark.parametrize("Q", [16, 24, 40])
def test_multi_chunk_waves_in_pair_mode(Q):
    """Short contexts (at most 256 positions: one worker per (sequence, KV head)
    pair, no split) with 2, 3 and 5 chunks of query tokens per sequence."""
    rng = np.random.default_rng(40 + Q)
    lens = np.array([Q, 256, 17, 0, 100, Q + 1, 200, 64], np.int32)
    qlens = np.minimum(np.array([Q, Q, 9, 0, Q - 3, 1, Q // 2, Q], np.int32), lens)
    case = wl.case_random(90 + Q, len(lens), 32, 8, 128, 16, lens)
    kp, vp = wl.host_pools(case)
    q = _q_with_nan_padding(rng, len(lens), Q, 32, 128, qlens)
    got = _run(case, q, kp, vp, qlens)
    ref = oracle.paged_attn_multi(q, kp, vp, case.block_tables, lens, qlens, 16, case.scale, 8)
    for s, T in enumerate(qlens):
        assert not got[s, T:].any(), "rows past the query tokens must be zero (seq %d)" % s
    assert_parity(got, ref, "multi pair mode Q=%d" % Q)


# (head_dim, block_size, q heads, kv heads, max query tokens) over fp8 pools
FP8_SHAPES = [(128, 16, 32, 8, 4), (128, 16, 32, 8, 8), (64, 8, 8, 8, 40), (128, 32, 16, 2, 3),
              (128, 16, 32, 8, 24)]


@pytest.mark.parametrize("long_ctx", [False, True])
@pytest.mark.parametrize("D,B,Hq,Hkv,Q", FP8_SHAPES)
def test_multi_over_fp8_pools_matches_the_oracle(D, B, Hq, Hkv, Q, long_ctx):
    import torch

    import paged_kv_cache_280_amd as pkv

    rng = np.random.default_rng(D + B + Q + 100 + long_ctx)
    lens = np.array([Q + 3, 5 * B + 1, Q, 0, 700, 2600 if long_ctx else 2000], np.int32)
    qlens = np.minimum(np.array([Q, 1, Q, 0, Q // 2, Q - 1], np.int32), lens)
    case = wl.case_random(D + Q + 7, len(lens), Hq, Hkv, D, B, lens)
    ks, vs = 0.043, 0.057
    kp8, vp8 = wl.host_pools_fp8(case, ks, vs)
    q = _q_with_nan_padding(rng, len(lens), Q, Hq, D, qlens)
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    out = pkv.paged_attn_multi(to_dev_bf16(q), u8(kp8), u8(vp8), to_dev_i32(case.block_tables),
                               to_dev_i32(lens), to_dev_i32(qlens), B, case.scale,
                               max_context_len=int(lens.max()), k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    got = bf16_to_f32(out)
    ref = oracle.paged_attn_multi_fp8(q, kp8, vp8, case.block_tables, lens, qlens, B, case.scale,
                                      ks, vs, Hkv)
    for s, T in enumerate(qlens):
        assert not got[s, T:].any()
    assert_parity(got, ref, "multi fp8 D=%d B=%d G=%d Q=%d long=%d" % (D, B, Hq // Hkv, Q, long_ctx))


def test_multi_over_fp8_pools_with_one_token_is_fp8_decode_bit_for_bit():
    import torch

    import paged_kv_cache_280_amd as pkv

    case = wl.case_chat(seed=12, num_seqs=20)
    ks, vs = 1 / 16, 1 / 16
    kp8, vp8 = wl.host_pools_fp8(case, ks, vs)
    q = wl.host_q(case)
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    kd, vd = u8(kp8), u8(vp8)
    tabs, lens = to_dev_i32(case.block_tables), to_dev_i32(case.context_lens)
    mx = int(case.context_lens.max())
    dec = pkv.paged_attn_decode_fp8(to_dev_bf16(q), kd, vd, tabs, lens, 16, case.scale, ks, vs,
                                    max_context_len=mx)
    multi = pkv.paged_attn_multi(to_dev_bf16(q[:, None]), kd, vd, tabs, lens,
                                 to_dev_i32(np.ones(case.num_seqs, np.int32)), 16, case.scale,
                                 max_context_len=mx, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    assert torch.equal(dec.view(torch.int16), multi[:, 0].contiguous().view(torch.int16))
