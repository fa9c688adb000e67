"""Census of logical blocks on the GPU (exact coverage of the block-table walk,
"PagedAttention (vLLM)", troisinh.com, section "Cơ chế Block Table": position t
of a sequence lives in logical block t / B, and every logical block must be read
exactly once).

With q = 0 every position gets the same weight, so with V one-hot by logical
block (V[t][d] = 1 when d = (t div B) mod D, else 0) each output is an exact share
count/L.  A dropped, doubled or misplaced 16-position tile moves an entry by at
least 8/count, which these tests see (bound: 2 bf16 ulps of count/L, 0 for zero
entries) while the 1e-2 parity gate would not at long contexts.  The keys variant
makes K one-hot by logical block too and puts the query on one dimension, so the
softmax mass lands on the blocks of that dimension only.

The shapes are those of the continuous-batching mix (256 sequences, 13 of them at
32,768 positions, 64 query / 8 KV heads, head_dim 128) and other batches of more
than 64 sequences, whose work split weighs each (sequence, KV head) pair; block
sizes 8, 16 and 32; bf16 and fp8 pools; decode with its append in the fused and
the two-launch form; multi-token attention.  Everything that must not be read
(unreferenced blocks, tails of last blocks, table padding) is NaN."""

import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import bf16_to_f32, to_dev_i32

pytestmark = pytest.mark.gpu

BF16_ONE = 0x3F80     # bf16 1.0 (as int16)
E4M3_ONE = 0x38       # E4M3FN 1.0
MIX_POOL = 6e9        # K+V bytes of the reduced mix pool (the live blocks are ~2 GB)


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (0 where x = 0)."""
    x = np.abs(np.asarray(x, np.float64))
    _, ex = np.frexp(x)
    return np.where(x > 0, np.ldexp(1.0, ex - 8), 0.0)


def census(L, B, D, n=None):
    """Exact shares of the first n (default L) positions of an L-position
    sequence, by dimension (t div B) mod D."""
    n = L if n is None else n
    counts = np.zeros(D, np.float64)
    full, rest = divmod(n, B)
    np.add.at(counts, np.arange(full) % D, B)
    if rest:
        counts[full % D] += rest
    return counts / n if n else counts


def assert_census(got, expect, label):
    err = np.abs(got.astype(np.float64) - expect)
    bad = err > 2 * bf16_ulp(expect)
    assert not bad.any(), "%s: %d entries off, worst %.3g at %s" % (
        label, int(bad.sum()), float(err.max()), np.unravel_index(np.argmax(err), err.shape))


def _live(case):
    """(block id, logical block index) of every referenced (sequence, block)."""
    B = case.block_size
    bs, js = [], []
    for s, L in enumerate(case.context_lens):
        n = -(-int(L) // B)
        bs.append(case.block_tables[s, :n])
        js.append(np.arange(n))
    return np.concatenate(bs).astype(np.int64), np.concatenate(js).astype(np.int64)


def census_pools_bf16(case, keys=False, dev="cuda:0"):
    """bf16 K and V pools on the GPU: V one-hot by logical block; K zero, or also
    one-hot with ``keys``; NaN everywhere that must not be read."""
    import torch

    NB, H, D, B = case.num_blocks, case.num_kv_heads, case.head_dim, case.block_size
    k = torch.full(wl.k_pool_shape(NB, H, D, B), -1, dtype=torch.int16, device=dev)
    v = torch.full(wl.v_pool_shape(NB, H, D, B), -1, dtype=torch.int16, device=dev)
    b, j = _live(case)
    bd = torch.from_numpy(b).to(dev)
    d = torch.from_numpy(j % D).to(dev)
    k[bd] = 0
    v[bd] = 0
    v.permute(0, 3, 1, 2, 4)[bd, d] = BF16_ONE          # [NB][D][Hkv][B/Bt][Bt]
    if keys:
        k.permute(0, 2, 4, 1, 3)[bd, d // 8, d % 8] = BF16_ONE   # [NB][D/8][8][Hkv][B]
    for blk, first in case.tail_slots():
        k[blk, :, :, first:, :] = -1
        wl.poison_v_tail(v, blk, first, -1)
    return k.view(torch.bfloat16), v.view(torch.bfloat16)


def census_pools_fp8(case, dev="cuda:0"):
    """fp8 pools on the GPU: K codes 0, V codes one-hot (E4M3 1.0) by logical
    block, the NaN code everywhere that must not be read."""
    import torch

    NB, H, D, B = case.num_blocks, case.num_kv_heads, case.head_dim, case.block_size
    k = torch.full(wl.k8_pool_shape(NB, H, D, B), wl.E4M3_NAN, dtype=torch.uint8, device=dev)
    v = torch.full(wl.v8_pool_shape(NB, H, D, B), wl.E4M3_NAN, dtype=torch.uint8, device=dev)
    b, j = _live(case)
    bd = torch.from_numpy(b).to(dev)
    d = torch.from_numpy(j % D).to(dev)
    k[bd] = 0
    v[bd] = 0
    # element (b, g, o, d) at [b][g][d%16][o/4][d/16][o%4] -> [NB][d%16][d/16][Hkv][B/4][4]
    v.permute(0, 2, 4, 1, 3, 5)[bd, d % 16, d // 16] = E4M3_ONE
    for blk, first in case.tail_slots():
        k[blk, :, :, first:, :] = wl.E4M3_NAN
        # slots o >= first: o/4 > first/4, or the same quad at o%4 >= first%4
        v[blk, :, :, first // 4 + (1 if first % 4 else 0):] = wl.E4M3_NAN
        if first % 4:
            v[blk, :, :, first // 4, :, first % 4:] = wl.E4M3_NAN
    return k, v


def expected_decode(case):
    S, Hq, D, B = case.num_seqs, case.num_q_heads, case.head_dim, case.block_size
    out = np.zeros((S, Hq, D))
    for s, L in enumerate(case.context_lens):
        out[s] = census(int(L), B, D)[None, :]
    return out


def _decode(case, k, v, fp8=False):
    import torch

    import paged_kv_cache_280_amd as pkv

    q = torch.zeros((case.num_seqs, case.num_q_heads, case.head_dim), dtype=torch.bfloat16,
                    device="cuda:0")
    tabs, lens = to_dev_i32(case.block_tables), to_dev_i32(case.context_lens)
    print("census decode %s S=%d B=%d fp8=%s" % (case.name, case.num_seqs, case.block_size, fp8),
          flush=True)
    if fp8:
        out = pkv.paged_attn_decode_fp8(q, k, v, tabs, lens, case.block_size, case.scale, 1.0, 1.0,
                                        max_context_len=case.max_context_len)
    else:
        out = pkv.paged_attn_decode(q, k, v, tabs, lens, case.block_size, case.scale,
                                    max_context_len=case.max_context_len)
    torch.cuda.synchronize()
    return bf16_to_f32(out)


@pytest.mark.parametrize("B", [8, 16, 32])
def test_census_at_the_mix_shape(B):
    case = wl.case_mix(1, B, pool_bytes=MIX_POOL)
    # the 13 long sequences grew by one position per churn step
    assert case.num_seqs > 64 and (case.context_lens >= 32768).sum() == 13
    k, v = census_pools_bf16(case)
    assert_census(_decode(case, k, v), expected_decode(case), "mix B=%d" % B)


@pytest.mark.parametrize("B", [8, 16, 32])
def test_census_at_the_mix_shape_over_fp8_pools(B):
    case = wl.case_mix(2, B, pool_bytes=MIX_POOL)
    k, v = census_pools_fp8(case)
    assert_census(_decode(case, k, v, fp8=True), expected_decode(case), "mix fp8 B=%d" % B)


def test_census_of_a_batch_past_the_register_held_length_chunks():
    """600 sequences: the plan reads the lengths of sequences past 256 again on
    every pass; long and empty sequences sit in the later chunks too."""
    rng = np.random.default_rng(9)
    lens = rng.integers(0, 900, 600).astype(np.int32)
    lens[[10, 300, 599]] = [20000, 16385, 9000]
    lens[[5, 400]] = 0
    case = wl.case_random(70, 600, 16, 2, 128, 16, lens)
    k, v = census_pools_bf16(case)
    assert_census(_decode(case, k, v), expected_decode(case), "600 seqs")


@pytest.mark.parametrize("B", [8, 16, 32])
def test_census_through_the_keys_at_the_mix_shape(B):
    """K and V one-hot by logical block, q[s] = alpha * e_j(s) with alpha * scale
    about 30: the weight of a position is e^(alpha*scale) on the blocks of dimension
    j(s) and 1 elsewhere, so the output is (up to e^-30 terms) e_j(s); a block
    gathered from the wrong place moves mass to another dimension."""
    import torch

    import paged_kv_cache_280_amd as pkv

    case = wl.case_mix(3, B, pool_bytes=MIX_POOL)
    S, Hq, D = case.num_seqs, case.num_q_heads, case.head_dim
    k, v = census_pools_bf16(case, keys=True)
    nblk = -(-case.context_lens.astype(np.int64) // B)
    jsel = np.array([s % max(1, min(int(n), D)) for s, n in enumerate(nblk)])
    alpha = float(wl.f32_from_bf16(wl.bf16_from_f32(np.float32(30.0 / case.scale))))
    qh = np.zeros((S, Hq, D), np.float32)
    qh[np.arange(S), :, jsel] = alpha
    q = torch.from_numpy(wl.bf16_from_f32(qh).reshape(qh.shape).view(np.int16)).to(
        "cuda:0").view(torch.bfloat16)
    print("census keys B=%d" % B, flush=True)
    out = pkv.paged_attn_decode(q, k, v, to_dev_i32(case.block_tables),
                                to_dev_i32(case.context_lens), B, case.scale,
                                max_context_len=case.max_context_len)
    torch.cuda.synchronize()
    got = bf16_to_f32(out)
    w = np.exp(np.float64(alpha) * np.float64(case.scale))
    for s, L in enumerate(case.context_lens):
        counts = census(int(L), B, D) * int(L)
        wd = np.where(np.arange(D) == jsel[s], w, 1.0)
        expect = counts * wd / (counts * wd).sum() if L > 0 else counts
        assert_census(got[s], np.broadcast_to(expect, (Hq, D)), "keys B=%d s=%d" % (B, s))


def _append_census(case, lens):
    """Decode with append over census pools: the newest position's slot is NaN
    before the call and its rows come from k_new = 0, v_new one-hot."""
    import torch

    import paged_kv_cache_280_amd as pkv

    S, Hq, Hkv, D, B = case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim, \
        case.block_size
    k, v = census_pools_bf16(case)
    kk, vv = k.view(torch.int16), v.view(torch.int16)
    bt = wl.v_half(B)
    vn = torch.zeros((S, Hkv, D), dtype=torch.int16, device="cuda:0")
    for s, L in enumerate(lens):
        if L < 1:
            continue
        p = int(L) - 1
        blk, o = int(case.block_tables[s, p // B]), p % B
        kk[blk, :, :, o, :] = -1
        vv[blk, :, o // bt, :, o % bt] = -1
        vn[s, :, (p // B) % D] = BF16_ONE
    kn = torch.zeros((S, Hkv, D), dtype=torch.bfloat16, device="cuda:0")
    q = torch.zeros((S, Hq, D), dtype=torch.bfloat16, device="cuda:0")
    tabs = to_dev_i32(case.block_tables)
    print("census decode+append S=%d B=%d" % (S, B), flush=True)
    out = pkv.paged_attn_decode_append(q, kn, vn.view(torch.bfloat16), k, v, tabs, to_dev_i32(lens),
                                       B, case.scale, max_context_len=int(lens.max()))
    torch.cuda.synchronize()
    got = bf16_to_f32(out)
    # every newest slot now holds the new rows
    for s, L in enumerate(lens):
        if L < 1:
            continue
        p = int(L) - 1
        blk, o = int(case.block_tables[s, p // B]), p % B
        assert (kk[blk, :, :, o, :] == 0).all()
        assert torch.equal(vv[blk, :, o // bt, :, o % bt], vn[s])
    return got


def test_census_of_decode_with_append_fused():
    """80 sequences x 8 KV heads = 640 pairs, no more than the workers: each pair's
    newest position is folded in by the worker holding its last tile, with the
    weighted split of batches over 64 sequences."""
    rng = np.random.default_rng(21)
    lens = wl.mix_lengths(rng, n=80, n_long=4)
    lens[:4] = [1, 16, 17, 0]
    case = wl.case_random(71, 80, 64, 8, 128, 16, lens)
    assert_census(_append_census(case, lens), expected_decode(case), "decode+append fused")


@pytest.mark.parametrize("B", [8, 16, 32])
def test_census_of_decode_with_append_at_the_mix_shape(B):
    """2,048 pairs, more than the workers: the call appends first, then decodes."""
    case = wl.case_mix(4, B, pool_bytes=MIX_POOL)
    lens = case.context_lens
    assert_census(_append_census(case, lens), expected_decode(case), "decode+append mix B=%d" % B)


@pytest.mark.parametrize("T", [4, 12, 24, 40])
def test_census_of_multi_token_attention_over_many_sequences(T):
    """100 sequences, G = 4, T query tokens each in chunks of 8 (12: two chunk waves
    per slot; 24: three of a launch of four; 40: a launch of four, then one): query
    token i of an L-position sequence sees positions 0 .. L-T+i."""
    import torch

    import paged_kv_cache_280_amd as pkv

    rng = np.random.default_rng(30 + T)
    S, Hq, Hkv, D, B = 100, 32, 8, 128, 16
    lens = wl.mix_lengths(rng, n=S, n_long=5, long_len=8192)
    lens = np.maximum(lens, 1)
    qlens = np.minimum(np.full(S, T, np.int32), lens).astype(np.int32)
    qlens[7] = 0
    case = wl.case_random(72 + T, S, Hq, Hkv, D, B, lens)
    k, v = census_pools_bf16(case)
    q = torch.zeros((S, T, Hq, D), dtype=torch.bfloat16, device="cuda:0")
    print("census multi T=%d" % T, flush=True)
    out = pkv.paged_attn_multi(q, k, v, to_dev_i32(case.block_tables), to_dev_i32(lens),
                               to_dev_i32(qlens), B, case.scale, max_context_len=int(lens.max()))
    torch.cuda.synchronize()
    got = bf16_to_f32(out)
    expect = np.zeros((S, T, Hq, D))
    for s, L in enumerate(lens):
        for i in range(int(qlens[s])):
            expect[s, i] = census(int(L), B, D, n=int(L) - int(qlens[s]) + i + 1)[None, :]
    assert_census(got, expect, "multi T=%d" % T)
