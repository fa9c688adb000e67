"""Pins for the CPU oracle: facts fixed by the pages or by mathematics, none of
which re-types the oracle's own loops.

Page references: P1 = "PagedAttention (vLLM) - Virtual memory cho AI"
(troisinh.com); P2 = the aiwiki.vn article on KV cache and PagedAttention.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from einops import rearrange

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")


def pages():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Brute force: contiguous attention via torch's fp64 scaled_dot_product_attention
# ---------------------------------------------------------------------------

def brute_force(case, q, kp, vp):
    """Gather every (seq, kv head) into contiguous [L][D] rows with einops and
    run the library routine in float64.  Returns float64 [S][Hq][D]."""
    kl = rearrange(wl.f32_from_bf16(kp).astype(np.float64), "n h c b e -> n h b (c e)")
    vl = rearrange(wl.f32_from_bf16(vp).astype(np.float64), "n h t d b -> n h (t b) d")
    qf = wl.f32_from_bf16(q).astype(np.float64)
    S, Hq, D = q.shape
    G = Hq // case.num_kv_heads
    out = np.zeros((S, Hq, D))
    for s in range(S):
        L = int(case.context_lens[s])
        if L == 0:
            continue
        nblk = -(-L // case.block_size)
        ids = case.block_tables[s, :nblk]
        for h in range(Hq):
            g = h // G
            K = kl[ids, g].reshape(-1, D)[:L]
            V = vl[ids, g].reshape(-1, D)[:L]
            o = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qf[s, h]).view(1, 1, 1, D), torch.from_numpy(K).view(1, 1, L, D),
                torch.from_numpy(V).view(1, 1, L, D), scale=case.scale)
            out[s, h] = o.view(D).numpy()
    return out


def run(oracle_lib, case, q, kp, vp, precision="f32"):
    return oracle_lib.paged_decode(q, kp, vp, case.block_tables, case.context_lens,
                                   case.block_size, case.scale, case.num_kv_heads, precision)


SHAPES = [
    # (S, Hq, Hkv, D, B, lens)
    (1, 4, 4, 64, 16, [100]),
    (3, 8, 2, 128, 16, [1, 17, 40]),
    (2, 8, 1, 64, 8, [9, 33]),
    (2, 4, 2, 128, 32, [31, 65]),
    (4, 6, 3, 64, 16, [16, 15, 2, 48]),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_oracle_matches_fp64_library_attention(oracle_lib, shape):
    S, Hq, Hkv, D, B, lens = shape
    case = wl.case_random(7, S, Hq, Hkv, D, B, lens)
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    got = run(oracle_lib, case, q, kp, vp)
    ref = brute_force(case, q, kp, vp)
    assert np.isfinite(got).all()
    assert np.abs(got - ref).max() <= 1e-5
    got64 = run(oracle_lib, case, q, kp, vp, "f64")
    assert np.abs(got64 - ref).max() <= 1e-12


def test_tiny_config_against_brute_force(oracle_lib):
    case = wl.case_tiny(0)
    assert case.block_tables[0, :7].tolist() != list(range(7))  # scattered placement
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    got = run(oracle_lib, case, q, kp, vp)
    ref = brute_force(case, q, kp, vp)
    assert np.abs(got - ref).max() <= 1e-5


def test_block_counts_match_pages():
    p = pages()
    r = p["request_100_tokens"]
    B = p["block_size_default"]["value"]
    assert -(-r["tokens"] // B) == r["blocks"] and r["blocks"] * B == r["slots"]
    r = p["request_4096_tokens"]
    assert -(-r["tokens"] // B) == r["blocks"]
    # the tiny workload is the pages' 100-token request
    case = wl.case_tiny(0)
    assert case.context_lens[0] == 100 and len(case.used_blocks()) == 7
    assert case.tail_slots() == [(int(case.block_tables[0, 6]), 4)]  # last block 4/16 full


def test_waste_only_in_last_block():
    for lens in ([100], list(range(1, 200, 7)), [16000], [32768, 1, 4095]):
        for B in (8, 16, 32):
            for L in lens:
                waste = -(-L // B) * B - L
                assert 0 <= waste <= B - 1


def test_kv_memory_formula_and_the_pages_halved_example():
    from paged_kv_cache_280_amd.accounting import kv_cache_bytes

    ex = pages()["kv_memory_example"]
    total = kv_cache_bytes(ex["layers"], ex["tokens"], ex["kv_heads"], ex["head_size"],
                           ex["bytes_per_element"])
    # the formula as printed: 2 x 32 x 16000 x 8 x 128 x 2
    assert total == 2_097_152_000
    # the printed "about 1.05 GB" is one of K or V, i.e. half the formula's value
    assert abs(total / 2 / 1e9 - ex["printed_gb"]) < 0.005
    assert abs(total / 1e9 - ex["printed_gb"]) > 1.0


def test_permutation_of_physical_blocks_is_bit_exact(oracle_lib):
    case = wl.case_random(3, 3, 8, 2, 128, 16, [5, 70, 33])
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    base = run(oracle_lib, case, q, kp, vp)
    rng = np.random.default_rng(11)
    perm = rng.permutation(case.num_blocks)          # new id of old block b = perm[b]
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    case.block_tables = perm[case.block_tables].astype(np.int32)
    again = run(oracle_lib, case, q, kp2, vp2)
    assert np.array_equal(base.view(np.uint32), again.view(np.uint32))


def test_softmax_weights_sum_to_one(oracle_lib):
    case = wl.case_random(5, 2, 4, 2, 64, 16, [1, 1000])
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    for s in range(2):
        L = int(case.context_lens[s])
        for h in range(4):
            _, p = oracle_lib.paged_decode_probs(q, kp, vp, case.block_tables, case.context_lens,
                                                 case.block_size, case.scale, case.num_kv_heads,
                                                 s, h)
            assert p.shape == (L,) and (p >= 0).all()
            assert abs(float(p.astype(np.float64).sum()) - 1.0) <= L * 2.0 ** -24


def test_q_zero_gives_mean_of_values(oracle_lib):
    case = wl.case_random(9, 2, 4, 2, 64, 8, [37, 12])
    q = np.zeros((2, 4, 64), np.uint16)  # +0.0
    kp, vp = wl.host_pools(case)
    got = run(oracle_lib, case, q, kp, vp, "f64")
    vl = rearrange(wl.f32_from_bf16(vp).astype(np.float64), "n h t d b -> n h (t b) d")
    for s in range(2):
        L = int(case.context_lens[s])
        ids = case.block_tables[s, : -(-L // 8)]
        for h in range(4):
            rows = vl[ids, h // 2].reshape(-1, 64)[:L]
            assert np.abs(got[s, h] - rows.mean(axis=0)).max() <= 1e-13


def test_single_token_returns_its_value_exactly(oracle_lib):
    case = wl.case_random(2, 3, 4, 4, 128, 16, [1, 1, 1])
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    got = run(oracle_lib, case, q, kp, vp)
    vl = rearrange(wl.f32_from_bf16(vp), "n h t d b -> n h (t b) d")
    for s in range(3):
        b = case.block_tables[s, 0]
        for h in range(4):
            assert np.array_equal(got[s, h], vl[b, h, 0])


def test_constant_values_give_constant_output(oracle_lib):
    case = wl.case_random(4, 2, 8, 2, 64, 16, [300, 7])
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    vp[...] = wl.bf16_from_f32(np.ones(1, np.float32))[0]
    got = run(oracle_lib, case, q, kp, vp)
    assert np.abs(got - 1.0).max() <= 300 * 2.0 ** -24


def test_argmax_limit(oracle_lib):
    # q = alpha * k_j with large alpha puts all weight on token j.
    case = wl.case_random(6, 1, 1, 1, 64, 16, [50])
    kp, vp = wl.host_pools(case)
    kl = rearrange(wl.f32_from_bf16(kp), "n h c b e -> n h b (c e)")
    vl = rearrange(wl.f32_from_bf16(vp), "n h t d b -> n h (t b) d")
    j = 23
    b, o = case.block_tables[0, j // 16], j % 16
    q = wl.bf16_from_f32(kl[b, 0, o] * 4.0).reshape(1, 1, 64)
    got = run(oracle_lib, case, q, kp, vp, "f64")
    assert np.abs(got[0, 0] - vl[b, 0, o]).max() <= 1e-6


def test_gqa_equals_expanded_mha(oracle_lib):
    case = wl.case_random(8, 2, 8, 2, 64, 16, [45, 20])
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    gqa = run(oracle_lib, case, q, kp, vp)
    # duplicate each KV head G = 4 times: head h of the MHA pool is KV head h // 4
    kp_m = np.ascontiguousarray(np.repeat(kp, 4, axis=1))
    vp_m = np.ascontiguousarray(np.repeat(vp, 4, axis=1))
    case.num_kv_heads = 8
    mha = run(oracle_lib, case, q, kp_m, vp_m)
    assert np.array_equal(gqa.view(np.uint32), mha.view(np.uint32))


@pytest.mark.parametrize("B", [8, 16, 32])
def test_census_of_logical_blocks(oracle_lib, B):
    """q = 0 and V one-hot at d = (logical block) mod D: out[d] = share of tokens
    whose logical block is congruent to d.  A dropped, repeated or misplaced
    block moves an entry by B/L."""
    D = 64
    lens = [1, B, 5 * B + 3, 70 * B + 1]
    case = wl.case_random(12, len(lens), 2, 1, D, B, lens)
    q = np.zeros((len(lens), 2, D), np.uint16)
    kp, vp = wl.host_pools(case)
    vl = np.zeros((case.num_blocks, 1, B, D), np.float32)
    for s, L in enumerate(lens):
        for j in range(-(-L // B)):
            vl[case.block_tables[s, j], 0, :, j % D] = 1.0
    vp = wl.v_to_pool(wl.bf16_from_f32(vl).reshape(vl.shape))
    wl.poison_host_pools(case, kp, vp)
    got = run(oracle_lib, case, q, kp, vp)
    for s, L in enumerate(lens):
        expect = np.zeros(D)
        for t in range(L):
            expect[(t // B) % D] += 1
        expect /= L
        assert np.abs(got[s, 0] - expect).max() <= 4 * L * 2.0 ** -24
        assert np.array_equal(got[s, 0], got[s, 1])


def test_census_through_the_keys(oracle_lib):
    """K one-hot at d = (logical block) mod D and q = a * e_j: the weight
    concentrates on blocks whose index is congruent to j, so with the one-hot V
    the output is close to e_j.  A K-gather error moves mass to another d."""
    D, B = 64, 16
    L = 40 * B
    case = wl.case_random(13, 1, 1, 1, D, B, [L])
    kl = np.zeros((case.num_blocks, 1, B, D), np.float32)
    vl = np.zeros_like(kl)
    for j in range(L // B):
        kl[case.block_tables[0, j], 0, :, j % D] = 1.0
        vl[case.block_tables[0, j], 0, :, j % D] = 1.0
    kp = wl.k_to_pool(wl.bf16_from_f32(kl).reshape(kl.shape))
    vp = wl.v_to_pool(wl.bf16_from_f32(vl).reshape(vl.shape))
    wl.poison_host_pools(case, kp, vp)
    for j in (0, 5, 39):
        qv = np.zeros((1, 1, D), np.float32)
        qv[0, 0, j] = 30.0 / case.scale
        got = run(oracle_lib, case, wl.bf16_from_f32(qv).reshape(1, 1, D), kp, vp)
        assert got[0, 0, j] > 1 - 1e-9 * L and abs(float(got[0, 0].sum()) - 1) < 1e-6


def test_never_reads_tail_padding_or_unused_blocks(oracle_lib):
    case = wl.case_random(14, 3, 4, 2, 64, 16, [3, 16, 50])
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case, poison=False)
    clean = run(oracle_lib, case, q, kp, vp)
    wl.poison_host_pools(case, kp, vp)
    assert np.isnan(wl.f32_from_bf16(kp)).any()
    poisoned = run(oracle_lib, case, q, kp, vp)
    assert np.array_equal(clean.view(np.uint32), poisoned.view(np.uint32))


def test_empty_sequence_gives_zeros(oracle_lib):
    case = wl.case_random(15, 3, 4, 2, 64, 16, [0, 20, 0])
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    got = run(oracle_lib, case, q, kp, vp)
    assert (got[0] == 0).all() and (got[2] == 0).all() and np.isfinite(got[1]).all()


def test_fp32_oracle_error_against_fp64_twin(oracle_lib):
    case = wl.case_chat(0, num_seqs=4)
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    a = run(oracle_lib, case, q, kp, vp)
    b = run(oracle_lib, case, q, kp, vp, "f64")
    assert np.abs(a - b).max() <= 2e-6


def test_oracle_rejects_out_of_pool_ids(oracle_lib):
    case = wl.case_random(16, 1, 1, 1, 64, 16, [20])
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    case.block_tables[0, 1] = case.num_blocks
    with pytest.raises(oracle_lib.OracleError):
        run(oracle_lib, case, q, kp, vp)


def test_oracle_copy_blocks_moves_exactly_the_named_blocks(oracle_lib):
    rng = np.random.default_rng(0)
    layers = 3
    ks = [rng.integers(0, 65535, size=(20, 2, 4, 8, 8), dtype=np.uint16) for _ in range(layers)]
    vs = [rng.integers(0, 65535, size=(20, 2, 32, 8), dtype=np.uint16) for _ in range(layers)]
    ks0 = [a.copy() for a in ks]
    vs0 = [a.copy() for a in vs]
    pairs = np.array([[3, 11], [3, 12], [7, 0]], np.int32)
    oracle_lib.copy_blocks(ks, vs, pairs)
    for l in range(layers):
        for src, dst in pairs:
            assert np.array_equal(ks[l][dst], ks0[l][src]) and np.array_equal(vs[l][dst], vs0[l][src])
        untouched = [b for b in range(20) if b not in pairs[:, 1]]
        assert np.array_equal(ks[l][untouched], ks0[l][untouched])
        assert np.array_equal(vs[l][untouched], vs0[l][untouched])
    oracle_lib.copy_blocks(ks, vs, np.zeros((0, 2), np.int32))


def test_oracle_kv_append_places_rows_by_the_table(oracle_lib):
    """Rows written through the table read back, through an independent layout view
    (einops), at (table[s][p // B], p % B); every other element is unchanged, and
    tokens outside the table are skipped."""
    rng = np.random.default_rng(21)
    for B, D in ((16, 128), (8, 64), (32, 128)):
        case = wl.case_random(int(B + D), 3, 4, 2, D, B, [3 * B + 5, B, 1])
        kp, vp = wl.host_pools(case, poison=False)
        kp0, vp0 = kp.copy(), vp.copy()
        seq = np.array([0, 0, 1, 2, 0, 1, 5, 0], np.int32)
        pos = np.array([0, 3 * B + 4, B - 1, 0, B, 0, 0, case.max_blocks_per_seq * B], np.int32)
        kn = wl.randn_bf16(rng, (8, 2, D))
        vn = wl.randn_bf16(rng, (8, 2, D))
        oracle_lib.kv_append(kn, vn, kp, vp, case.block_tables, seq, pos, B)
        kl = rearrange(kp, "n h c b e -> n h b (c e)")
        vl = rearrange(vp, "n h t d b -> n h (t b) d")
        kl0 = rearrange(kp0, "n h c b e -> n h b (c e)")
        vl0 = rearrange(vp0, "n h t d b -> n h (t b) d")
        touched = np.zeros(kl.shape[:3], bool)
        for i in range(6):                       # the last two tokens are out of range
            b, o = case.block_tables[seq[i], pos[i] // B], pos[i] % B
            assert np.array_equal(kl[b, :, o], kn[i]) and np.array_equal(vl[b, :, o], vn[i])
            touched[b, :, o] = True
        assert np.array_equal(kl[~touched], kl0[~touched]) and np.array_equal(vl[~touched], vl0[~touched])


@pytest.mark.parametrize("B,D,G,qmax", [(16, 128, 4, 4), (8, 64, 1, 16), (32, 128, 8, 2)])
def test_multi_query_oracle_matches_causal_library_attention(oracle_lib, B, D, G, qmax):
    """Each sequence's last query_lens[s] positions attend causally: torch's fp64
    scaled_dot_product_attention with an explicit mask on the contiguous gather."""
    lens = [qmax + 3, 5 * B + 1, qmax, 40]
    qlens = [qmax, 1, qmax, 0]
    case = wl.case_random(B + D + G, len(lens), 2 * G, 2, D, B, lens)
    rng = np.random.default_rng(qmax)
    q = wl.randn_bf16(rng, (len(lens), qmax, 2 * G, D))
    kp, vp = wl.host_pools(case)
    got = oracle_lib.paged_attn_multi(q, kp, vp, case.block_tables, case.context_lens, qlens,
                                      B, case.scale, 2)
    kl = rearrange(wl.f32_from_bf16(kp).astype(np.float64), "n h c b e -> n h b (c e)")
    vl = rearrange(wl.f32_from_bf16(vp).astype(np.float64), "n h t d b -> n h (t b) d")
    for s, (L, T) in enumerate(zip(lens, qlens)):
        ids = case.block_tables[s, : -(-L // B)]
        assert (got[s, T:] == 0).all()
        if T == 0:
            continue
        allowed = np.arange(L)[None, :] <= (L - T + np.arange(T))[:, None]   # [T][L]
        for h in range(2 * G):
            K = torch.from_numpy(kl[ids, h // G].reshape(-1, D)[:L])
            V = torch.from_numpy(vl[ids, h // G].reshape(-1, D)[:L])
            Q = torch.from_numpy(wl.f32_from_bf16(q[s, :T, h]).astype(np.float64))
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q[None, None], K[None, None], V[None, None],
                attn_mask=torch.from_numpy(allowed)[None, None], scale=case.scale)[0, 0].numpy()
            assert np.abs(got[s, :T, h] - ref).max() <= 1e-5


def test_multi_query_with_one_token_is_decode(oracle_lib):
    case = wl.case_random(31, 3, 8, 2, 128, 16, [17, 200, 1])
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    dec = run(oracle_lib, case, q, kp, vp)
    multi = oracle_lib.paged_attn_multi(q[:, None], kp, vp, case.block_tables, case.context_lens,
                                        np.ones(3, np.int32), 16, case.scale, 2)
    assert np.array_equal(multi[:, 0].view(np.uint32), dec.view(np.uint32))


# ---------------------------------------------------------------------------
# fp8 (E4M3FN) KV blocks
# ---------------------------------------------------------------------------

def test_fp8_decoding_of_every_code_matches_torch_float8(oracle_lib):
    """All 256 E4M3FN codes decode as torch's float8_e4m3fn does (NaN where it gives NaN)."""
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle_lib.fp8_e4m3_to_f32(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok].view(np.uint32), ref[ok].view(np.uint32))   # -0.0 included
    # landmarks of the format: 1.0, the largest finite, smallest normal and subnormal
    assert ours[0x38] == 1.0 and ours[0x7E] == 448.0 and ours[0x08] == 2.0 ** -6
    assert ours[0x01] == 2.0 ** -9 and np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


def brute_force_fp8(case, q, kp8, vp8, k_scale, v_scale):
    """fp8 pools decoded by torch (float8_e4m3fn -> float64, times the scale),
    gathered into contiguous rows with einops, attended by torch's fp64 SDPA."""
    def dec(a, scale):
        return torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).to(
            torch.float64).numpy() * scale
    kl = rearrange(dec(kp8, k_scale), "n h c b e -> n h b (c e)")
    vl = rearrange(dec(vp8, v_scale), "n h dl bq dc f -> n h (bq f) (dc dl)")
    qf = wl.f32_from_bf16(q).astype(np.float64)
    S, Hq, D = q.shape
    G = Hq // case.num_kv_heads
    out = np.zeros((S, Hq, D))
    for s in range(S):
        L = int(case.context_lens[s])
        if L == 0:
            continue
        ids = case.block_tables[s, :-(-L // case.block_size)]
        for h in range(Hq):
            K = kl[ids, h // G].reshape(-1, D)[:L]
            V = vl[ids, h // G].reshape(-1, D)[:L]
            o = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qf[s, h]).view(1, 1, 1, D), torch.from_numpy(K).view(1, 1, L, D),
                torch.from_numpy(V).view(1, 1, L, D), scale=case.scale)
            out[s, h] = o.view(D).numpy()
    return out


@pytest.mark.parametrize("B,D,G,scales", [(16, 128, 4, (0.037, 0.051)), (8, 64, 1, (1 / 16, 1 / 8)),
                                          (32, 128, 8, (0.02, 0.09))])
def test_fp8_oracle_matches_fp64_library_attention(oracle_lib, B, D, G, scales):
    Hkv = 2
    case = wl.case_random(B + D + G, 4, G * Hkv, Hkv, D, B, [3 * B + 5, 1, 0, 200])
    kp8, vp8 = wl.host_pools_fp8(case, *scales)           # NaN codes in every unread slot
    q = wl.randn_bf16(np.random.default_rng(B), (case.num_seqs, case.num_q_heads, D))
    got = oracle_lib.paged_decode_fp8(q, kp8, vp8, case.block_tables, case.context_lens, B,
                                      case.scale, scales[0], scales[1], Hkv)
    ref = brute_force_fp8(case, q, kp8, vp8, *scales)
    assert np.isfinite(got).all()
    assert np.abs(got - ref).max() <= 2e-5


def test_fp8_oracle_equals_bf16_oracle_on_the_same_values(oracle_lib):
    """With power-of-two scales every decoded value is a bf16 number; the fp8 oracle
    then performs exactly the bf16 oracle's arithmetic, bit for bit."""
    case = wl.case_random(21, 3, 8, 2, 128, 16, [70, 16, 5])
    ks, vs = 2.0 ** -4, 2.0 ** -3
    kp8, vp8 = wl.host_pools_fp8(case, ks, vs, poison=False)
    to_bf16 = lambda a, s: wl.bf16_from_f32(
        torch.from_numpy(a).view(torch.float8_e4m3fn).to(torch.float32).numpy() * np.float32(s))
    kp = wl.k_to_pool(to_bf16(wl.k8_from_pool(kp8), ks))
    vp = wl.v_to_pool(to_bf16(wl.v8_from_pool(vp8), vs))
    q = wl.randn_bf16(np.random.default_rng(4), (3, 8, 128))
    a = oracle_lib.paged_decode_fp8(q, kp8, vp8, case.block_tables, case.context_lens, 16,
                                    case.scale, ks, vs, 2)
    b = run(oracle_lib, case, q, kp, vp)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def _torch_e4m3(y):
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_encoding_matches_torch_float8_in_range(oracle_lib):
    """Nearest with ties to even, against torch's float32 -> float8_e4m3fn cast: random
    magnitudes over the whole range, every representable value, and every midpoint
    between neighbours (the ties)."""
    rng = np.random.default_rng(0)
    mags = np.exp2(rng.uniform(-12, np.log2(448.0), size=200000)).astype(np.float32)
    vals = oracle_lib.fp8_e4m3_to_f32(np.arange(0x7F, dtype=np.uint8))   # +0 .. 448
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    y = np.concatenate([mags, -mags, vals, -vals, mids, -mids])
    y = y[np.abs(y) <= 448.0]
    assert np.array_equal(oracle_lib.fp8_e4m3_from_f32(y), _torch_e4m3(y))


def test_fp8_encoding_saturates_and_round_trips(oracle_lib):
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle_lib.fp8_e4m3_to_f32(codes)
    ok = ~np.isnan(vals)
    assert np.array_equal(oracle_lib.fp8_e4m3_from_f32(vals[ok]), codes[ok])   # -0 -> 0x80
    big = np.array([448.0, 460.0, 464.0, 1e6, np.inf, -500.0, -np.inf], np.float32)
    assert oracle_lib.fp8_e4m3_from_f32(big).tolist() == [0x7E] * 5 + [0xFE] * 2
    assert oracle_lib.fp8_e4m3_from_f32(np.array([np.nan], np.float32)).tolist() == [0x7F]


def test_oracle_kv_append_fp8_quantises_into_the_right_slots(oracle_lib):
    """Rows land at (table[s][p/B], p%B) as the codes of x/scale: checked against a
    logical-layout rebuild with torch's cast (values kept inside the format's range)."""
    rng = np.random.default_rng(3)
    case = wl.case_random(5, 3, 8, 4, 64, 16, [40, 17, 3])
    ks, vs = 0.05, 0.03
    kp = np.full(wl.k8_pool_shape(case.num_blocks, 4, 64, 16), 0x7F, np.uint8)
    vp = np.full(wl.v8_pool_shape(case.num_blocks, 4, 64, 16), 0x7F, np.uint8)
    seq = np.array([0, 0, 1, 2, 2, 0], np.int32)
    pos = np.array([0, 39, 16, 2, 0, 17], np.int32)
    kn = wl.randn_bf16(rng, (6, 4, 64))
    vn = wl.randn_bf16(rng, (6, 4, 64))
    oracle_lib.kv_append_fp8(kn, vn, kp, vp, case.block_tables, seq, pos, 16, ks, vs)
    kl, vl = wl.k8_from_pool(kp), wl.v8_from_pool(vp)
    for i in range(6):
        b = case.block_tables[seq[i], pos[i] // 16]
        o = pos[i] % 16
        want_k = _torch_e4m3(wl.f32_from_bf16(kn[i]) / np.float32(ks))
        want_v = _torch_e4m3(wl.f32_from_bf16(vn[i]) / np.float32(vs))
        assert np.array_equal(kl[b, :, o, :], want_k) and np.array_equal(vl[b, :, o, :], want_v)
    written = sum(1 for _ in seq) * 4 * 64
    assert (kl != 0x7F).sum() == written and (vl != 0x7F).sum() == written


def test_fp8_multi_query_reduces_to_pinned_functions(oracle_lib):
    """Multi-token attention over fp8 pools: one query token is the fp8 decode bit for
    bit, and at power-of-two scales it is the bf16 multi-token oracle on the same
    (exactly representable) values bit for bit."""
    case = wl.case_random(31, 4, 16, 4, 128, 16, [45, 16, 7, 100])
    ks, vs = 2.0 ** -4, 2.0 ** -5
    kp8, vp8 = wl.host_pools_fp8(case, ks, vs, poison=False)
    rng = np.random.default_rng(6)
    q1 = wl.randn_bf16(rng, (4, 16, 128))
    one = oracle_lib.paged_attn_multi_fp8(q1[:, None], kp8, vp8, case.block_tables,
                                          case.context_lens, np.ones(4, np.int32), 16,
                                          case.scale, ks, vs, 4)
    dec = oracle_lib.paged_decode_fp8(q1, kp8, vp8, case.block_tables, case.context_lens, 16,
                                      case.scale, ks, vs, 4)
    assert np.array_equal(one[:, 0].view(np.uint32), dec.view(np.uint32))
    to_bf16 = lambda a, s: wl.bf16_from_f32(
        torch.from_numpy(a).view(torch.float8_e4m3fn).to(torch.float32).numpy() * np.float32(s))
    kp = wl.k_to_pool(to_bf16(wl.k8_from_pool(kp8), ks))
    vp = wl.v_to_pool(to_bf16(wl.v8_from_pool(vp8), vs))
    q = wl.randn_bf16(rng, (4, 5, 16, 128))
    qlens = np.array([5, 3, 0, 5], np.int32)
    a = oracle_lib.paged_attn_multi_fp8(q, kp8, vp8, case.block_tables, case.context_lens, qlens,
                                        16, case.scale, ks, vs, 4)
    b = oracle_lib.paged_attn_multi(q, kp, vp, case.block_tables, case.context_lens, qlens, 16,
                                    case.scale, 4)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
