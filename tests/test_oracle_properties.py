"""Property tests of the oracle's pins over drawn shapes (hypothesis, CPU only):
S in 1..4 sequences, Hkv in {1, 2, 4} KV heads, G in {1, 2, 4, 8} query heads per
KV head, head_dim in {64, 128}, block size in {8, 16, 32}, every context length in
[0, 5B + 3] (empty, single-token, block-boundary and ragged cases), seeded random
placement.  Each property pins the oracle to something other than itself: torch's
fp64 attention on contiguous gathers, the invariance of the result under a
renumbering of physical blocks ("PagedAttention (vLLM)", section "Ý tưởng cốt
lõi"), grouped-query attention as multi-head attention over repeated KV heads, the
closed form of q = 0 (the mean of the values), the census of logical blocks
(section "Cơ chế Block Table") and multi-token attention at one query token."""

import numpy as np
from einops import rearrange
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import workloads as wl
from tests.test_oracle_pins import brute_force

SETTINGS = settings(max_examples=50, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow])


@st.composite
def cases(draw, max_seqs=4):
    S = draw(st.integers(1, max_seqs))
    Hkv = draw(st.sampled_from([1, 2, 4]))
    G = draw(st.sampled_from([1, 2, 4, 8]))
    D = draw(st.sampled_from([64, 128]))
    B = draw(st.sampled_from([8, 16, 32]))
    lens = draw(st.lists(st.integers(0, 5 * B + 3), min_size=S, max_size=S))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return wl.case_random(seed, S, Hkv * G, Hkv, D, B, lens)


def decode(oracle_lib, case, q, kp, vp, precision="f32", num_kv_heads=None):
    return oracle_lib.paged_decode(q, kp, vp, case.block_tables, case.context_lens,
                                   case.block_size, case.scale,
                                   num_kv_heads or case.num_kv_heads, precision)


@SETTINGS
@given(cases())
def test_matches_fp64_library_attention(oracle_lib, case):
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    ref = brute_force(case, q, kp, vp)
    got = decode(oracle_lib, case, q, kp, vp)
    assert np.isfinite(got).all()
    assert np.abs(got - ref).max(initial=0.0) <= 1e-5
    got64 = decode(oracle_lib, case, q, kp, vp, "f64")
    assert np.abs(got64 - ref).max(initial=0.0) <= 1e-12


@SETTINGS
@given(cases(), st.integers(0, 2 ** 31 - 1))
def test_renumbering_physical_blocks_changes_no_bit(oracle_lib, case, seed):
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    base = decode(oracle_lib, case, q, kp, vp)
    perm = np.random.default_rng(seed).permutation(case.num_blocks)  # block b -> perm[b]
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    case.block_tables = perm[case.block_tables].astype(np.int32)
    again = decode(oracle_lib, case, q, kp2, vp2)
    assert np.array_equal(base.view(np.uint32), again.view(np.uint32))


@SETTINGS
@given(cases())
def test_grouped_query_attention_is_mha_over_repeated_kv_heads(oracle_lib, case):
    G = case.num_q_heads // case.num_kv_heads
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    got = decode(oracle_lib, case, q, kp, vp)
    kx, vx = np.repeat(kp, G, axis=1), np.repeat(vp, G, axis=1)   # KV head of query head h
    mha = decode(oracle_lib, case, q, kx, vx, num_kv_heads=case.num_q_heads)
    assert np.array_equal(got.view(np.uint32), mha.view(np.uint32))


@SETTINGS
@given(cases())
def test_zero_query_gives_the_mean_of_the_values(oracle_lib, case):
    q = np.zeros((case.num_seqs, case.num_q_heads, case.head_dim), np.uint16)   # +0.0
    kp, vp = wl.host_pools(case)
    got = decode(oracle_lib, case, q, kp, vp, "f64")
    vl = rearrange(wl.f32_from_bf16(vp).astype(np.float64), "n h t d b -> n h (t b) d")
    G, B, D = case.num_q_heads // case.num_kv_heads, case.block_size, case.head_dim
    for s, L in enumerate(case.context_lens):
        L = int(L)
        ids = case.block_tables[s, : -(-L // B)]
        for h in range(case.num_q_heads):
            expect = vl[ids, h // G].reshape(-1, D)[:L].mean(axis=0) if L else np.zeros(D)
            assert np.abs(got[s, h] - expect).max() <= 1e-13


@SETTINGS
@given(cases())
def test_census_of_logical_blocks(oracle_lib, case):
    """q = 0 and V one-hot by logical block (V[t][d] = 1 when d = (t div B) mod D):
    every output is the share of positions in the blocks of its dimension, which a
    dropped, doubled or misplaced block would change."""
    B, D, H = case.block_size, case.head_dim, case.num_kv_heads
    q = np.zeros((case.num_seqs, case.num_q_heads, D), np.uint16)
    kp, _ = wl.host_pools(case)
    vl = np.zeros((case.num_blocks, H, B, D), np.float32)
    for s, L in enumerate(case.context_lens):
        for j in range(-(-int(L) // B)):
            vl[case.block_tables[s, j], :, :, j % D] = 1.0
    vp = wl.v_to_pool(wl.bf16_from_f32(vl))
    got = decode(oracle_lib, case, q, kp, vp, "f64")
    for s, L in enumerate(case.context_lens):
        L = int(L)
        counts = np.zeros(D)
        for t in range(L):
            counts[(t // B) % D] += 1
        expect = counts / L if L else counts
        assert np.abs(got[s] - expect[None, :]).max() <= 1e-13


@SETTINGS
@given(cases())
def test_one_query_token_is_decode(oracle_lib, case):
    q = wl.host_q(case)
    kp, vp = wl.host_pools(case)
    dec = decode(oracle_lib, case, q, kp, vp)
    T = (case.context_lens > 0).astype(np.int32)
    multi = oracle_lib.paged_attn_multi(q[:, None], kp, vp, case.block_tables, case.context_lens,
                                        T, case.block_size, case.scale, case.num_kv_heads)
    assert np.array_equal(multi[:, 0].view(np.uint32), dec.view(np.uint32))
