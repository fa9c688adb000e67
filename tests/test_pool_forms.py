"""Host-side check of the pool forms the binding accepts: two contiguous pools, or
the paired form (the two halves of one [num_blocks][Hkv][2][tile] pool whose
(block, head) entries hold a K tile and then a V tile); any other strided view is
refused before the library is called."""

import torch

from paged_kv_cache_280_amd import pools_ok

NB, HKV, D, B = 6, 3, 64, 16
T = D * B


def _k(t):
    return t.view(NB, HKV, D // 8, B, 8)


def _v(t):
    return t.view(NB, HKV, D, B)


def test_contiguous_and_paired_pools_are_accepted():
    kv = torch.zeros((NB, HKV, 2, T), dtype=torch.bfloat16)
    assert pools_ok(_k(kv[:, :, 0]), _v(kv[:, :, 1]))
    assert pools_ok(_k(kv[:, :, 0].contiguous()), _v(kv[:, :, 1].contiguous()))
    codes = torch.zeros((NB, HKV, 2, T), dtype=torch.uint8)   # fp8 tiles: B*D bytes
    assert pools_ok(codes[:, :, 0].view(NB, HKV, D // 16, B, 16),
                    codes[:, :, 1].view(NB, HKV, 16, B // 4, D // 16, 4))


def test_other_strided_views_are_refused():
    kv = torch.zeros((NB, HKV, 2, T), dtype=torch.bfloat16)
    assert not pools_ok(_k(kv[:, :, 1]), _v(kv[:, :, 0]))          # V tile first
    blocks = torch.zeros((NB, 2, HKV, T), dtype=torch.bfloat16)   # whole blocks side by side
    assert not pools_ok(_k(blocks[:, 0]), _v(blocks[:, 1]))
    gap = torch.zeros((NB, HKV, 3, T), dtype=torch.bfloat16)      # a tile between K and V
    assert not pools_ok(_k(gap[:, :, 0]), _v(gap[:, :, 2]))
    assert not pools_ok(_k(gap[:, :, 0]), _v(gap[:, :, 1]))       # entries three tiles long
    other = torch.zeros_like(kv)                                  # halves of two pools
    assert not pools_ok(_k(kv[:, :, 0]), _v(other[:, :, 1]))
    mixed = torch.zeros((NB, HKV, 2, T), dtype=torch.float16)
    assert not pools_ok(_k(kv[:, :, 0]), _v(mixed[:, :, 1]))      # dtypes differ
