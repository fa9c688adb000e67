"""Seeded synthetic inputs for paged decode attention.

This module only draws random numbers and lays them out: it holds none of the
attention arithmetic, and both the GPU library's tests and the CPU oracle take
their inputs from here.  Nothing here imports the oracle or the product library.

Workload shapes follow the pages:
* "most answers are only 50-200 tokens" and contiguous reservation of a
  4096-token maximum (troisinh.com, section "Vấn đề");
* blocks of 16 tokens by default, 100 tokens -> 7 blocks (same page, section
  "Cơ chế Block Table");
* a 16,000-token context with 32 layers, 8 KV heads and head size 128 in the KV
  memory example (aiwiki.vn, paragraph on the memory formula);
* shared prompt prefixes for parallel sampling (troisinh.com, section
  "Copy-on-Write cho Beam Search");
* requests arriving and finishing at different times, leaving free blocks
  scattered (troisinh.com, sections "Vấn đề" and "Tại sao nó hoạt động").

Pool layout (the library's documented format, restated here so that inputs can
be written into it):  K [NB][Hkv][D/8][B][8] and V [NB][Hkv][B/Bt][D][Bt] with
Bt = min(B, 16), bf16.
Every slot that must never be read (unreferenced blocks, the unused tail of each
sequence's last block) holds a NaN; padding entries of a block-table row point
at a block that is entirely NaN.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

BF16_NAN = 0xFFFF  # a quiet NaN in bf16


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 bit patterns (round to nearest, ties to even); finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def f32_from_bf16(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def randn_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return bf16_from_f32(rng.standard_normal(shape, dtype=np.float32)).reshape(shape)


# ---------------------------------------------------------------------------
# Pool layout views (numpy): logical [NB][Hkv][B][D]  <->  library layout
# ---------------------------------------------------------------------------

def k_pool_shape(nb, hkv, d, b):
    return (nb, hkv, d // 8, b, 8)


def v_half(b):
    """Positions of one V run: the pool keeps each 16-position half of a block as
    its own [D][16] run (the whole block when B <= 16)."""
    return min(int(b), 16)


def v_pool_shape(nb, hkv, d, b):
    return (nb, hkv, b // v_half(b), d, v_half(b))


def k_to_pool(k_logical: np.ndarray) -> np.ndarray:
    nb, hkv, b, d = k_logical.shape
    return np.ascontiguousarray(k_logical.reshape(nb, hkv, b, d // 8, 8).transpose(0, 1, 3, 2, 4))


def v_to_pool(v_logical: np.ndarray) -> np.ndarray:
    nb, hkv, b, d = v_logical.shape
    bt = v_half(b)
    return np.ascontiguousarray(v_logical.reshape(nb, hkv, b // bt, bt, d).transpose(0, 1, 2, 4, 3))


def k_from_pool(k_pool: np.ndarray) -> np.ndarray:
    nb, hkv, dc, b, eight = k_pool.shape
    return np.ascontiguousarray(k_pool.transpose(0, 1, 3, 2, 4).reshape(nb, hkv, b, dc * eight))


def v_from_pool(v_pool: np.ndarray) -> np.ndarray:
    nb, hkv, nh, d, bt = v_pool.shape
    return np.ascontiguousarray(v_pool.transpose(0, 1, 2, 4, 3).reshape(nb, hkv, nh * bt, d))


def poison_v_tail(v, b, first, nan):
    """Set V positions first.. of block b (all heads, all dims) to ``nan``."""
    bt = v.shape[-1]
    for h in range(v.shape[2]):
        lo = max(first - h * bt, 0)
        if lo < bt:
            v[b, :, h, :, lo:] = nan


# ---------------------------------------------------------------------------
# Cases
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Case:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray          # int32 [S]
    block_tables: np.ndarray          # int32 [S][M]
    scale: float
    num_layers: int = 1
    poison_block: int = -1            # entirely-NaN block that padding entries point at
    seed: int = 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    def used_blocks(self) -> np.ndarray:
        """Sorted unique physical ids referenced by the valid part of the tables."""
        ids = [self.block_tables[s, : -(-int(L) // self.block_size)]
               for s, L in enumerate(self.context_lens)]
        return np.unique(np.concatenate(ids)) if ids else np.zeros(0, np.int32)

    def tail_slots(self):
        """(block id, first unused slot) of every sequence whose last block is partly full."""
        out = []
        B = self.block_size
        for s, L in enumerate(self.context_lens):
            L = int(L)
            if L > 0 and L % B:
                out.append((int(self.block_tables[s, (L - 1) // B]), L % B))
        return out


def _tables_from_lists(lists, m_min, pad_value):
    M = max([m_min] + [len(t) for t in lists])
    tab = np.full((len(lists), M), pad_value, np.int32)
    for s, t in enumerate(lists):
        tab[s, : len(t)] = t
    return tab


def _place(rng, lens, B, extra_blocks=1, pad_entries=1):
    """Random physical placement: the pool holds exactly the blocks needed plus
    ``extra_blocks`` NaN blocks; ids come from a seeded permutation."""
    need = [-(-int(L) // B) for L in lens]
    total = sum(need) + extra_blocks
    perm = rng.permutation(total).astype(np.int32)
    poison = int(perm[-1])
    lists, k = [], 0
    for n in need:
        lists.append(perm[k:k + n])
        k += n
    tab = _tables_from_lists(lists, max(need) + pad_entries if need else pad_entries, poison)
    return tab, total, poison


def case_tiny(seed=0) -> Case:
    """1 sequence of 100 tokens (7 blocks, the last 4/16 full), MHA 4/4 heads,
    head_dim 64, pool of 64 blocks at seeded random positions, scale 1/8."""
    rng = np.random.default_rng(seed)
    B, NB = 16, 64
    perm = rng.permutation(NB).astype(np.int32)
    ids = perm[:7]
    poison = int(perm[7])
    tab = np.full((1, 8), poison, np.int32)
    tab[0, :7] = ids
    return Case("tiny", 1, 4, 4, 64, B, NB, np.array([100], np.int32), tab, 1.0 / 8.0,
                poison_block=poison, seed=seed)


def chat_lengths(rng, n):
    """prompt ~ U_int[64, 1024] + answer ~ round(clip(LogNormal(ln 120, 0.5), 50, 2000))."""
    prompt = rng.integers(64, 1025, size=n)
    answer = np.rint(np.clip(rng.lognormal(math.log(120.0), 0.5, size=n), 50, 2000))
    return (prompt + answer).astype(np.int32)


def case_chat(seed=0, num_seqs=64, block_size=16) -> Case:
    """Chat-batch decode: GQA 32/8, head_dim 128, pool sized to total need."""
    rng = np.random.default_rng(seed)
    lens = chat_lengths(rng, num_seqs)
    tab, nb, poison = _place(rng, lens, block_size)
    return Case("chat", num_seqs, 32, 8, 128, block_size, nb, lens, tab, 1.0 / math.sqrt(128),
                poison_block=poison, seed=seed)


def case_long(seed=0, num_seqs=8, context_len=16000, num_layers=32, block_size=16) -> Case:
    """Long-context decode: 8 x 16,000 tokens, 32 layers (one table shared by all
    layers, one K and one V pool per layer), GQA 32/8, head_dim 128."""
    rng = np.random.default_rng(seed)
    lens = np.full(num_seqs, context_len, np.int32)
    tab, nb, poison = _place(rng, lens, block_size)
    return Case("long", num_seqs, 32, 8, 128, block_size, nb, lens, tab, 1.0 / math.sqrt(128),
                num_layers=num_layers, poison_block=poison, seed=seed)


def mix_lengths(rng, n=256, n_long=13, long_len=32768, median=150.0, sigma=1.0, max_len=4096):
    """Continuous-batching mix: n_long sequences at long_len, the rest
    round(clip(LogNormal(ln median, sigma), 1, max_len)); order shuffled."""
    short = np.rint(np.clip(rng.lognormal(math.log(median), sigma, size=n - n_long), 1, max_len))
    lens = np.concatenate([np.full(n_long, long_len), short]).astype(np.int32)
    rng.shuffle(lens)
    return lens


def case_mix(seed=0, block_size=16, num_seqs=256, n_long=13, long_len=32768,
             pool_bytes=100e9, churn_steps=64, num_blocks=None) -> Case:
    """Continuous-batching mix at pool scale: GQA 64/8, head_dim 128.  The pool
    (K+V) is sized to ``pool_bytes``; a churn warm-up (finish with p=1/64 per step,
    readmit, LIFO free list) scatters the live blocks before the batch is frozen."""
    rng = np.random.default_rng(seed)
    Hkv, D, B = 8, 128, block_size
    if num_blocks is None:
        num_blocks = int(pool_bytes // (2 * B * Hkv * D * 2))
    lens = mix_lengths(rng, num_seqs, n_long, long_len)
    is_long = lens == long_len
    free = list(rng.permutation(num_blocks).astype(np.int64))  # LIFO: pop() from the end
    tables = []
    for L in lens:
        tables.append([free.pop() for _ in range(-(-int(L) // B))])
    lens = lens.astype(np.int64)
    for _ in range(churn_steps):
        for s in range(num_seqs):
            if lens[s] % B == 0:
                tables[s].append(free.pop())
            lens[s] += 1
        for s in range(num_seqs):
            if not is_long[s] and rng.random() < 1.0 / 64:
                free.extend(reversed(tables[s]))
                newL = int(np.rint(np.clip(rng.lognormal(math.log(150.0), 1.0), 1, 4096)))
                tables[s] = [free.pop() for _ in range(-(-newL // B))]
                lens[s] = newL
    poison = int(free.pop())
    tab = _tables_from_lists(tables, max(len(t) for t in tables) + 1, poison)
    return Case("mix", num_seqs, 64, Hkv, D, B, num_blocks, lens.astype(np.int32), tab,
                1.0 / math.sqrt(D), poison_block=poison, seed=seed)


def case_random(seed, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, lens,
                extra_blocks=3, pad_entries=2) -> Case:
    """Arbitrary shape with the given lengths, random placement, scale 1/sqrt(D)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    tab, nb, poison = _place(rng, lens, block_size, extra_blocks, pad_entries)
    return Case("random", num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, nb, lens,
                tab, 1.0 / math.sqrt(head_dim), poison_block=poison, seed=seed)


@dataclasses.dataclass
class PrefixScript:
    """Parallel sampling with a shared prompt prefix: every prompt's prefix is
    stored once and forked to n_samples sequences, which then append divergent
    tails.  Block placement is left to the block manager (seeded free order)."""
    num_prompts: int
    num_samples: int
    prefix_len: int
    tails: np.ndarray          # int32 [num_prompts][num_samples]
    block_size: int
    num_blocks: int
    free_order: np.ndarray     # int32 permutation of the pool
    num_q_heads: int = 32
    num_kv_heads: int = 8
    head_dim: int = 128
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def prefix_script(seed=0, prefix_len=1020, num_prompts=16, num_samples=8, tail_max=256,
                  block_size=16, spare_blocks=8) -> PrefixScript:
    """16 prompts x 8 samples; tails ~ U_int[0, tail_max]; the pool holds what the
    script needs (prefix blocks once, each sample's tail blocks and one copy per
    sample that writes into a shared, partly filled block) plus spare blocks."""
    rng = np.random.default_rng(seed)
    tails = rng.integers(0, tail_max + 1, size=(num_prompts, num_samples)).astype(np.int32)
    B = block_size
    pre_blocks = -(-prefix_len // B)
    need = num_prompts * pre_blocks
    for p in range(num_prompts):
        for k in range(num_samples):
            need += -(-(prefix_len + int(tails[p, k])) // B) - pre_blocks
            need += 1 if (prefix_len % B and tails[p, k] > 0) else 0
    nb = need + spare_blocks
    return PrefixScript(num_prompts, num_samples, prefix_len, tails, B, nb,
                        rng.permutation(nb).astype(np.int32), seed=seed)


def token_kv(seed, tag, n_tokens, num_kv_heads, head_dim):
    """bf16 K and V rows [n_tokens][Hkv][D] for one tagged run of tokens."""
    rng = np.random.default_rng([seed, 3] + list(tag))
    k = randn_bf16(rng, (n_tokens, num_kv_heads, head_dim))
    v = randn_bf16(rng, (n_tokens, num_kv_heads, head_dim))
    return k, v


def write_tokens(k_pool, v_pool, slots, k_rows, v_rows):
    """Write token rows into (block, slot) positions of host pools in the library
    layout.  slots: sequence of (block, offset); rows: [n][Hkv][D] bf16 bits."""
    if len(slots) == 0:
        return
    b = np.array([s[0] for s in slots], dtype=np.int64)
    o = np.array([s[1] for s in slots], dtype=np.int64)
    n, hkv, d = k_rows.shape
    # K [NB][Hkv][D/8][B][8]: element (b, g, o, d) at [b, g, d // 8, o, d % 8]
    k_pool[b[:, None, None], np.arange(hkv)[None, :, None], (np.arange(d) // 8)[None, None, :],
           o[:, None, None], (np.arange(d) % 8)[None, None, :]] = k_rows
    # V [NB][Hkv][B/Bt][D][Bt]: element (b, g, o, d) at [b, g, o // Bt, d, o % Bt]
    bt = v_pool.shape[-1]
    v_pool[b[:, None, None], np.arange(hkv)[None, :, None], (o // bt)[:, None, None],
           np.arange(d)[None, None, :], (o % bt)[:, None, None]] = v_rows


# ---------------------------------------------------------------------------
# Host materialisation (numpy)
# ---------------------------------------------------------------------------

def host_q(case: Case, layer=0) -> np.ndarray:
    rng = np.random.default_rng([case.seed, 1, layer])
    return randn_bf16(rng, (case.num_seqs, case.num_q_heads, case.head_dim))


def host_pools(case: Case, layer=0, poison=True):
    """(k_pool, v_pool) as uint16 numpy arrays in the library layout.  Referenced
    blocks hold bf16 N(0,1); with ``poison`` everything that must not be read is NaN."""
    rng = np.random.default_rng([case.seed, 2, layer])
    NB, H, D, B = case.num_blocks, case.num_kv_heads, case.head_dim, case.block_size
    k = randn_bf16(rng, k_pool_shape(NB, H, D, B))
    v = randn_bf16(rng, v_pool_shape(NB, H, D, B))
    if poison:
        poison_host_pools(case, k, v)
    return k, v


def poison_host_pools(case: Case, k: np.ndarray, v: np.ndarray) -> None:
    used = np.zeros(case.num_blocks, bool)
    used[case.used_blocks()] = True
    k[~used] = BF16_NAN
    v[~used] = BF16_NAN
    for b, first in case.tail_slots():
        k[b, :, :, first:, :] = BF16_NAN
        poison_v_tail(v, b, first, BF16_NAN)


# ---------------------------------------------------------------------------
# Device materialisation (torch on a GPU); used where pools are too big for the host
# ---------------------------------------------------------------------------

def device_tensors(case: Case, device, layer=0, poison=True):
    """q, k_pool, v_pool as bf16 torch tensors on ``device``; block_tables and
    context_lens as int32 tensors.  Random values come from a seeded torch
    generator on the device (different numbers from the host path)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(case.seed) * 1000003 + int(layer))
    NB, H, D, B = case.num_blocks, case.num_kv_heads, case.head_dim, case.block_size
    q = torch.randn((case.num_seqs, case.num_q_heads, D), generator=g, device=device,
                    dtype=torch.float32).to(torch.bfloat16)
    k = torch.empty(k_pool_shape(NB, H, D, B), dtype=torch.bfloat16, device=device)
    v = torch.empty(v_pool_shape(NB, H, D, B), dtype=torch.bfloat16, device=device)
    fill_device_pools(case, k, v, g, poison)
    tables = torch.from_numpy(case.block_tables).to(device)
    lens = torch.from_numpy(case.context_lens).to(device)
    return q, k, v, tables, lens


def fill_device_pools(case: Case, k, v, g, poison=True) -> None:
    import torch

    used = torch.from_numpy(case.used_blocks().astype(np.int64)).to(k.device)
    if poison:
        k.view(torch.int16).fill_(-1)   # 0xFFFF: NaN
        v.view(torch.int16).fill_(-1)
    chunk = 1 << 14
    for i in range(0, used.numel(), chunk):
        ids = used[i:i + chunk]
        k[ids] = torch.randn((ids.numel(),) + tuple(k.shape[1:]), generator=g, device=k.device,
                             dtype=torch.float32).to(torch.bfloat16)
        v[ids] = torch.randn((ids.numel(),) + tuple(v.shape[1:]), generator=g, device=v.device,
                             dtype=torch.float32).to(torch.bfloat16)
    if poison:
        kk, vv = k.view(torch.int16), v.view(torch.int16)
        for b, first in case.tail_slots():
            kk[b, :, :, first:, :] = -1
            poison_v_tail(vv, b, first, -1)


# ---------------------------------------------------------------------------
# fp8 (OCP E4M3FN) pools: one byte per element, a scale per pool
# ---------------------------------------------------------------------------
# Layouts (the library's documented fp8 format, restated so that inputs can be
# written into it):  K [NB][Hkv][D/16][B][16] and V [NB][Hkv][16][B/4][D/16][4],
# element (b, g, o, d) of V at [b][g][d%16][o/4][d/16][o%4].  Codes come from
# torch's float8_e4m3fn conversion of N(0,1)/scale (input generation only).

E4M3_NAN = 0x7F


def k8_pool_shape(nb, hkv, d, b):
    return (nb, hkv, d // 16, b, 16)


def v8_pool_shape(nb, hkv, d, b):
    return (nb, hkv, 16, b // 4, d // 16, 4)


def k8_to_pool(k_logical: np.ndarray) -> np.ndarray:
    nb, hkv, b, d = k_logical.shape
    return np.ascontiguousarray(k_logical.reshape(nb, hkv, b, d // 16, 16).transpose(0, 1, 3, 2, 4))


def v8_to_pool(v_logical: np.ndarray) -> np.ndarray:
    nb, hkv, b, d = v_logical.shape
    x = v_logical.reshape(nb, hkv, b // 4, 4, d // 16, 16)      # [o/4][o%4][d/16][d%16]
    return np.ascontiguousarray(x.transpose(0, 1, 5, 2, 4, 3))   # [d%16][o/4][d/16][o%4]


def k8_from_pool(k_pool: np.ndarray) -> np.ndarray:
    nb, hkv, dc, b, sixteen = k_pool.shape
    return np.ascontiguousarray(k_pool.transpose(0, 1, 3, 2, 4).reshape(nb, hkv, b, dc * sixteen))


def v8_from_pool(v_pool: np.ndarray) -> np.ndarray:
    nb, hkv, sixteen, bq, dc, four = v_pool.shape
    x = v_pool.transpose(0, 1, 3, 5, 4, 2)                       # [o/4][o%4][d/16][d%16]
    return np.ascontiguousarray(x.reshape(nb, hkv, bq * four, dc * sixteen))


def e4m3_codes(x: np.ndarray, scale: float) -> np.ndarray:
    """uint8 E4M3FN codes of x / scale (torch's conversion; values clipped to the
    format's range first)."""
    import torch

    y = np.clip(np.asarray(x, dtype=np.float32) / np.float32(scale), -448.0, 448.0)
    return torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def host_pools_fp8(case: Case, k_scale: float, v_scale: float, layer=0, poison=True):
    """(k_pool, v_pool) as uint8 numpy arrays in the fp8 layouts: codes of bf16-free
    N(0,1) draws divided by the scales; with ``poison`` every slot that must not be
    read holds the NaN code."""
    rng = np.random.default_rng([case.seed, 5, layer])
    NB, H, D, B = case.num_blocks, case.num_kv_heads, case.head_dim, case.block_size
    k = e4m3_codes(rng.standard_normal((NB, H, B, D), dtype=np.float32), k_scale)
    v = e4m3_codes(rng.standard_normal((NB, H, B, D), dtype=np.float32), v_scale)
    if poison:
        used = np.zeros(NB, bool)
        used[case.used_blocks()] = True
        for a in (k, v):
            a[~used] = E4M3_NAN
            for b, first in case.tail_slots():
                a[b, :, first:, :] = E4M3_NAN
    return k8_to_pool(k), v8_to_pool(v)


def device_pools_fp8(case: Case, device, k_scale: float, v_scale: float, layer=0, poison=True):
    """fp8 K and V pools (uint8 torch tensors in the fp8 layouts) on ``device``,
    filled for the referenced blocks from a seeded device generator; with
    ``poison`` everything else (and each last block's unused tail) is the NaN code."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(case.seed) * 1000003 + 7919 + int(layer))
    NB, H, D, B = case.num_blocks, case.num_kv_heads, case.head_dim, case.block_size
    k = torch.full(k8_pool_shape(NB, H, D, B), E4M3_NAN if poison else 0, dtype=torch.uint8,
                   device=device)
    v = torch.full(v8_pool_shape(NB, H, D, B), E4M3_NAN if poison else 0, dtype=torch.uint8,
                   device=device)
    used = torch.from_numpy(case.used_blocks().astype(np.int64)).to(device)
    tails = {b: first for b, first in case.tail_slots()} if poison else {}

    def codes(n, scale):
        x = torch.randn((n, H, B, D), generator=g, device=device, dtype=torch.float32) / scale
        return x.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)

    chunk = 1 << 13
    for i in range(0, used.numel(), chunk):
        ids = used[i:i + chunk]
        kl, vl = codes(ids.numel(), k_scale), codes(ids.numel(), v_scale)
        if tails:
            for j, b in enumerate(ids.tolist()):
                if b in tails:
                    kl[j, :, tails[b]:, :] = E4M3_NAN
                    vl[j, :, tails[b]:, :] = E4M3_NAN
        n = ids.numel()
        k[ids] = kl.reshape(n, H, B, D // 16, 16).permute(0, 1, 3, 2, 4).contiguous()
        v[ids] = vl.reshape(n, H, B // 4, 4, D // 16, 16).permute(0, 1, 5, 2, 4, 3).contiguous()
    return k, v


# ---------------------------------------------------------------------------
# K/V rows that depend on a token history (prefix caching and beam search tests)
# ---------------------------------------------------------------------------

def history_kv(tokens, num_kv_heads, head_dim):
    """bf16 K and V rows [Hkv][D] of the last position of ``tokens``, drawn from a
    generator seeded by the whole history (as a model's K/V depend on every
    earlier token): equal histories give equal rows."""
    import hashlib

    digest = hashlib.sha256(np.asarray(tokens, dtype="<i8").tobytes()).digest()
    rng = np.random.default_rng(np.frombuffer(digest[:16], dtype=np.uint32).tolist())
    return (randn_bf16(rng, (num_kv_heads, head_dim)), randn_bf16(rng, (num_kv_heads, head_dim)))


def private_layout(histories, num_kv_heads, head_dim, block_size):
    """Every sequence's K/V (rows from history_kv) in blocks of its own, numbered in
    order; returns (k_pool, v_pool, block_tables, context_lens) with NaN in the
    unused tail slots and in one extra block that table padding points at."""
    B = block_size
    nblk = [-(-len(h) // B) for h in histories]
    NB = sum(nblk) + 1
    kp = np.full(k_pool_shape(NB, num_kv_heads, head_dim, B), BF16_NAN, np.uint16)
    vp = np.full(v_pool_shape(NB, num_kv_heads, head_dim, B), BF16_NAN, np.uint16)
    tables = np.full((len(histories), max(nblk + [1]) + 1), NB - 1, np.int32)
    nxt = 0
    for i, h in enumerate(histories):
        slots = []
        for j in range(nblk[i]):
            tables[i, j] = nxt + j
        for p in range(len(h)):
            slots.append((nxt + p // B, p % B))
        rows = [history_kv(h[:p + 1], num_kv_heads, head_dim) for p in range(len(h))]
        if rows:
            write_tokens(kp, vp, slots, np.stack([r[0] for r in rows]), np.stack([r[1] for r in rows]))
        nxt += nblk[i]
    lens = np.array([len(h) for h in histories], np.int32)
    return kp, vp, tables, lens
