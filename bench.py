"""Benchmark of paged decode attention on one MI355X.

Default workload (one step = one decode token for every sequence through every
layer): 8 sequences x 16,000 tokens, 32 layers each with its own K and V pool,
32 query heads / 8 KV heads, head_dim 128, block size 16, random physical
placement.  Inputs are synthetic (seeded bf16 N(0,1)) and resident in HBM before
timing starts.  The 32 pools hold 16.8 GB, far beyond the 256 MB last-level
cache, so every layer's blocks come from HBM (the chat workload keeps 16 layers of
pools for the same reason; the mix reads 2 GB per call from a 100 GB pool).

Prints one JSON line: decode tokens/s (value), KV GB/s, the roofline of the main
decode kernel (HIP events around every launch in the timed region) and the CPU
oracle timed on a bounded sample of the same workload.

Other workloads (--workload chat|mix|prefix|tiny) are for measurements beside the
headline; prefix also times the copy-on-write copy_blocks call, and counts the
shared prefix's bytes once (unique positions read) beside the logical bytes.
--query-tokens T > 1 times multi-token attention instead of decode: every
sequence verifies T query tokens (its last T positions, causal), as a
speculative decoding step does; value is then query tokens/s.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode: achieved KV GB/s (% of HBM peak) + decode tokens/s, 1 GPU"
METRIC_MULTI = ("paged multi-token attention (T causal query tokens per sequence): achieved KV "
                "GB/s (% of HBM peak) + query tokens/s, 1 GPU")
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
FP8_SCALE = 1.0 / 16   # K and V pool scales of the fp8 runs (N(0,1) values * 16 fit E4M3)
CSRC = os.path.join(ROOT, "paged_kv_cache_280_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long",
                    choices=["long", "chat", "mix", "prefix", "tiny", "append"])
    ap.add_argument("--shared-prefix", action="store_true",
                    help="with --workload prefix: paged_attn_decode_shared over the batch's "
                         "sharing groups (each prompt's prefix read once per call)")
    ap.add_argument("--with-append", action="store_true",
                    help="each layer call also appends the new token's K/V: the full "
                         "per-layer decode step")
    ap.add_argument("--append-mode", default="fused", choices=["fused", "separate"],
                    help="with --with-append: one paged_attn_decode_append call (fused), or "
                         "kv_append then the decode (separate; always so for --query-tokens > 1)")
    ap.add_argument("--block-size", type=int, default=16)
    ap.add_argument("--kv-dtype", default="bf16", choices=["bf16", "fp8"],
                    help="fp8: K/V pools of E4M3FN codes with a scale of 1/16 each")
    ap.add_argument("--kv-layout", default="separate", choices=["separate", "paired"],
                    help="paired: K and V as the two halves of one pool whose (block, head) "
                         "entries hold a K tile and then a V tile")
    ap.add_argument("--query-tokens", type=int, default=1,
                    help="T > 1: multi-token attention, T causal query tokens per sequence")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--timeline", action="store_true",
                    help="per-worker timeline of --steps eager decode calls from the "
                         "PKV_TIMELINE build (libpkv_timeline.so) instead of the timed run")
    ap.add_argument("--timeline-raw", default="", metavar="NPZ",
                    help="with --timeline: also save every call's worker stamps to NPZ")
    ap.add_argument("--probe-sweep", action="store_true",
                    help="only run the read-stream probe on the workload's K/V units, "
                         "sweeping waves per CU and units in flight, and print it")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes three times (the "
                         "reference kernel that scales hardware byte counters) and exit")
    return ap.parse_args()


def copy_calibration(nbytes):
    import torch

    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes,
                      "launches": 3}), flush=True)


def source_sha():
    """Hash of the library sources (a counter summary is used only for the code it
    was taken on)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_key):
    """HBM bytes per decode call (decode kernel + merge kernel, read + written) from
    the committed rocprofv3 counter summary, if it was taken on the current kernel
    source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload_key)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != source_sha():
        return None
    return t.get("hbm_bytes_per_call")


def prefix_case(args):
    """Shared-prefix parallel sampling: 16 prompts x 8 samples, a 1020-token prefix
    stored once per prompt, tails U_int[0, 256], built by the block manager (which
    queues the copy-on-write pairs).  Returns (case, pairs, unique positions,
    fragmentation, sharing groups of the batch (group offsets, prefix lengths))."""
    import workloads as wl
    from paged_kv_cache_280_amd.block_manager import BlockManager

    sc = wl.prefix_script(args.seed, prefix_len=1020, block_size=args.block_size)
    bm = BlockManager(sc.num_blocks, sc.block_size, sc.free_order)
    seqs = []
    for p in range(sc.num_prompts):
        bm.add(("prompt", p), sc.prefix_len)
        for k in range(sc.num_samples):
            bm.fork(("prompt", p), (p, k))
            seqs.append((p, k))
        bm.free(("prompt", p))
    for (p, k) in seqs:
        bm.append((p, k), int(sc.tails[p, k]))
    pairs = bm.take_copies()
    pad = int(bm.free_ids()[0]) if bm.num_free else 0
    tables, lens = bm.batch(seqs, pad_block=pad)
    B = sc.block_size
    pos = np.concatenate([tables[i, np.arange(L) // B].astype(np.int64) * B + np.arange(L) % B
                          for i, L in enumerate(lens)])
    case = wl.Case("prefix", len(seqs), sc.num_q_heads, sc.num_kv_heads, sc.head_dim, B,
                   sc.num_blocks, lens, tables, sc.scale, num_layers=16, poison_block=pad,
                   seed=args.seed)
    # slots of the distinct blocks the batch holds that hold no token (a shared block
    # counts once, as it is stored once)
    held = np.unique(pos // B).size * B
    frag = round((held - np.unique(pos).size) / held, 5)
    return case, pairs, int(np.unique(pos).size), frag, bm.shared_groups(seqs, sc.num_samples)


def build_workload(args, dev):
    import torch

    import workloads as wl

    extra = {}
    if args.workload == "long":
        case = wl.case_long(args.seed, block_size=args.block_size)
        layers = case.num_layers
        desc = ("long-context decode: 8 seqs x 16000 tokens, 32 layers, 32 q / 8 KV heads, "
                "head_dim 128, block %d" % case.block_size)
    elif args.workload == "chat":
        # 16 layers with their own pools: 2.9 GB of K+V per step, so every call
        # streams from HBM (one layer's 178 MB would otherwise sit in the 256 MB
        # last-level cache)
        case = wl.case_chat(args.seed, block_size=args.block_size)
        layers = 16
        desc = ("chat-batch decode: 64 seqs, 16 layers, 32 q / 8 KV heads, head_dim 128, "
                "block %d" % case.block_size)
    elif args.workload == "prefix":
        # 16 layers with their own pools (2.2 GB), so the unique 134 MB of a layer
        # is not served from the last-level cache by the previous step
        case, pairs, unique, frag, groups = prefix_case(args)
        layers = case.num_layers
        extra = {"pairs": pairs, "unique_tokens": unique, "fragmentation": frag,
                 "groups": groups}
        desc = ("shared-prefix sampling: 16 prompts x 8 samples, prefix 1020 stored once, tails "
                "U[0,256], 16 layers, 32 q / 8 KV heads, head_dim 128, block %d" % case.block_size)
    elif args.workload == "tiny":
        case = wl.case_tiny(args.seed)
        layers = 1
        desc = "tiny decode: 1 seq x 100 tokens, 4 q / 4 KV heads, head_dim 64, block 16"
    else:
        case = wl.case_mix(args.seed, args.block_size)
        layers = 1
        desc = ("continuous-batching mix: 256 seqs (13 at 32768), 64 q / 8 KV heads, head_dim 128, "
                "block %d, 100 GB pool" % case.block_size)
    pools = []
    for layer in range(layers):
        q, k, v, tabs, lens = wl.device_tensors(case, dev, layer=layer)
        if args.kv_dtype == "fp8":
            del k, v
            k, v = wl.device_pools_fp8(case, dev, FP8_SCALE, FP8_SCALE, layer=layer)
        if args.kv_layout == "paired":
            k, v = pair_pools(k, v)
        pools.append((q, k, v))
    torch.cuda.synchronize()
    if args.kv_dtype == "fp8":
        desc += ", fp8 E4M3 K/V"
    if args.kv_layout == "paired":
        desc += ", K and V tiles paired in one pool"
    return case, layers, desc, pools, tabs, lens, extra


def pair_pools(k, v):
    """The paired form of two device pools: one [NB][Hkv][2][tile] pool holding
    both, each (block, head) entry a K tile and then a V tile, returned as its two
    halves viewed in the K and V layouts (the separate pools are freed)."""
    import torch

    NB, H = int(k.shape[0]), int(k.shape[1])
    tile = k.numel() // (NB * H)
    kv = torch.empty((NB, H, 2, tile), dtype=k.dtype, device=k.device)
    kv[:, :, 0] = k.reshape(NB, H, tile)
    kv[:, :, 1] = v.reshape(NB, H, tile)
    return kv[:, :, 0].view(k.shape), kv[:, :, 1].view(v.shape)


def cpu_baseline(case, pools, layers, args):
    """The oracle on the host cores over a bounded sample of the same workload:
    whole (layer, sequence) pairs in order until about ``--cpu-seconds`` of oracle
    time, scaled by context tokens to the full step.  With several query tokens the
    oracle's multi-token attention runs on the same q rows the GPU reads; with fp8
    pools, the oracle's fp8 decode."""
    import torch

    import oracle

    fp8 = args.kv_dtype == "fp8"

    def run_oracle(qh, kh, vh, tab, L, threads):
        lens = np.array([L], np.int32)
        if args.query_tokens > 1 and fp8:
            oracle.paged_attn_multi_fp8(qh, kh, vh, tab, lens,
                                        np.array([args.query_tokens], np.int32), case.block_size,
                                        case.scale, FP8_SCALE, FP8_SCALE, case.num_kv_heads,
                                        threads=threads)
        elif args.query_tokens > 1:
            oracle.paged_attn_multi(qh, kh, vh, tab, lens, np.array([args.query_tokens], np.int32),
                                    case.block_size, case.scale, case.num_kv_heads, threads=threads)
        elif fp8:
            oracle.paged_decode_fp8(qh, kh, vh, tab, lens, case.block_size, case.scale, FP8_SCALE,
                                    FP8_SCALE, case.num_kv_heads, threads=threads)
        else:
            oracle.paged_decode(qh, kh, vh, tab, lens, case.block_size, case.scale,
                                case.num_kv_heads, threads=threads)

    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    done_tokens = 0
    elapsed = 0.0
    pairs_done = 0
    for layer in range(layers):
        q, kd, vd = pools[layer]
        for s in range(case.num_seqs):
            L = int(case.context_lens[s])
            nb = -(-L // case.block_size)
            idx = torch.from_numpy(case.block_tables[s, :nb].astype(np.int64)).to(kd.device)
            if fp8:
                kh, vh = kd[idx].cpu().numpy(), vd[idx].cpu().numpy()
            else:
                kh = kd[idx].view(torch.int16).cpu().numpy().view(np.uint16)
                vh = vd[idx].view(torch.int16).cpu().numpy().view(np.uint16)
            qh = q[s:s + 1].view(torch.int16).cpu().numpy().view(np.uint16)
            tab = np.arange(nb, dtype=np.int32)[None, :]
            t0 = time.perf_counter()
            run_oracle(qh, kh, vh, tab, L, threads)
            elapsed += time.perf_counter() - t0
            done_tokens += L
            pairs_done += 1
            if elapsed >= args.cpu_seconds:
                break
        if elapsed >= args.cpu_seconds:
            break
    total_tokens = int(case.context_lens.sum()) * layers
    step_seconds = elapsed * total_tokens / max(done_tokens, 1)
    # one core: the last sampled pair again, single-threaded
    t0 = time.perf_counter()
    run_oracle(qh, kh, vh, tab, L, 1)
    one_core_step = (time.perf_counter() - t0) * total_tokens / max(L, 1)
    return {
        "value": round(case.num_seqs * args.query_tokens / step_seconds, 4),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d of %d (layer, sequence) pairs, %d context tokens, %.1f s of oracle time on "
                  "%d threads, scaled by context tokens to the full step"
                  % (pairs_done, case.num_seqs * layers, done_tokens, elapsed, threads),
        "one_core_value": round(case.num_seqs * args.query_tokens / one_core_step, 4),
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def copy_blocks_timing(pools, pairs, args):
    """The copy-on-write copy_blocks call of the shared-prefix workload (every
    layer's K and V pool in one call), timed with HIP events: back to back (warm:
    the sources stay in the last-level cache) and cold (a 2 GiB buffer is read and
    written before each call, outside the timed events, so the sources come from
    HBM).  Copying again is harmless: sources are never destinations."""
    import torch

    import paged_kv_cache_280_amd as pkv

    dev = pools[0][1].device
    pd = torch.from_numpy(np.ascontiguousarray(pairs, dtype=np.int32)).to(dev)
    ks, vs = [p[1] for p in pools], [p[2] for p in pools]
    for _ in range(3):
        pkv.copy_blocks(ks, vs, pd)
    torch.cuda.synchronize()
    reps = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        pkv.copy_blocks(ks, vs, pd)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    flush = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(10):
        flush.fill_(i)                     # evicts the 256 MB last-level cache
        e0.record()
        pkv.copy_blocks(ks, vs, pd)
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) * 1e3)
    del flush
    torch.cuda.empty_cache()
    block_bytes = ks[0][0].numel() * ks[0].element_size()
    moved = 2 * 2 * len(pairs) * len(ks) * block_bytes  # K and V: read src, write dst
    us_cold = float(np.median(cold))
    return {"pairs": int(len(pairs)), "layers": len(ks), "us_per_call": round(us, 2),
            "bytes_per_call": int(moved), "gbs": round(moved / us / 1e3, 1),
            "cold_us_per_call": round(us_cold, 2), "cold_gbs": round(moved / us_cold / 1e3, 1)}


STREAM_LIB = os.path.join(ROOT, "paged_kv_cache_280_amd", "libpkv_stream.so")
TIMELINE_LIB = os.path.join(ROOT, "paged_kv_cache_280_amd", "libpkv_timeline.so")


def stream_library():
    """The HBM read-stream probe (include/pkv_stream.h), loaded after torch's HIP runtime."""
    import ctypes

    import torch  # noqa: F401

    if not os.path.exists(STREAM_LIB):
        raise RuntimeError("libpkv_stream.so is not built; run python -m "
                           "paged_kv_cache_280_amd.build --stream-probe")
    lib = ctypes.CDLL(STREAM_LIB)
    p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.pkv_stream_read.argtypes = [p, ctypes.c_size_t, p, i32, p]
    lib.pkv_stream_read.restype = i32
    lib.pkv_stream_read_pairs.argtypes = [p, p, i64, p, i32, i32, i32, p, i32, i32, p]
    lib.pkv_stream_read_pairs.restype = i32
    return lib


def decode_units(case, elem_bytes):
    """Unit ids of the K/V reads of one decode call in the decode kernel's order
    ((sequence, KV head) pairs sequence-major, then positions), one unit per
    16-position run of a block (a whole block of 8 positions at B = 8), and the
    unit size in bytes."""
    B, H, D = case.block_size, case.num_kv_heads, case.head_dim
    run = min(B, 16)
    halves = B // run
    ids = []
    for s, L in enumerate(case.context_lens):
        nb = -(-int(L) // B)
        blocks = case.block_tables[s, :nb].astype(np.int64)
        for g in range(H):
            base = (blocks * H + g) * halves
            n_runs = -(-int(L) // run)
            ids.append((base[:, None] + np.arange(halves)[None, :]).reshape(-1)[:n_runs])
    return np.concatenate(ids).astype(np.int32), run * D * elem_bytes


def attainable_bandwidth(case, pools, elem_bytes, reps=10, seq_bytes=4 << 30, sweep=False):
    """The probe kernels of libpkv_stream.so on the same GPU in the same run: a
    sequential 4 GiB read, and the decode call's own K/V reads (in the decode
    kernel's order and unit size, 3 waves per CU, three units in flight) with 8- and
    16-byte V loads, one call's bytes per launch.  Launch r reads the pools of layer
    r mod layers, as the timed steps do, so that no launch finds the previous one's
    bytes in the 256 MB last-level cache.  Best of ``reps`` HIP-event-timed launches
    each.  ``sweep`` adds other wave counts and in-flight depths."""
    import ctypes

    import torch

    lib = stream_library()
    dev = pools[0][1].device
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cu = torch.cuda.get_device_properties(dev).multi_processor_count

    def best(fn, moved):
        fn(reps)
        torch.cuda.synchronize()
        t = []
        for r in range(reps):
            e0.record(stream)
            fn(r)
            e1.record(stream)
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) / 1e3)
        return round(moved / min(t) / 1e9, 1)

    res = {}
    x = torch.empty(seq_bytes, dtype=torch.uint8, device=dev)
    x.fill_(1)
    groups = cu * 8
    sink = torch.empty(groups * 256, dtype=torch.int32, device=dev)

    def seq(r):
        assert lib.pkv_stream_read(x.data_ptr(), seq_bytes, sink.data_ptr(), groups, sh) == 0

    res["read_gbs"] = best(seq, seq_bytes)
    del x
    torch.cuda.empty_cache()
    ids, unit = decode_units(case, elem_bytes)
    k0 = pools[0][1]
    pool_units = k0.numel() * k0.element_size() // unit
    if not k0.is_contiguous():
        # paired pools: a (block, head) entry is `halves` K units and then as many V
        # units, so K unit (entry e, half h) is unit 2*e*halves + h of the pool and
        # its V lies one tile (halves units) later; the clamp bound keeps V inside
        halves = case.block_size // min(case.block_size, 16)
        ids, pool_units = 2 * ids - ids % halves, 2 * pool_units - halves
    idd = torch.from_numpy(ids).to(dev)
    sink = torch.empty(max(groups * 256, 16 * cu * 64), dtype=torch.int32, device=dev)

    def pairs_gbs(idv, vb, waves, depth):
        def run(r):
            _, k_pool, v_pool = pools[r % len(pools)]
            assert lib.pkv_stream_read_pairs(k_pool.data_ptr(), v_pool.data_ptr(), pool_units,
                                             idv.data_ptr(), idv.numel(), unit, vb,
                                             sink.data_ptr(), waves, depth, sh) == 0
        return best(run, 2 * idv.numel() * unit)

    for vb in (8, 16):
        res["pairs_v%d_gbs" % vb] = pairs_gbs(idd, vb, 3 * cu, 3)
    if sweep:
        res["call_sweep_v8"] = {"%dw_d%d" % (wpc, depth): pairs_gbs(idd, 8, wpc * cu, depth)
                                for wpc in (2, 3, 4, 6, 8) for depth in (3, 6)}
    res["pair_units"] = int(len(ids))
    res["unit_bytes"] = int(unit)
    res["kernels"] = ("libpkv_stream.so: sequential 4 GiB read, 16-byte lane loads (read_gbs); "
                      "this workload's K/V units in decode order, 16-byte K loads and 8- or "
                      "16-byte V loads, %d waves, 3 units in flight, one call's bytes per "
                      "launch, launches cycling over the %d layers' pools (pairs_v8_gbs, "
                      "pairs_v16_gbs)" % (3 * cu, len(pools)))
    return res


def internal_fragmentation(lens, block_size):
    """Share of the slots held by the batch's blocks that hold no token: only each
    sequence's last block has empty slots."""
    lens = np.asarray(lens, np.int64)
    held = int((-(-lens // block_size)).sum()) * block_size
    return 0.0 if held == 0 else round((held - int(lens.sum())) / held, 5)


def append_bench(args):
    """kv_append (or kv_append_fp8 with --kv-dtype fp8) of a prefill-sized chunk:
    8 sequences x 2048 new tokens into a pool with random block placement (GQA 8 KV
    heads, head_dim 128).  Prints one JSON line with the call time and the bytes
    moved (bf16 rows read + slots written)."""
    import torch

    import paged_kv_cache_280_amd as pkv
    import workloads as wl

    dev = torch.device("cuda:0")
    fp8 = args.kv_dtype == "fp8"
    S, chunk, H, D, B = 8, 2048, 8, 128, args.block_size
    case = wl.case_random(args.seed, S, 32, H, D, B, [chunk] * S)
    if fp8:
        kd, vd = wl.device_pools_fp8(case, dev, FP8_SCALE, FP8_SCALE, poison=False)
        tabs = torch.from_numpy(case.block_tables).to(dev)
        call = lambda: pkv.kv_append_fp8(k_new, v_new, kd, vd, tabs, seq, pos, B, FP8_SCALE,
                                         FP8_SCALE)
    else:
        _, kd, vd, tabs, _ = wl.device_tensors(case, dev, poison=False)
        call = lambda: pkv.kv_append(k_new, v_new, kd, vd, tabs, seq, pos, B)
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    T = S * chunk
    k_new = torch.randn((T, H, D), generator=g, device=dev).to(torch.bfloat16)
    v_new = torch.randn((T, H, D), generator=g, device=dev).to(torch.bfloat16)
    seq = torch.arange(S, device=dev, dtype=torch.int32).repeat_interleave(chunk)
    pos = torch.arange(chunk, device=dev, dtype=torch.int32).repeat(S)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    moved = 2 * T * H * D * (2 + (1 if fp8 else 2))   # K and V: bf16 rows read, slots written
    print(json.dumps({"workload": "kv_append%s %d tokens (8 seqs x %d), 8 KV heads, head_dim 128, "
                      "block %d" % ("_fp8" if fp8 else "", T, chunk, B),
                      "us_per_call": round(us, 2), "bytes_per_call": moved,
                      "gbs": round(moved / us / 1e3, 1)}), flush=True)


STAMP = np.dtype([("t_entry", "<u8"), ("d_plan", "<u4"), ("d_first", "<u4"), ("d_end", "<u4"),
                  ("xcc", "<u4"), ("tiles", "<u4"), ("group", "<u4")])


def timeline(args):
    """Per-worker timeline of decode calls from the PKV_TIMELINE build of the library
    (libpkv_timeline.so): every worker's entry, plan, first-tile and end times on the
    100 MHz s_memrealtime clock and the XCC it ran on, read back from the workspace
    after each eagerly launched call of the workload's layers.  Prints one JSON line
    of medians over the calls (microseconds after the first worker's entry)."""
    import torch

    from paged_kv_cache_280_amd import _binding

    if not os.path.exists(TIMELINE_LIB):
        raise RuntimeError("libpkv_timeline.so is not built; run python -m "
                           "paged_kv_cache_280_amd.build --timeline")
    if args.query_tokens != 1 or args.with_append or args.workload in ("append", "tiny"):
        raise SystemExit("--timeline covers the split decode call (one query token, no append)")
    _binding.load_library(TIMELINE_LIB)   # every binding call below uses this build
    import paged_kv_cache_280_amd as pkv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case, layers, desc, pools, tabs, lens, extra = build_workload(args, dev)
    S, Hq, Hkv, D, B = (case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim,
                        case.block_size)
    fp8 = args.kv_dtype == "fp8"
    max_ctx = case.max_context_len
    ws = pkv.new_workspace(S, Hq, Hkv, D, B, max_ctx, dev)
    cu = torch.cuda.get_device_properties(dev).multi_processor_count
    wpc = int(os.environ.get("PKV_WAVES_PER_CU", "0") or 0) or (4 if fp8 else 3)
    n = min(cu * wpc, S * Hkv * (-(-max_ctx // 16)))
    G = Hq // Hkv
    rec_bytes = n * 2 * (G * D + ((2 * G + 3) // 4) * 4) * 4
    off = rec_bytes + 16 * n   # past the descriptors
    out = torch.empty_like(pools[0][0])
    stats, raw = [], []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for c in range(args.warmup + args.steps):
        q, k, v = pools[c % layers]
        e0.record()
        if fp8:
            pkv.paged_attn_decode_fp8(q, k, v, tabs, lens, B, case.scale, FP8_SCALE, FP8_SCALE,
                                      out, workspace=ws, max_context_len=max_ctx)
        else:
            pkv.paged_attn_decode(q, k, v, tabs, lens, B, case.scale, out, workspace=ws,
                                  max_context_len=max_ctx)
        e1.record()
        torch.cuda.synchronize()
        if c < args.warmup:
            continue
        st = np.frombuffer(ws[off:off + n * STAMP.itemsize].cpu().numpy().tobytes(), dtype=STAMP)
        assert (st["group"] == np.arange(n) // 4).all(), "stamps missing: n_workers mismatch"
        raw.append(st.copy())
        t0 = int(st["t_entry"].min())
        us = lambda ticks: np.asarray(ticks, np.float64) * 0.01
        entry = us(st["t_entry"] - t0)
        has = st["d_first"] != 0xFFFFFFFF
        end = entry + us(st["d_end"])
        first = entry[has] + us(st["d_first"][has])
        per_xcc = {int(x): end[st["xcc"] == x] for x in np.unique(st["xcc"])}
        stats.append({
            "call_us": e0.elapsed_time(e1) * 1e3,
            "entry_max": entry.max(), "plan_median": float(np.median(entry + us(st["d_plan"]))),
            "first_tile_median": float(np.median(first)), "first_tile_max": float(first.max()),
            "end_min": end.min(), "end_p10": float(np.percentile(end, 10)),
            "end_median": float(np.median(end)), "end_p90": float(np.percentile(end, 90)),
            "end_max": end.max(), "end_mean": end.mean(),
            "xcc_end_median": {x: float(np.median(e)) for x, e in per_xcc.items()},
            "xcc_end_max": {x: float(e.max()) for x, e in per_xcc.items()},
            "workers_per_xcc": {x: int(len(e)) for x, e in per_xcc.items()},
            "tiles_min": int(st["tiles"][has].min()), "tiles_max": int(st["tiles"][has].max()),
        })
    med = lambda key: round(float(np.median([x[key] for x in stats])), 2)
    xccs = sorted(stats[0]["xcc_end_median"])
    line = {
        "timeline": desc, "workers": n, "calls": len(stats),
        "call_us_median": med("call_us"),
        "entry_spread_us": med("entry_max"), "plan_done_us": med("plan_median"),
        "first_tile_us": {"median": med("first_tile_median"), "max": med("first_tile_max")},
        "worker_end_us": {k: med("end_" + k) for k in ("min", "p10", "median", "mean", "p90",
                                                        "max")},
        "xcc_end_median_us": {x: round(float(np.median([s_["xcc_end_median"][x] for s_ in stats])),
                                       2) for x in xccs},
        "slowest_xcc_per_call": [max(s_["xcc_end_median"], key=s_["xcc_end_median"].get)
                                 for s_ in stats],
        "xcc_spread_us_per_call": [round(max(s_["xcc_end_median"].values()) -
                                         min(s_["xcc_end_median"].values()), 2) for s_ in stats],
        "workers_per_xcc": stats[0]["workers_per_xcc"],
        "tiles_per_worker": [stats[0]["tiles_min"], stats[0]["tiles_max"]],
        "clock": "s_memrealtime, 100 MHz",
    }
    print(json.dumps(line), flush=True)
    if args.timeline_raw:
        np.savez(args.timeline_raw, stamps=np.stack(raw), call_us=[x["call_us"] for x in stats])


def main():
    args = parse()
    if args.timeline:
        timeline(args)
        return
    if args.probe_sweep:
        import torch

        dev = torch.device("cuda:0")
        case, layers, desc, pools, tabs, lens, extra = build_workload(args, dev)
        res = attainable_bandwidth(case, pools, 1 if args.kv_dtype == "fp8" else 2, sweep=True)
        print(json.dumps({"probe": desc, **res}), flush=True)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.workload == "append":
        append_bench(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library's decode runs on a single device "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import paged_kv_cache_280_amd as pkv
    from paged_kv_cache_280_amd.accounting import decode_algorithmic_bytes

    pkv.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case, layers, desc, pools, tabs, lens, extra = build_workload(args, dev)
    S, Hq, Hkv, D, B = (case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim,
                        case.block_size)
    max_ctx = case.max_context_len
    T = args.query_tokens
    multi = T > 1
    fp8 = args.kv_dtype == "fp8"
    if multi:
        # q of every layer becomes [S][T][Hq][D]; each sequence's last T positions
        # are its query tokens
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed + 29)
        pools = [(torch.randn((S, T, Hq, D), generator=gen, device=dev).to(torch.bfloat16), k, v)
                 for (_, k, v) in pools]
        qlens = torch.full((S,), T, dtype=torch.int32, device=dev)
        desc += ", %d causal query tokens per sequence" % T
        ws = pkv.new_multi_workspace(S, Hq, Hkv, D, B, max_ctx, T, dev)
    else:
        ws = pkv.new_workspace(S, Hq, Hkv, D, B, max_ctx, dev)
    shared = args.shared_prefix
    if shared:
        if "groups" not in extra or multi or fp8 or args.with_append:
            raise SystemExit("--shared-prefix: bf16 decode of --workload prefix only")
        gf_h, pl_h = extra["groups"]
        max_group = int(np.diff(gf_h).max())
        max_prefix = int(pl_h.max())
        gfirst = torch.from_numpy(gf_h).to(dev)
        plens = torch.from_numpy(pl_h).to(dev)
        ws = torch.empty(pkv.paged_attn_decode_shared_workspace_bytes(
            S, Hq, Hkv, D, B, max_ctx, len(gf_h) - 1, max_group, max_prefix), dtype=torch.uint8,
            device=dev)
        desc += ", shared-prefix decode (groups of %d, prefix %d)" % (max_group, max_prefix)
    outs = [torch.empty_like(p[0]) for p in pools]
    kv_elem = 1 if fp8 else 2
    per_call_bytes = decode_algorithmic_bytes(case.context_lens, Hq, Hkv, D, B, query_tokens=T,
                                              unique_tokens=extra.get("unique_tokens"),
                                              kv_elem_bytes=kv_elem)
    logical_bytes = decode_algorithmic_bytes(case.context_lens, Hq, Hkv, D, B, query_tokens=T,
                                             kv_elem_bytes=kv_elem)

    stream = torch.cuda.current_stream(dev)
    n_ev = args.steps * layers
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_ev)]

    # --with-append: the K/V of every sequence's newest T positions (T = 1: the
    # token being decoded, position L-1) are written into their slots before the
    # layer's attention
    if args.with_append:
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed + 17)
        new_k = [torch.randn((S * T, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
                 for _ in range(layers)]
        new_v = [torch.randn((S * T, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
                 for _ in range(layers)]
        # the T newest positions of every sequence (T = 1: the token being decoded)
        tok_seq = torch.arange(S, device=dev, dtype=torch.int32).repeat_interleave(T)
        tok_pos = (lens.repeat_interleave(T) - T +
                   torch.arange(T, device=dev, dtype=torch.int32).repeat(S)).to(torch.int32)

    fused_append = args.with_append and args.append_mode == "fused" and not multi

    def step(timed_events=None):
        for layer in range(layers):
            q, k, v = pools[layer]
            if fused_append:
                e = timed_events[layer] if timed_events is not None else None
                if e is not None:
                    e[0].record(stream)
                sc = dict(k_scale=FP8_SCALE, v_scale=FP8_SCALE) if fp8 else {}
                pkv.paged_attn_decode_append(q, new_k[layer], new_v[layer], k, v, tabs, lens, B,
                                             case.scale, outs[layer], workspace=ws,
                                             max_context_len=max_ctx, **sc)
                if e is not None:
                    e[1].record(stream)
                continue
            if args.with_append and fp8:
                pkv.kv_append_fp8(new_k[layer], new_v[layer], k, v, tabs, tok_seq, tok_pos, B,
                                  FP8_SCALE, FP8_SCALE)
            elif args.with_append:
                pkv.kv_append(new_k[layer], new_v[layer], k, v, tabs, tok_seq, tok_pos, B)
            e = timed_events[layer] if timed_events is not None else None
            if e is not None:
                e[0].record(stream)
            if multi:
                sc = dict(k_scale=FP8_SCALE, v_scale=FP8_SCALE) if fp8 else {}
                pkv.paged_attn_multi(q, k, v, tabs, lens, qlens, B, case.scale, outs[layer],
                                     workspace=ws, max_context_len=max_ctx, **sc)
            elif shared:
                pkv.paged_attn_decode_shared(q, k, v, tabs, lens, gfirst, plens, B, case.scale,
                                             outs[layer], max_group_size=max_group,
                                             max_prefix_len=max_prefix, workspace=ws,
                                             max_context_len=max_ctx)
            elif fp8:
                pkv.paged_attn_decode_fp8(q, k, v, tabs, lens, B, case.scale, FP8_SCALE, FP8_SCALE,
                                          outs[layer], workspace=ws, max_context_len=max_ctx)
            else:
                pkv.paged_attn_decode(q, k, v, tabs, lens, B, case.scale, outs[layer],
                                      workspace=ws, max_context_len=max_ctx)
            if e is not None:
                e[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The step (all layers' launches) is captured once into a HIP graph and
    # replayed: the timed region then holds GPU work only, no Python per launch.
    graph = None
    try:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
    except Exception as e:  # capture unsupported: time eager launches instead
        print("graph capture failed (%s); timing eager launches" % e, file=sys.stderr)
        graph = None

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # Per-launch duration of the main decode kernel: HIP events around every
    # launch of eager steps on the same stream.
    for i in range(args.steps):
        step(ev[i * layers:(i + 1) * layers])
    torch.cuda.synchronize()

    ms_per_step = elapsed * 1e3 / args.steps
    kern_ms = [a.elapsed_time(b) for a, b in ev]
    kern_avg_s = float(np.mean(kern_ms)) / 1e3
    p10, p50, p90 = (float(x) * 1e3 for x in np.percentile(kern_ms, [10, 50, 90]))
    copy_line = copy_blocks_timing(pools, extra["pairs"], args) if "pairs" in extra else None
    attain = attainable_bandwidth(case, pools, kv_elem)
    # the probe read shaped like this decode: 16-byte K loads, and V loads of 8 bytes
    # (bf16 pools) or 16 bytes (fp8 pools)
    attain_key = "pairs_v16_gbs" if fp8 else "pairs_v8_gbs"
    step_bytes = per_call_bytes * layers
    tokens_per_s = S * T / (ms_per_step / 1e3)
    kv_gbs = step_bytes / (ms_per_step / 1e3) / 1e9
    achieved = per_call_bytes / kern_avg_s / 1e9
    traffic = measured_traffic(args.workload + ("_shared" if shared else "") +
                               ("_q%d" % T if multi else "") + ("_fp8" if fp8 else "") +
                               ("_paired" if args.kv_layout == "paired" else ""))

    line = {
        "metric": METRIC_MULTI if multi else METRIC,
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 q/out, fp8 e4m3 K/V" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": desc, "num_seqs": S, "context_len": int(case.context_lens.max()),
                   "layers": layers, "block_size": B, "num_q_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": D, "query_tokens": T, "kv_layout": args.kv_layout},
        "graph": graph is not None,
        "with_append": ("fused" if fused_append else "separate") if args.with_append else False,
        "kv_gbs": round(kv_gbs, 1),
        "hbm_frac": round(kv_gbs / HBM_PEAK_GBS, 4),
        "us_per_call": {"mean": round(kern_avg_s * 1e6, 2), "p10": round(p10, 2),
                        "median": round(p50, 2), "p90": round(p90, 2),
                        "calls": len(kern_ms)},
        "attainable": attain,
        "roofline": {"bound": "hbm",
                     "kernel": ("paged_attn_decode_shared (prefix and tail passes, each "
                                "decode_kernel + merge_kernel)" if shared else
                                ("paged_attn_multi" if multi else
                                 "paged_attn_decode_fp8" if fp8 else "paged_attn_decode") +
                                " (decode_kernel + merge_kernel)"),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "frac_of_attainable": round(achieved / attain[attain_key], 4),
                     "attainable_kernel": attain_key,
                     "algorithmic_bytes_per_launch": int(per_call_bytes),
                     "avg_launch_us": round(kern_avg_s * 1e6, 2)},
        "cpu_baseline": None,
        "internal_fragmentation": extra.get("fragmentation",
                                            internal_fragmentation(case.context_lens, B)),
    }
    if "unique_tokens" in extra:
        line["logical_kv_gbs"] = round(logical_bytes * layers / (ms_per_step / 1e3) / 1e9, 1)
        line["copy_blocks"] = copy_line
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, pools, layers, args)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
