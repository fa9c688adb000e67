"""ctypes binding of ``libpkv.so`` (C ABI declared in ``include/pkv.h``).

Argument marshalling only: shapes are read from the torch tensors, pointers and
the current HIP stream are handed to the library, and every step of the
computation runs in the library's kernels.  There is no fallback: without the
built library every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# PKV_LIBRARY names another build of the library (the CPU tests use it for the
# sanitized host-side build); unset, the in-tree libpkv.so
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(PKG, "libpkv.so")

_lib = None

STATUS_NAMES = {
    0: "PKV_OK", -1: "PKV_ERR_NULL", -2: "PKV_ERR_SHAPE", -3: "PKV_ERR_UNSUPPORTED",
    -4: "PKV_ERR_WORKSPACE", -5: "PKV_ERR_ALIGNMENT", -6: "PKV_ERR_DEVICE", -7: "PKV_ERR_LAUNCH",
}

EXPORTS = ("pkv_abi_version", "pkv_status_string", "paged_attn_decode_workspace_bytes",
           "paged_attn_decode", "paged_attn_decode_fp8", "paged_attn_multi_workspace_bytes",
           "paged_attn_multi", "paged_attn_multi_fp8",
           "kv_append", "kv_append_fp8", "copy_blocks", "pkv_check_batch",
           "paged_attn_decode_append", "paged_attn_decode_append_fp8",
           "paged_attn_decode_noalloc", "paged_attn_decode_shared_workspace_bytes",
           "paged_attn_decode_shared")


class PkvError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        text = load_library().pkv_status_string(status).decode()
        super().__init__("%s%s (%s)" % (what + ": " if what else "", text,
                                        STATUS_NAMES.get(status, status)))


def load_library(path: str = LIB_PATH):
    """Load the built library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libpkv.so is not built (%s); run `python -m paged_kv_cache_280_amd.build`"
                           % path)
    # torch ships its own HIP runtime: load it first, so that the library binds to
    # the runtime that owns torch's device memory and streams (loaded alone, the
    # library would bind to the system runtime and fail to query the device)
    import torch  # noqa: F401

    lib = ctypes.CDLL(path)
    p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.pkv_abi_version.argtypes = []
    lib.pkv_abi_version.restype = i32
    lib.pkv_status_string.argtypes = [i32]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.paged_attn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.paged_attn_decode_workspace_bytes.restype = sz
    decode_args = [p, p, p, p, p, i32, ctypes.c_float, p, i32, i32, i32, i32, i32, i64, i32, p,
                   sz, p]
    lib.paged_attn_decode.argtypes = decode_args
    lib.paged_attn_decode.restype = i32
    lib.paged_attn_decode_noalloc.argtypes = decode_args[:15] + [p]
    lib.paged_attn_decode_noalloc.restype = i32
    f32 = ctypes.c_float
    lib.paged_attn_decode_fp8.argtypes = [p, p, p, p, p, i32, f32, f32, f32, p, i32, i32, i32, i32,
                                          i32, i64, i32, p, sz, p]
    lib.paged_attn_decode_fp8.restype = i32
    lib.paged_attn_multi_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.paged_attn_multi_workspace_bytes.restype = sz
    lib.paged_attn_multi.argtypes = [p, p, p, p, p, p, i32, i32, ctypes.c_float, p, i32, i32, i32,
                                     i32, i32, i64, i32, p, sz, p]
    lib.paged_attn_multi.restype = i32
    lib.paged_attn_multi_fp8.argtypes = [p, p, p, p, p, p, i32, i32, ctypes.c_float, ctypes.c_float,
                                         ctypes.c_float, p, i32, i32, i32, i32, i32, i64, i32, p,
                                         sz, p]
    lib.paged_attn_multi_fp8.restype = i32
    lib.kv_append.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i64, p]
    lib.kv_append.restype = i32
    lib.kv_append_fp8.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i64, f32, f32,
                                  p]
    lib.kv_append_fp8.restype = i32
    lib.copy_blocks.argtypes = [p, p, i32, i64, i64, p, i32, p]
    lib.copy_blocks.restype = i32
    lib.pkv_check_batch.argtypes = [p, p, p, i32, i32, i64, i32, i32, p, p]
    lib.pkv_check_batch.restype = i32
    lib.paged_attn_decode_append.argtypes = [p, p, p, p, p, p, p, i32, f32, p, i32, i32, i32, i32,
                                             i32, i64, i32, p, sz, p]
    lib.paged_attn_decode_append.restype = i32
    lib.paged_attn_decode_append_fp8.argtypes = [p, p, p, p, p, p, p, i32, f32, f32, f32, p, i32,
                                                 i32, i32, i32, i32, i64, i32, p, sz, p]
    lib.paged_attn_decode_append_fp8.restype = i32
    lib.paged_attn_decode_shared_workspace_bytes.argtypes = [i32] * 9
    lib.paged_attn_decode_shared_workspace_bytes.restype = sz
    lib.paged_attn_decode_shared.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, f32, p, i32,
                                             i32, i32, i32, i32, i64, i32, p, sz, p]
    lib.paged_attn_decode_shared.restype = i32
    _lib = lib
    return lib


def abi_version() -> int:
    return int(load_library().pkv_abi_version())


def status_string(status: int) -> str:
    return load_library().pkv_status_string(int(status)).decode()


def _stream_handle(tensor, stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(tensor.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _on_stream(tensor, stream):
    """Context for one call: tensor's device current, and the stream the kernels
    run on (``stream``, default torch's current one) current too, so that any
    temporary the call allocates (workspace, output) belongs to that stream in
    torch's caching allocator and is not handed to other work while the kernels
    still use it."""
    import contextlib

    import torch

    ctx = contextlib.ExitStack()
    ctx.enter_context(torch.cuda.device(tensor.device))
    if stream is not None:
        ctx.enter_context(torch.cuda.stream(stream))
    return ctx


def _check(cond, msg):
    if not cond:
        raise ValueError(msg)


def _v_pool_ok(v_cache, NB, Hkv, D, B):
    """bf16 V pool [NB][Hkv][B/Bt][D][Bt], Bt = min(B, 16); for B <= 16 the same
    memory may also come as [NB][Hkv][D][B]."""
    bt = min(B, 16)
    shape = tuple(v_cache.shape)
    return shape == (NB, Hkv, B // bt, D, bt) or (B <= 16 and shape == (NB, Hkv, D, B))


V_POOL_TEXT = "v_cache must be [num_blocks][Hkv][block_size/Bt][D][Bt], Bt = min(block_size, 16)"
POOLS_TEXT = "k_cache/v_cache: two contiguous pools, or the two halves of one paired pool"


def _dense_strides(shape):
    out, acc = [], 1
    for n in reversed(tuple(shape)):
        out.append(acc)
        acc *= int(n)
    return tuple(reversed(out))


def pools_ok(k_cache, v_cache):
    """True for two contiguous pools, or for the paired form: the two halves of one
    pool [num_blocks][Hkv][2][tile] whose (block, head) entries hold a K tile and
    then a V tile (e.g. ``kv[:, :, 0]`` and ``kv[:, :, 1]`` viewed in the K and V
    layouts), so that v_cache starts one tile after k_cache."""
    if k_cache.is_contiguous() and v_cache.is_contiguous():
        return True
    if k_cache.dim() < 3 or v_cache.dim() < 3 or k_cache.dtype != v_cache.dtype:
        return False
    NB, Hkv = int(k_cache.shape[0]), int(k_cache.shape[1])
    if tuple(v_cache.shape[:2]) != (NB, Hkv):
        return False
    tile = math.prod(int(n) for n in k_cache.shape[2:])
    if math.prod(int(n) for n in v_cache.shape[2:]) != tile:
        return False
    for t in (k_cache, v_cache):
        want = (2 * Hkv * tile, 2 * tile) + _dense_strides(t.shape[2:])
        if any(n > 1 and st != w for n, st, w in zip(t.shape, t.stride(), want)):
            return False
    return (v_cache.data_ptr() - k_cache.data_ptr() == tile * k_cache.element_size()
            and k_cache.untyped_storage().data_ptr() == v_cache.untyped_storage().data_ptr())


def decode_shapes(q, k_cache, v_cache, block_tables, context_lens, block_size):
    """(S, Hq, Hkv, D, NB, M) of a decode call, after host-side checks of the tensors."""
    import torch

    _check(q.dim() == 3, "q must be [num_seqs][num_q_heads][head_dim]")
    S, Hq, D = q.shape
    B = int(block_size)
    _check(k_cache.dim() == 5 and k_cache.shape[2] * 8 == D and k_cache.shape[3] == B
           and k_cache.shape[4] == 8, "k_cache must be [num_blocks][Hkv][D/8][block_size][8]")
    NB, Hkv = int(k_cache.shape[0]), int(k_cache.shape[1])
    _check(_v_pool_ok(v_cache, NB, Hkv, D, B), V_POOL_TEXT)
    _check(block_tables.dim() == 2 and block_tables.shape[0] == S,
           "block_tables must be [num_seqs][max_blocks_per_seq]")
    _check(context_lens.dim() == 1 and context_lens.shape[0] == S, "context_lens must be [num_seqs]")
    for t in (q, k_cache, v_cache):
        _check(t.dtype == torch.bfloat16, "q/k_cache/v_cache: bf16")
    _check(q.is_contiguous(), "q must be contiguous")
    _check(pools_ok(k_cache, v_cache), POOLS_TEXT)
    for t in (block_tables, context_lens):
        _check(t.dtype == torch.int32 and t.is_contiguous(), "tables/lengths: contiguous int32")
    devs = {t.device for t in (q, k_cache, v_cache, block_tables, context_lens)}
    _check(len(devs) == 1 and q.is_cuda, "all tensors must be on one GPU")
    return S, Hq, Hkv, D, NB, int(block_tables.shape[1])


def paged_attn_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                      max_context_len) -> int:
    return int(load_library().paged_attn_decode_workspace_bytes(
        int(num_seqs), int(num_q_heads), int(num_kv_heads), int(head_dim), int(block_size),
        int(max_context_len)))


def new_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
                  device):
    """A workspace tensor for paged_attn_decode with these sizes."""
    import torch

    with torch.cuda.device(device):
        need = paged_attn_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                 block_size, max_context_len)
        return torch.empty(max(need, 16), dtype=torch.uint8, device=device)


def paged_attn_decode(q, k_cache, v_cache, block_tables, context_lens, block_size, scale,
                      out=None, *, max_context_len=None, workspace=None, stream=None):
    """Paged decode attention (see ``include/pkv.h``).  Returns ``out``.

    ``max_context_len`` defaults to ``max_blocks_per_seq * block_size`` (a bound
    known without reading the lengths back); ``workspace`` (see ``new_workspace``)
    is allocated when not given; ``stream`` defaults to torch's current stream on
    q's device."""
    import torch

    lib = load_library()
    S, Hq, Hkv, D, NB, M = decode_shapes(q, k_cache, v_cache, block_tables, context_lens,
                                         block_size)
    if max_context_len is None:
        max_context_len = M * int(block_size)
    with _on_stream(q, stream):
        if out is None:
            out = torch.empty_like(q)
        _check(out.shape == q.shape and out.dtype == torch.bfloat16 and out.is_contiguous()
               and out.device == q.device, "out must match q")
        if workspace is None:
            workspace = new_workspace(S, Hq, Hkv, D, block_size, max_context_len, q.device)
        _check(workspace.is_cuda and workspace.device == q.device and workspace.is_contiguous(),
               "workspace must be a contiguous tensor on q's device")
        ws_bytes = workspace.numel() * workspace.element_size()
        rc = lib.paged_attn_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                   block_tables.data_ptr(), context_lens.data_ptr(),
                                   int(block_size), float(scale), out.data_ptr(), S, Hq, Hkv, D,
                                   M, NB, int(max_context_len), workspace.data_ptr(), ws_bytes,
                                   _stream_handle(q, stream))
    if rc != 0:
        raise PkvError(rc, "paged_attn_decode")
    return out


def paged_attn_decode_shared_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                             block_size, max_context_len, num_groups,
                                             max_group_size, max_prefix_len) -> int:
    return int(load_library().paged_attn_decode_shared_workspace_bytes(
        int(num_seqs), int(num_q_heads), int(num_kv_heads), int(head_dim), int(block_size),
        int(max_context_len), int(num_groups), int(max_group_size), int(max_prefix_len)))


def paged_attn_decode_shared(q, k_cache, v_cache, block_tables, context_lens, group_first,
                             prefix_lens, block_size, scale, out=None, *, max_group_size,
                             max_prefix_len, max_context_len=None, workspace=None, stream=None):
    """Paged decode over a batch whose groups of consecutive sequences share a prefix
    (see ``include/pkv.h``): ``group_first`` int32 [num_groups + 1] (device) are
    the group offsets, ``prefix_lens`` int32 [num_seqs] (device) each sequence's
    shared positions; ``max_group_size`` and ``max_prefix_len`` are host-side
    bounds (``BlockManager.shared_groups`` gives all four).  Returns ``out``."""
    import torch

    lib = load_library()
    S, Hq, Hkv, D, NB, M = decode_shapes(q, k_cache, v_cache, block_tables, context_lens,
                                         block_size)
    _check(group_first.dim() == 1 and group_first.shape[0] >= 1, "group_first: [num_groups + 1]")
    _check(prefix_lens.dim() == 1 and prefix_lens.shape[0] == S, "prefix_lens: [num_seqs]")
    for t in (group_first, prefix_lens):
        _check(t.dtype == torch.int32 and t.is_contiguous() and t.device == q.device,
               "group_first/prefix_lens: contiguous int32 on q's device")
    NG = int(group_first.shape[0]) - 1
    if max_context_len is None:
        max_context_len = M * int(block_size)
    with _on_stream(q, stream):
        if out is None:
            out = torch.empty_like(q)
        _check(out.shape == q.shape and out.dtype == torch.bfloat16 and out.is_contiguous()
               and out.device == q.device, "out must match q")
        if workspace is None:
            need = paged_attn_decode_shared_workspace_bytes(S, Hq, Hkv, D, block_size,
                                                            max_context_len, NG, max_group_size,
                                                            max_prefix_len)
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        _check(workspace.is_cuda and workspace.device == q.device and workspace.is_contiguous(),
               "workspace must be a contiguous tensor on q's device")
        ws_bytes = workspace.numel() * workspace.element_size()
        rc = lib.paged_attn_decode_shared(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                          block_tables.data_ptr(), context_lens.data_ptr(),
                                          group_first.data_ptr(), prefix_lens.data_ptr(), NG,
                                          int(max_group_size), int(max_prefix_len),
                                          int(block_size), float(scale), out.data_ptr(), S, Hq,
                                          Hkv, D, M, NB, int(max_context_len),
                                          workspace.data_ptr(), ws_bytes,
                                          _stream_handle(q, stream))
    if rc != 0:
        raise PkvError(rc, "paged_attn_decode_shared")
    return out


NOALLOC_SCRATCH_BYTES = 8 << 20   # PKV_NOALLOC_SCRATCH_BYTES of include/pkv.h


def paged_attn_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, block_size, scale,
                              out, *, max_context_len=None, stream=None):
    """paged_attn_decode through the entry point that allocates nothing (see
    ``include/pkv.h``): the split-K scratch is the library's own per-GPU array, and
    ``out`` must be given.  Calls whose work overlaps in time on one GPU race on
    that scratch.  Returns ``out``."""
    import torch

    lib = load_library()
    S, Hq, Hkv, D, NB, M = decode_shapes(q, k_cache, v_cache, block_tables, context_lens,
                                         block_size)
    _check(out is not None and out.shape == q.shape and out.dtype == torch.bfloat16
           and out.is_contiguous() and out.device == q.device, "out must match q")
    if max_context_len is None:
        max_context_len = M * int(block_size)
    with torch.cuda.device(q.device):
        rc = lib.paged_attn_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                           block_tables.data_ptr(), context_lens.data_ptr(),
                                           int(block_size), float(scale), out.data_ptr(), S, Hq,
                                           Hkv, D, M, NB, int(max_context_len),
                                           _stream_handle(q, stream))
    if rc != 0:
        raise PkvError(rc, "paged_attn_decode_noalloc")
    return out


def paged_attn_decode_fp8(q, k_cache, v_cache, block_tables, context_lens, block_size, scale,
                          k_scale, v_scale, out=None, *, max_context_len=None, workspace=None,
                          stream=None):
    """Paged decode attention over fp8 (E4M3FN) pools (see ``include/pkv.h``).
    ``k_cache`` uint8 [num_blocks][Hkv][D/16][block_size][16], ``v_cache`` uint8
    [num_blocks][Hkv][16][block_size/4][D/16][4]; keys are code * k_scale, values
    code * v_scale.  Workspace as for paged_attn_decode.  Returns ``out``."""
    import torch

    lib = load_library()
    _check(q.dim() == 3, "q must be [num_seqs][num_q_heads][head_dim]")
    S, Hq, D = q.shape
    B = int(block_size)
    _check(k_cache.dim() == 5 and k_cache.shape[2] * 16 == D and k_cache.shape[3] == B
           and k_cache.shape[4] == 16, "k_cache must be [num_blocks][Hkv][D/16][block_size][16]")
    NB, Hkv = int(k_cache.shape[0]), int(k_cache.shape[1])
    _check(tuple(v_cache.shape) == (NB, Hkv, 16, B // 4, D // 16, 4),
           "v_cache must be [num_blocks][Hkv][16][block_size/4][D/16][4]")
    _check(q.dtype == torch.bfloat16 and q.is_contiguous(), "q: contiguous bf16")
    _check(k_cache.dtype == torch.uint8 and v_cache.dtype == torch.uint8
           and pools_ok(k_cache, v_cache), "fp8 pools: uint8 codes; " + POOLS_TEXT)
    _check(block_tables.dim() == 2 and block_tables.shape[0] == S,
           "block_tables must be [num_seqs][max_blocks_per_seq]")
    _check(context_lens.dim() == 1 and context_lens.shape[0] == S, "context_lens must be [num_seqs]")
    for t in (block_tables, context_lens):
        _check(t.dtype == torch.int32 and t.is_contiguous(), "tables/lengths: contiguous int32")
    devs = {t.device for t in (q, k_cache, v_cache, block_tables, context_lens)}
    _check(len(devs) == 1 and q.is_cuda, "all tensors must be on one GPU")
    M = int(block_tables.shape[1])
    if max_context_len is None:
        max_context_len = M * B
    with _on_stream(q, stream):
        if out is None:
            out = torch.empty_like(q)
        _check(out.shape == q.shape and out.dtype == torch.bfloat16 and out.is_contiguous()
               and out.device == q.device, "out must match q")
        if workspace is None:
            workspace = new_workspace(S, Hq, Hkv, D, B, max_context_len, q.device)
        _check(workspace.is_cuda and workspace.device == q.device and workspace.is_contiguous(),
               "workspace must be a contiguous tensor on q's device")
        ws_bytes = workspace.numel() * workspace.element_size()
        rc = lib.paged_attn_decode_fp8(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                       block_tables.data_ptr(), context_lens.data_ptr(), B,
                                       float(scale), float(k_scale), float(v_scale),
                                       out.data_ptr(), S, Hq, Hkv, D, M, NB,
                                       int(max_context_len), workspace.data_ptr(), ws_bytes,
                                       _stream_handle(q, stream))
    if rc != 0:
        raise PkvError(rc, "paged_attn_decode_fp8")
    return out


def paged_attn_decode_append(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                             block_size, scale, out=None, *, max_context_len=None, workspace=None,
                             k_scale=None, v_scale=None, stream=None):
    """One decode step with its KV append (see ``include/pkv.h``): the rows
    k_new / v_new (bf16 [num_seqs][Hkv][D]) of each sequence's newest position
    (context_lens[s] - 1) go into their slots, and attention runs over all
    context_lens[s] positions.  With ``k_scale`` / ``v_scale`` the pools are fp8
    (layouts as in paged_attn_decode_fp8).  Returns ``out``."""
    import torch

    lib = load_library()
    fp8 = k_scale is not None or v_scale is not None
    _check(q.dim() == 3, "q must be [num_seqs][num_q_heads][head_dim]")
    S, Hq, D = q.shape
    B = int(block_size)
    if fp8:
        _check(k_scale is not None and v_scale is not None, "fp8 pools need k_scale and v_scale")
        _check(k_cache.dim() == 5 and k_cache.shape[2] * 16 == D and k_cache.shape[3] == B
               and k_cache.shape[4] == 16, "k_cache must be [num_blocks][Hkv][D/16][block_size][16]")
        NB, Hkv = int(k_cache.shape[0]), int(k_cache.shape[1])
        _check(tuple(v_cache.shape) == (NB, Hkv, 16, B // 4, D // 16, 4),
               "v_cache must be [num_blocks][Hkv][16][block_size/4][D/16][4]")
        _check(k_cache.dtype == torch.uint8 and v_cache.dtype == torch.uint8
               and pools_ok(k_cache, v_cache), "fp8 pools: uint8 codes; " + POOLS_TEXT)
        _check(q.dtype == torch.bfloat16 and q.is_contiguous(), "q: contiguous bf16")
        _check(block_tables.dim() == 2 and block_tables.shape[0] == S
               and context_lens.dim() == 1 and context_lens.shape[0] == S,
               "block_tables [num_seqs][max_blocks_per_seq], context_lens [num_seqs]")
        for t in (block_tables, context_lens):
            _check(t.dtype == torch.int32 and t.is_contiguous(), "tables/lengths: contiguous int32")
        M = int(block_tables.shape[1])
    else:
        S, Hq, Hkv, D, NB, M = decode_shapes(q, k_cache, v_cache, block_tables, context_lens, B)
    for t in (k_new, v_new):
        _check(tuple(t.shape) == (S, Hkv, D) and t.dtype == torch.bfloat16 and t.is_contiguous(),
               "k_new/v_new must be contiguous bf16 [num_seqs][Hkv][D]")
    devs = {t.device for t in (q, k_new, v_new, k_cache, v_cache, block_tables, context_lens)}
    _check(len(devs) == 1 and q.is_cuda, "all tensors must be on one GPU")
    if max_context_len is None:
        max_context_len = M * B
    with _on_stream(q, stream):
        if out is None:
            out = torch.empty_like(q)
        _check(out.shape == q.shape and out.dtype == torch.bfloat16 and out.is_contiguous()
               and out.device == q.device, "out must match q")
        if workspace is None:
            workspace = new_workspace(S, Hq, Hkv, D, B, max_context_len, q.device)
        _check(workspace.is_cuda and workspace.device == q.device and workspace.is_contiguous(),
               "workspace must be a contiguous tensor on q's device")
        ws_bytes = workspace.numel() * workspace.element_size()
        head = (q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
                v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), B,
                float(scale))
        tail = (out.data_ptr(), S, Hq, Hkv, D, M, NB, int(max_context_len), workspace.data_ptr(),
                ws_bytes, _stream_handle(q, stream))
        if fp8:
            rc = lib.paged_attn_decode_append_fp8(*head, float(k_scale), float(v_scale), *tail)
        else:
            rc = lib.paged_attn_decode_append(*head, *tail)
    if rc != 0:
        raise PkvError(rc, "paged_attn_decode_append_fp8" if fp8 else "paged_attn_decode_append")
    return out


def paged_attn_multi_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                     max_context_len, max_query_len) -> int:
    return int(load_library().paged_attn_multi_workspace_bytes(
        int(num_seqs), int(num_q_heads), int(num_kv_heads), int(head_dim), int(block_size),
        int(max_context_len), int(max_query_len)))


def new_multi_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                        max_context_len, max_query_len, device):
    """A workspace tensor for paged_attn_multi with these sizes."""
    import torch

    with torch.cuda.device(device):
        need = paged_attn_multi_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                block_size, max_context_len, max_query_len)
        return torch.empty(max(need, 16), dtype=torch.uint8, device=device)


def _fp8_pool_shapes(q3, k_cache, v_cache, block_tables, context_lens, block_size):
    """(Hkv, NB, M) of fp8 pools after host-side checks (q3: q seen as [S][rows][D])."""
    import torch

    S, _, D = q3.shape
    B = int(block_size)
    _check(k_cache.dim() == 5 and k_cache.shape[2] * 16 == D and k_cache.shape[3] == B
           and k_cache.shape[4] == 16, "k_cache must be [num_blocks][Hkv][D/16][block_size][16]")
    NB, Hkv = int(k_cache.shape[0]), int(k_cache.shape[1])
    _check(tuple(v_cache.shape) == (NB, Hkv, 16, B // 4, D // 16, 4),
           "v_cache must be [num_blocks][Hkv][16][block_size/4][D/16][4]")
    _check(q3.dtype == torch.bfloat16 and q3.is_contiguous(), "q: contiguous bf16")
    _check(k_cache.dtype == torch.uint8 and v_cache.dtype == torch.uint8
           and pools_ok(k_cache, v_cache), "fp8 pools: uint8 codes; " + POOLS_TEXT)
    _check(block_tables.dim() == 2 and block_tables.shape[0] == S,
           "block_tables must be [num_seqs][max_blocks_per_seq]")
    _check(context_lens.dim() == 1 and context_lens.shape[0] == S, "context_lens must be [num_seqs]")
    for t in (block_tables, context_lens):
        _check(t.dtype == torch.int32 and t.is_contiguous(), "tables/lengths: contiguous int32")
    devs = {t.device for t in (q3, k_cache, v_cache, block_tables, context_lens)}
    _check(len(devs) == 1 and q3.is_cuda, "all tensors must be on one GPU")
    return Hkv, NB, int(block_tables.shape[1])


def paged_attn_multi(q, k_cache, v_cache, block_tables, context_lens, query_lens, block_size,
                     scale, out=None, *, max_context_len=None, workspace=None, stream=None,
                     k_scale=None, v_scale=None):
    """Multi-token paged attention with a causal mask (see ``include/pkv.h``).
    ``q`` is [num_seqs][max_query_len][num_q_heads][head_dim] bf16, ``query_lens``
    int32 [num_seqs].  Returns ``out`` (same shape as q; rows past a sequence's
    query tokens are zero).  With ``k_scale``/``v_scale`` given, the pools are fp8
    (E4M3FN codes in the fp8 layouts) and ``paged_attn_multi_fp8`` runs."""
    import torch

    lib = load_library()
    _check(q.dim() == 4, "q must be [num_seqs][max_query_len][num_q_heads][head_dim]")
    S, Q, Hq, D = q.shape
    _check(q.is_contiguous(), "q must be contiguous")
    fp8 = k_scale is not None or v_scale is not None
    _check(not fp8 or (k_scale is not None and v_scale is not None), "give both k_scale and v_scale")
    # the pools, tables and lengths are checked as for decode, on q seen as [S][Q*Hq][D]
    if fp8:
        Hkv, NB, M = _fp8_pool_shapes(q.view(S, Q * Hq, D), k_cache, v_cache, block_tables,
                                      context_lens, block_size)
    else:
        _, _, Hkv, _, NB, M = decode_shapes(q.view(S, Q * Hq, D), k_cache, v_cache, block_tables,
                                            context_lens, block_size)
    _check(query_lens.dim() == 1 and query_lens.shape[0] == S and query_lens.dtype == torch.int32
           and query_lens.is_contiguous() and query_lens.device == q.device,
           "query_lens must be contiguous int32 [num_seqs] on q's device")
    if max_context_len is None:
        max_context_len = M * int(block_size)
    with _on_stream(q, stream):
        if out is None:
            out = torch.empty_like(q)
        _check(out.shape == q.shape and out.dtype == torch.bfloat16 and out.is_contiguous()
               and out.device == q.device, "out must match q")
        if workspace is None:
            workspace = new_multi_workspace(S, Hq, Hkv, D, block_size, max_context_len, Q, q.device)
        _check(workspace.is_cuda and workspace.device == q.device and workspace.is_contiguous(),
               "workspace must be a contiguous tensor on q's device")
        ws_bytes = workspace.numel() * workspace.element_size()
        ptrs = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                context_lens.data_ptr(), query_lens.data_ptr(), Q, int(block_size), float(scale))
        rest = (out.data_ptr(), S, Hq, Hkv, D, M, NB, int(max_context_len), workspace.data_ptr(),
                ws_bytes, _stream_handle(q, stream))
        if fp8:
            rc = lib.paged_attn_multi_fp8(*ptrs, float(k_scale), float(v_scale), *rest)
        else:
            rc = lib.paged_attn_multi(*ptrs, *rest)
    if rc != 0:
        raise PkvError(rc, "paged_attn_multi_fp8" if fp8 else "paged_attn_multi")
    return out


def kv_append(k_new, v_new, k_cache, v_cache, block_tables, token_seq, token_pos, block_size,
              stream=None):
    """Write new tokens' K/V rows ([T][Hkv][D] bf16) into their slots through the
    block table (see ``include/pkv.h``).  token_seq/token_pos: int32 [T]."""
    import torch

    lib = load_library()
    _check(k_new.dim() == 3 and v_new.shape == k_new.shape, "k_new/v_new must be [T][Hkv][D]")
    T, Hkv, D = k_new.shape
    B = int(block_size)
    _check(k_cache.dim() == 5 and tuple(k_cache.shape[1:]) == (Hkv, D // 8, B, 8),
           "k_cache must be [num_blocks][Hkv][D/8][block_size][8]")
    NB = int(k_cache.shape[0])
    _check(_v_pool_ok(v_cache, NB, Hkv, D, B), V_POOL_TEXT)
    for t in (k_new, v_new, k_cache, v_cache):
        _check(t.dtype == torch.bfloat16, "bf16 tensors")
    _check(k_new.is_contiguous() and v_new.is_contiguous(), "k_new/v_new must be contiguous")
    _check(pools_ok(k_cache, v_cache), POOLS_TEXT)
    for t in (block_tables, token_seq, token_pos):
        _check(t.dtype == torch.int32 and t.is_contiguous(), "int32 contiguous tensors")
    _check(token_seq.numel() == T and token_pos.numel() == T, "one sequence id and position per token")
    _check(block_tables.dim() == 2, "block_tables must be [num_seqs][max_blocks_per_seq]")
    devs = {t.device for t in (k_new, v_new, k_cache, v_cache, block_tables, token_seq, token_pos)}
    _check(len(devs) == 1 and k_cache.is_cuda, "all tensors must be on one GPU")
    with _on_stream(k_cache, stream):
        rc = lib.kv_append(k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
                           v_cache.data_ptr(), block_tables.data_ptr(), token_seq.data_ptr(),
                           token_pos.data_ptr(), T, int(block_tables.shape[0]), Hkv, D, B,
                           int(block_tables.shape[1]), NB, _stream_handle(k_cache, stream))
    if rc != 0:
        raise PkvError(rc, "kv_append")


def kv_append_fp8(k_new, v_new, k_cache, v_cache, block_tables, token_seq, token_pos, block_size,
                  k_scale, v_scale, stream=None):
    """Quantise new tokens' K/V rows ([T][Hkv][D] bf16) into fp8 pools through the
    block table (see ``include/pkv.h``): code = E4M3(x / scale), nearest even,
    saturating.  token_seq/token_pos: int32 [T]."""
    import torch

    lib = load_library()
    _check(k_new.dim() == 3 and v_new.shape == k_new.shape, "k_new/v_new must be [T][Hkv][D]")
    T, Hkv, D = k_new.shape
    B = int(block_size)
    _check(k_cache.dim() == 5 and tuple(k_cache.shape[1:]) == (Hkv, D // 16, B, 16),
           "k_cache must be [num_blocks][Hkv][D/16][block_size][16]")
    NB = int(k_cache.shape[0])
    _check(tuple(v_cache.shape) == (NB, Hkv, 16, B // 4, D // 16, 4),
           "v_cache must be [num_blocks][Hkv][16][block_size/4][D/16][4]")
    for t in (k_new, v_new):
        _check(t.dtype == torch.bfloat16 and t.is_contiguous(), "k_new/v_new: contiguous bf16")
    _check(k_cache.dtype == torch.uint8 and v_cache.dtype == torch.uint8
           and pools_ok(k_cache, v_cache), "fp8 pools: uint8 codes; " + POOLS_TEXT)
    for t in (block_tables, token_seq, token_pos):
        _check(t.dtype == torch.int32 and t.is_contiguous(), "int32 contiguous tensors")
    _check(token_seq.numel() == T and token_pos.numel() == T, "one sequence id and position per token")
    _check(block_tables.dim() == 2, "block_tables must be [num_seqs][max_blocks_per_seq]")
    devs = {t.device for t in (k_new, v_new, k_cache, v_cache, block_tables, token_seq, token_pos)}
    _check(len(devs) == 1 and k_cache.is_cuda, "all tensors must be on one GPU")
    with _on_stream(k_cache, stream):
        rc = lib.kv_append_fp8(k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
                               v_cache.data_ptr(), block_tables.data_ptr(), token_seq.data_ptr(),
                               token_pos.data_ptr(), T, int(block_tables.shape[0]), Hkv, D, B,
                               int(block_tables.shape[1]), NB, float(k_scale), float(v_scale),
                               _stream_handle(k_cache, stream))
    if rc != 0:
        raise PkvError(rc, "kv_append_fp8")


def copy_blocks(k_caches, v_caches, src_dst_pairs, stream=None):
    """Copy-on-write block copy over every layer's K and V pool (see ``include/pkv.h``).
    ``k_caches``/``v_caches``: sequences of per-layer pool tensors of equal shape;
    ``src_dst_pairs``: int32 [num_pairs][2] on the pools' device."""
    import torch

    lib = load_library()
    k_caches, v_caches = list(k_caches), list(v_caches)
    _check(len(k_caches) == len(v_caches), "as many K pools as V pools")
    n_layers = len(k_caches)
    _check(src_dst_pairs.dtype == torch.int32 and src_dst_pairs.is_contiguous()
           and src_dst_pairs.dim() == 2 and src_dst_pairs.shape[1] == 2,
           "src_dst_pairs must be contiguous int32 [num_pairs][2]")
    n_pairs = int(src_dst_pairs.shape[0])
    if n_layers == 0 or n_pairs == 0:
        return
    ref = k_caches[0]
    nb = int(ref.shape[0])
    nbytes = ref.numel() * ref.element_size()
    for t in k_caches + v_caches:
        _check(t.device == ref.device and t.shape[0] == nb
               and t.numel() * t.element_size() == nbytes, "pools must match in shape and device")
    for k, v in zip(k_caches, v_caches):
        _check(pools_ok(k, v), POOLS_TEXT)
    _check(src_dst_pairs.device == ref.device, "src_dst_pairs must be on the pools' device")
    kp = (ctypes.c_void_p * n_layers)(*[t.data_ptr() for t in k_caches])
    vp = (ctypes.c_void_p * n_layers)(*[t.data_ptr() for t in v_caches])
    with _on_stream(ref, stream):
        rc = lib.copy_blocks(ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(vp, ctypes.c_void_p),
                             n_layers, nb, nbytes // nb, src_dst_pairs.data_ptr(), n_pairs,
                             _stream_handle(ref, stream))
    if rc != 0:
        raise PkvError(rc, "copy_blocks")


CHECK_KINDS = {1: "context length outside [0, max_blocks_per_seq*block_size]",
               2: "block-table entry outside [0, num_blocks)",
               3: "query length outside [0, min(context length, max_query_len)]"}


def check_batch(block_tables, context_lens, block_size, num_blocks, query_lens=None,
                max_query_len=0, stream=None):
    """Check the table contract on the device (see ``pkv_check_batch`` in
    ``include/pkv.h``).  Waits for the stream and returns None when every sequence
    meets it, else ``(sequence, kind, text)`` for the first one that does not."""
    import torch

    lib = load_library()
    for t in (block_tables, context_lens) + ((query_lens,) if query_lens is not None else ()):
        _check(t.dtype == torch.int32 and t.is_contiguous() and t.is_cuda, "int32 contiguous GPU tensors")
    _check(block_tables.dim() == 2 and context_lens.numel() == block_tables.shape[0],
           "block_tables [num_seqs][max_blocks_per_seq] and context_lens [num_seqs]")
    S, M = int(block_tables.shape[0]), int(block_tables.shape[1])
    if query_lens is not None:
        _check(query_lens.numel() == S, "query_lens [num_seqs]")
    with _on_stream(block_tables, stream):
        st = torch.cuda.current_stream(block_tables.device)
        result = torch.empty(1, dtype=torch.int32, device=block_tables.device)
        rc = lib.pkv_check_batch(block_tables.data_ptr(), context_lens.data_ptr(),
                                 query_lens.data_ptr() if query_lens is not None else None, S, M,
                                 int(num_blocks), int(block_size), int(max_query_len),
                                 result.data_ptr(), ctypes.c_void_p(st.cuda_stream))
        if rc != 0:
            raise PkvError(rc, "pkv_check_batch")
        st.synchronize()
    code = int(result.item())
    if code < 0:
        return None
    return code // 4, code % 4, CHECK_KINDS.get(code % 4, "unknown")
