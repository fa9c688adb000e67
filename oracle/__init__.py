"""CPU oracle for paged decode attention and the copy-on-write block copy.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library (``paged_kv_cache_280_amd``) never imports it, and the two share no code.

``oracle.cpp`` holds the plain loops (fp32 oracle, fp64 twin, per-row debug form
with the softmax weights, multi-token causal attention, decode over fp8 blocks and
the E4M3FN decoding, KV append, byte copy of blocks).  This module compiles it with
``g++ -O2 -fopenmp`` (no fast-math) and exposes numpy-level wrappers.

Parity pins (what fixes the oracle other than itself) live in
``tests/test_oracle_pins.py``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
# PKV_ORACLE_LIBRARY names another build of oracle.cpp to load (the CPU tests use the
# sanitized build of build_sanitized); unset, liboracle.so beside this file
_LIB_OVERRIDE = os.environ.get("PKV_ORACLE_LIBRARY")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.cpp`` into ``liboracle.so`` beside it and return the path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(out: str) -> str:
    """Compile ``oracle.cpp`` with AddressSanitizer and UndefinedBehaviorSanitizer (any
    finding aborts) into ``out``; the process that loads it must preload GCC's
    libasan (``g++ -print-file-name=libasan.so``)."""
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fopenmp", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", _SRC, "-o", out]
    subprocess.run(cmd, check=True)
    return out


def _bind(lib):
    p = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.oracle_paged_decode_f32.argtypes = [p, p, p, p, p, i32, ctypes.c_float, p, i32, i32,
                                            i32, i32, i32, i64, i32]
    lib.oracle_paged_decode_f32.restype = ctypes.c_int
    lib.oracle_paged_decode_f64.argtypes = [p, p, p, p, p, i32, ctypes.c_double, p, i32, i32,
                                            i32, i32, i32, i64, i32]
    lib.oracle_paged_decode_f64.restype = ctypes.c_int
    lib.oracle_paged_decode_probs_f32.argtypes = [p, p, p, p, p, i32, ctypes.c_float, i32,
                                                  i32, i32, i32, i32, i64, i32, i32, p, p]
    lib.oracle_paged_decode_probs_f32.restype = ctypes.c_int
    lib.oracle_paged_attn_multi_f32.argtypes = [p, p, p, p, p, p, i32, i32, ctypes.c_float, p,
                                                 i32, i32, i32, i32, i32, i64, i32]
    lib.oracle_paged_attn_multi_f32.restype = ctypes.c_int
    lib.oracle_paged_decode_fp8_f32.argtypes = [p, p, p, p, p, i32, ctypes.c_float,
                                                ctypes.c_float, ctypes.c_float, p, i32, i32, i32,
                                                i32, i32, i64, i32]
    lib.oracle_paged_decode_fp8_f32.restype = ctypes.c_int
    lib.oracle_fp8_e4m3_to_f32.argtypes = [p, p, i64]
    lib.oracle_fp8_e4m3_to_f32.restype = None
    lib.oracle_fp8_e4m3_from_f32.argtypes = [p, p, i64]
    lib.oracle_fp8_e4m3_from_f32.restype = None
    lib.oracle_kv_append_fp8.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i64,
                                         ctypes.c_float, ctypes.c_float]
    lib.oracle_kv_append_fp8.restype = ctypes.c_int
    lib.oracle_paged_attn_multi_fp8_f32.argtypes = [p, p, p, p, p, p, i32, i32, ctypes.c_float,
                                                    ctypes.c_float, ctypes.c_float, p, i32, i32,
                                                    i32, i32, i32, i64, i32]
    lib.oracle_paged_attn_multi_fp8_f32.restype = ctypes.c_int
    lib.oracle_kv_append.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i64]
    lib.oracle_kv_append.restype = ctypes.c_int
    lib.oracle_copy_blocks.argtypes = [p, p, i32, i64, i64, p, i32]
    lib.oracle_copy_blocks.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            _lib = _bind(ctypes.CDLL(_LIB_OVERRIDE))
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _u16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        a = a.view(np.uint16)
    return a


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


class OracleError(RuntimeError):
    pass


def paged_decode(q, k_pool, v_pool, block_tables, context_lens, block_size, scale,
                 num_kv_heads, precision="f32", threads=0, lib=None):
    """Reference decode.  Arrays are numpy; q/k_pool/v_pool hold bf16 bit patterns
    (uint16 or int16).  Shapes: q [S][Hq][D]; k_pool [NB][Hkv][D/8][B][8];
    v_pool [NB][Hkv][B/Bt][D][Bt], Bt = min(B, 16); block_tables [S][M] int32;
    context_lens [S] int32.
    Returns float32 (or float64) [S][Hq][D]."""
    q, kp, vp = _u16(q), _u16(k_pool), _u16(v_pool)
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    S, Hq, D = q.shape
    M = tables.shape[1] if tables.ndim == 2 else 0
    NB = kp.shape[0]
    B = int(block_size)
    if kp.size != NB * num_kv_heads * D * B or vp.size != kp.size:
        raise OracleError("pool size does not match [NB][Hkv][..] with D=%d B=%d" % (D, B))
    lib = lib or _load()
    if precision == "f32":
        out = np.zeros((S, Hq, D), np.float32)
        rc = lib.oracle_paged_decode_f32(_ptr(q), _ptr(kp), _ptr(vp), _ptr(tables), _ptr(lens),
                                         B, float(scale), _ptr(out), S, Hq, num_kv_heads, D, M,
                                         NB, int(threads))
    elif precision == "f64":
        out = np.zeros((S, Hq, D), np.float64)
        rc = lib.oracle_paged_decode_f64(_ptr(q), _ptr(kp), _ptr(vp), _ptr(tables), _ptr(lens),
                                         B, float(scale), _ptr(out), S, Hq, num_kv_heads, D, M,
                                         NB, int(threads))
    else:
        raise ValueError(precision)
    if rc != 0:
        raise OracleError("oracle_paged_decode returned %d" % rc)
    return out


def paged_attn_multi(q, k_pool, v_pool, block_tables, context_lens, query_lens, block_size,
                     scale, num_kv_heads, threads=0, lib=None):
    """Reference multi-token attention.  q: bf16 bits [S][Qmax][Hq][D]; the last
    query_lens[s] positions of sequence s are its query tokens, each attending
    causally.  Returns float32 [S][Qmax][Hq][D] (rows past query_lens[s] are 0)."""
    q, kp, vp = _u16(q), _u16(k_pool), _u16(v_pool)
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    qlens = np.ascontiguousarray(query_lens, dtype=np.int32)
    S, Qmax, Hq, D = q.shape
    out = np.zeros((S, Qmax, Hq, D), np.float32)
    rc = (lib or _load()).oracle_paged_attn_multi_f32(
        _ptr(q), _ptr(kp), _ptr(vp), _ptr(tables), _ptr(lens), _ptr(qlens), Qmax,
        int(block_size), float(scale), _ptr(out), S, Hq, num_kv_heads, D, tables.shape[1],
        kp.shape[0], int(threads))
    if rc != 0:
        raise OracleError("oracle_paged_attn_multi returned %d" % rc)
    return out


def paged_attn_multi_fp8(q, k_pool, v_pool, block_tables, context_lens, query_lens, block_size,
                         scale, k_scale, v_scale, num_kv_heads, threads=0, lib=None):
    """Reference multi-token attention over fp8 pools (layouts as paged_decode_fp8;
    q bf16 bits [S][Qmax][Hq][D]).  Returns float32 [S][Qmax][Hq][D]."""
    q = _u16(q)
    kp = np.ascontiguousarray(k_pool, dtype=np.uint8)
    vp = np.ascontiguousarray(v_pool, dtype=np.uint8)
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    qlens = np.ascontiguousarray(query_lens, dtype=np.int32)
    S, Qmax, Hq, D = q.shape
    out = np.zeros((S, Qmax, Hq, D), np.float32)
    rc = (lib or _load()).oracle_paged_attn_multi_fp8_f32(
        _ptr(q), _ptr(kp), _ptr(vp), _ptr(tables), _ptr(lens), _ptr(qlens), Qmax,
        int(block_size), float(scale), float(k_scale), float(v_scale), _ptr(out), S, Hq,
        num_kv_heads, D, tables.shape[1], kp.shape[0], int(threads))
    if rc != 0:
        raise OracleError("oracle_paged_attn_multi_fp8 returned %d" % rc)
    return out


def paged_decode_probs(q, k_pool, v_pool, block_tables, context_lens, block_size, scale,
                       num_kv_heads, seq, head, lib=None):
    """Debug form: (out_row float32 [D], softmax weights float32 [L]) for one (seq, head)."""
    q, kp, vp = _u16(q), _u16(k_pool), _u16(v_pool)
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    S, Hq, D = q.shape
    M = tables.shape[1]
    L = int(lens[seq])
    out = np.zeros(D, np.float32)
    probs = np.zeros(max(L, 1), np.float32)
    rc = (lib or _load()).oracle_paged_decode_probs_f32(_ptr(q), _ptr(kp), _ptr(vp), _ptr(tables),
                                               _ptr(lens), int(block_size), float(scale), S, Hq,
                                               num_kv_heads, D, M, kp.shape[0], int(seq),
                                               int(head), _ptr(out), _ptr(probs))
    if rc != 0:
        raise OracleError("oracle_paged_decode_probs returned %d" % rc)
    return out, probs[:L]


def paged_decode_fp8(q, k_pool, v_pool, block_tables, context_lens, block_size, scale, k_scale,
                     v_scale, num_kv_heads, threads=0, lib=None):
    """Reference decode over fp8 pools: q bf16 bits [S][Hq][D]; k_pool uint8
    [NB][Hkv][D/16][B][16]; v_pool uint8 [NB][Hkv][16][B/4][D/16][4]; each code is
    an E4M3FN number, times k_scale (keys) or v_scale (values).  Returns float32
    [S][Hq][D]."""
    q = _u16(q)
    kp = np.ascontiguousarray(k_pool, dtype=np.uint8)
    vp = np.ascontiguousarray(v_pool, dtype=np.uint8)
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    S, Hq, D = q.shape
    NB, B = kp.shape[0], int(block_size)
    if kp.size != NB * num_kv_heads * D * B or vp.size != kp.size:
        raise OracleError("pool size does not match [NB][Hkv][..] with D=%d B=%d" % (D, B))
    out = np.zeros((S, Hq, D), np.float32)
    rc = (lib or _load()).oracle_paged_decode_fp8_f32(
        _ptr(q), _ptr(kp), _ptr(vp), _ptr(tables), _ptr(lens), B, float(scale), float(k_scale),
        float(v_scale), _ptr(out), S, Hq, num_kv_heads, D, tables.shape[1], NB, int(threads))
    if rc != 0:
        raise OracleError("oracle_paged_decode_fp8 returned %d" % rc)
    return out


def fp8_e4m3_to_f32(codes, lib=None):
    """The oracle's E4M3FN decoding of uint8 codes (float32, same shape)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.zeros(c.shape, np.float32)
    (lib or _load()).oracle_fp8_e4m3_to_f32(_ptr(c), _ptr(out), c.size)
    return out


def fp8_e4m3_from_f32(x, lib=None):
    """The oracle's E4M3FN encoding (nearest, ties to even, saturating at 448) of
    float32 values: uint8 codes, same shape."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(a.shape, np.uint8)
    (lib or _load()).oracle_fp8_e4m3_from_f32(_ptr(a), _ptr(out), a.size)
    return out


def kv_append_fp8(k_new, v_new, k_pool, v_pool, block_tables, token_seq, token_pos, block_size,
                  k_scale, v_scale, lib=None):
    """Quantise new tokens' rows (bf16 bits [T][Hkv][D]) into uint8 fp8 pools in place."""
    kn, vn = _u16(k_new), _u16(v_new)
    for a in (k_pool, v_pool):
        if a.dtype != np.uint8 or not a.flags["C_CONTIGUOUS"]:
            raise OracleError("fp8 pools must be contiguous uint8 arrays (written in place)")
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    seq = np.ascontiguousarray(token_seq, dtype=np.int32)
    pos = np.ascontiguousarray(token_pos, dtype=np.int32)
    T, H, D = kn.shape
    rc = (lib or _load()).oracle_kv_append_fp8(
        _ptr(kn), _ptr(vn), _ptr(k_pool), _ptr(v_pool), _ptr(tables), _ptr(seq), _ptr(pos), T,
        tables.shape[0], H, D, int(block_size), tables.shape[1], k_pool.shape[0], float(k_scale),
        float(v_scale))
    if rc != 0:
        raise OracleError("oracle_kv_append_fp8 returned %d" % rc)


def kv_append(k_new, v_new, k_pool, v_pool, block_tables, token_seq, token_pos, block_size,
              lib=None):
    """Write new tokens' rows (bf16 bits [T][Hkv][D]) into host pools in place."""
    kn, vn = _u16(k_new), _u16(v_new)
    if k_pool.dtype != np.uint16 or not k_pool.flags["C_CONTIGUOUS"] or \
            v_pool.dtype != np.uint16 or not v_pool.flags["C_CONTIGUOUS"]:
        raise OracleError("pools must be contiguous uint16 arrays (written in place)")
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    seq = np.ascontiguousarray(token_seq, dtype=np.int32)
    pos = np.ascontiguousarray(token_pos, dtype=np.int32)
    T, H, D = kn.shape
    rc = (lib or _load()).oracle_kv_append(_ptr(kn), _ptr(vn), _ptr(k_pool), _ptr(v_pool),
                                           _ptr(tables), _ptr(seq), _ptr(pos), T,
                                           tables.shape[0], H, D, int(block_size),
                                           tables.shape[1], k_pool.shape[0])
    if rc != 0:
        raise OracleError("oracle_kv_append returned %d" % rc)


def copy_blocks(k_pools, v_pools, pairs, lib=None):
    """Byte copy of whole blocks, in place, on lists of numpy pools (one per layer).
    ``pairs`` is int32 [P][2] of (src, dst)."""
    pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    n_layers = len(k_pools)
    if n_layers == 0 or pairs.shape[0] == 0:
        return
    nb = k_pools[0].shape[0]
    block_bytes = k_pools[0].nbytes // nb
    for a in list(k_pools) + list(v_pools):
        if not a.flags["C_CONTIGUOUS"] or a.nbytes != nb * block_bytes:
            raise OracleError("pools must be contiguous and of equal size")
    kp = (ctypes.c_void_p * n_layers)(*[_ptr(a) for a in k_pools])
    vp = (ctypes.c_void_p * n_layers)(*[_ptr(a) for a in v_pools])
    rc = (lib or _load()).oracle_copy_blocks(ctypes.cast(kp, ctypes.c_void_p),
                                    ctypes.cast(vp, ctypes.c_void_p), n_layers, nb, block_bytes,
                                    _ptr(pairs), pairs.shape[0])
    if rc != 0:
        raise OracleError("oracle_copy_blocks returned %d" % rc)


class Variant:
    """The same wrappers bound to another build of ``oracle.cpp`` (used by the
    tests that plant a mistake in a copy of the oracle and check that a pin fails)."""

    OracleError = OracleError

    def __init__(self, path: str):
        self._lib = _bind(ctypes.CDLL(path))

    def paged_decode(self, *args, **kwargs):
        return paged_decode(*args, lib=self._lib, **kwargs)

    def paged_decode_probs(self, *args, **kwargs):
        return paged_decode_probs(*args, lib=self._lib, **kwargs)

    def copy_blocks(self, *args, **kwargs):
        return copy_blocks(*args, lib=self._lib, **kwargs)

    def kv_append(self, *args, **kwargs):
        return kv_append(*args, lib=self._lib, **kwargs)

    def paged_attn_multi(self, *args, **kwargs):
        return paged_attn_multi(*args, lib=self._lib, **kwargs)

    def paged_attn_multi_fp8(self, *args, **kwargs):
        return paged_attn_multi_fp8(*args, lib=self._lib, **kwargs)

    def paged_decode_fp8(self, *args, **kwargs):
        return paged_decode_fp8(*args, lib=self._lib, **kwargs)

    def fp8_e4m3_to_f32(self, *args, **kwargs):
        return fp8_e4m3_to_f32(*args, lib=self._lib, **kwargs)

    def fp8_e4m3_from_f32(self, *args, **kwargs):
        return fp8_e4m3_from_f32(*args, lib=self._lib, **kwargs)

    def kv_append_fp8(self, *args, **kwargs):
        return kv_append_fp8(*args, lib=self._lib, **kwargs)
