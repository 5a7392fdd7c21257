"""fp64 CPU oracle for fused scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``attention_tiled_fmha_amd``) never imports, links or calls it, and the two
share no code: only the seeded input arrays pass between them.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over
(batch, head); no BLAS, no fast-math) and computes the plain definition
softmax(scale * Q K^T) V with the full score matrix materialised, as stated in
"FlashInfer kernel library ..." (zyxy.net/archives/24491), section 1.
``brute.py`` holds a pure-Python restatement for tiny shapes.

Inputs are numpy arrays: float64, float32, or uint16 holding bf16 bit patterns.
Outputs are always float64.

Every function here is pinned by ``tests/test_oracle_pins.py`` against closed
forms, invariants, a hand-derived example and scipy's softmax/logsumexp.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_F64, _F32, _BF16 = 0, 1, 2


def build(out_path=_LIB_PATH, src_path=_SRC, quiet=True):
    """Compile oracle.c with gcc into a shared library (plain -O2, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           src_path, "-o", out_path, "-lm"]
    subprocess.run(cmd, check=True, capture_output=quiet)
    return out_path


def load(path=_LIB_PATH):
    """Load a compiled oracle library and declare its signatures."""
    lib = ctypes.CDLL(path)
    vp, dp, ip = ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.c_int
    lib.oracle_attention.restype = ip
    lib.oracle_attention.argtypes = [vp, vp, vp, ip, dp, dp, ip, ip, ip, ip, ip,
                                     ip, ip, ctypes.c_double, ip]
    lib.oracle_decode_paged.restype = ip
    lib.oracle_decode_paged.argtypes = [vp, vp, vp, ip, vp, vp, dp, dp, ip, ip,
                                        ip, ip, ip, ip, ctypes.c_long,
                                        ctypes.c_double, ip]
    lib.oracle_prefill_paged.restype = ip
    lib.oracle_prefill_paged.argtypes = [vp, vp, vp, ip, vp, vp, dp, dp, ip, ip, ip, ip, ip,
                                         ip, ip, ctypes.c_long, ip, ctypes.c_double, ip]
    lib.oracle_flat_gemm.restype = ip
    lib.oracle_flat_gemm.argtypes = [vp, vp, ip, dp, ip, ip, ip, ip]
    lib.oracle_decode_paged_fp8.restype = ip
    cd = ctypes.c_double
    lib.oracle_decode_paged_fp8.argtypes = [vp, ip, vp, vp, cd, cd, vp, vp, dp, dp, ip, ip, ip,
                                            ip, ip, ip, ctypes.c_long, cd, ip]
    lib.oracle_e4m3_value.restype = cd
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_merge_states.restype = None
    lib.oracle_merge_states.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.c_long, ip]
    lib.oracle_unified_fallback_count.restype = ctypes.c_long
    lib.oracle_unified_fallback_count.argtypes = [vp, vp, ip, vp, vp, ip, ip, ip, ip, ip, ip,
                                                  ctypes.c_double, ip, ctypes.c_double,
                                                  ctypes.c_double]
    return lib


def _get():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        _lib = load()
    return _lib


def default_threads():
    return len(os.sched_getaffinity(0))


def _dtype_code(a):
    if a.dtype == np.float64:
        return _F64
    if a.dtype == np.float32:
        return _F32
    if a.dtype == np.uint16:
        return _BF16
    raise TypeError("oracle inputs must be float64, float32 or uint16 (bf16 bits), "
                    f"got {a.dtype}")


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def attention(q, k, v, causal, scale, threads=None, lib=None):
    """Dense attention.  q [B,Hq,Tq,D]; k, v [B,Hkv,Tk,D].

    Returns (o [B,Hq,Tq,D] fp64, lse [B,Hq,Tq] fp64), lse = ln sum_j exp(s_ij).
    """
    lib = lib or _get()
    q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k, v must share one element type")
    B, Hq, Tq, D = q.shape
    Bk, Hkv, Tk, Dk = k.shape
    if Bk != B or Dk != D or v.shape != k.shape:
        raise ValueError("shape mismatch")
    o = np.zeros((B, Hq, Tq, D), np.float64)
    lse = np.zeros((B, Hq, Tq), np.float64)
    rc = lib.oracle_attention(_ptr(q), _ptr(k), _ptr(v), dt, _dptr(o), _dptr(lse),
                              B, Hq, Hkv, Tq, Tk, D, int(bool(causal)),
                              float(scale), threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_attention failed ({rc})")
    return o, lse


def decode_paged(q, k_pages, v_pages, block_table, kv_lens, scale, threads=None,
                 lib=None):
    """One query row per (sequence, head) over a paged cache.

    q [B,Hq,D]; k_pages, v_pages [P,Hkv,page,D]; block_table int32 [B,maxp];
    kv_lens int32 [B].  Returns (o [B,Hq,D], lse [B,Hq]) in fp64.
    """
    lib = lib or _get()
    q = np.ascontiguousarray(q)
    k_pages = np.ascontiguousarray(k_pages)
    v_pages = np.ascontiguousarray(v_pages)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    kl = np.ascontiguousarray(kv_lens, dtype=np.int32)
    dt = _dtype_code(q)
    if _dtype_code(k_pages) != dt or _dtype_code(v_pages) != dt:
        raise TypeError("q and the pages must share one element type")
    B, Hq, D = q.shape
    P, Hkv, page, Dk = k_pages.shape
    if Dk != D or v_pages.shape != k_pages.shape or bt.shape[0] != B or kl.shape != (B,):
        raise ValueError("shape mismatch")
    o = np.zeros((B, Hq, D), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    rc = lib.oracle_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), dt,
                                 _ptr(bt), _ptr(kl), _dptr(o), _dptr(lse),
                                 B, Hq, Hkv, D, page, bt.shape[1], P,
                                 float(scale), threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_decode_paged failed ({rc})")
    return o, lse


def prefill_paged(q, k_pages, v_pages, block_table, kv_lens, causal, scale, threads=None,
                  lib=None):
    """Prefill of Tq new tokens per sequence against a paged cache.

    q [B,Hq,Tq,D] (the last Tq positions of each sequence); k_pages, v_pages
    [P,Hkv,page,D]; block_table int32 [B,maxp]; kv_lens int32 [B] (keys per
    sequence, the new tokens included).  Causal: query i sees key j when
    j <= i + kv_lens[b] - Tq.  Returns (o [B,Hq,Tq,D], lse [B,Hq,Tq]) in fp64.
    """
    lib = lib or _get()
    q = np.ascontiguousarray(q)
    k_pages = np.ascontiguousarray(k_pages)
    v_pages = np.ascontiguousarray(v_pages)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    kl = np.ascontiguousarray(kv_lens, dtype=np.int32)
    dt = _dtype_code(q)
    if _dtype_code(k_pages) != dt or _dtype_code(v_pages) != dt:
        raise TypeError("q and the pages must share one element type")
    B, Hq, Tq, D = q.shape
    P, Hkv, page, Dk = k_pages.shape
    if Dk != D or v_pages.shape != k_pages.shape or bt.shape[0] != B or kl.shape != (B,):
        raise ValueError("shape mismatch")
    o = np.zeros((B, Hq, Tq, D), np.float64)
    lse = np.zeros((B, Hq, Tq), np.float64)
    rc = lib.oracle_prefill_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), dt, _ptr(bt),
                                  _ptr(kl), _dptr(o), _dptr(lse), B, Hq, Hkv, Tq, D, page,
                                  bt.shape[1], P, int(bool(causal)), float(scale),
                                  threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_prefill_paged failed ({rc})")
    return o, lse


def flat_gemm(a, w, threads=None, lib=None):
    """C = A W^T: a [m,k], w [n,k] (bf16 bits, fp32 or fp64).  Returns fp64 [m,n]."""
    lib = lib or _get()
    a = np.ascontiguousarray(a)
    w = np.ascontiguousarray(w)
    dt = _dtype_code(a)
    if _dtype_code(w) != dt:
        raise TypeError("a and w must share one element type")
    m, k = a.shape
    n, kw = w.shape
    if kw != k:
        raise ValueError("shape mismatch")
    c = np.zeros((m, n), np.float64)
    rc = lib.oracle_flat_gemm(_ptr(a), _ptr(w), dt, _dptr(c), m, n, k,
                              threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_flat_gemm failed ({rc})")
    return c


def e4m3_value(byte, lib=None):
    """Value of one OCP FP8 E4M3 byte (NaN for S.1111.111), from oracle.c."""
    lib = lib or _get()
    return lib.oracle_e4m3_value(int(byte) & 0xFF)


def decode_paged_fp8(q, k_pages, v_pages, k_scale, v_scale, block_table, kv_lens, scale,
                     threads=None, lib=None):
    """Paged decode over an FP8 (OCP E4M3) cache with per-tensor scales.

    q [B,Hq,D] (bf16 bits as uint16, or fp32/fp64); k_pages, v_pages uint8
    [P,Hkv,page,D] holding E4M3 bytes, dequantised as scale * e4m3(byte);
    block_table int32 [B,maxp]; kv_lens int32 [B].  Returns (o, lse) in fp64.
    """
    lib = lib or _get()
    q = np.ascontiguousarray(q)
    k_pages = np.ascontiguousarray(k_pages, dtype=np.uint8)
    v_pages = np.ascontiguousarray(v_pages, dtype=np.uint8)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    kl = np.ascontiguousarray(kv_lens, dtype=np.int32)
    B, Hq, D = q.shape
    P, Hkv, page, Dk = k_pages.shape
    if Dk != D or v_pages.shape != k_pages.shape or bt.shape[0] != B or kl.shape != (B,):
        raise ValueError("shape mismatch")
    o = np.zeros((B, Hq, D), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    rc = lib.oracle_decode_paged_fp8(_ptr(q), _dtype_code(q), _ptr(k_pages), _ptr(v_pages),
                                     float(k_scale), float(v_scale), _ptr(bt), _ptr(kl),
                                     _dptr(o), _dptr(lse), B, Hq, Hkv, D, page, bt.shape[1], P,
                                     float(scale), threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_decode_paged_fp8 failed ({rc})")
    return o, lse


def unified_fallback_count(q, k_pages, block_table, kv_lens, scale, split_tokens, phi,
                           window=60.0, lib=None):
    """Number of (query row, chunk) pairs whose largest scaled score leaves
    [phi - window, phi + window]: the fallback model of the unified-max
    softmax.  Same input layout as decode_paged."""
    lib = lib or _get()
    q = np.ascontiguousarray(q)
    k_pages = np.ascontiguousarray(k_pages)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    kl = np.ascontiguousarray(kv_lens, dtype=np.int32)
    dt = _dtype_code(q)
    if _dtype_code(k_pages) != dt:
        raise TypeError("q and the pages must share one element type")
    B, Hq, D = q.shape
    P, Hkv, page, Dk = k_pages.shape
    if Dk != D or bt.shape[0] != B or kl.shape != (B,):
        raise ValueError("shape mismatch")
    n = lib.oracle_unified_fallback_count(_ptr(q), _ptr(k_pages), dt, _ptr(bt), _ptr(kl),
                                          B, Hq, Hkv, D, page, bt.shape[1], float(scale),
                                          int(split_tokens), float(phi), float(window))
    if n < 0:
        raise RuntimeError("oracle_unified_fallback_count: bad arguments")
    return int(n)


def merge_states(o_a, lse_a, o_b, lse_b, lib=None):
    """State of the union of two disjoint key sets, from their partial states."""
    lib = lib or _get()
    o_a = np.ascontiguousarray(o_a, np.float64)
    o_b = np.ascontiguousarray(o_b, np.float64)
    lse_a = np.ascontiguousarray(lse_a, np.float64)
    lse_b = np.ascontiguousarray(lse_b, np.float64)
    if o_a.shape != o_b.shape or lse_a.shape != lse_b.shape or \
            o_a.shape[:-1] != lse_a.shape:
        raise ValueError("shape mismatch")
    D = o_a.shape[-1]
    rows = int(np.prod(lse_a.shape))
    o = np.empty_like(o_a)
    lse = np.empty_like(lse_a)
    lib.oracle_merge_states(_dptr(o_a), _dptr(lse_a), _dptr(o_b), _dptr(lse_b),
                            _dptr(o), _dptr(lse), rows, D)
    return o, lse


def cascade_decode(q, k_pages, v_pages, prefix_pages, prefix_len, suffix_table,
                   suffix_lens, scale, threads=None, lib=None):
    """Shared-prefix decode by definition: every request attends the
    concatenation prefix + its own suffix (one table per request)."""
    page = k_pages.shape[2]
    if prefix_len % page:
        raise ValueError("the concatenated table needs a page-aligned prefix")
    B = q.shape[0]
    npre = prefix_len // page
    table = np.concatenate(
        [np.broadcast_to(np.asarray(prefix_pages[:npre], np.int32), (B, npre)),
         np.asarray(suffix_table, np.int32)], axis=1)
    lens = np.asarray(suffix_lens, np.int64) + prefix_len
    return decode_paged(q, k_pages, v_pages, table, lens.astype(np.int32), scale,
                        threads=threads, lib=lib)
