"""Python binding of libattn.so (the C ABI in include/attn.h).

Argument marshalling only: shapes and element types are read off torch
device tensors, pointers and the current HIP stream are passed through
ctypes, and a non-zero status becomes an :class:`AttnError`.  Every step of
the computation runs in the library's HIP kernels; there is no fallback.  If
libattn.so has not been built, the first call raises.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")
# the same interface with device-side index checks and an error word
CHECKED_LIB_PATH = os.path.join(_PKG, "libattn_checked.so")

BF16, F32, FP8_E4M3 = 0, 1, 2
DEV_ERR_KV_LEN, DEV_ERR_PAGE = 1, 2      # the checked library's error-word bits
_lib = None
_libs = {}

# Every symbol include/attn.h declares, with (restype, argtypes).
_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_ip = ctypes.POINTER(ctypes.c_int)
SIGNATURES = {
    "attn_status_str": (ctypes.c_char_p, [_i]),
    "attn_prefill": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _vp]),
    "attn_decode_plan": (_i, [_i, _i, _i, _i, _i, _ip, _ip]),
    "attn_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "attn_decode_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                               _i, _i, _f, _vp, _sz, _vp]),
    "attn_decode_paged_ex": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                  _i, _i, _i, _f, _vp, _sz, _vp, _vp]),
    "attn_decode_paged_fp8": (_i, [_vp, _vp, _vp, _f, _f, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                                   _i, _i, _i, _i, _f, _vp, _sz, _vp, _vp]),
    "attn_merge_states": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _vp]),
    "attn_shared_prefix_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "attn_decode_shared_prefix": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i,
                                       _i, _i, _f, _vp, _sz, _vp]),
    "attn_prefill_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                               _i, _i, _f, _vp]),
    "attn_decode_shared_prefix_fp8": (_i, [_vp, _vp, _vp, _f, _f, _vp, _i, _vp, _vp, _i, _i, _i,
                                           _i, _i, _i, _f, _vp, _sz, _vp]),
    "attn_flat_gemm_plan": (_i, [_i, _i, _i, _i, _vp, _ip, _ip, _ip]),
    "attn_flat_gemm_workspace_bytes": (_sz, [_i, _i, _i, _vp]),
    "attn_flat_gemm": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _sz, _vp, _vp]),
    "attn_decode_paged_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                       _i, _i, _i, _i, _f, _vp]),
    "attn_cascade_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "attn_decode_cascade": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                 _i, _i, _i, _i, _f, _f, _f, _vp, _sz, _vp]),
    "attn_checked_build": (_i, []),
    "attn_device_errors": (_i, [ctypes.POINTER(ctypes.c_uint), _i]),
    "attn_device_pool_pages": (_i, [_vp, _sz, ctypes.POINTER(ctypes.c_int)]),
    "attn_probe_block_bytes": (_i, []),
    "attn_probe_hbm_read": (_i, [_vp, _vp, _i, _vp, _vp]),
}

NOALLOC_SCRATCH_BYTES = 32 << 20


class AttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


class DecodeOpts(ctypes.Structure):
    _fields_ = [("split_tokens", ctypes.c_int), ("use_unified_max", ctypes.c_int),
                ("phi", ctypes.c_float), ("reserved0", ctypes.c_int),
                ("fallback_count", ctypes.c_void_p), ("reserved", ctypes.c_int * 4)]


def load(path=None):
    """The library the calls of this module go to, with every exported
    signature declared.  With no path: the one in use, else libattn.so, or
    libattn_checked.so when the environment sets ATTN_CHECKED=1.  With a
    path: that library, which then stays in use."""
    global _lib
    if path is None:
        if _lib is not None:
            return _lib
        path = CHECKED_LIB_PATH if os.environ.get("ATTN_CHECKED") == "1" else LIB_PATH
    if path not in _libs:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build() or "
                               "python -m attention_tiled_fmha_amd.build")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _libs[path] = lib
    _lib = _libs[path]
    return _lib


def device_errors(clear=True):
    """The checked library's device error word (ATTN_DEV_ERR_* bits) after
    the device has finished its work; clears it by default."""
    flags = ctypes.c_uint(0)
    _check(load().attn_device_errors(ctypes.byref(flags), int(clear)), "attn_device_errors")
    return flags.value


def device_pool_pages(pages):
    """The page bound the checked library holds indices into `pages` to."""
    n = ctypes.c_int(0)
    page_bytes = pages[0].numel() * pages.element_size() if pages.shape[0] else 0
    _check(load().attn_device_pool_pages(_p(pages), page_bytes, ctypes.byref(n)),
           "attn_device_pool_pages")
    return n.value


def status_str(status):
    return load().attn_status_str(int(status)).decode()


def _check(status, where):
    if status != 0:
        raise AttnError(status, where)


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported element type {t.dtype}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _workspace(need, device, stream):
    """A workspace of ``need`` bytes for one call.  It is allocated on the
    stream the call is enqueued on: torch's caching allocator hands a freed
    block only to later work of the stream it was allocated on, which runs
    after this call's kernels, so releasing it on return is safe."""
    if stream is None:
        return torch.empty(need, dtype=torch.uint8, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(need, dtype=torch.uint8, device=device)


def _dense(t, name):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


# ---------------------------------------------------------------------------

def attn_prefill(q, k, v, o, lse=None, causal=False, scale=None, stream=None):
    """q, o [B,Hq,Tq,D]; k, v [B,Hkv,Tk,D]; lse fp32 [B,Hq,Tq] or None."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _dense(t, n)
    B, Hq, Tq, D = q.shape
    _, Hkv, Tk, _ = k.shape
    if o.shape != q.shape or v.shape != k.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("shape mismatch")
    if lse is not None:
        _dense(lse, "lse")
        if lse.shape != (B, Hq, Tq) or lse.dtype != torch.float32:
            raise ValueError("lse must be fp32 [B, Hq, Tq]")
    dt = _dtype(q)
    if not (_dtype(k) == _dtype(v) == _dtype(o) == dt):
        raise TypeError("q, k, v, o must share one element type")
    scale = D ** -0.5 if scale is None else scale
    _check(load().attn_prefill(_p(q), _p(k), _p(v), _p(o), _p(lse), B, Hq, Hkv, Tq, Tk, D, dt,
                               int(bool(causal)), float(scale), _stream(stream)), "attn_prefill")


def attn_prefill_paged(q, k_pages, v_pages, block_table, kv_lens, o, lse=None, causal=True,
                       scale=None, stream=None):
    """Chunked prefill: q, o bf16 [B,Hq,Tq,D] (each sequence's last Tq
    positions); k_pages, v_pages bf16 [P,Hkv,16,D]; block_table int32
    [B,maxp]; kv_lens int32 [B] (keys per sequence, the chunk included);
    lse fp32 [B,Hq,Tq] or None."""
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"),
                 (block_table, "block_table"), (kv_lens, "kv_lens"), (o, "o")):
        _dense(t, n)
    B, Hq, Tq, D = q.shape
    P, Hkv, page, _ = k_pages.shape
    if o.shape != q.shape or v_pages.shape != k_pages.shape or k_pages.shape[3] != D:
        raise ValueError("shape mismatch")
    if block_table.dtype != torch.int32 or kv_lens.dtype != torch.int32:
        raise TypeError("block_table and kv_lens must be int32")
    if block_table.shape[0] != B or kv_lens.shape != (B,):
        raise ValueError("block_table / kv_lens shape mismatch")
    if lse is not None:
        _dense(lse, "lse")
        if lse.shape != (B, Hq, Tq) or lse.dtype != torch.float32:
            raise ValueError("lse must be fp32 [B, Hq, Tq]")
    dt = _dtype(q)
    if not (_dtype(k_pages) == _dtype(v_pages) == dt):
        raise TypeError("q and the pages must share one element type")
    scale = D ** -0.5 if scale is None else scale
    _check(load().attn_prefill_paged(
        _p(q), _p(k_pages), _p(v_pages), _p(block_table), _p(kv_lens), _p(o), _p(lse), B, Hq,
        Hkv, Tq, D, page, block_table.shape[1], dt, int(bool(causal)), float(scale),
        _stream(stream)), "attn_prefill_paged")


def attn_decode_plan(batch, heads_kv, max_kv_len, num_cus=0, requested_split=0):
    split, max_splits = ctypes.c_int(), ctypes.c_int()
    _check(load().attn_decode_plan(batch, heads_kv, max_kv_len, num_cus, requested_split,
                                   ctypes.byref(split), ctypes.byref(max_splits)),
           "attn_decode_plan")
    return split.value, max_splits.value


def attn_decode_workspace_bytes(batch, heads_q, heads_kv, head_dim, max_kv_len, split_tokens=0):
    return load().attn_decode_workspace_bytes(batch, heads_q, heads_kv, head_dim, max_kv_len,
                                              split_tokens)


def attn_decode_paged(q, k_pages, v_pages, block_table, kv_lens, o, lse=None, max_kv_len=None,
                      scale=None, workspace=None, split_tokens=0, stream=None,
                      unified_max=False, phi=0.0, fallback_count=None):
    """q, o [B,Hq,D]; k_pages, v_pages [P,Hkv,16,D]; block_table int32 [B,maxp];
    kv_lens int32 [B]; lse fp32 [B,Hq] or None.  max_kv_len is the host-side
    bound of kv_lens (required).  A workspace of the needed size is allocated
    with torch when none is given.  unified_max selects the unified-max
    softmax with value phi; fallback_count (a device int32 tensor of one
    element, or None) receives the number of (row, chunk) pairs that fell
    back to the exact path, added to its value."""
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"),
                 (block_table, "block_table"), (kv_lens, "kv_lens"), (o, "o")):
        _dense(t, n)
    if max_kv_len is None:
        raise ValueError("max_kv_len (host-side bound of kv_lens) is required")
    B, Hq, D = q.shape
    P, Hkv, page, _ = k_pages.shape
    if o.shape != q.shape or v_pages.shape != k_pages.shape or k_pages.shape[3] != D:
        raise ValueError("shape mismatch")
    if block_table.dtype != torch.int32 or kv_lens.dtype != torch.int32:
        raise TypeError("block_table and kv_lens must be int32")
    if block_table.shape[0] != B or kv_lens.shape != (B,):
        raise ValueError("block_table / kv_lens shape mismatch")
    if lse is not None:
        _dense(lse, "lse")
        if lse.shape != (B, Hq) or lse.dtype != torch.float32:
            raise ValueError("lse must be fp32 [B, Hq]")
    dt = _dtype(q)
    if not (_dtype(k_pages) == _dtype(v_pages) == dt):
        raise TypeError("q and the pages must share one element type")
    scale = D ** -0.5 if scale is None else scale
    need = attn_decode_workspace_bytes(B, Hq, Hkv, D, max_kv_len, split_tokens)
    if workspace is None and need:
        workspace = _workspace(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if fallback_count is not None:
        _dense(fallback_count, "fallback_count")
        if fallback_count.dtype != torch.int32 or fallback_count.numel() != 1:
            raise TypeError("fallback_count must be one int32 element")
    opts = DecodeOpts(split_tokens=int(split_tokens), use_unified_max=int(bool(unified_max)),
                      phi=float(phi), fallback_count=_p(fallback_count))
    _check(load().attn_decode_paged_ex(
        _p(q), _p(k_pages), _p(v_pages), _p(block_table), _p(kv_lens), _p(o), _p(lse),
        B, Hq, Hkv, D, page, block_table.shape[1], int(max_kv_len), dt, _dtype(o),
        float(scale), _p(workspace), ws_bytes, _stream(stream), ctypes.byref(opts)),
        "attn_decode_paged")


def attn_decode_paged_noalloc(q, k_pages, v_pages, block_table, kv_lens, o, lse=None,
                              max_kv_len=None, scale=None, stream=None):
    """attn_decode_paged without a workspace: the split partials go to the
    library's fixed device array (NOALLOC_SCRATCH_BYTES per GPU; larger plans
    raise AttnError with ATTN_E_SCRATCH).  Calls that overlap on one GPU
    share that array and race."""
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"),
                 (block_table, "block_table"), (kv_lens, "kv_lens"), (o, "o")):
        _dense(t, n)
    if max_kv_len is None:
        raise ValueError("max_kv_len (host-side bound of kv_lens) is required")
    B, Hq, D = q.shape
    P, Hkv, page, _ = k_pages.shape
    if o.shape != q.shape or v_pages.shape != k_pages.shape or k_pages.shape[3] != D:
        raise ValueError("shape mismatch")
    if block_table.dtype != torch.int32 or kv_lens.dtype != torch.int32:
        raise TypeError("block_table and kv_lens must be int32")
    if block_table.shape[0] != B or kv_lens.shape != (B,):
        raise ValueError("block_table / kv_lens shape mismatch")
    if lse is not None:
        _dense(lse, "lse")
        if lse.shape != (B, Hq) or lse.dtype != torch.float32:
            raise ValueError("lse must be fp32 [B, Hq]")
    dt = _dtype(q)
    if not (_dtype(k_pages) == _dtype(v_pages) == dt):
        raise TypeError("q and the pages must share one element type")
    scale = D ** -0.5 if scale is None else scale
    _check(load().attn_decode_paged_noalloc(
        _p(q), _p(k_pages), _p(v_pages), _p(block_table), _p(kv_lens), _p(o), _p(lse),
        B, Hq, Hkv, D, page, block_table.shape[1], int(max_kv_len), dt, _dtype(o),
        float(scale), _stream(stream)), "attn_decode_paged_noalloc")


def attn_decode_paged_fp8(q, k_pages, v_pages, k_scale, v_scale, block_table, kv_lens, o,
                          lse=None, max_kv_len=None, scale=None, workspace=None, split_tokens=0,
                          stream=None, unified_max=False, phi=0.0, fallback_count=None):
    """attn_decode_paged over an FP8 cache: q bf16 [B,Hq,D]; k_pages, v_pages
    uint8 [P,Hkv,16,D] holding OCP E4M3 bytes, the cached values being
    k_scale * e4m3 and v_scale * e4m3; o bf16 or fp32 [B,Hq,D]."""
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"),
                 (block_table, "block_table"), (kv_lens, "kv_lens"), (o, "o")):
        _dense(t, n)
    if max_kv_len is None:
        raise ValueError("max_kv_len (host-side bound of kv_lens) is required")
    B, Hq, D = q.shape
    P, Hkv, page, _ = k_pages.shape
    if o.shape != q.shape or v_pages.shape != k_pages.shape or k_pages.shape[3] != D:
        raise ValueError("shape mismatch")
    if q.dtype != torch.bfloat16 or k_pages.dtype != torch.uint8 or v_pages.dtype != torch.uint8:
        raise TypeError("q must be bf16 and the pages uint8 (E4M3 bytes)")
    if block_table.dtype != torch.int32 or kv_lens.dtype != torch.int32:
        raise TypeError("block_table and kv_lens must be int32")
    if block_table.shape[0] != B or kv_lens.shape != (B,):
        raise ValueError("block_table / kv_lens shape mismatch")
    if lse is not None:
        _dense(lse, "lse")
        if lse.shape != (B, Hq) or lse.dtype != torch.float32:
            raise ValueError("lse must be fp32 [B, Hq]")
    scale = D ** -0.5 if scale is None else scale
    need = attn_decode_workspace_bytes(B, Hq, Hkv, D, max_kv_len, split_tokens)
    if workspace is None and need:
        workspace = _workspace(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if fallback_count is not None:
        _dense(fallback_count, "fallback_count")
        if fallback_count.dtype != torch.int32 or fallback_count.numel() != 1:
            raise TypeError("fallback_count must be one int32 element")
    opts = DecodeOpts(split_tokens=int(split_tokens), use_unified_max=int(bool(unified_max)),
                      phi=float(phi), fallback_count=_p(fallback_count))
    _check(load().attn_decode_paged_fp8(
        _p(q), _p(k_pages), _p(v_pages), float(k_scale), float(v_scale), _p(block_table),
        _p(kv_lens), _p(o), _p(lse), B, Hq, Hkv, D, page, block_table.shape[1], int(max_kv_len),
        _dtype(o), float(scale), _p(workspace), ws_bytes, _stream(stream), ctypes.byref(opts)),
        "attn_decode_paged_fp8")


def attn_merge_states(o_a, lse_a, o_b, lse_b, stream=None):
    """In place into (o_a, lse_a); o_* [rows..., D], lse_* fp32 [rows...]."""
    for t, n in ((o_a, "o_a"), (lse_a, "lse_a"), (o_b, "o_b"), (lse_b, "lse_b")):
        _dense(t, n)
    if o_a.shape != o_b.shape or lse_a.shape != lse_b.shape or o_a.shape[:-1] != lse_a.shape:
        raise ValueError("shape mismatch")
    if lse_a.dtype != torch.float32 or lse_b.dtype != torch.float32:
        raise TypeError("lse must be fp32")
    dt = _dtype(o_a)
    if _dtype(o_b) != dt:
        raise TypeError("o_a and o_b must share one element type")
    D = o_a.shape[-1]
    rows = lse_a.numel()
    _check(load().attn_merge_states(_p(o_a), _p(lse_a), _p(o_b), _p(lse_b), rows, D, dt,
                                    _stream(stream)), "attn_merge_states")


def attn_shared_prefix_workspace_bytes(batch, heads_q, heads_kv, head_dim, prefix_len, dtype=BF16):
    return load().attn_shared_prefix_workspace_bytes(batch, heads_q, heads_kv, head_dim,
                                                     prefix_len, dtype)


def attn_decode_shared_prefix(q, k_pages, v_pages, prefix_pages, prefix_len, o, lse=None,
                              scale=None, workspace=None, stream=None):
    """q, o [B,Hq,D]; prefix_pages int32 [ceil(prefix_len/16)]; lse fp32 [B,Hq]."""
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"), (o, "o")):
        _dense(t, n)
    B, Hq, D = q.shape
    P, Hkv, page, _ = k_pages.shape
    if o.shape != q.shape or v_pages.shape != k_pages.shape or k_pages.shape[3] != D:
        raise ValueError("shape mismatch")
    if prefix_len > 0:
        _dense(prefix_pages, "prefix_pages")
        if prefix_pages.dtype != torch.int32 or prefix_pages.numel() * page < prefix_len:
            raise ValueError("prefix_pages must be int32 covering prefix_len tokens")
    if lse is not None:
        _dense(lse, "lse")
        if lse.shape != (B, Hq) or lse.dtype != torch.float32:
            raise ValueError("lse must be fp32 [B, Hq]")
    dt = _dtype(q)
    scale = D ** -0.5 if scale is None else scale
    need = attn_shared_prefix_workspace_bytes(B, Hq, Hkv, D, prefix_len, dt)
    if workspace is None and need:
        workspace = _workspace(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().attn_decode_shared_prefix(
        _p(q), _p(k_pages), _p(v_pages), _p(prefix_pages), int(prefix_len), _p(o), _p(lse),
        B, Hq, Hkv, D, page, dt, _dtype(o), float(scale), _p(workspace), ws_bytes,
        _stream(stream)), "attn_decode_shared_prefix")


def attn_decode_shared_prefix_fp8(q, k_pages, v_pages, k_scale, v_scale, prefix_pages,
                                  prefix_len, o, lse=None, scale=None, workspace=None,
                                  stream=None):
    """attn_decode_shared_prefix over an FP8 cache: q bf16 [B,Hq,D]; k_pages,
    v_pages uint8 [P,Hkv,16,D] (E4M3 bytes, values k_scale * e4m3 and
    v_scale * e4m3); o bf16 or fp32 [B,Hq,D]."""
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"), (o, "o")):
        _dense(t, n)
    if q.dtype != torch.bfloat16 or k_pages.dtype != torch.uint8 or v_pages.dtype != torch.uint8:
        raise TypeError("q must be bf16 and the pages uint8 (E4M3 bytes)")
    B, Hq, D = q.shape
    P, Hkv, page, _ = k_pages.shape
    if o.shape != q.shape or v_pages.shape != k_pages.shape or k_pages.shape[3] != D:
        raise ValueError("shape mismatch")
    if prefix_len > 0:
        _dense(prefix_pages, "prefix_pages")
        if prefix_pages.dtype != torch.int32 or prefix_pages.numel() * page < prefix_len:
            raise ValueError("prefix_pages must be int32 covering prefix_len tokens")
    if lse is not None:
        _dense(lse, "lse")
        if lse.shape != (B, Hq) or lse.dtype != torch.float32:
            raise ValueError("lse must be fp32 [B, Hq]")
    scale = D ** -0.5 if scale is None else scale
    need = attn_shared_prefix_workspace_bytes(B, Hq, Hkv, D, prefix_len, FP8_E4M3)
    if workspace is None and need:
        workspace = _workspace(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().attn_decode_shared_prefix_fp8(
        _p(q), _p(k_pages), _p(v_pages), float(k_scale), float(v_scale), _p(prefix_pages),
        int(prefix_len), _p(o), _p(lse), B, Hq, Hkv, D, page, _dtype(o), float(scale),
        _p(workspace), ws_bytes, _stream(stream)), "attn_decode_shared_prefix_fp8")


def attn_cascade_workspace_bytes(batch, heads_q, heads_kv, head_dim, prefix_len, max_suffix_len,
                                 dtype=BF16):
    return load().attn_cascade_workspace_bytes(batch, heads_q, heads_kv, head_dim, prefix_len,
                                               max_suffix_len, dtype)


def attn_decode_cascade(q, k_pages, v_pages, prefix_pages, prefix_len, suffix_table, suffix_lens,
                        o, lse=None, max_suffix_len=None, scale=None, k_scale=1.0, v_scale=1.0,
                        workspace=None, stream=None):
    """Shared-prefix cascade decode in one call (prefix stage, own-token
    decode and one combine over both's chunk states): q, o [B,Hq,D]; pages
    [P,Hkv,16,D] bf16, or uint8 E4M3 bytes (values k_scale * e4m3,
    v_scale * e4m3); prefix_pages int32 [ceil(prefix_len/16)];
    suffix_table int32 [B, max_pages]; suffix_lens int32 [B] or None."""
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"), (o, "o")):
        _dense(t, n)
    B, Hq, D = q.shape
    P, Hkv, page, _ = k_pages.shape
    if o.shape != q.shape or v_pages.shape != k_pages.shape or k_pages.shape[3] != D:
        raise ValueError("shape mismatch")
    if q.dtype != torch.bfloat16:
        raise TypeError("q must be bf16")
    if k_pages.dtype == torch.uint8 and v_pages.dtype == torch.uint8:
        dt = FP8_E4M3
    elif k_pages.dtype == torch.bfloat16 and v_pages.dtype == torch.bfloat16:
        dt = BF16
    else:
        raise TypeError("the pages must both be bf16 or both uint8 (E4M3 bytes)")
    if prefix_len > 0:
        _dense(prefix_pages, "prefix_pages")
        if prefix_pages.dtype != torch.int32 or prefix_pages.numel() * page < prefix_len:
            raise ValueError("prefix_pages must be int32 covering prefix_len tokens")
    _dense(suffix_table, "suffix_table")
    if suffix_table.dtype != torch.int32 or suffix_table.dim() != 2 or suffix_table.shape[0] != B:
        raise ValueError("suffix_table must be int32 [B, max_pages]")
    if suffix_lens is not None:
        _dense(suffix_lens, "suffix_lens")
        if suffix_lens.dtype != torch.int32 or suffix_lens.shape != (B,):
            raise ValueError("suffix_lens must be int32 [B]")
    if max_suffix_len is None:
        max_suffix_len = int(suffix_lens.max().item()) if (suffix_lens is not None and B) else 0
    if lse is not None:
        _dense(lse, "lse")
        if lse.shape != (B, Hq) or lse.dtype != torch.float32:
            raise ValueError("lse must be fp32 [B, Hq]")
    scale = D ** -0.5 if scale is None else scale
    need = attn_cascade_workspace_bytes(B, Hq, Hkv, D, prefix_len, max_suffix_len, dt)
    if workspace is None and need:
        workspace = _workspace(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().attn_decode_cascade(
        _p(q), _p(k_pages), _p(v_pages), _p(prefix_pages), int(prefix_len), _p(suffix_table),
        _p(suffix_lens), _p(o), _p(lse), B, Hq, Hkv, D, page, suffix_table.shape[1],
        int(max_suffix_len), dt, _dtype(o), float(scale), float(k_scale), float(v_scale),
        _p(workspace), ws_bytes, _stream(stream)), "attn_decode_cascade")


class FlatGemmOpts(ctypes.Structure):
    _fields_ = [("splits", ctypes.c_int), ("rows_per_workgroup", ctypes.c_int),
                ("waves_per_workgroup", ctypes.c_int), ("kernel", ctypes.c_int),
                ("reserved", ctypes.c_int * 4)]


# attn_flat_gemm_opts.kernel
FG_REGISTER, FG_LDS = 1, 2


def _fg_opts(splits, rows, waves=0, kernel=0):
    return ctypes.byref(FlatGemmOpts(int(splits), int(rows), int(waves), int(kernel)))


def attn_flat_gemm_plan(m, n, k, num_cus=0, splits=0, rows_per_workgroup=0, kernel=0):
    """Host-only: (k slices, rows of W per workgroup, kernel) the planner
    picks for C = A W^T (kernel FG_REGISTER or FG_LDS)."""
    s, r, kn = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _check(load().attn_flat_gemm_plan(m, n, k, num_cus,
                                      _fg_opts(splits, rows_per_workgroup, 0, kernel),
                                      ctypes.byref(s), ctypes.byref(r), ctypes.byref(kn)),
           "attn_flat_gemm_plan")
    return s.value, r.value, kn.value


def attn_flat_gemm_workspace_bytes(m, n, k, splits=0, rows_per_workgroup=0, waves_per_workgroup=0,
                                   kernel=0):
    return load().attn_flat_gemm_workspace_bytes(
        m, n, k, _fg_opts(splits, rows_per_workgroup, waves_per_workgroup, kernel))


def attn_flat_gemm(a, w, c, splits=0, rows_per_workgroup=0, waves_per_workgroup=0,
                   workspace=None, stream=None, kernel=0):
    """C = A W^T: a bf16 [m, k], w bf16 [n, k], c bf16 or fp32 [m, n]."""
    for t, nm in ((a, "a"), (w, "w"), (c, "c")):
        _dense(t, nm)
    if a.dim() != 2 or w.dim() != 2 or c.dim() != 2:
        raise ValueError("a, w, c must be 2-D")
    m, k = a.shape
    n, kw = w.shape
    if kw != k or tuple(c.shape) != (m, n):
        raise ValueError("shape mismatch")
    if a.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise TypeError("a and w must be bf16")
    need = attn_flat_gemm_workspace_bytes(m, n, k, splits, rows_per_workgroup, waves_per_workgroup,
                                          kernel)
    if workspace is None and need:
        workspace = _workspace(need, a.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().attn_flat_gemm(_p(a), _p(w), _p(c), m, n, k, BF16, _dtype(c), _p(workspace),
                                 ws_bytes, _stream(stream),
                                 _fg_opts(splits, rows_per_workgroup, waves_per_workgroup, kernel)),
           "attn_flat_gemm")


def attn_probe_hbm_read(buf, order=None, sink=None, stream=None):
    """Read the uint8 device tensor buf (a multiple of attn_probe_block_bytes()
    bytes) as 4 KiB blocks in the int32 order (None: in place order); one
    kernel on the stream, for timing with events."""
    _dense(buf, "buf")
    blk = load().attn_probe_block_bytes()
    nbytes = buf.numel() * buf.element_size()
    if nbytes % blk:
        raise ValueError(f"buf must be a multiple of {blk} bytes")
    n = nbytes // blk
    if order is not None:
        _dense(order, "order")
        if order.dtype != torch.int32 or order.numel() != n:
            raise ValueError("order must be int32 with one entry per block")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check(load().attn_probe_hbm_read(_p(buf), _p(order), int(n), _p(sink), _stream(stream)),
           "attn_probe_hbm_read")
