"""Seeded synthetic inputs for the attention hot path.

This module holds no attention arithmetic: it draws random numbers, rounds
them to the storage type, and lays out paged caches and block tables.  Both
the HIP path and the CPU oracle consume what it produces, so it is the only
code they have in common.

Storage conventions (see ``include/attn.h``):

* dense prefill tensors are [B, H, T, D], row-major;
* a paged cache is [num_pages, Hkv, page_size, D], one [page_size, D] tile per
  (page, kv head) contiguous in memory;
* block tables are int32 [B, max_pages]; entries past a sequence's last page
  hold 0 (a valid page, never read);
* bf16 tensors are carried on the host as uint16 bit patterns;
* FP8 caches are OCP E4M3 bytes (uint8) with one scale per tensor.

Draw order for a workload (one ``numpy.random.Generator(PCG64(seed))``):
lengths, page permutation, Q, K pool, V pool.  Large pools are drawn in
fixed-size chunks, each from its own PCG64 stream seeded by the parent
generator, so the values do not depend on how many threads draw them.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

PAGE_SIZE = 16
_CHUNK = 1 << 22

# Values written into the unused slots of each sequence's last page.  They are
# large so that reading a slot past kv_len shows up in any result.
TAIL_K = 30.0
TAIL_V = 1000.0


def generator(seed):
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits(x):
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16.  NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def e4m3_bits(x, scale=1.0):
    """Quantise x / scale (computed in float32) to OCP FP8 E4M3 bytes (uint8):
    round to nearest, ties to even, saturating at +-448; the stored value is
    scale * e4m3(byte).  E4M3 keeps 3 mantissa bits; its exponent field
    (bias 7) spans 2^-6 .. 2^8, with subnormals in steps of 2^-9 below 2^-6."""
    one = np.float32(1.0)
    y = np.asarray(x, np.float32) / np.float32(scale)
    a = np.minimum(np.abs(y), np.float32(448.0))
    _, e = np.frexp(a)                          # a = f * 2^e, f in [0.5, 1)
    e = np.clip(e - 1, -6, 8)
    step = np.ldexp(one, e - 3).astype(np.float32)   # spacing of E4M3 values there
    r = np.minimum(np.rint(a / step) * step, np.float32(448.0))   # rint: ties to even
    _, er = np.frexp(r)
    er = er - 1
    normal = r >= np.float32(2.0 ** -6)
    exp_field = np.where(normal, er + 7, 0)
    mant = np.where(normal, r / np.ldexp(one, er).astype(np.float32) * 8 - 8, r * np.float32(512.0))
    code = (exp_field.astype(np.int32) << 3) | np.rint(mant).astype(np.int32)
    code = np.where(np.signbit(y) & (r > 0), code | 0x80, code)
    return code.astype(np.uint8)


def bf16_to_f32(bits):
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def normal(gen, shape, dtype, e4m3_scale=1.0):
    """N(0,1) draws of ``shape`` in storage ``dtype`` ('bf16' -> uint16 bits,
    'f32' -> float32, 'e4m3' -> uint8 E4M3 bytes of x / e4m3_scale).  Drawn in
    fixed chunks from child streams."""
    n = int(np.prod(shape)) if len(shape) else 1
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)
    seeds = gen.integers(0, 2**63 - 1, size=nchunks, dtype=np.int64)
    out = np.empty(n, dtype={"bf16": np.uint16, "e4m3": np.uint8}.get(dtype, np.float32))

    def fill(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        x = generator(int(seeds[c])).standard_normal(hi - lo, dtype=np.float32)
        if dtype == "bf16":
            out[lo:hi] = bf16_bits(x)
        elif dtype == "e4m3":
            out[lo:hi] = e4m3_bits(x, e4m3_scale)
        else:
            out[lo:hi] = x

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def _const(value, dtype):
    if dtype == "e4m3":
        return 0x7E            # the largest E4M3 code
    return bf16_bits(np.float32(value)).item() if dtype == "bf16" else np.float32(value)


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def prefill_inputs(B, Hq, Hkv, Tq, Tk, D, dtype, seed):
    """Q [B,Hq,Tq,D], K and V [B,Hkv,Tk,D], i.i.d. N(0,1)."""
    gen = generator(seed)
    q = normal(gen, (B, Hq, Tq, D), dtype)
    k = normal(gen, (B, Hkv, Tk, D), dtype)
    v = normal(gen, (B, Hkv, Tk, D), dtype)
    return dict(q=q, k=k, v=v, B=B, Hq=Hq, Hkv=Hkv, Tq=Tq, Tk=Tk, D=D,
                dtype=dtype, scale=1.0 / math.sqrt(D), seed=seed)


# ---------------------------------------------------------------------------
# paged decode
# ---------------------------------------------------------------------------

def uniform_lengths(gen, n, lo, hi):
    """Integer lengths uniform on [lo, hi] (both ends included)."""
    return gen.integers(lo, hi, size=n, endpoint=True).astype(np.int32)


def log_uniform_lengths(gen, n, lo, hi):
    """floor(exp(U(ln lo, ln hi))), clamped to [lo, hi]."""
    x = np.floor(np.exp(gen.uniform(math.log(lo), math.log(hi), size=n)))
    return np.clip(x, lo, hi).astype(np.int32)


def pages_for(lengths, page_size=PAGE_SIZE):
    return (np.asarray(lengths, np.int64) + page_size - 1) // page_size


def _tables(lengths, physical, page_size, max_pages=None):
    """Block tables that map each sequence's logical pages, in order, onto
    consecutive entries of ``physical``."""
    npages = pages_for(lengths, page_size)
    maxp = int(max_pages if max_pages is not None else max(1, int(npages.max(initial=1))))
    table = np.zeros((len(lengths), maxp), np.int32)
    pos = 0
    for b, n in enumerate(npages):
        table[b, :n] = physical[pos:pos + n]
        pos += n
    return table


def _fill_tails(k_pages, v_pages, table, lengths, page_size, dtype):
    """Write the tail-slot sentinels past each sequence's last token."""
    kt, vt = _const(TAIL_K, dtype), _const(TAIL_V, dtype)
    for b, L in enumerate(np.asarray(lengths)):
        if L % page_size:
            pg = table[b, (L - 1) // page_size]
            k_pages[pg, :, L % page_size:, :] = kt
            v_pages[pg, :, L % page_size:, :] = vt


def paged_decode_inputs(B, Hq, Hkv, D, dtype, seed, lengths=None,
                        length_range=(512, 8192), length_dist="uniform",
                        page_size=PAGE_SIZE, tail_garbage=True, permute=True):
    """One query token per sequence over a paged cache.

    The physical pool holds exactly sum(ceil(L_b / page_size)) pages; logical
    pages map through one random permutation of the pool (identity if
    ``permute`` is False).
    """
    gen = generator(seed)
    if lengths is None:
        lo, hi = length_range
        draw = uniform_lengths if length_dist == "uniform" else log_uniform_lengths
        lengths = draw(gen, B, lo, hi)
    lengths = np.asarray(lengths, np.int32)
    total_pages = int(pages_for(lengths, page_size).sum())
    pool = max(1, total_pages)
    physical = gen.permutation(pool).astype(np.int32) if permute else \
        np.arange(pool, dtype=np.int32)
    table = _tables(lengths, physical, page_size)
    q = normal(gen, (B, Hq, D), dtype)
    k_pages = normal(gen, (pool, Hkv, page_size, D), dtype)
    v_pages = normal(gen, (pool, Hkv, page_size, D), dtype)
    if tail_garbage:
        _fill_tails(k_pages, v_pages, table, lengths, page_size, dtype)
    return dict(q=q, k_pages=k_pages, v_pages=v_pages, block_table=table,
                kv_lens=lengths, B=B, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                page_size=page_size, scale=1.0 / math.sqrt(D), seed=seed,
                max_kv_len=int(lengths.max(initial=0)))


def paged_prefill_inputs(B, Hq, Hkv, Tq, D, dtype, seed, lengths=None,
                         length_range=(1024, 8192), length_dist="uniform",
                         page_size=PAGE_SIZE, tail_garbage=True, permute=True):
    """Chunked prefill: Tq new query tokens per sequence (its last Tq
    positions, q [B,Hq,Tq,D]) over the paged cache of ``paged_decode_inputs``
    (same seed, same draws), whose kv_lens count the new tokens too."""
    d = paged_decode_inputs(B, Hq, Hkv, D, dtype, seed, lengths, length_range, length_dist,
                            page_size, tail_garbage, permute)
    d["q"] = normal(generator(seed + 7919), (B, Hq, Tq, D), dtype)
    d["Tq"] = Tq
    return d


def paged_decode_fp8_inputs(B, Hq, Hkv, D, seed, lengths=None, length_range=(512, 8192),
                            length_dist="uniform", kv_scale=1.0 / 32, page_size=PAGE_SIZE,
                            tail_garbage=True):
    """Paged decode over an FP8 (OCP E4M3) cache: bf16 queries; K and V are
    N(0,1) draws quantised to E4M3 bytes with one per-tensor scale each
    (``kv_scale``: stored value = kv_scale * e4m3(byte)).  Same draw order and
    layout as ``paged_decode_inputs``; the unused slots of each last page hold
    the largest code (448 * kv_scale) so that any read past kv_len shows."""
    gen = generator(seed)
    if lengths is None:
        lo, hi = length_range
        draw = uniform_lengths if length_dist == "uniform" else log_uniform_lengths
        lengths = draw(gen, B, lo, hi)
    lengths = np.asarray(lengths, np.int32)
    pool = max(1, int(pages_for(lengths, page_size).sum()))
    physical = gen.permutation(pool).astype(np.int32)
    table = _tables(lengths, physical, page_size)
    q = normal(gen, (B, Hq, D), "bf16")
    k = normal(gen, (pool, Hkv, page_size, D), "e4m3", kv_scale)
    v = normal(gen, (pool, Hkv, page_size, D), "e4m3", kv_scale)
    if tail_garbage:
        for b, L in enumerate(lengths):
            if L % page_size:
                pg = table[b, (L - 1) // page_size]
                k[pg, :, L % page_size:, :] = 0x7E
                v[pg, :, L % page_size:, :] = 0x7E
    return dict(q=q, k_pages=k, v_pages=v, block_table=table, kv_lens=lengths, B=B, Hq=Hq,
                Hkv=Hkv, D=D, dtype="fp8", page_size=page_size, scale=1.0 / math.sqrt(D),
                seed=seed, max_kv_len=int(lengths.max(initial=0)), k_scale=kv_scale,
                v_scale=kv_scale)


def cascade_inputs(R, H, D, dtype, seed, prefix_len=4096, suffix_range=(128, 1024),
                   suffix_lens=None, page_size=PAGE_SIZE, Hkv=None,
                   tail_garbage=True, kv_scale=1.0 / 32):
    """Shared-prefix decode: R requests share one prefix of ``prefix_len``
    tokens, stored once, plus their own suffixes.  Prefix and suffix pages
    are all placed by one permutation of the pool.  dtype 'fp8': bf16
    queries over an E4M3 cache with per-tensor scale ``kv_scale`` (as
    ``paged_decode_fp8_inputs``)."""
    if dtype == "fp8":
        c = cascade_inputs(R, H, D, "e4m3", seed, prefix_len, suffix_range, suffix_lens,
                           page_size, Hkv, tail_garbage, kv_scale)
        return c | dict(dtype="fp8", k_scale=kv_scale, v_scale=kv_scale)
    Hkv = Hkv or H
    gen = generator(seed)
    if suffix_lens is None:
        suffix_lens = uniform_lengths(gen, R, *suffix_range)
    suffix_lens = np.asarray(suffix_lens, np.int32)
    npre = (prefix_len + page_size - 1) // page_size
    total = npre + int(pages_for(suffix_lens, page_size).sum())
    physical = gen.permutation(max(1, total)).astype(np.int32)
    prefix_pages = physical[:npre].copy()
    suffix_table = _tables(suffix_lens, physical[npre:], page_size)
    q = normal(gen, (R, H, D), "bf16" if dtype == "e4m3" else dtype)
    k_pages = normal(gen, (max(1, total), Hkv, page_size, D), dtype, kv_scale)
    v_pages = normal(gen, (max(1, total), Hkv, page_size, D), dtype, kv_scale)
    if tail_garbage:
        _fill_tails(k_pages, v_pages, suffix_table, suffix_lens, page_size, dtype)
        if prefix_len % page_size:
            pg = prefix_pages[-1]
            k_pages[pg, :, prefix_len % page_size:, :] = _const(TAIL_K, dtype)
            v_pages[pg, :, prefix_len % page_size:, :] = _const(TAIL_V, dtype)
    return dict(q=q, k_pages=k_pages, v_pages=v_pages, prefix_pages=prefix_pages,
                prefix_len=prefix_len, suffix_table=suffix_table,
                suffix_lens=suffix_lens, R=R, H=H, Hkv=Hkv, D=D, dtype=dtype,
                page_size=page_size, scale=1.0 / math.sqrt(D), seed=seed)


# ---------------------------------------------------------------------------
# the named workloads
# ---------------------------------------------------------------------------

PREFILL_F32 = "prefill_f32_b1_h1_t128_d64"
PREFILL_CAUSAL = "prefill_causal_b4_h32_t1024_d128"
DECODE_MHA = "decode_mha_b32_h32_d128"
DECODE_GQA = "decode_gqa_b128_hq32_hkv8_d128"
CASCADE = "cascade_r64_prefix4096_h32_d128"

WORKLOADS = {
    PREFILL_F32: "non-causal prefill B1 H1 T128 D64 fp32",
    PREFILL_CAUSAL: "causal prefill B4 H32 T1024 D128 bf16 (Llama2-7B attention shape)",
    DECODE_MHA: "paged decode MHA B32 H32 D128 bf16, L~U[512,8192], page 16",
    DECODE_GQA: "paged decode GQA B128 Hq32 Hkv8 D128 bf16, L~logU[1024,32768], page 16, "
                "split <= 512",
    CASCADE: "shared-prefix cascade decode, 64 requests, prefix 4096, suffix U[128,1024], "
             "H32 D128 bf16, page 16",
}

FP8_WORKLOADS = {
    DECODE_MHA: "paged decode MHA B32 H32 D128, FP8 E4M3 cache (scale 1/32), bf16 q/o, "
                "L~U[512,8192], page 16",
    DECODE_GQA: "paged decode GQA B128 Hq32 Hkv8 D128, FP8 E4M3 cache (scale 1/32), bf16 q/o, "
                "L~logU[1024,32768], page 16, split <= 512",
    CASCADE: "shared-prefix cascade decode, 64 requests, prefix 4096, suffix U[128,1024], "
             "H32 D128, FP8 E4M3 cache (scale 1/32), bf16 q/o, page 16",
}

# default seeds (PCG64), one per workload
SEEDS = {PREFILL_F32: 1001, PREFILL_CAUSAL: 1002, DECODE_MHA: 1003, DECODE_GQA: 1004, CASCADE: 1005}


def fp8_workload(name, seed=None):
    """The decode and cascade workloads over an FP8 cache (same shapes and
    length draws as the bf16 ones)."""
    seed = SEEDS[name] if seed is None else seed
    if name == CASCADE:
        return cascade_inputs(64, 32, 128, "fp8", seed)
    if name == DECODE_MHA:
        return paged_decode_fp8_inputs(32, 32, 32, 128, seed, length_range=(512, 8192),
                                       length_dist="uniform")
    if name == DECODE_GQA:
        return paged_decode_fp8_inputs(128, 32, 8, 128, seed, length_range=(1024, 32768),
                                       length_dist="log-uniform") | dict(split_tokens=512)
    raise ValueError(f"no FP8 workload {name}")


def workload(name, seed=None):
    """Inputs of the named workload, seeded from SEEDS by default."""
    seed = SEEDS[name] if seed is None else seed
    if name == PREFILL_F32:
        return prefill_inputs(1, 1, 1, 128, 128, 64, "f32", seed) | dict(causal=False)
    if name == PREFILL_CAUSAL:
        return prefill_inputs(4, 32, 32, 1024, 1024, 128, "bf16", seed) | dict(causal=True)
    if name == DECODE_MHA:
        return paged_decode_inputs(32, 32, 32, 128, "bf16", seed,
                                   length_range=(512, 8192), length_dist="uniform")
    if name == DECODE_GQA:
        return paged_decode_inputs(128, 32, 8, 128, "bf16", seed,
                                   length_range=(1024, 32768), length_dist="log-uniform") \
            | dict(split_tokens=512)
    if name == CASCADE:
        return cascade_inputs(64, 32, 128, "bf16", seed)
    raise ValueError(f"no workload {name}")


# ---------------------------------------------------------------------------
# flat GEMM of the decode phase
# ---------------------------------------------------------------------------

# Weight shapes [n, k] of the four projections of one Llama2-7B layer
# (hidden size 4096, FFN size 11008): fused K/Q/V, O, fused gate + up, down.
LLAMA2_7B_PROJECTIONS = {
    "qkv": (12288, 4096),
    "o": (4096, 4096),
    "gate_up": (22016, 4096),
    "down": (4096, 11008),
}


def flat_gemm_inputs(m, n, k, seed):
    """A [m, k] (the m tokens of one decode step) and W [n, k] (a projection's
    weight), bf16 i.i.d. N(0,1); drawn in that order."""
    gen = generator(seed)
    a = normal(gen, (m, k), "bf16")
    w = normal(gen, (n, k), "bf16")
    return dict(a=a, w=w, m=m, n=n, k=k, seed=seed)
