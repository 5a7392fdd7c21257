"""GPU parity of paged decode over an FP8 (OCP E4M3) KV cache against the
fp64 oracle, through the C ABI (attn_decode_paged_fp8).

The kernel widens the E4M3 bytes to bf16 in registers (exact) and otherwise
computes as the bf16 path (P rounded to bf16, fp32 accumulation), so the bf16
tolerances apply to both output types."""
import numpy as np
import pytest
import torch

import oracle
from attention_tiled_fmha_amd import attn
from attention_tiled_fmha_amd import workloads as wl
from gpu_util import assert_close, dev, empty_like_out, host, require_gpu

pytestmark = pytest.mark.gpu


def run_fp8(d, split_tokens=0, o_dtype="bf16", k_scale=None, v_scale=None, table=None):
    q = dev(d["q"])
    o = empty_like_out(q.shape, o_dtype)
    lse = torch.full(q.shape[:2], float("nan"), device="cuda")
    bt = dev(d["block_table"] if table is None else table)
    attn.attn_decode_paged_fp8(q, dev(d["k_pages"]), dev(d["v_pages"]),
                               d["k_scale"] if k_scale is None else k_scale,
                               d["v_scale"] if v_scale is None else v_scale,
                               bt, dev(d["kv_lens"]), o, lse,
                               max_kv_len=int(d["kv_lens"].max(initial=0)), scale=d["scale"],
                               split_tokens=split_tokens)
    torch.cuda.synchronize()
    return host(o), host(lse)


def oracle_fp8(d, rows=None, k_scale=None, v_scale=None):
    ks = d["k_scale"] if k_scale is None else k_scale
    vs = d["v_scale"] if v_scale is None else v_scale
    if rows is None:
        return oracle.decode_paged_fp8(d["q"], d["k_pages"], d["v_pages"], ks, vs,
                                       d["block_table"], d["kv_lens"], d["scale"])
    return oracle.decode_paged_fp8(d["q"][rows], d["k_pages"], d["v_pages"], ks, vs,
                                   d["block_table"][rows], d["kv_lens"][rows], d["scale"])


LENS = [0, 1, 15, 16, 17, 63, 64, 65, 200, 511, 512, 513, 1000, 1500]


@pytest.mark.parametrize("o_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("heads", [(4, 4), (8, 2), (32, 8), (6, 2), (32, 2), (8, 1)])
@pytest.mark.parametrize("D", [64, 128])
def test_fp8_decode_shapes(o_dtype, heads, D):
    """Ragged lengths (empty, one token, page and chunk edges), MHA and GQA
    groups 1..16 (including 3 and 16), both head sizes, random page
    placement, the largest code in unused page slots."""
    require_gpu()
    Hq, Hkv = heads
    d = wl.paged_decode_fp8_inputs(len(LENS), Hq, Hkv, D, 40 + Hq + D, lengths=LENS)
    o, lse = run_fp8(d, o_dtype=o_dtype)
    ro, rl = oracle_fp8(d)
    assert_close(o, ro, "bf16", "O")
    assert_close(lse, rl, "bf16", "lse")
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0])), "empty sequence"


@pytest.mark.parametrize("split", [64, 128, 192, 512, 1024])
def test_fp8_forced_splits(split):
    require_gpu()
    d = wl.paged_decode_fp8_inputs(6, 8, 2, 128, 7, lengths=[1, 100, 511, 700, 1024, 2049])
    o, lse = run_fp8(d, split_tokens=split)
    ro, rl = oracle_fp8(d)
    assert_close(o, ro, "bf16", f"O split {split}")
    assert_close(lse, rl, "bf16", f"lse split {split}")


def test_fp8_scales():
    """Unequal, non-power-of-two key and value scales (the bytes encode
    32 x N(0,1), so these scales give keys ~1.4 and values ~0.9 x N(0,1))."""
    require_gpu()
    d = wl.paged_decode_fp8_inputs(5, 8, 4, 128, 8, lengths=[3, 90, 400, 1300, 17])
    o, lse = run_fp8(d, k_scale=0.0437, v_scale=0.0291)
    ro, rl = oracle_fp8(d, k_scale=0.0437, v_scale=0.0291)
    assert_close(o, ro, "bf16", "O")
    assert_close(lse, rl, "bf16", "lse")


def test_fp8_every_code():
    """Every finite E4M3 code (normals, subnormals, both signs, zeros) as a
    value element and as a key element: the widening of each byte matches the
    oracle's decoding of the format."""
    require_gpu()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)   # 254
    L, D = 64, 128
    d = wl.paged_decode_fp8_inputs(2, 4, 2, D, 9, lengths=[L, L])
    n = d["k_pages"].size
    d["v_pages"] = np.resize(codes, n).reshape(d["v_pages"].shape)
    d["k_pages"] = np.resize(codes[::-1], n).reshape(d["k_pages"].shape)
    # scaled so that values stay within +-1.75 and keys within +-0.875
    o, lse = run_fp8(d, k_scale=1.0 / 512, v_scale=1.0 / 256)
    ro, rl = oracle_fp8(d, k_scale=1.0 / 512, v_scale=1.0 / 256)
    assert_close(o, ro, "bf16", "O")
    assert_close(lse, rl, "bf16", "lse")


def test_fp8_equals_bf16_decode_of_the_dequantised_cache():
    """With power-of-two scales the dequantised cache is exact in bf16, and
    the FP8 path computes the same scores and weights as the bf16 path on
    that cache; only the order in which pages reach the wavefronts differs
    (FP8 pages go in pairs), which changes each wavefront's softmax reference
    and so the bf16 rounding of P: the outputs agree to the bf16 tolerance
    (a wrong widening or scale would be far outside it)."""
    require_gpu()
    d = wl.paged_decode_fp8_inputs(8, 32, 8, 128, 10, lengths=[1, 17, 300, 511, 512, 1025, 2000, 64])
    table = np.array([oracle.e4m3_value(b) for b in range(256)])
    kb = wl.bf16_bits((d["k_scale"] * table[d["k_pages"]]).astype(np.float32))
    vb = wl.bf16_bits((d["v_scale"] * table[d["v_pages"]]).astype(np.float32))
    for split in (0, 128):
        o8, l8 = run_fp8(d, split_tokens=split, o_dtype="f32")
        q = dev(d["q"])
        o = empty_like_out(q.shape, "f32")
        lse = torch.empty(q.shape[:2], device="cuda")
        attn.attn_decode_paged(q, dev(kb), dev(vb), dev(d["block_table"]), dev(d["kv_lens"]),
                               o, lse, max_kv_len=int(d["kv_lens"].max()), scale=d["scale"],
                               split_tokens=split)
        torch.cuda.synchronize()
        assert_close(o8, host(o), "bf16", f"O vs the bf16 path (split {split})")
        assert_close(l8, host(lse), "bf16", f"lse vs the bf16 path (split {split})")


def test_fp8_page_placement_invariance():
    """Physical page placement does not change a single bit."""
    require_gpu()
    lens = [700, 33, 1500]
    a = wl.paged_decode_fp8_inputs(3, 8, 2, 128, 11, lengths=lens)
    # the same logical cache under another physical placement
    P = a["k_pages"].shape[0]
    perm = np.random.default_rng(3).permutation(P).astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(P, dtype=np.int32)
    b = dict(a, k_pages=a["k_pages"][inv], v_pages=a["v_pages"][inv])
    table_b = perm[a["block_table"]].astype(np.int32)
    oa, la = run_fp8(a)
    ob, lb = run_fp8(b, table=table_b)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb), "placement changed the result"


@pytest.mark.parametrize("name", [wl.DECODE_MHA, wl.DECODE_GQA])
def test_fp8_workloads_full_size_sampled(name):
    """The MHA (B32) and GQA (32/8, B128, chunks of 512) decode shapes over
    FP8 caches at full size, in the bench's launch configuration; the oracle
    checks a sample of sequences element by element."""
    require_gpu()
    d = wl.fp8_workload(name)
    o, lse = run_fp8(d, split_tokens=d.get("split_tokens", 0))
    rows = [0, 1, int(np.argmax(d["kv_lens"])), int(np.argmin(d["kv_lens"])), d["B"] - 1]
    ro, rl = oracle_fp8(d, rows)
    assert_close(o[rows], ro, "bf16", f"O rows {rows}")
    assert_close(lse[rows], rl, "bf16", f"lse rows {rows}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


# --- shared-prefix cascade over an FP8 cache ----------------------------------

@pytest.mark.parametrize("R,H,Hkv,plen,D", [
    (3, 4, 4, 15, 128), (5, 8, 2, 100, 128), (70, 4, 4, 300, 128), (9, 4, 1, 517, 64),
    (64, 32, 32, 4096, 128), (16, 2, 2, 20000, 128),
])
@pytest.mark.parametrize("o_dtype", ["bf16", "f32"])
def test_fp8_shared_prefix(R, H, Hkv, plen, D, o_dtype):
    """The MFMA prefix stage over an FP8 cache against per-request decode of
    the prefix: more than 64 query rows per kv head, GQA groups, ragged
    prefix lengths, one and many prefix chunks."""
    require_gpu()
    c = wl.cascade_inputs(R, H, D, "fp8", 31 + R + plen, prefix_len=plen, suffix_range=(1, 2),
                          Hkv=Hkv)
    q = dev(c["q"])
    o = empty_like_out(q.shape, o_dtype)
    lse = torch.full(q.shape[:2], float("nan"), device="cuda")
    attn.attn_decode_shared_prefix_fp8(q, dev(c["k_pages"]), dev(c["v_pages"]), c["k_scale"],
                                       c["v_scale"], dev(c["prefix_pages"]), plen, o, lse,
                                       scale=c["scale"])
    torch.cuda.synchronize()
    table = np.broadcast_to(c["prefix_pages"], (R, len(c["prefix_pages"]))).copy()
    ro, rl = oracle.decode_paged_fp8(c["q"], c["k_pages"], c["v_pages"], c["k_scale"],
                                     c["v_scale"], table, np.full(R, plen, np.int32), c["scale"])
    assert_close(host(o), ro, "bf16", "prefix O")
    assert_close(host(lse), rl, "bf16", "prefix lse")


def run_cascade_fp8(c):
    q = dev(c["q"])
    kp, vp = dev(c["k_pages"]), dev(c["v_pages"])
    o_p, o_s = torch.empty_like(q), torch.empty_like(q)
    l_p = torch.empty(q.shape[:2], device="cuda")
    l_s = torch.empty(q.shape[:2], device="cuda")
    attn.attn_decode_shared_prefix_fp8(q, kp, vp, c["k_scale"], c["v_scale"],
                                       dev(c["prefix_pages"]), c["prefix_len"], o_p, l_p,
                                       scale=c["scale"])
    attn.attn_decode_paged_fp8(q, kp, vp, c["k_scale"], c["v_scale"], dev(c["suffix_table"]),
                               dev(c["suffix_lens"]), o_s, l_s,
                               max_kv_len=int(c["suffix_lens"].max()), scale=c["scale"])
    attn.attn_merge_states(o_p, l_p, o_s, l_s)
    torch.cuda.synchronize()
    return host(o_p), host(l_p)


def test_fp8_cascade_r64_prefix4096_full_size():
    """The cascade shape over an FP8 cache (64 requests, 4096-token prefix,
    suffixes U[128, 1024]): prefix stage, suffix decode and merge against the
    plain decode of each request's whole key sequence."""
    require_gpu()
    c = wl.fp8_workload(wl.CASCADE)
    o, lse = run_cascade_fp8(c)
    rows = [0, 1, 31, 63]
    npre = len(c["prefix_pages"])
    table = np.stack([np.concatenate([c["prefix_pages"], c["suffix_table"][r]]) for r in rows])
    lens = (c["prefix_len"] + c["suffix_lens"][rows]).astype(np.int32)
    assert c["prefix_len"] == npre * 16
    ro, rl = oracle.decode_paged_fp8(c["q"][rows], c["k_pages"], c["v_pages"], c["k_scale"],
                                     c["v_scale"], table.astype(np.int32), lens, c["scale"])
    assert_close(o[rows], ro, "bf16", "cascade O")
    assert_close(lse[rows], rl, "bf16", "cascade lse")


# --- unified max (asynchronous softmax) over an FP8 cache ----------------------

def run_fp8_unified(d, phi, split_tokens):
    q = dev(d["q"])
    o = empty_like_out(q.shape, "bf16")
    lse = torch.full(q.shape[:2], float("nan"), device="cuda")
    count = torch.zeros(1, dtype=torch.int32, device="cuda")
    attn.attn_decode_paged_fp8(q, dev(d["k_pages"]), dev(d["v_pages"]), d["k_scale"],
                               d["v_scale"], dev(d["block_table"]), dev(d["kv_lens"]), o, lse,
                               max_kv_len=int(d["kv_lens"].max(initial=0)), scale=d["scale"],
                               split_tokens=split_tokens, unified_max=True, phi=phi,
                               fallback_count=count)
    torch.cuda.synchronize()
    return host(o), host(lse), int(count.item())


def fp8_model_count(d, split, phi):
    """The oracle's fp64 fallback model on the dequantised cache (each E4M3
    byte decoded by the oracle, times k_scale); the case must not sit within
    0.01 of the window edge."""
    table = np.array([oracle.e4m3_value(b) for b in range(256)], np.float64)
    k = (table[d["k_pages"]] * d["k_scale"]).astype(np.float32)
    q = wl.bf16_to_f32(d["q"]).astype(np.float32)
    args = (q, k, d["block_table"], d["kv_lens"], d["scale"], split, phi)
    n = oracle.unified_fallback_count(*args)
    assert n == oracle.unified_fallback_count(*args, window=59.99) == \
        oracle.unified_fallback_count(*args, window=60.01), "case too close to the window edge"
    return n


UNI_LENS = [0, 1, 16, 17, 300, 512, 513, 1000, 2049]


@pytest.mark.parametrize("phi", [0.0, 100.0, -100.0])
@pytest.mark.parametrize("heads", [(8, 8), (32, 8)])
def test_fp8_unified_max(phi, heads):
    """The unified-max softmax over an FP8 cache: the window test uses the
    scaled score scale * q.(k_scale * e4m3).  With phi = 0 no (row, chunk)
    pair of N(0,1)-sized scores falls back, with phi = +-100 every pair does;
    either way the result is the plain attention and the GPU's fallback
    count is the fp64 model's."""
    require_gpu()
    Hq, Hkv = heads
    split = 256
    d = wl.paged_decode_fp8_inputs(len(UNI_LENS), Hq, Hkv, 128, 60 + Hq, lengths=UNI_LENS)
    o, lse, n = run_fp8_unified(d, phi, split)
    ro, rl = oracle_fp8(d)
    assert_close(o, ro, "bf16", "O")
    assert_close(lse, rl, "bf16", "lse")
    pairs = Hq * sum((L + split - 1) // split for L in UNI_LENS)
    assert n == fp8_model_count(d, split, phi) == (0 if phi == 0.0 else pairs)


def test_fp8_unified_max_mixed_fallback():
    """Queries of half the sequences scaled by 50 (scores up to a few hundred
    against a window of +-60 around phi = 0): those pairs are recomputed, the
    count matches the model and the result the oracle."""
    require_gpu()
    split = 128
    lens = [33, 200, 700, 1500, 64, 129, 900, 2000]
    d = wl.paged_decode_fp8_inputs(len(lens), 16, 4, 128, 67, lengths=lens)
    q = wl.bf16_to_f32(d["q"])
    q[::2] *= 50.0
    d["q"] = wl.bf16_bits(q)
    o, lse, n = run_fp8_unified(d, 0.0, split)
    ro, rl = oracle_fp8(d)
    assert_close(o, ro, "bf16", "O")
    assert_close(lse, rl, "bf16", "lse")
    assert n == fp8_model_count(d, split, 0.0)
    assert 0 < n < 16 * sum((L + split - 1) // split for L in lens)
