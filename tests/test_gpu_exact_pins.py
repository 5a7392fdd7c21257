"""Exact pins of page, chunk and tile coverage on the kernels that run the
bf16 and FP8 workloads (the MFMA decode, the MFMA shared-prefix stage, the
state merge and the bf16 MFMA prefill), through the C ABI.

With every key of a kv head identical, every score of a query row is the
same number s, so the softmax weights are all exactly 1 (exp of 0, which
bf16 holds exactly) and

    O[c] = (1/n) * sum of V[t][c] over the n keys the row attends,
    lse  = s + ln n.

Values V[t][c] = bit (c mod 16) of (t + 7*kvh), complemented in odd groups
of 16 dimensions, are 0 or 1, so the sums are exact integers and O is a
closed form that names which tokens were read (a skipped, repeated or
misplaced page or tile, a read past kv_len, a transposed dimension group or
the wrong kv head all change it).  At these lengths the bf16 tolerance of
the workloads cannot see one page (16 tokens move lse by about 16/n); these
pins can: O is read in fp32 and held to 2e-6, lse to 1e-5 (decode) and 1e-4
(prefill, whose O is bf16 and whose lse also carries the rounding of
m + log2 l).  Queries are multiples of 1/8 and keys 1/4, so s is exact in
fp32 and the tolerance only covers the final scaling, division and log.

The expected values are computed here from the closed forms alone; no
oracle or kernel output enters them.
"""
import functools
import math

import numpy as np
import pytest
import torch

from attention_tiled_fmha_amd import attn
from attention_tiled_fmha_amd import workloads as wl
from gpu_util import dev, host, require_gpu

pytestmark = pytest.mark.gpu

O_TOL, LSE_TOL, PREFILL_LSE_TOL = 2e-6, 1e-5, 1e-4
KEY = 0.25
BF16_ONE, BF16_KEY = 0x3F80, 0x3E80            # 1.0 and 0.25
E4M3_ONE = 0x38                                # 1.0 (exponent field 7 = bias)


def vbits(t, D, kvh):
    """V[t][c] in {0, 1}: bit (c % 16) of (t + 7 kvh), inverted for odd c // 16."""
    t = np.asarray(t, np.int64)[:, None] + 7 * kvh
    c = np.arange(D)
    bit = (t >> (c % 16)) & 1
    return np.where((c // 16) % 2 == 1, 1 - bit, bit)


@functools.lru_cache(maxsize=None)
def expected_o(n, D, kvh, t0=0):
    """Closed-form mean of V over tokens t0 .. t0 + n - 1 (exact integer sums)."""
    if n == 0:
        return np.zeros(D)
    return vbits(np.arange(t0, t0 + n), D, kvh).sum(0) / n


def eighths(gen, shape):
    """Queries that are multiples of 1/8 in [-4, 4] (bf16-exact)."""
    return np.clip(np.rint(gen.standard_normal(shape) * 8), -32, 32) / 8.0


def q_bits(qv):
    return wl.bf16_bits(qv.astype(np.float32))


def fill_cache(k_pages, v_pages, table, lens, D, fp8, t_offsets=None):
    """Overwrite the valid slots of every sequence: identical keys, bit-pattern
    values (token index t counted from t_offsets[b]); unused slots keep the
    generator's tail sentinels."""
    Hkv = k_pages.shape[1]
    for b, L in enumerate(lens):
        if L == 0:
            continue
        t = np.arange(L)
        pg, sl = table[b, t // 16], t % 16
        t0 = 0 if t_offsets is None else t_offsets[b]
        for g in range(Hkv):
            bits = vbits(t + t0, D, g)
            if fp8:
                k_pages[pg, g, sl, :] = E4M3_ONE
                v_pages[pg, g, sl, :] = np.where(bits == 1, E4M3_ONE, 0).astype(np.uint8)
            else:
                k_pages[pg, g, sl, :] = BF16_KEY
                v_pages[pg, g, sl, :] = np.where(bits == 1, BF16_ONE, 0).astype(np.uint16)


def check_rows(o, lse, qv, ns, scale, key, vscale, G, D, t0s=None, what=""):
    """o [B,Hq,D] fp32, lse [B,Hq]; ns[b] tokens attended by sequence b."""
    B, Hq, _ = o.shape
    for b in range(B):
        n = int(ns[b])
        for h in range(Hq):
            kvh = h // G
            eo = vscale * expected_o(n, D, kvh, 0 if t0s is None else int(t0s[b]))
            s = scale * key * float(qv[b, h].sum())
            el = s + math.log(n) if n > 0 else -math.inf
            err_o = float(np.abs(o[b, h] - eo).max())
            assert err_o <= O_TOL, f"{what} O: b={b} h={h} n={n} max err {err_o:.3e}"
            if n == 0:
                assert np.isneginf(lse[b, h]), f"{what} lse of an empty row"
            else:
                err_l = abs(float(lse[b, h]) - el)
                assert err_l <= LSE_TOL, f"{what} lse: b={b} h={h} n={n} err {err_l:.3e}"


DECODE_LENS = [1, 15, 16, 17, 511, 512, 513, 1023, 1024, 1025, 4097, 8191, 32768]


def decode_pin_inputs(G, D, fp8, seed, lens=DECODE_LENS, Hkv=2):
    Hq = G * Hkv
    if fp8:
        d = wl.paged_decode_fp8_inputs(len(lens), Hq, Hkv, D, seed, lengths=lens)
    else:
        d = wl.paged_decode_inputs(len(lens), Hq, Hkv, D, "bf16", seed, lengths=lens)
    qv = eighths(wl.generator(seed + 1), (len(lens), Hq, D))
    d["q"] = q_bits(qv)
    fill_cache(d["k_pages"], d["v_pages"], d["block_table"], lens, D, fp8)
    return d, qv


@pytest.mark.parametrize("split", [0, 128, 256, 512])
@pytest.mark.parametrize("G", [1, 4, 16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_decode_token_set_and_lse_exact(split, G, D, fp8):
    """Paged decode (MFMA kernel, bf16 or E4M3 cache, fp32 output) over
    lengths at and around page, chunk and item edges up to 32768, random
    page placement, with the planner's split and forced 128/256/512-token
    chunks (two-chunk items at 512)."""
    require_gpu()
    d, qv = decode_pin_inputs(G, D, fp8, 300 + 10 * G + D + int(fp8))
    q = dev(d["q"])
    o = torch.full(q.shape, float("nan"), device="cuda")
    lse = torch.full(q.shape[:2], float("nan"), device="cuda")
    args = (dev(d["block_table"]), dev(d["kv_lens"]), o, lse)
    kw = dict(max_kv_len=int(max(DECODE_LENS)), scale=d["scale"], split_tokens=split)
    if fp8:
        # key byte 1.0 x k_scale 0.25 = 0.25; value bytes 0 / 1.0 x v_scale 2
        attn.attn_decode_paged_fp8(q, dev(d["k_pages"]), dev(d["v_pages"]), 0.25, 2.0, *args, **kw)
    else:
        attn.attn_decode_paged(q, dev(d["k_pages"]), dev(d["v_pages"]), *args, **kw)
    torch.cuda.synchronize()
    check_rows(host(o), host(lse), qv, d["kv_lens"], d["scale"], KEY, 2.0 if fp8 else 1.0, G, D,
               what=f"decode split={split}")


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("R,H,Hkv,plen", [(16, 4, 4, 4096), (70, 4, 1, 4096), (8, 2, 2, 20000),
                                          (64, 32, 32, 4096)])
def test_cascade_token_set_and_lse_exact(fp8, R, H, Hkv, plen):
    """Shared-prefix stage (MFMA), suffix decode and attn_merge_states, each
    pinned: the prefix alone attends tokens 0 .. P-1, the suffix P .. P+L-1,
    the merged state all P + L of them."""
    require_gpu()
    D, G = 128, H // Hkv
    gen = wl.generator(400 + R + plen)
    suffix = gen.integers(1, 1025, size=R).astype(np.int32)
    suffix[0] = 1
    c = wl.cascade_inputs(R, H, D, "fp8" if fp8 else "bf16", 401 + R + plen, prefix_len=plen,
                          suffix_lens=suffix, Hkv=Hkv)
    qv = eighths(gen, (R, H, D))
    c["q"] = q_bits(qv)
    npre = (plen + 15) // 16
    pre_table = c["prefix_pages"][None, :]
    fill_cache(c["k_pages"], c["v_pages"], pre_table, [plen], D, fp8)
    fill_cache(c["k_pages"], c["v_pages"], c["suffix_table"], suffix, D, fp8,
               t_offsets=[plen] * R)
    assert len(c["prefix_pages"]) == npre
    q, kp, vp = dev(c["q"]), dev(c["k_pages"]), dev(c["v_pages"])
    o_p = torch.full(q.shape, float("nan"), device="cuda")
    l_p = torch.full(q.shape[:2], float("nan"), device="cuda")
    o_s, l_s = torch.full_like(o_p, float("nan")), torch.full_like(l_p, float("nan"))
    vs = 2.0 if fp8 else 1.0
    if fp8:
        attn.attn_decode_shared_prefix_fp8(q, kp, vp, 0.25, vs, dev(c["prefix_pages"]), plen, o_p,
                                           l_p, scale=c["scale"])
        attn.attn_decode_paged_fp8(q, kp, vp, 0.25, vs, dev(c["suffix_table"]), dev(suffix), o_s,
                                   l_s, max_kv_len=int(suffix.max()), scale=c["scale"])
    else:
        attn.attn_decode_shared_prefix(q, kp, vp, dev(c["prefix_pages"]), plen, o_p, l_p,
                                       scale=c["scale"])
        attn.attn_decode_paged(q, kp, vp, dev(c["suffix_table"]), dev(suffix), o_s, l_s,
                               max_kv_len=int(suffix.max()), scale=c["scale"])
    torch.cuda.synchronize()
    check_rows(host(o_p), host(l_p), qv, [plen] * R, c["scale"], KEY, vs, G, D, what="prefix")
    check_rows(host(o_s), host(l_s), qv, suffix, c["scale"], KEY, vs, G, D, t0s=[plen] * R,
               what="suffix")
    attn.attn_merge_states(o_p, l_p, o_s, l_s)
    torch.cuda.synchronize()
    check_rows(host(o_p), host(l_p), qv, plen + suffix, c["scale"], KEY, vs, G, D, what="merged")


# --- bf16 MFMA prefill --------------------------------------------------------

def prefill_pin(B, Hq, Hkv, T, D, causal, seed):
    gen = wl.generator(seed)
    qv = eighths(gen, (B, Hq, T, D))
    k = np.full((B, Hkv, T, D), BF16_KEY, np.uint16)
    v = np.stack([np.stack([np.where(vbits(np.arange(T), D, g) == 1, BF16_ONE, 0)
                            for g in range(Hkv)]) for _ in range(B)]).astype(np.uint16)
    q = dev(q_bits(qv))
    o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full(q.shape[:3], float("nan"), device="cuda")
    attn.attn_prefill(q, dev(k), dev(v), o, lse, causal=causal, scale=D ** -0.5)
    torch.cuda.synchronize()
    return qv, host(o), host(lse)


def prefill_expect(T, D, kvh, causal):
    """[T, D] expected O: the running mean (causal) or the full mean."""
    bits = vbits(np.arange(T), D, kvh)
    if causal:
        return np.cumsum(bits, 0) / np.arange(1, T + 1)[:, None]
    return np.broadcast_to(bits.sum(0) / T, (T, D))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(4, 32, 32, 1024, 128), (1, 2, 1, 16384, 128),
                                   (2, 4, 2, 1000, 64), (1, 3, 1, 4099, 128)])
def test_prefill_token_set_and_lse_exact(causal, shape):
    """bf16 MFMA prefill at the causal-workload shape (B4 H32 T1024 D128), at
    T = 16384, with grouped heads and ragged T: every row's lse is s + ln n
    to 1e-4 (one 32-key tile moves it by >= 2e-3 at n = 16384) and O is the
    exact mean of the visible values up to the bf16 rounding of the output."""
    require_gpu()
    B, Hq, Hkv, T, D = shape
    G = Hq // Hkv
    qv, o, lse = prefill_pin(B, Hq, Hkv, T, D, causal, 500 + T + D + int(causal))
    scale = D ** -0.5
    n = np.arange(1, T + 1) if causal else np.full(T, T)
    for h in range(Hq):
        eo = prefill_expect(T, D, h // G, causal)
        for b in range(B):
            s = scale * KEY * qv[b, h].sum(-1)
            err_l = np.abs(lse[b, h] - (s + np.log(n))).max()
            assert err_l <= PREFILL_LSE_TOL, f"lse b={b} h={h}: {err_l:.3e}"
            # bf16 output (8 significant bits): RNE is within 2^-8 |x| of x
            err_o = np.abs(o[b, h] - eo) - 2.0 ** -8 * np.abs(eo)
            assert err_o.max() <= 1e-6, f"O b={b} h={h}: {err_o.max():.3e} past bf16 rounding"


def decode_vs_prefill_row(d, L, D, H):
    """The same rows through the bf16 MFMA decode (fp32 output) and the bf16
    MFMA prefill with one query (bf16 output)."""
    q = dev(d["q"])
    o = torch.full(q.shape, float("nan"), device="cuda")
    lse = torch.full(q.shape[:2], float("nan"), device="cuda")
    attn.attn_decode_paged(q, dev(d["k_pages"]), dev(d["v_pages"]), dev(d["block_table"]),
                           dev(d["kv_lens"]), o, lse, max_kv_len=L, scale=d["scale"])
    t = np.arange(L)
    pg, sl = d["block_table"][0, t // 16], t % 16
    K = d["k_pages"][pg, :, sl].transpose(1, 0, 2)[None].copy()     # [1, H, L, D]
    V = d["v_pages"][pg, :, sl].transpose(1, 0, 2)[None].copy()
    pq = dev(d["q"][:, :, None, :].copy())
    po = torch.full(pq.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    pl = torch.full(pq.shape[:3], float("nan"), device="cuda")
    attn.attn_prefill(pq, dev(K), dev(V), po, pl, causal=False, scale=d["scale"])
    torch.cuda.synchronize()
    return host(o)[0], host(lse)[0], host(po)[0, :, 0], host(pl)[0, :, 0], V


@pytest.mark.parametrize("D", [64, 128])
def test_decode_equals_last_prefill_row_bf16(D):
    """Decode = the last prefill row, on the bf16 MFMA kernels.

    Pin inputs (identical keys, bit-pattern values): both reach the closed
    form, the decode to 2e-6 in fp32 and the prefill to its bf16 rounding.

    Random N(0,1) inputs: the kernels differ only in summation order and in
    the reference each takes its exponentials against, so each rounds its
    P = exp(s - m) to bf16 differently (relative error <= 2^-8 per weight).
    That moves each lse by at most ln(1 + 2^-8) and each O by at most
    2 * 2^-8 * max|V| (weights w_j(1 + d_j) / (1 + mean d)); the comparison
    allows both kernels' share plus the prefill's bf16 output rounding."""
    require_gpu()
    L, H = 1500, 8
    d, qv = decode_pin_inputs(1, D, False, 700 + D, lens=[L], Hkv=H)
    od, ld, op, lp, _ = decode_vs_prefill_row(d, L, D, H)
    check_rows(od[None], ld[None], qv, [L], d["scale"], KEY, 1.0, 1, D, what="decode")
    for h in range(H):
        eo = expected_o(L, D, h)
        assert np.all(np.abs(op[h] - eo) <= 2.0 ** -8 * np.abs(eo) + 1e-6), f"prefill O h={h}"
        s = d["scale"] * KEY * float(qv[0, h].sum())
        assert abs(lp[h] - (s + math.log(L))) <= PREFILL_LSE_TOL, f"prefill lse h={h}"

    d = wl.paged_decode_inputs(1, H, H, D, "bf16", 77 + D, lengths=[L])
    od, ld, op, lp, V = decode_vs_prefill_row(d, L, D, H)
    vmax = np.abs(wl.bf16_to_f32(V)).max()
    assert np.abs(ld - lp).max() <= 2 * math.log1p(2.0 ** -8)
    err = np.abs(od - op) - 2.0 ** -8 * np.abs(op)
    assert err.max() <= 2 * 2 * 2.0 ** -8 * vmax, f"decode vs prefill O: {err.max():.3e}"


def test_two_streams_with_internal_workspaces():
    """Two decode calls that each need a workspace (forced 256-token chunks),
    one on a side stream and one on the current stream, both with the
    binding allocating the workspace: each call's workspace belongs to its
    own stream, so repeated runs are bit-identical and match one-stream runs."""
    require_gpu()
    d, qv = decode_pin_inputs(4, 128, False, 600, lens=[700, 3000, 9000, 1])
    q = dev(d["q"])
    kp, vp, bt, kl = dev(d["k_pages"]), dev(d["v_pages"]), dev(d["block_table"]), dev(d["kv_lens"])
    kw = dict(max_kv_len=9000, scale=d["scale"], split_tokens=256)
    o_ref = torch.empty(q.shape, device="cuda")
    l_ref = torch.empty(q.shape[:2], device="cuda")
    attn.attn_decode_paged(q, kp, vp, bt, kl, o_ref, l_ref, **kw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for _ in range(4):
        o_a, o_b = torch.empty_like(o_ref), torch.empty_like(o_ref)
        l_a, l_b = torch.empty_like(l_ref), torch.empty_like(l_ref)
        side.wait_stream(torch.cuda.current_stream())
        attn.attn_decode_paged(q, kp, vp, bt, kl, o_a, l_a, stream=side, **kw)
        attn.attn_decode_paged(q, kp, vp, bt, kl, o_b, l_b, **kw)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for o, l in ((o_a, l_a), (o_b, l_b)):
            assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    check_rows(host(o_ref), host(l_ref), qv, d["kv_lens"], d["scale"], KEY, 1.0, 4, 128,
               what="two streams")
