"""Pins for the fp64 oracle: checks that fix what it computes by something
other than itself -- closed forms, invariants, a hand-derived example, scipy's
softmax/logsumexp, and a pure-Python brute force on tiny shapes.

Each check takes a loaded oracle library so that the same checks can run
against copies of the oracle with a planted mistake (tests/test_oracle_mutations.py).
A check raises AssertionError when the oracle disagrees.
"""
import json
import math
import os

import numpy as np
import scipy.special

import oracle
from oracle import brute
from attention_tiled_fmha_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(err)) and err.max(initial=0.0) <= tol, \
        f"{what}: max err {err.max(initial=0.0):.3e} > {tol:.1e}"


def _rng(seed):
    return np.random.default_rng(seed)


# --- 1. hand-derived example --------------------------------------------------

def check_hand_2x2(lib):
    with open(os.path.join(GOLDEN, "attn_2x2.json")) as f:
        g = json.load(f)
    env = {"e": math.e, "log": math.log}
    q = np.array(g["q"], np.float64)[None, None]
    k = np.array(g["k"], np.float64)[None, None]
    v = np.array(g["v"], np.float64)[None, None]
    for mode, causal in (("noncausal", False), ("causal", True)):
        exp_o = np.array([[eval(x, env) for x in row] for row in g[mode]["o_expr"]])
        exp_l = np.array([eval(x, env) for x in g[mode]["lse_expr"]])
        _close(exp_o, g[mode]["o"], 1e-15, f"fixture {mode} o")
        o, lse = oracle.attention(q, k, v, causal, g["scale"], lib=lib)
        _close(o[0, 0], exp_o, 1e-14, f"2x2 {mode} o")
        _close(lse[0, 0], exp_l, 1e-14, f"2x2 {mode} lse")


# --- 2. identical keys ---------------------------------------------------------

def check_identical_keys(lib):
    r = _rng(1)
    T, D = 37, 8
    q = r.standard_normal((1, 2, T, D))
    key = r.standard_normal(D)
    k = np.broadcast_to(key, (1, 2, T, D)).copy()
    v = r.standard_normal((1, 2, T, D))
    scale = 0.3
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, causal, scale, lib=lib)
        for h in range(2):
            for i in range(T):
                n = i + 1 if causal else T
                s = scale * math.fsum(q[0, h, i] * key)
                exp_o = [math.fsum(v[0, h, :n, c]) / n for c in range(D)]
                _close(o[0, h, i], exp_o, 1e-13, "identical keys o")
                _close(lse[0, h, i], s + math.log(n), 1e-13, "identical keys lse")


# --- 3. one dominant score -----------------------------------------------------

def check_dominant_score(lib):
    r = _rng(2)
    n, D = 9, 4
    v = r.standard_normal((n, D))
    jstar = 5
    for a, scale in ((1.0, 1.0), (2.0, 0.5), (6.0, 1.0 / 8.0), (math.sqrt(40.0), 1.0)):
        q = np.zeros((1, 1, 1, D)); q[0, 0, 0, 0] = a
        k = np.zeros((1, 1, n, D)); k[0, 0, jstar, 0] = a
        o, lse = oracle.attention(q, k, v[None, None], False, scale, lib=lib)
        delta = scale * a * a
        w = math.exp(delta)
        others = [j for j in range(n) if j != jstar]
        exp_o = [(w * v[jstar, c] + math.fsum(v[j, c] for j in others)) / (w + n - 1)
                 for c in range(D)]
        _close(o[0, 0, 0], exp_o, 1e-13, f"dominant score o (delta={delta})")
        _close(lse[0, 0, 0], math.log(w + n - 1), 1e-13, "dominant score lse")
        if delta >= 40:
            _close(o[0, 0, 0], v[jstar], 1e-15, "dominant score limit")


# --- 4/5. single key, causal row 0 ---------------------------------------------

def check_single_key_and_row0(lib):
    r = _rng(3)
    D = 16
    q = r.standard_normal((2, 3, 1, D))
    k = r.standard_normal((2, 3, 1, D))
    v = r.standard_normal((2, 3, 1, D))
    o, lse = oracle.attention(q, k, v, False, 0.25, lib=lib)
    _close(o, v, 1e-15, "T=1 o")
    _close(lse, 0.25 * np.einsum("bhid,bhid->bhi", q, k), 1e-14, "T=1 lse")
    # causal: row 0 sees key 0 only
    q = r.standard_normal((1, 2, 6, D))
    k = r.standard_normal((1, 2, 6, D))
    v = r.standard_normal((1, 2, 6, D))
    o, lse = oracle.attention(q, k, v, True, 0.25, lib=lib)
    _close(o[:, :, 0], v[:, :, 0], 1e-15, "causal row 0 o")
    _close(lse[:, :, 0], 0.25 * np.sum(q[:, :, 0] * k[:, :, 0], -1), 1e-14,
           "causal row 0 lse")


# --- 6. scale zero -------------------------------------------------------------

def check_scale_zero(lib):
    r = _rng(4)
    T, D = 21, 8
    q = r.standard_normal((1, 1, T, D)) * 100
    k = r.standard_normal((1, 1, T, D)) * 100
    v = r.standard_normal((1, 1, T, D))
    o, lse = oracle.attention(q, k, v, False, 0.0, lib=lib)
    _close(o[0, 0], np.broadcast_to(v[0, 0].mean(0), (T, D)), 1e-14, "scale 0 o")
    _close(lse[0, 0], np.full(T, math.log(T)), 1e-14, "scale 0 lse")


# --- 7. brute force at tiny sizes ----------------------------------------------

def check_brute_force(lib):
    r = _rng(5)
    for (B, Hq, Hkv, Tq, Tk, D) in ((1, 1, 1, 1, 1, 1), (1, 2, 1, 3, 4, 2),
                                    (2, 2, 2, 4, 4, 3), (1, 4, 2, 2, 3, 4),
                                    (1, 1, 1, 4, 2, 4)):
        q = r.standard_normal((B, Hq, Tq, D))
        k = r.standard_normal((B, Hkv, Tk, D))
        v = r.standard_normal((B, Hkv, Tk, D))
        for causal in (False, True):
            o, lse = oracle.attention(q, k, v, causal, 0.7, lib=lib)
            bo, bl = brute.attention(q.tolist(), k.tolist(), v.tolist(), causal, 0.7)
            _close(o, bo, 1e-14, f"brute o {B,Hq,Hkv,Tq,Tk,D} causal={causal}")
            _close(lse, bl, 1e-14, f"brute lse {B,Hq,Hkv,Tq,Tk,D} causal={causal}")


# --- scipy: the softmax and logsumexp library routines --------------------------

def check_scipy(lib):
    r = _rng(6)
    B, Hq, Hkv, Tq, Tk, D = 2, 4, 2, 19, 23, 16
    q = r.standard_normal((B, Hq, Tq, D))
    k = r.standard_normal((B, Hkv, Tk, D))
    v = r.standard_normal((B, Hkv, Tk, D))
    scale = 1 / math.sqrt(D)
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, causal, scale, lib=lib)
        for b in range(B):
            for h in range(Hq):
                kk, vv = k[b, h // 2], v[b, h // 2]
                s = scale * (q[b, h] @ kk.T)
                if causal:
                    i = np.arange(Tq)[:, None]
                    j = np.arange(Tk)[None, :]
                    s = np.where(j > i + (Tk - Tq), -np.inf, s)
                _close(lse[b, h], scipy.special.logsumexp(s, axis=1), 1e-12, "scipy lse")
                _close(o[b, h], scipy.special.softmax(s, axis=1) @ vv, 1e-12, "scipy o")


# --- softmax rows sum to one ---------------------------------------------------

def check_rows_sum_to_one(lib):
    r = _rng(7)
    T = 16
    q = r.standard_normal((1, 1, T, T)) * 3
    k = r.standard_normal((1, 1, T, T)) * 3
    # V = identity: O row i is the probability row P_i itself
    v = np.eye(T)[None, None]
    for causal in (False, True):
        o, _ = oracle.attention(q, k, v, causal, 1.0, lib=lib)
        p = o[0, 0]
        assert np.all(p >= 0), "negative probability"
        _close(p.sum(1), np.ones(T), 1e-14, "softmax row sum")
        if causal:
            assert np.all(np.triu(p, 1) == 0), "causal mask leaked"


# --- 8. permutation invariance -------------------------------------------------

def check_permutation(lib):
    r = _rng(8)
    T, D = 40, 8
    q = r.standard_normal((1, 2, 5, D))
    k = r.standard_normal((1, 2, T, D))
    v = r.standard_normal((1, 2, T, D))
    perm = r.permutation(T)
    o1, l1 = oracle.attention(q, k, v, False, 0.5, lib=lib)
    o2, l2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], False, 0.5, lib=lib)
    _close(o1, o2, 1e-14, "permuted keys o")
    _close(l1, l2, 1e-14, "permuted keys lse")
    # paged: the same logical cache under a random and an identity placement
    a = wl.paged_decode_inputs(3, 4, 2, 8, "f32", 11, lengths=[35, 16, 1], permute=True)
    b = wl.paged_decode_inputs(3, 4, 2, 8, "f32", 11, lengths=[35, 16, 1], permute=False)
    # re-place b's pool so that its logical content equals a's
    kb = np.zeros_like(a["k_pages"]); vb = np.zeros_like(a["v_pages"])
    for s in range(3):
        for p in range(int(wl.pages_for([a["kv_lens"][s]])[0])):
            kb[b["block_table"][s, p]] = a["k_pages"][a["block_table"][s, p]]
            vb[b["block_table"][s, p]] = a["v_pages"][a["block_table"][s, p]]
    oa, la = oracle.decode_paged(a["q"], a["k_pages"], a["v_pages"], a["block_table"],
                                 a["kv_lens"], a["scale"], lib=lib)
    ob, lb = oracle.decode_paged(a["q"], kb, vb, b["block_table"], b["kv_lens"],
                                 a["scale"], lib=lib)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb), "page placement changed result"


# --- 9. merge(split(x)) = x ------------------------------------------------------

def check_merge_split(lib):
    r = _rng(9)
    T, D = 13, 6
    q = r.standard_normal((1, 3, 2, D))
    k = r.standard_normal((1, 3, T, D))
    v = r.standard_normal((1, 3, T, D))
    full_o, full_l = oracle.attention(q, k, v, False, 0.6, lib=lib)
    for n in range(T + 1):
        oa, la = oracle.attention(q, k[:, :, :n], v[:, :, :n], False, 0.6, lib=lib)
        ob, lb = oracle.attention(q, k[:, :, n:], v[:, :, n:], False, 0.6, lib=lib)
        o, l = oracle.merge_states(oa, la, ob, lb, lib=lib)
        _close(o, full_o, 1e-13, f"merge(split at {n}) o")
        _close(l, full_l, 1e-13, f"merge(split at {n}) lse")
    # a three-way split folded in order
    parts = [(0, 4), (4, 9), (9, T)]
    acc = None
    for lo, hi in parts:
        st = oracle.attention(q, k[:, :, lo:hi], v[:, :, lo:hi], False, 0.6, lib=lib)
        acc = st if acc is None else oracle.merge_states(*acc, *st, lib=lib)
    _close(acc[0], full_o, 1e-13, "3-way merge o")
    _close(acc[1], full_l, 1e-13, "3-way merge lse")


# --- 10. merge algebra -----------------------------------------------------------

def check_merge_algebra(lib):
    r = _rng(10)
    rows, D = 7, 5
    st = [(r.standard_normal((rows, D)), r.standard_normal(rows) * 3) for _ in range(3)]
    a, b, c = st
    ab = oracle.merge_states(*a, *b, lib=lib)
    ba = oracle.merge_states(*b, *a, lib=lib)
    _close(ab[0], ba[0], 1e-14, "commutative o"); _close(ab[1], ba[1], 1e-14, "commutative lse")
    l1 = oracle.merge_states(*ab, *c, lib=lib)
    l2 = oracle.merge_states(*a, *oracle.merge_states(*b, *c, lib=lib), lib=lib)
    _close(l1[0], l2[0], 1e-13, "associative o"); _close(l1[1], l2[1], 1e-13, "associative lse")
    empty = (np.full((rows, D), np.nan), np.full(rows, -np.inf))
    e1 = oracle.merge_states(*a, *empty, lib=lib)
    _close(e1[0], a[0], 0.0, "identity o"); _close(e1[1], a[1], 0.0, "identity lse")
    e2 = oracle.merge_states(*empty, *a, lib=lib)
    _close(e2[0], a[0], 0.0, "identity (left) o")
    aa = oracle.merge_states(*a, *a, lib=lib)
    _close(aa[0], a[0], 1e-15, "self merge o")
    _close(aa[1], a[1] + math.log(2.0), 1e-14, "self merge lse")
    ee = oracle.merge_states(*empty, *empty, lib=lib)
    assert np.all(ee[0] == 0) and np.all(ee[1] == -np.inf), "empty+empty"
    # closed form on one row: lse of the union is ln(e^la + e^lb)
    la, lb = 0.3, -1.2
    oa, ob = np.array([[1.0, 0.0]]), np.array([[0.0, 1.0]])
    o, l = oracle.merge_states(oa, np.array([la]), ob, np.array([lb]), lib=lib)
    wa = math.exp(la) / (math.exp(la) + math.exp(lb))
    _close(o[0], [wa, 1 - wa], 1e-15, "merge weights")
    _close(l, [math.log(math.exp(la) + math.exp(lb))], 1e-15, "merge lse closed form")


# --- 11. cascade = concatenation -------------------------------------------------

def check_cascade(lib):
    c = wl.cascade_inputs(5, 4, 8, "f32", 12, prefix_len=64, suffix_range=(1, 40))
    direct = oracle.cascade_decode(c["q"], c["k_pages"], c["v_pages"], c["prefix_pages"],
                                   c["prefix_len"], c["suffix_table"], c["suffix_lens"],
                                   c["scale"], lib=lib)
    R = c["q"].shape[0]
    pre_tab = np.broadcast_to(c["prefix_pages"], (R, len(c["prefix_pages"]))).copy()
    pre = oracle.decode_paged(c["q"], c["k_pages"], c["v_pages"], pre_tab,
                              np.full(R, c["prefix_len"], np.int32), c["scale"], lib=lib)
    suf = oracle.decode_paged(c["q"], c["k_pages"], c["v_pages"], c["suffix_table"],
                              c["suffix_lens"], c["scale"], lib=lib)
    o, l = oracle.merge_states(*pre, *suf, lib=lib)
    _close(o, direct[0], 1e-13, "cascade o")
    _close(l, direct[1], 1e-13, "cascade lse")


# --- 12. decode = last prefill row -----------------------------------------------

def check_decode_vs_prefill(lib):
    d = wl.paged_decode_inputs(4, 4, 2, 16, "f32", 13, lengths=[1, 17, 32, 50])
    o, lse = oracle.decode_paged(d["q"], d["k_pages"], d["v_pages"], d["block_table"],
                                 d["kv_lens"], d["scale"], lib=lib)
    for b in range(4):
        L = int(d["kv_lens"][b])
        K = np.stack([d["k_pages"][d["block_table"][b, t // 16], :, t % 16] for t in range(L)], 1)
        V = np.stack([d["v_pages"][d["block_table"][b, t // 16], :, t % 16] for t in range(L)], 1)
        po, pl = oracle.attention(d["q"][b][None, :, None], K[None], V[None], False,
                                  d["scale"], lib=lib)
        _close(o[b], po[0, :, 0], 1e-14, "decode vs prefill o")
        _close(lse[b], pl[0, :, 0], 1e-14, "decode vs prefill lse")
        # causal prefill whose last query row is this token gives the same
        Tq = 3
        qq = np.zeros((1, 4, Tq, 16), np.float32); qq[0, :, -1] = d["q"][b]
        co, cl = oracle.attention(qq, K[None], V[None], True, d["scale"], lib=lib)
        _close(co[0, :, -1], o[b], 1e-14, "causal last row vs decode")


# --- 13. GQA head mapping ------------------------------------------------------

def check_gqa_mapping(lib):
    Hq, Hkv = 8, 2
    G = Hq // Hkv
    d = wl.paged_decode_inputs(2, Hq, Hkv, 4, "f32", 14, lengths=[20, 33])
    v = np.empty_like(d["v_pages"])
    for g in range(Hkv):
        v[:, g] = g + 1
    o, _ = oracle.decode_paged(d["q"], d["k_pages"], v, d["block_table"], d["kv_lens"],
                               d["scale"], lib=lib)
    for h in range(Hq):
        _close(o[:, h], np.full((2, 4), h // G + 1.0), 1e-14, f"GQA head {h}")
    # dense form too
    q = np.random.default_rng(0).standard_normal((1, Hq, 3, 4))
    k = np.random.default_rng(1).standard_normal((1, Hkv, 5, 4))
    vv = np.stack([np.full((5, 4), g + 1.0) for g in range(Hkv)])[None]
    o, _ = oracle.attention(q, k, vv, True, 1.0, lib=lib)
    for h in range(Hq):
        _close(o[0, h], np.full((3, 4), h // G + 1.0), 1e-14, f"dense GQA head {h}")


# --- 14. which tokens were read ----------------------------------------------------

def check_token_set(lib):
    D = 12
    lens = [1, 15, 16, 17, 100, 1000]
    d = wl.paged_decode_inputs(len(lens), 2, 2, D, "f32", 15, lengths=lens,
                               tail_garbage=True)
    k = d["k_pages"].copy(); v = d["v_pages"].copy()
    for b, L in enumerate(lens):
        for t in range(L):
            pg, sl = d["block_table"][b, t // 16], t % 16
            k[pg, :, sl] = 0.25
            v[pg, :, sl] = [(t >> c) & 1 for c in range(D)]
    o, lse = oracle.decode_paged(d["q"], k, v, d["block_table"], d["kv_lens"],
                                 d["scale"], lib=lib)
    for b, L in enumerate(lens):
        exp_o = [sum((t >> c) & 1 for t in range(L)) / L for c in range(D)]
        for h in range(2):
            _close(o[b, h], exp_o, 1e-14, f"token set L={L}")
            s = d["scale"] * 0.25 * math.fsum(d["q"][b, h].astype(np.float64))
            _close(lse[b, h], s + math.log(L), 1e-13, f"token-set lse L={L}")


# --- 15. lse sees a dropped page -------------------------------------------------

def check_lse_dropped_page(lib):
    L, D = 4096, 8
    d = wl.paged_decode_inputs(1, 1, 1, D, "f32", 16, lengths=[L])
    k = np.full_like(d["k_pages"], 0.5)
    o, lse = oracle.decode_paged(d["q"], k, d["v_pages"], d["block_table"], d["kv_lens"],
                                 d["scale"], lib=lib)
    s = d["scale"] * 0.5 * math.fsum(d["q"][0, 0].astype(np.float64))
    _close(lse[0, 0], s + math.log(L), 1e-12, "lse = s + ln L")
    # the same cache with one page fewer moves lse by ln((L-16)/L)
    o2, lse2 = oracle.decode_paged(d["q"], k, d["v_pages"], d["block_table"],
                                   np.array([L - 16], np.int32), d["scale"], lib=lib)
    _close(lse2[0, 0] - lse[0, 0], math.log((L - 16) / L), 1e-12, "dropped page shift")


# --- 16. tail garbage ------------------------------------------------------------

def check_tail_garbage(lib):
    lens = [5, 16, 23]
    a = wl.paged_decode_inputs(3, 2, 1, 8, "f32", 17, lengths=lens, tail_garbage=True)
    b = wl.paged_decode_inputs(3, 2, 1, 8, "f32", 17, lengths=lens, tail_garbage=False)
    kn, vn = a["k_pages"].copy(), a["v_pages"].copy()
    for bb, L in enumerate(lens):
        if L % 16:
            pg = a["block_table"][bb, (L - 1) // 16]
            kn[pg, :, L % 16:] = np.nan
            vn[pg, :, L % 16:] = np.nan
    ra = oracle.decode_paged(a["q"], a["k_pages"], a["v_pages"], a["block_table"], a["kv_lens"], a["scale"], lib=lib)
    rb = oracle.decode_paged(b["q"], b["k_pages"], b["v_pages"], b["block_table"], b["kv_lens"], b["scale"], lib=lib)
    rn = oracle.decode_paged(a["q"], kn, vn, a["block_table"], a["kv_lens"], a["scale"], lib=lib)
    for r, what in ((rb, "zeros"), (rn, "NaN")):
        assert np.array_equal(ra[0], r[0]) and np.array_equal(ra[1], r[1]), \
            f"tail slots ({what}) changed the result"


# --- bf16 widening ---------------------------------------------------------------

def check_bf16_widening(lib):
    r = _rng(18)
    x = r.standard_normal((1, 2, 9, 8)).astype(np.float32)
    bits = [wl.bf16_bits(x) for _ in range(3)]
    wide = [wl.bf16_to_f32(b) for b in bits]
    o1, l1 = oracle.attention(bits[0], bits[1], bits[2], True, 0.4, lib=lib)
    o2, l2 = oracle.attention(wide[0], wide[1], wide[2], True, 0.4, lib=lib)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "bf16 widening"


# --- 17. fallback model of the unified-max softmax ----------------------------

def check_unified_fallback(lib):
    """The (row, chunk) pairs that leave phi +- 60 (the reading of the unified
    max of the FlashDecoding++ summary, sections 1 and 3): closed forms from
    constant and one-hot scores, and the brute force on random tiny cases."""
    D, split, Hq, Hkv = 8, 32, 4, 2
    lens = [40, 16, 100]                        # 2 + 1 + 4 chunks of 32
    d = wl.paged_decode_inputs(len(lens), Hq, Hkv, D, "f32", 21, lengths=lens)
    bt, kl = d["block_table"], d["kv_lens"]
    pairs = Hq * sum((L + split - 1) // split for L in lens)
    # every score s = 1 * (2 e0) . (5 e0) = 10 exactly
    k = np.zeros_like(d["k_pages"]); k[..., 0] = 5.0
    q = np.zeros_like(d["q"]); q[..., 0] = 2.0
    for phi, expect in ((0.0, 0), (100.0, pairs), (-55.0, pairs), (-45.0, 0), (69.0, 0), (71.0, pairs)):
        n = oracle.unified_fallback_count(q, k, bt, kl, 1.0, split, phi, lib=lib)
        assert n == expect, f"constant scores, phi {phi}: {n} != {expect}"
    # one key with score 100 (sequence 2, token 37 = chunk 1, kv head 1) and
    # every other score 0: only heads 2 and 3 of that chunk fall back
    k = np.zeros_like(d["k_pages"])
    k[bt[2][37 // 16], 1, 37 % 16, 0] = 100.0
    q = np.zeros_like(d["q"]); q[..., 0] = 1.0
    n = oracle.unified_fallback_count(q, k, bt, kl, 1.0, split, 0.0, lib=lib)
    assert n == 2, f"one dominant key: {n} != 2"
    # brute force: random scores spread over a few hundred around phi
    g = _rng(22)
    for case in range(3):
        lens = [int(x) for x in g.integers(1, 70, size=3)]
        d = wl.paged_decode_inputs(3, Hq, Hkv, D, "f32", 30 + case, lengths=lens)
        scale, phi = float(g.uniform(20, 60)), float(g.uniform(-50, 50))
        n = oracle.unified_fallback_count(d["q"], d["k_pages"], d["block_table"], d["kv_lens"],
                                          scale, 16, phi, lib=lib)
        keys = [[[d["k_pages"][d["block_table"][b][t // 16], kvh, t % 16].tolist()
                  for t in range(lens[b])] for kvh in range(Hkv)] for b in range(3)]
        ref = brute.unified_fallback_count(d["q"].tolist(), keys, lens, scale, 16, phi)
        assert n == ref, f"brute force case {case}: {n} != {ref}"
        assert 0 < ref < Hq * sum((L + 15) // 16 for L in lens), "case should mix in and out"


# --- 18. FP8 (OCP E4M3) caches ------------------------------------------------

def check_e4m3_values(lib):
    """Values that the OCP 8-bit floating point format fixes for E4M3: 1.0 is
    0x38, the largest finite value 448 is 0x7E, the smallest normal 2^-6 is
    0x08, the smallest subnormal 2^-9 is 0x01, S.1111.111 is NaN, the top bit
    is the sign; the positive codes increase strictly; the generator's own
    round-to-nearest encoder inverts the decoder on every finite nonzero code;
    every value is exact in bf16."""
    v = [oracle.e4m3_value(b, lib=lib) for b in range(256)]
    assert v[0x00] == 0.0 and math.copysign(1.0, v[0x80]) == -1.0, "zeros"
    assert v[0x38] == 1.0 and v[0x40] == 2.0 and v[0x30] == 0.5, "one, two, half"
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0, "largest finite"
    assert v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9, \
        "normal / subnormal boundary"
    assert math.isnan(v[0x7F]) and math.isnan(v[0xFF]), "NaN codes"
    pos = v[0x00:0x7F]
    assert all(a < b for a, b in zip(pos, pos[1:])), "positive codes not increasing"
    assert all(v[b | 0x80] == -v[b] for b in range(0x7F)), "sign bit"
    fin = [b for b in range(256) if not math.isnan(v[b]) and v[b] != 0.0]
    assert list(wl.e4m3_bits(np.array([v[b] for b in fin]))) == fin, "encoder round trip"
    x = np.array([v[b] for b in fin], np.float32)
    assert np.array_equal(wl.bf16_to_f32(wl.bf16_bits(x)), x), "E4M3 values exact in bf16"


def check_decode_fp8(lib):
    """The FP8 decode is the plain decode of the dequantised cache: it equals
    oracle.decode_paged on scale * value arrays (built here from the pinned
    value table) for GQA, ragged lengths and unequal k / v scales; and with
    every key equal the weights are uniform (closed form for O and lse)."""
    table = np.array([oracle.e4m3_value(b, lib=lib) for b in range(256)])
    lens = [1, 15, 16, 17, 70]
    Hq, Hkv, D = 4, 2, 16
    d = wl.paged_decode_fp8_inputs(len(lens), Hq, Hkv, D, 31, lengths=lens)
    ks, vs = 0.75, 1.0 / 16
    bt, kl, sc = d["block_table"], d["kv_lens"], d["scale"]
    o8, l8 = oracle.decode_paged_fp8(d["q"], d["k_pages"], d["v_pages"], ks, vs, bt, kl, sc,
                                     lib=lib)
    qf = wl.bf16_to_f32(d["q"]).astype(np.float64)
    o, l = oracle.decode_paged(qf, ks * table[d["k_pages"]], vs * table[d["v_pages"]], bt, kl,
                               sc, lib=lib)
    _close(o8, o, 1e-14, "fp8 decode vs dequantised decode")
    _close(l8, l, 1e-13, "fp8 decode lse")
    k1 = np.full_like(d["k_pages"], 0x38)          # every key = 1.0 * 2.0
    o1, l1 = oracle.decode_paged_fp8(d["q"], k1, d["v_pages"], 2.0, vs, bt, kl, sc, lib=lib)
    for b, L in enumerate(lens):
        for h in range(Hq):
            kvh = h // (Hq // Hkv)
            vals = [vs * table[d["v_pages"][bt[b, t // 16], kvh, t % 16]] for t in range(L)]
            _close(o1[b, h], np.mean(vals, axis=0), 1e-14, f"fp8 uniform O L={L}")
            s = sc * 2.0 * math.fsum(qf[b, h])
            _close(l1[b, h], s + math.log(L), 1e-13, f"fp8 uniform lse L={L}")


# --- prefill against a paged cache (chunked prefill) -----------------------------

def _tiny_paged(r, B, Hkv, D, page, lens):
    """A random pool holding each sequence's pages at permuted places."""
    npages = [-(-L // page) for L in lens]
    pool = max(1, sum(npages))
    phys = r.permutation(pool).astype(np.int32)
    table = np.zeros((B, max(1, max(npages))), np.int32)
    at = 0
    for b, n in enumerate(npages):
        table[b, :n] = phys[at:at + n]
        at += n
    kp = r.standard_normal((pool, Hkv, page, D))
    vp = r.standard_normal((pool, Hkv, page, D))
    return kp, vp, table


def check_prefill_paged_brute(lib):
    """Gather through the table and bottom-right causal offset against the
    pure-Python brute force on each sequence's logical keys."""
    r = _rng(41)
    for (B, Hq, Hkv, Tq, D, page, lens) in ((2, 2, 1, 3, 3, 2, [5, 3]),
                                            (3, 2, 2, 2, 2, 4, [1, 7, 2]),
                                            (1, 4, 2, 4, 2, 2, [4])):
        kp, vp, table = _tiny_paged(r, B, Hkv, D, page, lens)
        q = r.standard_normal((B, Hq, Tq, D))
        kl = np.asarray(lens, np.int32)
        for causal in (False, True):
            o, lse = oracle.prefill_paged(q, kp, vp, table, kl, causal, 0.6, lib=lib)
            for b, L in enumerate(lens):
                K = [[[float(x) for x in kp[table[b, t // page], h, t % page]] for t in range(L)]
                     for h in range(Hkv)]
                V = [[[float(x) for x in vp[table[b, t // page], h, t % page]] for t in range(L)]
                     for h in range(Hkv)]
                bo, bl = brute.attention([q[b].tolist()], [K], [V], causal, 0.6)
                _close(o[b], bo[0], 1e-14, f"paged prefill brute o b={b} causal={causal}")
                _close(lse[b], bl[0], 1e-14, f"paged prefill brute lse b={b} causal={causal}")


def check_prefill_paged_identical_keys(lib):
    """Identical keys: query i of the chunk sees n_i = kv_len - Tq + i + 1 keys
    (causal, bottom-right) or all kv_len, so O_i is the mean of those value
    rows and lse_i = s_i + ln n_i, a closed form in the offset."""
    r = _rng(43)
    B, Hq, Hkv, Tq, D, page = 2, 2, 1, 5, 4, 4
    lens = [9, 5]
    kp, vp, table = _tiny_paged(r, B, Hkv, D, page, lens)
    k0 = np.array([0.5, -1.0, 0.25, 2.0])
    kp[:] = k0
    q = r.standard_normal((B, Hq, Tq, D))
    kl = np.asarray(lens, np.int32)
    for causal in (False, True):
        o, lse = oracle.prefill_paged(q, kp, vp, table, kl, causal, 0.8, lib=lib)
        for b, L in enumerate(lens):
            vrows = np.stack([vp[table[b, t // page], 0, t % page] for t in range(L)])
            for h in range(Hq):
                for i in range(Tq):
                    n = L - Tq + i + 1 if causal else L
                    s = 0.8 * float(q[b, h, i] @ k0)
                    _close(o[b, h, i], vrows[:n].mean(0), 1e-13, f"identical keys o {b,h,i}")
                    _close(lse[b, h, i], s + math.log(n), 1e-13, f"identical keys lse {b,h,i}")


def check_prefill_paged_placement_and_decode(lib):
    """The same logical cache under two physical placements gives the same
    bits, and a one-token chunk is the paged decode of that token."""
    r = _rng(47)
    B, Hq, Hkv, D, page = 3, 4, 2, 8, 4
    lens = [13, 4, 9]
    kp, vp, table = _tiny_paged(r, B, Hkv, D, page, lens)
    q = r.standard_normal((B, Hq, 3, D))
    kl = np.asarray(lens, np.int32)
    # move every page to a new place
    perm = r.permutation(kp.shape[0])
    kp2 = np.empty_like(kp); vp2 = np.empty_like(vp)
    kp2[perm] = kp; vp2[perm] = vp
    table2 = perm[table].astype(np.int32)
    for causal in (False, True):
        o1, l1 = oracle.prefill_paged(q, kp, vp, table, kl, causal, 0.4, lib=lib)
        o2, l2 = oracle.prefill_paged(q, kp2, vp2, table2, kl, causal, 0.4, lib=lib)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "page placement changed result"
    o, l = oracle.prefill_paged(q[:, :, 2:], kp, vp, table, kl, True, 0.4, lib=lib)
    od, ld = oracle.decode_paged(q[:, :, 2], kp, vp, table, kl, 0.4, lib=lib)
    _close(o[:, :, 0], od, 1e-15, "one-token chunk vs decode o")
    _close(l[:, :, 0], ld, 1e-15, "one-token chunk vs decode lse")


# --- flat GEMM of the decode phase ----------------------------------------------

def check_flat_gemm(lib):
    """C = A W^T against a pure-Python triple loop (math.fsum) on tiny shapes,
    a one-hot A that selects columns of W (fixes which operand is transposed
    and the index order), and numpy's matmul of the widened values."""
    r = _rng(53)
    for (m, n, k) in ((1, 1, 1), (2, 3, 4), (3, 5, 2), (4, 2, 7)):
        a = r.standard_normal((m, k))
        w = r.standard_normal((n, k))
        c = oracle.flat_gemm(a, w, lib=lib)
        ref = [[math.fsum(a[i, t] * w[j, t] for t in range(k)) for j in range(n)] for i in range(m)]
        _close(c, ref, 1e-14, f"flat gemm brute {(m, n, k)}")
    m, n, k = 3, 6, 5
    w = r.standard_normal((n, k))
    a = np.zeros((m, k))
    picks = [4, 0, 2]
    for i, t in enumerate(picks):
        a[i, t] = 1.0
    c = oracle.flat_gemm(a, w, lib=lib)
    assert np.array_equal(c, w[:, picks].T), "one-hot rows must select columns of W"
    a = wl.normal(wl.generator(54), (16, 256), "bf16")
    w = wl.normal(wl.generator(55), (48, 256), "bf16")
    c = oracle.flat_gemm(a, w, lib=lib)
    af = wl.bf16_to_f32(a).astype(np.float64)
    wf = wl.bf16_to_f32(w).astype(np.float64)
    _close(c, af @ wf.T, 1e-12, "flat gemm vs numpy matmul (bf16 inputs)")


ALL_CHECKS = [
    check_hand_2x2, check_identical_keys, check_dominant_score,
    check_single_key_and_row0, check_scale_zero, check_brute_force, check_scipy,
    check_rows_sum_to_one, check_permutation, check_merge_split, check_merge_algebra,
    check_cascade, check_decode_vs_prefill, check_gqa_mapping, check_token_set,
    check_lse_dropped_page, check_tail_garbage, check_bf16_widening, check_unified_fallback,
    check_e4m3_values, check_decode_fp8, check_prefill_paged_brute,
    check_prefill_paged_identical_keys, check_prefill_paged_placement_and_decode,
    check_flat_gemm,
]
