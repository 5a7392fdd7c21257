"""GPU parity of paged decode, state merging and shared-prefix cascade
decode against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from attention_tiled_fmha_amd import attn
from attention_tiled_fmha_amd import workloads as wl
from gpu_util import assert_close, dev, empty_like_out, host, require_gpu

pytestmark = pytest.mark.gpu


def run_decode(d, split_tokens=0, o_dtype=None, table=None):
    o_dtype = o_dtype or d["dtype"]
    q = dev(d["q"])
    o = empty_like_out(q.shape, o_dtype)
    lse = torch.full(q.shape[:2], float("nan"), device="cuda")
    bt = dev(d["block_table"] if table is None else table)
    attn.attn_decode_paged(q, dev(d["k_pages"]), dev(d["v_pages"]), bt, dev(d["kv_lens"]), o,
                           lse, max_kv_len=int(d["kv_lens"].max(initial=0)), scale=d["scale"],
                           split_tokens=split_tokens)
    torch.cuda.synchronize()
    return host(o), host(lse)


def oracle_decode(d, rows=None):
    if rows is None:
        return oracle.decode_paged(d["q"], d["k_pages"], d["v_pages"], d["block_table"],
                                   d["kv_lens"], d["scale"])
    return oracle.decode_paged(d["q"][rows], d["k_pages"], d["v_pages"], d["block_table"][rows],
                               d["kv_lens"][rows], d["scale"])


LENS = [0, 1, 15, 16, 17, 63, 64, 65, 200, 511, 512, 513, 1000, 1500]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("heads", [(4, 4), (8, 4), (16, 4), (32, 8), (8, 1)])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_shapes(dtype, heads, D):
    """Ragged lengths (empty, one token, page edges, chunk edges), MHA and
    GQA groups 2/4/8/1->8, both head sizes, random page placement, garbage
    in unused page slots."""
    require_gpu()
    Hq, Hkv = heads
    d = wl.paged_decode_inputs(len(LENS), Hq, Hkv, D, dtype, 21 + Hq + D, lengths=LENS)
    o, lse = run_decode(d)
    ro, rl = oracle_decode(d)
    assert_close(o, ro, dtype, "O")
    assert_close(lse, rl, dtype, "lse")
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0])), "empty sequence"


@pytest.mark.parametrize("split", [64, 128, 192, 512, 1024])
def test_decode_forced_splits(split):
    """Any chunk length gives the same result (merge(split(x)) = x)."""
    require_gpu()
    d = wl.paged_decode_inputs(6, 8, 2, 128, "f32", 5, lengths=[1, 100, 511, 700, 1024, 2049])
    o, lse = run_decode(d, split_tokens=split)
    ro, rl = oracle_decode(d)
    assert_close(o, ro, "f32", f"O split {split}")
    assert_close(lse, rl, "f32", f"lse split {split}")


def test_decode_fp32_output_of_bf16_cache():
    require_gpu()
    d = wl.paged_decode_inputs(4, 8, 8, 128, "bf16", 6, lengths=[5, 300, 1200, 64])
    o, lse = run_decode(d, o_dtype="f32")
    ro, rl = oracle_decode(d)
    assert_close(o, ro, "bf16", "O")


def test_decode_page_placement_invariance():
    """A random physical placement and the identity placement of the same
    logical cache agree to fp32 reordering (here: bit-identical)."""
    require_gpu()
    lens = [37, 800, 1600]
    a = wl.paged_decode_inputs(3, 4, 4, 128, "bf16", 9, lengths=lens, permute=True)
    kb = np.zeros_like(a["k_pages"]); vb = np.zeros_like(a["v_pages"])
    ident = np.zeros_like(a["block_table"])
    pos = 0
    for s, L in enumerate(lens):
        for p in range(-(-L // 16)):
            kb[pos] = a["k_pages"][a["block_table"][s, p]]
            vb[pos] = a["v_pages"][a["block_table"][s, p]]
            ident[s, p] = pos
            pos += 1
    b = dict(a, k_pages=kb, v_pages=vb, block_table=ident)
    oa, la = run_decode(a)
    ob, lb = run_decode(b)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_decode_gqa_mapping_exact():
    require_gpu()
    d = wl.paged_decode_inputs(3, 32, 8, 128, "bf16", 10, lengths=[17, 600, 2000])
    for g in range(8):
        d["v_pages"][:, g] = wl.bf16_bits(np.float32(g + 1))
    o, _ = run_decode(d)
    for h in range(32):
        assert np.all(o[:, h] == h // 4 + 1), f"head {h}"


def test_decode_token_set_and_lse_of_every_page():
    """Identical keys and V[t][c] = bit c of t (fp32): O[c] is the share of
    the first L tokens with bit c set, and lse = s + ln L exactly -- a
    skipped or repeated page or a read past kv_len changes both."""
    require_gpu()
    D = 64
    lens = [1, 16, 17, 100, 1000, 4097, 8191]
    d = wl.paged_decode_inputs(len(lens), 2, 2, D, "f32", 12, lengths=lens)
    for b, L in enumerate(lens):
        for t in range(L):
            pg, sl = d["block_table"][b, t // 16], t % 16
            d["k_pages"][pg, :, sl] = 0.25
            d["v_pages"][pg, :, sl] = [(t >> c) & 1 for c in range(D)]
    o, lse = run_decode(d)
    for b, L in enumerate(lens):
        expect = np.array([sum((t >> c) & 1 for t in range(L)) / L for c in range(D)])
        s = d["scale"] * 0.25 * d["q"][b].astype(np.float64).sum(-1)
        for h in range(2):
            assert np.abs(o[b, h] - expect).max() <= 1e-6, f"token set L={L}"
            assert abs(lse[b, h] - (s[h] + np.log(L))) <= 2e-6, f"lse L={L}"


def test_decode_equals_last_prefill_row():
    require_gpu()
    L, D = 700, 128
    d = wl.paged_decode_inputs(1, 4, 4, D, "f32", 13, lengths=[L])
    o, lse = run_decode(d)
    K = np.stack([d["k_pages"][d["block_table"][0, t // 16], :, t % 16] for t in range(L)], 1)
    V = np.stack([d["v_pages"][d["block_table"][0, t // 16], :, t % 16] for t in range(L)], 1)
    q = torch.from_numpy(d["q"][0][None, :, None].copy()).cuda()
    po = torch.empty_like(q)
    pl = torch.empty((1, 4, 1), device="cuda")
    attn.attn_prefill(q, dev(K[None].copy()), dev(V[None].copy()), po, pl, causal=False,
                      scale=d["scale"])
    torch.cuda.synchronize()
    assert_close(o[0], host(po)[0, :, 0], "f32", "decode vs prefill O")
    assert_close(lse[0], host(pl)[0, :, 0], "f32", "decode vs prefill lse")


@pytest.mark.parametrize("name", [wl.DECODE_MHA, wl.DECODE_GQA])
def test_decode_workloads_full_size_sampled(name):
    """The MHA (B32 H32, L~U[512,8192]) and GQA (B128 32/8, L~logU[1024,32768],
    chunks of 512) decode workloads at full size in the bench's launch
    configuration; the oracle checks a sample of sequences element by
    element."""
    require_gpu()
    d = wl.workload(name)
    o, lse = run_decode(d, split_tokens=d.get("split_tokens", 0))
    rows = [0, 1, int(np.argmax(d["kv_lens"])), int(np.argmin(d["kv_lens"])), d["B"] - 1]
    ro, rl = oracle_decode(d, rows)
    assert_close(o[rows], ro, "bf16", f"O rows {rows}")
    assert_close(lse[rows], rl, "bf16", f"lse rows {rows}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


# ---------------------------------------------------------------------------
# attn_merge_states
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_merge_states(dtype, D):
    require_gpu()
    r = np.random.default_rng(D)
    rows = 1000
    oa = r.standard_normal((rows, D)).astype(np.float32)
    ob = r.standard_normal((rows, D)).astype(np.float32)
    la = (r.standard_normal(rows) * 5).astype(np.float32)
    lb = (r.standard_normal(rows) * 5).astype(np.float32)
    la[::7] = -np.inf
    lb[::11] = -np.inf
    ob[::11] = np.nan          # an empty side's o is never read
    if dtype == "bf16":
        oa_h, ob_h = wl.bf16_bits(oa), wl.bf16_bits(ob)
        oa_r, ob_r = wl.bf16_to_f32(oa_h), wl.bf16_to_f32(ob_h)
    else:
        oa_h, ob_h, oa_r, ob_r = oa, ob, oa, ob
    to, tl = dev(oa_h), dev(la)
    attn.attn_merge_states(to, tl, dev(ob_h), dev(lb))
    torch.cuda.synchronize()
    ro, rl = oracle.merge_states(oa_r, la, ob_r, lb)
    assert_close(host(to), ro, dtype, "merged O")
    assert_close(host(tl), rl, "f32", "merged lse")
    both = np.isneginf(la) & np.isneginf(lb)
    assert np.all(host(to)[both] == 0)


def test_merge_states_self_alias():
    require_gpu()
    r = np.random.default_rng(1)
    o = r.standard_normal((64, 128)).astype(np.float32)
    l = r.standard_normal(64).astype(np.float32)
    to, tl = dev(o), dev(l)
    attn.attn_merge_states(to, tl, to, tl)
    torch.cuda.synchronize()
    assert np.abs(host(to) - o).max() <= 1e-6
    assert np.abs(host(tl) - (l.astype(np.float64) + np.log(2))).max() <= 1e-6


# ---------------------------------------------------------------------------
# shared-prefix cascade
# ---------------------------------------------------------------------------

def run_cascade(c, o_dtype="bf16"):
    q = dev(c["q"])
    kp, vp = dev(c["k_pages"]), dev(c["v_pages"])
    R, H, D = q.shape
    o_p = empty_like_out(q.shape, o_dtype)
    l_p = torch.empty((R, H), device="cuda")
    attn.attn_decode_shared_prefix(q, kp, vp, dev(c["prefix_pages"]), c["prefix_len"], o_p, l_p,
                                   scale=c["scale"])
    o_s = empty_like_out(q.shape, o_dtype)
    l_s = torch.empty((R, H), device="cuda")
    attn.attn_decode_paged(q, kp, vp, dev(c["suffix_table"]), dev(c["suffix_lens"]), o_s, l_s,
                           max_kv_len=int(c["suffix_lens"].max()), scale=c["scale"])
    attn.attn_merge_states(o_p, l_p, o_s, l_s)
    torch.cuda.synchronize()
    return host(o_p), host(l_p)


def test_cascade_small_fp32():
    require_gpu()
    c = wl.cascade_inputs(9, 4, 128, "f32", 14, prefix_len=160, suffix_range=(1, 300))
    o, lse = run_cascade(c, o_dtype="f32")
    ro, rl = oracle.cascade_decode(c["q"], c["k_pages"], c["v_pages"], c["prefix_pages"],
                                   c["prefix_len"], c["suffix_table"], c["suffix_lens"], c["scale"])
    assert_close(o, ro, "f32", "cascade O")
    assert_close(lse, rl, "f32", "cascade lse")


def test_cascade_r64_prefix4096_full_size():
    """64 requests sharing a 4096-token prefix, suffixes U[128, 1024]."""
    require_gpu()
    c = wl.workload(wl.CASCADE)
    o, lse = run_cascade(c)
    rows = [0, 1, 31, 63]
    sub = dict(c, q=c["q"][rows], suffix_table=c["suffix_table"][rows],
               suffix_lens=c["suffix_lens"][rows])
    ro, rl = oracle.cascade_decode(sub["q"], c["k_pages"], c["v_pages"], c["prefix_pages"],
                                   c["prefix_len"], sub["suffix_table"], sub["suffix_lens"],
                                   c["scale"])
    assert_close(o[rows], ro, "bf16", "cascade O")
    assert_close(lse[rows], rl, "bf16", "cascade lse")


def test_cascade_two_streams():
    """The prefix stage on a second stream, concurrent with the suffix decode
    on the first (the two stages share nothing but the read-only cache), then
    the merge once both are done: the same result as one stream."""
    require_gpu()
    c = wl.workload(wl.CASCADE)
    q = dev(c["q"])
    kp, vp = dev(c["k_pages"]), dev(c["v_pages"])
    R, H, D = q.shape
    o_p, o_s = torch.empty_like(q), torch.empty_like(q)
    l_p, l_s = (torch.empty((R, H), device="cuda") for _ in range(2))
    pp, st, sl = dev(c["prefix_pages"]), dev(c["suffix_table"]), dev(c["suffix_lens"])
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    for rep in range(3):
        side.wait_stream(main)
        attn.attn_decode_shared_prefix(q, kp, vp, pp, c["prefix_len"], o_p, l_p, scale=c["scale"],
                                       stream=side)
        attn.attn_decode_paged(q, kp, vp, st, sl, o_s, l_s, max_kv_len=int(c["suffix_lens"].max()),
                               scale=c["scale"])
        main.wait_stream(side)
        attn.attn_merge_states(o_p, l_p, o_s, l_s)
        torch.cuda.synchronize()
        o, lse = host(o_p), host(l_p)
        if rep == 0:
            first = (o.copy(), lse.copy())
        else:
            # the same kernels on the same data: bit-identical on every repetition
            assert np.array_equal(o, first[0])
            assert np.array_equal(lse, first[1])
    rows = [0, 17, 63]
    ro, rl = oracle.cascade_decode(c["q"][rows], c["k_pages"], c["v_pages"], c["prefix_pages"],
                                   c["prefix_len"], c["suffix_table"][rows], c["suffix_lens"][rows],
                                   c["scale"])
    assert_close(o[rows], ro, "bf16", "cascade O")
    assert_close(lse[rows], rl, "bf16", "cascade lse")


@pytest.mark.parametrize("R,H,Hkv,plen,D", [
    (1, 1, 1, 1, 128), (3, 4, 4, 15, 128), (5, 8, 2, 100, 128), (70, 4, 4, 300, 128),
    (40, 8, 2, 1000, 128), (9, 4, 1, 517, 64), (64, 32, 32, 4096, 128), (16, 2, 2, 20000, 128),
])
@pytest.mark.parametrize("o_dtype", ["bf16", "f32"])
def test_shared_prefix_bf16(R, H, Hkv, plen, D, o_dtype):
    """The MFMA prefix stage against per-request decode of the prefix: more
    than 64 query rows per kv head, GQA groups, ragged prefix lengths, one
    and many prefix chunks."""
    require_gpu()
    c = wl.cascade_inputs(R, H, D, "bf16", 31 + R + plen, prefix_len=plen, suffix_range=(1, 2),
                          Hkv=Hkv)
    q = dev(c["q"])
    o = empty_like_out(q.shape, o_dtype)
    lse = torch.full(q.shape[:2], float("nan"), device="cuda")
    attn.attn_decode_shared_prefix(q, dev(c["k_pages"]), dev(c["v_pages"]), dev(c["prefix_pages"]),
                                   plen, o, lse, scale=c["scale"])
    torch.cuda.synchronize()
    table = np.broadcast_to(c["prefix_pages"], (R, len(c["prefix_pages"]))).copy()
    ro, rl = oracle.decode_paged(c["q"], c["k_pages"], c["v_pages"], table,
                                 np.full(R, plen, np.int32), c["scale"])
    assert_close(host(o), ro, "bf16", "prefix O")
    assert_close(host(lse), rl, "bf16", "prefix lse")


# --- unified-max softmax (asynchronous softmax with recompute fallback) -------

def run_decode_unified(d, phi, split_tokens):
    q = dev(d["q"])
    o = empty_like_out(q.shape, d["dtype"])
    lse = torch.full(q.shape[:2], float("nan"), device="cuda")
    count = torch.zeros(1, dtype=torch.int32, device="cuda")
    attn.attn_decode_paged(q, dev(d["k_pages"]), dev(d["v_pages"]), dev(d["block_table"]),
                           dev(d["kv_lens"]), o, lse, max_kv_len=int(d["kv_lens"].max(initial=0)),
                           scale=d["scale"], split_tokens=split_tokens, unified_max=True, phi=phi,
                           fallback_count=count)
    torch.cuda.synchronize()
    return host(o), host(lse), int(count.item())


def model_count(d, split, phi):
    """The fp64 fallback model; the case must not sit within 0.01 of the
    window edge, where fp32 and fp64 scores could decide differently."""
    args = (d["q"], d["k_pages"], d["block_table"], d["kv_lens"], d["scale"], split, phi)
    n = oracle.unified_fallback_count(*args)
    assert n == oracle.unified_fallback_count(*args, window=59.99) == \
        oracle.unified_fallback_count(*args, window=60.01), "case too close to the window edge"
    return n


UNI_LENS = [0, 1, 16, 17, 300, 512, 513, 1000, 2049]


@pytest.mark.parametrize("phi", [0.0, 100.0, -100.0])
@pytest.mark.parametrize("heads", [(8, 8), (32, 8)])
def test_unified_max(phi, heads):
    """With phi = 0 no (row, chunk) pair of N(0,1) scores leaves the window
    and none falls back; with phi = +-100 every pair does.  Either way the
    result is the plain attention, and the GPU's fallback count is the fp64
    model's."""
    require_gpu()
    Hq, Hkv = heads
    split = 256
    d = wl.paged_decode_inputs(len(UNI_LENS), Hq, Hkv, 128, "bf16", 40 + Hq, lengths=UNI_LENS)
    o, lse, n = run_decode_unified(d, phi, split)
    ro, rl = oracle_decode(d)
    assert_close(o, ro, "bf16", "O")
    assert_close(lse, rl, "bf16", "lse")
    pairs = Hq * sum((L + split - 1) // split for L in UNI_LENS)
    assert n == model_count(d, split, phi) == (0 if phi == 0.0 else pairs)


def test_unified_max_mixed_fallback():
    """Queries of half the sequences scaled by 50: their (row, chunk) pairs
    leave the window around phi = 0 (the others stay inside) and are
    recomputed; the count matches the model and the result the oracle."""
    require_gpu()
    split = 128
    lens = [33, 200, 700, 1500, 64, 129, 900, 2000]
    d = wl.paged_decode_inputs(len(lens), 16, 4, 128, "bf16", 47, lengths=lens)
    q = wl.bf16_to_f32(d["q"])
    q[::2] *= 50.0
    d["q"] = wl.bf16_bits(q)
    o, lse, n = run_decode_unified(d, 0.0, split)
    ro, rl = oracle_decode(d)
    assert_close(o, ro, "bf16", "O")
    assert_close(lse, rl, "bf16", "lse")
    assert n == model_count(d, split, 0.0)
    assert 0 < n < 16 * sum((L + split - 1) // split for L in lens)


def test_unified_max_default_split():
    """Planner-chosen chunks, GQA 4, fp32 output: same result as the plain path."""
    require_gpu()
    d = wl.paged_decode_inputs(6, 32, 8, 128, "bf16", 48, lengths=[5, 600, 1100, 3000, 64, 4096])
    o, lse, n = run_decode_unified(d, 0.0, 0)
    ro, rl = oracle_decode(d)
    assert_close(o, ro, "bf16", "O")
    assert n == 0


def test_decode_longest_context():
    """A 131072-token sequence (128 chunks of 1024 tokens, a 128-way combine)
    next to a 70001-token one (ragged last page), GQA 32/8, every row against
    the oracle, with the planner's split and with forced 512-token chunks."""
    require_gpu()
    d = wl.paged_decode_inputs(2, 32, 8, 128, "bf16", 71, lengths=[131072, 70001])
    assert attn.attn_decode_plan(2, 8, 131072) == (1024, 128)
    ro, rl = oracle_decode(d)
    for split in (0, 512):
        o, lse = run_decode(d, split_tokens=split)
        assert_close(o, ro, "bf16", f"O split {split}")
        assert_close(lse, rl, "bf16", f"lse split {split}")
