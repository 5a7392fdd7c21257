"""attn_decode_cascade (the prefix stage's chunk states and the requests' own
chunk states in one workspace, merged by one combine) through the C ABI.

Parity: against the fp64 oracle's cascade (prefix + suffix attention, the
same definition the three-call path is checked against) at the bf16
tolerance, over GQA groups, ragged prefixes (shorter than one chunk, many
chunks), requests with no own tokens, D = 64 and 128, bf16 and fp32
outputs and FP8 caches; exact pins (identical keys, V[t][c] = bit c of t)
that see a dropped or doubled page; bit-exact repeats; graph replay."""
import numpy as np
import pytest
import torch

import oracle
from attention_tiled_fmha_amd import attn
from attention_tiled_fmha_amd import workloads as wl
from gpu_util import assert_close, dev, empty_like_out, host, require_gpu
from test_gpu_exact_pins import KEY, check_rows, eighths, fill_cache, q_bits

pytestmark = pytest.mark.gpu


def fused(c, o_dtype="bf16", k_scale=1.0, v_scale=1.0, lens=None):
    q = dev(c["q"])
    kp, vp = dev(c["k_pages"]), dev(c["v_pages"])
    o = empty_like_out(q.shape, o_dtype)
    lse = torch.full(q.shape[:2], float("nan"), device="cuda")
    sl = c["suffix_lens"] if lens is None else lens
    attn.attn_decode_cascade(q, kp, vp, dev(c["prefix_pages"]), c["prefix_len"],
                             dev(c["suffix_table"]), dev(sl), o, lse,
                             max_suffix_len=int(np.max(sl, initial=0)), scale=c["scale"],
                             k_scale=k_scale, v_scale=v_scale)
    torch.cuda.synchronize()
    return host(o), host(lse)


def oracle_cascade(c, lens, fp8):
    """The oracle's decode of the prefix alone (every request the same pages)
    and of each request's own tokens, merged by the oracle's state merge:
    attention over the union of the two key sets for any prefix length."""
    R = c["q"].shape[0]
    npre = len(c["prefix_pages"])
    pre_table = np.broadcast_to(c["prefix_pages"], (R, max(npre, 1))).astype(np.int32).copy()
    pre_lens = np.full(R, c["prefix_len"], np.int32)
    lens = np.asarray(lens, np.int32)
    if fp8:
        ks, vs = c["k_scale"], c["v_scale"]
        dec = lambda t, n: oracle.decode_paged_fp8(c["q"], c["k_pages"], c["v_pages"], ks, vs,
                                                   t, n, c["scale"])
    else:
        dec = lambda t, n: oracle.decode_paged(c["q"], c["k_pages"], c["v_pages"], t, n,
                                               c["scale"])
    po, pl = dec(pre_table, pre_lens)
    so, sl = dec(c["suffix_table"].astype(np.int32), lens)
    return oracle.merge_states(po, pl, so, sl)


@pytest.mark.parametrize("R,H,Hkv,plen,D", [
    (1, 1, 1, 1, 128), (3, 4, 4, 15, 128), (5, 8, 2, 100, 128), (70, 4, 1, 300, 128),
    (40, 8, 2, 1000, 128), (9, 4, 1, 517, 64), (16, 2, 2, 5000, 128),
])
@pytest.mark.parametrize("o_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_fused_cascade(fp8, R, H, Hkv, plen, D, o_dtype):
    """More than 16 query rows per kv head (several 16-row prefix blocks, a
    ragged last one), GQA groups, ragged prefixes, suffixes of 0 .. 700
    tokens, one and many chunks on both sides."""
    require_gpu()
    c = wl.cascade_inputs(R, H, D, "fp8" if fp8 else "bf16", 61 + R + plen, prefix_len=plen,
                          suffix_range=(1, 700), Hkv=Hkv)
    lens = c["suffix_lens"].copy()
    lens[::3] = 0                      # requests with no own tokens: the prefix alone
    kw = dict(k_scale=c["k_scale"], v_scale=c["v_scale"]) if fp8 else {}
    o, lse = fused(c, o_dtype, lens=lens, **kw)
    ro, rl = oracle_cascade(c, lens, fp8)
    assert_close(o, ro, "bf16", "fused cascade O")
    assert_close(lse, rl, "bf16", "fused cascade lse")


def test_fused_cascade_r64_prefix4096_full_size():
    """The cascade workload (64 requests, 4096-token prefix, suffixes
    U[128, 1024]) in the launch configuration the bench times; sampled rows
    against the oracle, and every row against the three-call path."""
    require_gpu()
    c = wl.workload(wl.CASCADE)
    o, lse = fused(c)
    rows = [0, 1, 31, 63]
    ro, rl = oracle.cascade_decode(c["q"][rows], c["k_pages"], c["v_pages"], c["prefix_pages"],
                                   c["prefix_len"], c["suffix_table"][rows],
                                   c["suffix_lens"][rows], c["scale"])
    assert_close(o[rows], ro, "bf16", "fused cascade O")
    assert_close(lse[rows], rl, "bf16", "fused cascade lse")
    from test_gpu_decode import run_cascade
    o3, l3 = run_cascade(c)
    assert_close(o, o3, "bf16", "fused against three calls O")
    assert np.abs(lse - l3).max() <= 1e-3


def test_fused_cascade_fp8_full_size():
    """The cascade workload over an FP8 cache against the plain decode of
    each request's whole key sequence."""
    require_gpu()
    c = wl.fp8_workload(wl.CASCADE)
    o, lse = fused(c, k_scale=c["k_scale"], v_scale=c["v_scale"])
    rows = [0, 1, 31, 63]
    table = np.stack([np.concatenate([c["prefix_pages"], c["suffix_table"][r]]) for r in rows])
    lens = (c["prefix_len"] + c["suffix_lens"][rows]).astype(np.int32)
    assert c["prefix_len"] == len(c["prefix_pages"]) * 16
    ro, rl = oracle.decode_paged_fp8(c["q"][rows], c["k_pages"], c["v_pages"], c["k_scale"],
                                     c["v_scale"], table.astype(np.int32), lens, c["scale"])
    assert_close(o[rows], ro, "bf16", "fused FP8 cascade O")
    assert_close(lse[rows], rl, "bf16", "fused FP8 cascade lse")


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("R,H,Hkv,plen", [(16, 4, 4, 4096), (70, 4, 1, 4096), (8, 2, 2, 20000),
                                          (64, 32, 32, 4096), (5, 2, 1, 37)])
def test_fused_cascade_token_set_and_lse_exact(fp8, R, H, Hkv, plen):
    """Identical keys and V[t][c] = bit c of t over the prefix and each
    request's own tokens: the output is the mean of exactly the tokens
    0 .. P + L - 1 (fp32 output, exact) and lse = s + ln(P + L)."""
    require_gpu()
    D, G = 128, H // Hkv
    gen = wl.generator(700 + R + plen)
    suffix = gen.integers(1, 1025, size=R).astype(np.int32)
    suffix[0] = 1
    suffix[-1] = 0                     # the prefix alone
    c = wl.cascade_inputs(R, H, D, "fp8" if fp8 else "bf16", 701 + R + plen, prefix_len=plen,
                          suffix_lens=np.maximum(suffix, 1), Hkv=Hkv)
    qv = eighths(gen, (R, H, D))
    c["q"] = q_bits(qv)
    fill_cache(c["k_pages"], c["v_pages"], c["prefix_pages"][None, :], [plen], D, fp8)
    fill_cache(c["k_pages"], c["v_pages"], c["suffix_table"], suffix, D, fp8,
               t_offsets=[plen] * R)
    vs = 2.0 if fp8 else 1.0
    o, lse = fused(c, "f32", k_scale=0.25 if fp8 else 1.0, v_scale=vs, lens=suffix)
    check_rows(o, lse, qv, plen + suffix, c["scale"], KEY, vs, G, D, what="fused")


def test_fused_cascade_repeats_bit_exact():
    """The same input four times with other GPU work in between: identical
    bits (every sum runs in a fixed order)."""
    require_gpu()
    c = wl.workload(wl.CASCADE)
    first = fused(c)
    junk = torch.randn(1 << 24, device="cuda")
    for _ in range(3):
        (junk * 2).sum()
        o, lse = fused(c)
        assert np.array_equal(o, first[0]) and np.array_equal(lse, first[1])


def test_fused_cascade_graph_replay():
    """Captured in a HIP graph (no allocation, synchronisation or memset in the
    call) and replayed three times with eager work between: every replay
    matches the eager result bit for bit."""
    require_gpu()
    c = wl.workload(wl.CASCADE)
    q = dev(c["q"])
    kp, vp = dev(c["k_pages"]), dev(c["v_pages"])
    pp, st, sl = dev(c["prefix_pages"]), dev(c["suffix_table"]), dev(c["suffix_lens"])
    R, H, D = q.shape
    maxlen = int(c["suffix_lens"].max())
    need = attn.attn_cascade_workspace_bytes(R, H, c["Hkv"], D, c["prefix_len"], maxlen)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    o, lse = torch.empty_like(q), torch.empty((R, H), device="cuda")

    def call():
        attn.attn_decode_cascade(q, kp, vp, pp, c["prefix_len"], st, sl, o, lse,
                                 max_suffix_len=maxlen, scale=c["scale"], workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    want_o, want_l = o.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(3):
        o.zero_(); lse.zero_()
        (torch.randn(1 << 20, device="cuda") * 2).sum()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, want_o) and torch.equal(lse, want_l)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_fused_cascade_edges(fp8):
    """No prefix (the call is the paged decode of the requests' own tokens);
    no own tokens at all (max_suffix_len 0: the prefix alone); suffix_lens
    NULL (every request has max_suffix_len tokens); 16 query heads per kv
    head (the largest group)."""
    require_gpu()
    dt = "fp8" if fp8 else "bf16"
    # no prefix
    c = wl.cascade_inputs(6, 4, 128, dt, 811, prefix_len=0, suffix_range=(1, 900), Hkv=2)
    kw = dict(k_scale=c["k_scale"], v_scale=c["v_scale"]) if fp8 else {}
    o, lse = fused(c, "f32", **kw)
    if fp8:
        ro, rl = oracle.decode_paged_fp8(c["q"], c["k_pages"], c["v_pages"], c["k_scale"],
                                         c["v_scale"], c["suffix_table"], c["suffix_lens"],
                                         c["scale"])
    else:
        ro, rl = oracle.decode_paged(c["q"], c["k_pages"], c["v_pages"], c["suffix_table"],
                                     c["suffix_lens"], c["scale"])
    assert_close(o, ro, "bf16", "no prefix O")
    assert_close(lse, rl, "bf16", "no prefix lse")
    # no own tokens: max_suffix_len 0
    c = wl.cascade_inputs(5, 4, 128, dt, 812, prefix_len=1000, suffix_range=(1, 2), Hkv=4)
    kw = dict(k_scale=c["k_scale"], v_scale=c["v_scale"]) if fp8 else {}
    zeros = np.zeros(5, np.int32)
    o, lse = fused(c, "f32", lens=zeros, **kw)
    ro, rl = oracle_cascade(c, zeros, fp8)
    assert_close(o, ro, "bf16", "prefix alone O")
    assert_close(lse, rl, "bf16", "prefix alone lse")
    # suffix_lens NULL, G = 16
    L = 300
    c = wl.cascade_inputs(3, 16, 64, dt, 813, prefix_len=700, suffix_lens=np.full(3, L, np.int32),
                          Hkv=1)
    q = dev(c["q"])
    o = torch.full(q.shape, float("nan"), device="cuda")
    lse = torch.full(q.shape[:2], float("nan"), device="cuda")
    kw = dict(k_scale=c["k_scale"], v_scale=c["v_scale"]) if fp8 else {}
    attn.attn_decode_cascade(q, dev(c["k_pages"]), dev(c["v_pages"]), dev(c["prefix_pages"]),
                             c["prefix_len"], dev(c["suffix_table"]), None, o, lse,
                             max_suffix_len=L, scale=c["scale"], **kw)
    torch.cuda.synchronize()
    ro, rl = oracle_cascade(c, c["suffix_lens"], fp8)
    assert_close(host(o), ro, "bf16", "suffix_lens NULL, G = 16 O")
    assert_close(host(lse), rl, "bf16", "suffix_lens NULL, G = 16 lse")
