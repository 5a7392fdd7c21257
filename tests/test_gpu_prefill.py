"""GPU parity of attn_prefill against the fp64 oracle, through the C ABI."""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_tiled_fmha_amd import attn
from attention_tiled_fmha_amd import workloads as wl
from gpu_util import assert_close, dev, empty_like_out, host, require_gpu

pytestmark = pytest.mark.gpu


def run_prefill(inp, causal, with_lse=True):
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    o = empty_like_out(q.shape, inp["dtype"])
    lse = torch.full(q.shape[:3], float("nan"), device="cuda") if with_lse else None
    attn.attn_prefill(q, k, v, o, lse, causal=causal, scale=inp["scale"])
    torch.cuda.synchronize()
    return host(o), (host(lse) if with_lse else None)


def check(inp, causal, bh_sample=None):
    o, lse = run_prefill(inp, causal)
    q, k, v = inp["q"], inp["k"], inp["v"]
    if bh_sample is not None:
        G = inp["Hq"] // inp["Hkv"]
        for b, h in bh_sample:
            ro, rl = oracle.attention(q[b:b + 1, h:h + 1], k[b:b + 1, h // G:h // G + 1],
                                      v[b:b + 1, h // G:h // G + 1], causal, inp["scale"])
            assert_close(o[b, h], ro[0, 0], inp["dtype"], f"O (b={b},h={h})")
            assert_close(lse[b, h], rl[0, 0], inp["dtype"], f"lse (b={b},h={h})")
    else:
        ro, rl = oracle.attention(q, k, v, causal, inp["scale"])
        assert_close(o, ro, inp["dtype"], "O")
        assert_close(lse, rl, inp["dtype"], "lse")


def test_prefill_f32_b1h1t128d64_noncausal():
    """B1 H1 T128 D64 fp32, non-causal: max-abs <= 1e-5."""
    require_gpu()
    check(wl.workload(wl.PREFILL_F32), causal=False)


@pytest.mark.parametrize("shape", [
    (1, 1, 1, 1, 1, 64), (1, 2, 2, 37, 37, 64), (2, 4, 2, 129, 129, 128),
    (1, 2, 1, 200, 77, 128), (1, 1, 1, 50, 300, 64), (2, 8, 8, 256, 256, 128),
])
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_mode_shapes(shape, causal):
    """fp32 test mode on ragged shapes (tiles plus a tail), GQA, Tq != Tk."""
    require_gpu()
    B, Hq, Hkv, Tq, Tk, D = shape
    check(wl.prefill_inputs(B, Hq, Hkv, Tq, Tk, D, "f32", 7 + Tq), causal)


@pytest.mark.parametrize("shape", [
    (1, 1, 1, 1, 1, 128), (1, 2, 2, 33, 33, 64), (2, 4, 4, 300, 300, 128),
    (1, 4, 2, 257, 257, 128), (1, 2, 1, 100, 400, 128), (1, 2, 2, 512, 512, 64),
    (2, 2, 2, 640, 640, 128),
    # groups of 8 query heads with batch x kv heads not a multiple of the 8
    # XCDs (the workgroup-to-head map), Tq > Tk, and 8 query tiles of 256
    (3, 16, 2, 200, 200, 128), (2, 6, 3, 96, 160, 64), (1, 2, 2, 300, 100, 128),
    (1, 2, 1, 2048, 2048, 128),
])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_shapes(shape, causal):
    """bf16 MFMA kernel on ragged shapes spanning several tiles, grouped heads
    and Tq != Tk (bottom-right causal alignment)."""
    require_gpu()
    B, Hq, Hkv, Tq, Tk, D = shape
    check(wl.prefill_inputs(B, Hq, Hkv, Tq, Tk, D, "bf16", 11 + Tq), causal)


def test_prefill_causal_b4h32t1024d128_full_size_sampled():
    """Causal B4 H32 T1024 D128 bf16 at full size, as launched by the bench;
    the oracle checks a sample of (b, h) pairs element by element."""
    require_gpu()
    inp = wl.workload(wl.PREFILL_CAUSAL)
    check(inp, causal=True, bh_sample=[(0, 0), (1, 17), (2, 31), (3, 8)])


def test_prefill_identical_keys_closed_form():
    """All keys equal: every row is the running mean of V (causal), lse = s + ln n."""
    require_gpu()
    T, D = 300, 128
    inp = wl.prefill_inputs(1, 2, 2, T, T, D, "bf16", 3)
    inp["k"][:] = inp["k"][:, :, :1, :]
    o, lse = run_prefill(inp, causal=True)
    vf = wl.bf16_to_f32(inp["v"]).astype(np.float64)
    qf = wl.bf16_to_f32(inp["q"]).astype(np.float64)
    kf = wl.bf16_to_f32(inp["k"]).astype(np.float64)
    n = np.arange(1, T + 1)[None, :, None]
    mean = np.cumsum(vf[0], axis=1) / n
    s = inp["scale"] * np.einsum("htd,hd->ht", qf[0], kf[0, :, 0])
    assert_close(o[0], mean, "bf16", "running mean")
    assert_close(lse[0], s + np.log(np.arange(1, T + 1))[None], "bf16", "lse")


def test_prefill_gqa_mapping_exact():
    """V of kv head g is the constant g + 1: O of query head h is h // G + 1."""
    require_gpu()
    inp = wl.prefill_inputs(1, 8, 2, 70, 70, 128, "bf16", 4)
    for g in range(2):
        inp["v"][:, g] = wl.bf16_bits(np.float32(g + 1))
    o, _ = run_prefill(inp, causal=True)
    for h in range(8):
        assert np.all(o[0, h] == h // 4 + 1), f"head {h}"


def test_prefill_dominant_score():
    """One key dominates by ~Delta = 30: O equals that key's V row."""
    require_gpu()
    T, D = 96, 128
    inp = wl.prefill_inputs(1, 1, 1, T, T, D, "f32", 5)
    inp["q"][:] = 0
    inp["k"][:] = 0
    inp["q"][0, 0, :, 0] = math.sqrt(30 * math.sqrt(D))
    inp["k"][0, 0, 40, 0] = math.sqrt(30 * math.sqrt(D))
    o, _ = run_prefill(inp, causal=False)
    w = math.exp(30.0)
    expect = (w * inp["v"][0, 0, 40].astype(np.float64) + inp["v"][0, 0].sum(0) -
              inp["v"][0, 0, 40]) / (w + T - 1)
    assert_close(o[0, 0], np.broadcast_to(expect, (T, D)), "f32", "dominant")


def test_prefill_lse_none_and_empty_keys():
    """lse may be omitted; with no keys at all O is 0 and lse is -inf."""
    require_gpu()
    for dt in ("bf16", "f32"):
        inp = wl.prefill_inputs(1, 2, 2, 40, 40, 64, dt, 6)
        o, _ = run_prefill(inp, causal=True, with_lse=False)
        ro, _ = oracle.attention(inp["q"], inp["k"], inp["v"], True, inp["scale"])
        assert_close(o, ro, dt, "O without lse")
        # seq_kv = 0
        q = dev(inp["q"])
        kv = torch.empty((1, 2, 0, 64), dtype=q.dtype, device="cuda")
        o = empty_like_out(q.shape, dt)
        lse = torch.zeros(q.shape[:3], device="cuda")
        attn.attn_prefill(q, kv, kv, o, lse, causal=False, scale=0.125)
        torch.cuda.synchronize()
        assert torch.all(o.float() == 0) and torch.all(torch.isneginf(lse))


def test_prefill_causal_rows_without_keys():
    """Bottom-right causal with Tq > Tk: the first Tq - Tk rows see no key."""
    require_gpu()
    for dt in ("bf16", "f32"):
        inp = wl.prefill_inputs(1, 2, 2, 90, 50, 128, dt, 8)
        o, lse = run_prefill(inp, causal=True)
        ro, rl = oracle.attention(inp["q"], inp["k"], inp["v"], True, inp["scale"])
        assert np.all(o[:, :, :40] == 0) and np.all(np.isneginf(lse[:, :, :40]))
        assert_close(o, ro, dt, "O")
        assert_close(lse, rl, dt, "lse")


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_long_sequence_sampled_rows(causal):
    """T = 16384 (64 query tiles of 256, 512 key tiles of 32) with grouped
    heads: sampled query rows (the first and last, both sides of tile
    boundaries, random ones) against the oracle.  A causal row i is the
    non-causal attention of query i over keys 0..i, so each sampled row is
    checked on exactly the keys it may see."""
    require_gpu()
    B, Hq, Hkv, T, D = 1, 4, 2, 16384, 128
    inp = wl.prefill_inputs(B, Hq, Hkv, T, T, D, "bf16", 61 + int(causal))
    o, lse = run_prefill(inp, causal)
    rng = np.random.default_rng(62)
    rows = sorted(set([0, 1, 31, 32, 255, 256, 257, 8191, 8192, T - 257, T - 256, T - 1]
                      + rng.integers(0, T, 20).tolist()))
    for h in (0, 3):
        kvh = h // (Hq // Hkv)
        for i in rows:
            n = i + 1 if causal else T
            ro, rl = oracle.attention(inp["q"][:, h:h + 1, i:i + 1], inp["k"][:, kvh:kvh + 1, :n],
                                      inp["v"][:, kvh:kvh + 1, :n], False, inp["scale"])
            assert_close(o[0, h, i], ro[0, 0, 0], "bf16", f"O (h={h}, row {i})")
            assert_close(lse[0, h, i:i + 1], rl[0, 0], "bf16", f"lse (h={h}, row {i})")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_late_dominant_key_bf16(causal, D):
    """The bf16 kernel takes each row's exponent reference from its first key
    tile; a key later in the sequence whose score is far above that reference
    (here key 700, scores 23 to 32 above the others) makes the kernel recompute
    the query tile against the exact row maxima.  Rows that see the key, rows
    that do not (causal rows before 700), and tiles without it must all match
    the oracle."""
    require_gpu()
    B, H, T = 1, 2, 1000
    inp = wl.prefill_inputs(B, H, H, T, T, D, "bf16", 90 + D + int(causal))
    kf = wl.bf16_to_f32(inp["k"])
    qf = wl.bf16_to_f32(inp["q"])
    kf[0, :, 700] = 0.0
    kf[0, :, 700, 0] = 16.0                # key 700 = 16 e_0
    qf[0, :, 300:, 0] = 16.0               # rows 300..: score 256 / sqrt(D) on it,
    #                                        over 30 log2 units above the rest
    inp["k"], inp["q"] = wl.bf16_bits(kf), wl.bf16_bits(qf)
    check(inp, causal)


@pytest.mark.parametrize("Tk", [300, 700])
def test_prefill_paired_tiles_with_empty_rows(Tk):
    """B4 H32 Tq1024 D128 causal bf16 with fewer keys than queries
    (bottom-right diagonal at Tk - Tq): 1024 query tiles of 128 rows, so
    each workgroup takes two, and with Tk = 300 both tiles of some workgroups see no key at
    all while others pair an empty tile with a full one.  Rows before
    Tq - Tk are O = 0 with lse = -inf; sampled (b, h) pairs match the
    oracle."""
    require_gpu()
    B, H, Tq, D = 4, 32, 1024, 128
    inp = wl.prefill_inputs(B, H, H, Tq, Tk, D, "bf16", 71 + Tk)
    o, lse = run_prefill(inp, causal=True)
    assert np.all(o[:, :, :Tq - Tk] == 0) and np.all(np.isneginf(lse[:, :, :Tq - Tk]))
    for b, h in [(0, 0), (1, 5), (2, 17), (3, 30), (3, 31)]:
        ro, rl = oracle.attention(inp["q"][b:b + 1, h:h + 1], inp["k"][b:b + 1, h:h + 1],
                                  inp["v"][b:b + 1, h:h + 1], True, inp["scale"])
        assert_close(o[b, h], ro[0, 0], "bf16", f"O (b={b},h={h})")
        assert_close(lse[b, h], rl[0, 0], "bf16", f"lse (b={b},h={h})")


@pytest.mark.gpu
@pytest.mark.parametrize("Hkv,D", [(32, 128), (8, 128), (32, 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_paired_odd_tile_count_ragged(Hkv, D, causal):
    """B5 Hq32 T840: seven 128-row query tiles per (b, h), the last holding
    72 rows, and 1120 tiles in all, enough for workgroups to take tiles p and
    6 - p; the middle workgroup of each (b, h) takes tile 3 alone.  Sampled
    (b, h) pairs, one per kv group where grouped, match the oracle."""
    require_gpu()
    B, Hq, T = 5, 32, 840
    inp = wl.prefill_inputs(B, Hq, Hkv, T, T, D, "bf16", 930 + Hkv + D + int(causal))
    o, lse = run_prefill(inp, causal=causal)
    G = Hq // Hkv
    for b, h in [(0, 0), (1, 9), (2, 18), (3, 27), (4, 31)]:
        kh = h // G
        ro, rl = oracle.attention(inp["q"][b:b + 1, h:h + 1], inp["k"][b:b + 1, kh:kh + 1],
                                  inp["v"][b:b + 1, kh:kh + 1], causal, inp["scale"])
        assert_close(o[b, h], ro[0, 0], "bf16", f"O (b={b},h={h})")
        assert_close(lse[b, h], rl[0, 0], "bf16", f"lse (b={b},h={h})")
