"""GPU parity of the flat GEMM of the decode phase, C = A W^T, against the
fp64 oracle, through the C ABI (attn_flat_gemm).

Tolerance, from the arithmetic: every product of two bf16 values is exact in
fp32 and the k products of an output are added in fp32, so
|C - C_exact| <= k * 2^-24 * sum_t |a_t| |w_t| (the classic bound for a
floating-point sum of k terms); a bf16 output adds its rounding, at most
2^-9 |C| (we allow 2^-8).  The bound is computed per element from the
oracle's product of |A| and |W|."""
import numpy as np
import pytest
import torch

import oracle
from attention_tiled_fmha_amd import attn
from attention_tiled_fmha_amd import workloads as wl
from gpu_util import dev, host, require_gpu

pytestmark = pytest.mark.gpu


def run(d, c_dtype="bf16", splits=0, cols=None, rows=0, waves=0, kernel=0, c_offset=0):
    a, w = dev(d["a"]), dev(d["w"])
    # c_offset > 0: C starts that many elements into its buffer (a pointer
    # aligned to 4 bytes only, which rules out the vector stores)
    buf = torch.full((d["m"] * d["n"] + c_offset,), float("nan"),
                     dtype=torch.bfloat16 if c_dtype == "bf16" else torch.float32, device="cuda")
    c = buf[c_offset:].view(d["m"], d["n"])
    attn.attn_flat_gemm(a, w, c, splits=splits, rows_per_workgroup=rows, waves_per_workgroup=waves,
                        kernel=kernel)
    torch.cuda.synchronize()
    out = host(c)
    return out if cols is None else out[:, cols]


def check(got, d, c_dtype, cols=None, what=""):
    a, w = d["a"], d["w"] if cols is None else d["w"][cols]
    ref = oracle.flat_gemm(a, w)
    s_abs = oracle.flat_gemm(a & 0x7FFF, w & 0x7FFF)   # |A| |W|^T (sign bits cleared)
    k = d["k"]
    bound = k * 2.0 ** -24 * s_abs + (2.0 ** -8 * np.abs(ref) if c_dtype == "bf16" else 0.0)
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    worst = float((err - bound).max(initial=-1.0))
    assert (err <= bound).all(), f"{what}: error exceeds the bound by {worst:.3e}"


SHAPES = [(1, 1, 8), (1, 15, 40), (5, 100, 264), (16, 16, 32), (17, 33, 96),
          (32, 200, 520), (40, 64, 1024), (64, 1000, 1024), (3, 4096, 4096), (16, 4096, 4096)]


@pytest.mark.parametrize("rows", [0, 16, 32, 64])
@pytest.mark.parametrize("c_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_flat_gemm_shapes(shape, c_dtype, rows):
    """Ragged m (1 .. 64, every token-tile count), n off the 16- and 64-row
    blocks, k off the 32-wide steps (a multiple of 8), up to n = k = 4096;
    the planner's choice and both forced row-block widths."""
    require_gpu()
    m, n, k = shape
    d = wl.flat_gemm_inputs(m, n, k, 300 + m + n)
    check(run(d, c_dtype, rows=rows), d, c_dtype, what=f"{shape} {c_dtype} rows {rows}")


@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("rows", [16, 32, 64])
@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64])
def test_flat_gemm_forced_splits(splits, rows, waves):
    """k cut into slices across workgroups (fp32 partials in the workspace,
    added in slice order) and over 4, 8 or 16 wavefronts per workgroup
    gives the same result to the bound."""
    require_gpu()
    for m in (9, 40):
        d = wl.flat_gemm_inputs(m, 300, 2048, 77)
        for c_dtype in ("bf16", "f32"):
            check(run(d, c_dtype, splits=splits, rows=rows, waves=waves), d, c_dtype,
                  what=f"m {m} splits {splits} rows {rows} waves {waves} {c_dtype}")


LDS_SHAPES = [(1, 100, 264), (8, 300, 520), (16, 1000, 1032), (17, 33, 96), (32, 200, 520),
              (40, 1000, 1032), (48, 300, 264), (64, 1000, 1024), (64, 4200, 2056), (33, 4096, 64)]


@pytest.mark.parametrize("rows", [64, 128, 256])
@pytest.mark.parametrize("splits", [0, 1, 3, 7])
@pytest.mark.parametrize("shape", LDS_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_flat_gemm_lds_kernel(shape, splits, rows):
    """The LDS-tiled kernel: 64, 128 or 256 rows of W per workgroup, k in
    64-wide chunks (ragged tails of 8 .. 56), k slices with partials, n off
    every tile, 1 .. 4 token tiles (m from 1 to 64); bf16 and fp32 C, and C
    at a 4-byte offset (scalar stores)."""
    require_gpu()
    m, n, k = shape
    d = wl.flat_gemm_inputs(m, n, k, 500 + m + n + k)
    # offsets of 4 bytes: C keeps the 4-byte alignment the interface asks for
    for c_dtype, off in (("bf16", 0), ("f32", 0), ("bf16", 2), ("f32", 1)):
        check(run(d, c_dtype, splits=splits, rows=rows, kernel=attn.FG_LDS, c_offset=off), d,
              c_dtype, what=f"{shape} splits {splits} rows {rows} {c_dtype} offset {off}")


@pytest.mark.parametrize("m", [17, 40, 64])
def test_flat_gemm_register_kernel_forced(m):
    """The register-streaming kernel stays available for m > 16."""
    require_gpu()
    d = wl.flat_gemm_inputs(m, 1000, 1024, 600 + m)
    for c_dtype in ("bf16", "f32"):
        check(run(d, c_dtype, kernel=attn.FG_REGISTER), d, c_dtype, what=f"m {m} {c_dtype}")


def test_flat_gemm_planner_splits_small_n():
    """A short, deep weight (n = 256, k = 8192) leaves CUs idle with whole-k
    row blocks, so the planner slices k; the result still matches."""
    require_gpu()
    assert attn.attn_flat_gemm_plan(16, 256, 8192)[0] > 1
    assert attn.attn_flat_gemm_workspace_bytes(16, 256, 8192) > 0
    d = wl.flat_gemm_inputs(16, 256, 8192, 78)
    check(run(d, "f32"), d, "f32", what="planner splits")


def test_flat_gemm_one_hot_selects_columns():
    """A one-hot row of A picks one column of W: C[i][j] = W[j][t_i] exactly
    (all other products are exact zeros), which fixes the operand order and
    every index, including tokens past 16 and rows past 4096."""
    require_gpu()
    m, n, k = 40, 4200, 264
    d = wl.flat_gemm_inputs(m, n, k, 79)
    picks = np.random.default_rng(5).integers(0, k, size=m)
    a = np.zeros((m, k), np.uint16)
    a[np.arange(m), picks] = wl.bf16_bits(np.float32(1.0)).item()
    d["a"] = a
    want = wl.bf16_to_f32(d["w"][:, picks].T).astype(np.float64)
    for rows in (16, 64):
        assert np.array_equal(run(d, "f32", rows=rows), want), f"rows {rows}"
    for rows in (128, 256):
        for splits in (0, 3):
            got = run(d, "f32", rows=rows, splits=splits, kernel=attn.FG_LDS)
            assert np.array_equal(got, want), f"LDS rows {rows} splits {splits}"


def test_flat_gemm_lds_zero_k():
    """k = 0 on the LDS-tiled kernel (planner's and forced, with slices):
    C = 0 exactly."""
    require_gpu()
    for kw in (dict(), dict(kernel=attn.FG_LDS), dict(kernel=attn.FG_LDS, splits=3, rows_per_workgroup=256)):
        c = torch.full((40, 300), float("nan"), device="cuda")
        a = torch.empty((40, 0), dtype=torch.bfloat16, device="cuda")
        w = torch.empty((300, 0), dtype=torch.bfloat16, device="cuda")
        attn.attn_flat_gemm(a, w, c, **kw)
        torch.cuda.synchronize()
        assert (c == 0).all(), kw


def test_flat_gemm_zero_k_and_empty():
    require_gpu()
    c = torch.full((3, 5), float("nan"), device="cuda")
    a = torch.empty((3, 0), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((5, 0), dtype=torch.bfloat16, device="cuda")
    attn.attn_flat_gemm(a, w, c)
    torch.cuda.synchronize()
    assert (c == 0).all()
    c0 = torch.empty((0, 5), device="cuda")
    attn.attn_flat_gemm(torch.empty((0, 8), dtype=torch.bfloat16, device="cuda"),
                        torch.zeros((5, 8), dtype=torch.bfloat16, device="cuda"), c0)


@pytest.mark.parametrize("name", list(wl.LLAMA2_7B_PROJECTIONS))
@pytest.mark.parametrize("m", [1, 16, 64])
def test_flat_gemm_llama2_7b_shapes_sampled(name, m):
    """Full decode projection shapes of one Llama2-7B layer, in the launch
    configuration the bench times; 97 sampled output columns (the first,
    the last and random ones) are checked against the oracle."""
    require_gpu()
    n, k = wl.LLAMA2_7B_PROJECTIONS[name]
    d = wl.flat_gemm_inputs(m, n, k, 400 + m)
    cols = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(m).integers(0, n, 95)]))
    for c_dtype in ("bf16", "f32"):
        check(run(d, c_dtype, cols=cols), d, c_dtype, cols=cols, what=f"{name} m{m} {c_dtype}")
