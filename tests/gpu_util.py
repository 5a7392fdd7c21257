"""Helpers of the GPU parity tests: host<->device transfer of the seeded
inputs and the element-by-element comparison against the oracle.

Tolerances (the contract for this path): bf16 I/O with fp32 accumulation,
max-abs <= 2e-2 and mean-abs <= 2e-3 on O; fp32 test mode, max-abs <= 1e-5.
The same bounds are applied to lse.
"""
import sys

import numpy as np
import pytest
import torch

BF16_MAX, BF16_MEAN = 2e-2, 2e-3
F32_MAX = 1e-5


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this process")


def dev(a):
    """numpy (uint16 bf16 bits / float32 / int32) -> device tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    """device tensor -> float64 numpy."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def empty_like_out(shape, dtype):
    return torch.full(shape, float("nan"), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                      device="cuda")


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    both_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(got - ref))
    finite = np.isfinite(err)
    if not finite.all():
        return np.inf, np.inf, int(np.argmax(~finite.ravel()))
    return float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0, int(np.argmax(err))


def assert_close(got, ref, dtype, what):
    mx, mean, where = errors(got, ref)
    print(f"  {what}: max {mx:.3e} mean {mean:.3e}", file=sys.stderr)
    if dtype == "bf16":
        assert mx <= BF16_MAX and mean <= BF16_MEAN, \
            f"{what}: max-abs {mx:.3e} / mean-abs {mean:.3e} (at flat index {where})"
    else:
        assert mx <= F32_MAX, f"{what}: max-abs {mx:.3e} (at flat index {where})"
