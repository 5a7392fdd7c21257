"""Run-to-run determinism of the kernels that run the workloads: the same
input launched several times, with other launches in between, must give the
same bits.  Each kernel fixes its order of summation (wavefront order,
chunk order, merge order), so any difference between two runs is a hazard
(a read before its data arrived, a race on shared memory or on the
workspace), which a tolerance test could miss."""
import math

import numpy as np
import pytest
import torch

from attention_tiled_fmha_amd import attn
from attention_tiled_fmha_amd import workloads as wl
from gpu_util import dev, require_gpu

pytestmark = pytest.mark.gpu

REPEATS = 4


def same_bits(runs, what):
    first = runs[0]
    for i, r in enumerate(runs[1:], 1):
        for a, b, name in zip(first, r, ("O", "lse")):
            if a is None:
                continue
            ok = torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                             b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))
            assert ok, f"{what}: run {i} differs from run 0 in {name}"


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("split", [0, 512])
def test_decode_gqa_repeats_bit_exact(fp8, split):
    """GQA decode (Hq32 Hkv8 D128, lengths log-uniform in [1024, 32768]) with
    the planner's chunks and with 512-token chunks (two-chunk items), bf16
    and FP8 caches."""
    require_gpu()
    B, Hq, Hkv, D = 24, 32, 8, 128
    if fp8:
        d = wl.paged_decode_fp8_inputs(B, Hq, Hkv, D, 401, length_range=(1024, 32768), length_dist="log")
    else:
        d = wl.paged_decode_inputs(B, Hq, Hkv, D, "bf16", 401, length_range=(1024, 32768), length_dist="log")
    q, kp, vp = dev(d["q"]), dev(d["k_pages"]), dev(d["v_pages"])
    bt, kl = dev(d["block_table"]), dev(d["kv_lens"])
    maxlen = int(d["kv_lens"].max())
    runs = []
    for i in range(REPEATS):
        o = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full(q.shape[:2], float("nan"), device="cuda")
        if fp8:
            attn.attn_decode_paged_fp8(q, kp, vp, d["k_scale"], d["v_scale"], bt, kl, o, lse,
                                       max_kv_len=maxlen, scale=d["scale"], split_tokens=split)
        else:
            attn.attn_decode_paged(q, kp, vp, bt, kl, o, lse, max_kv_len=maxlen,
                                   scale=d["scale"], split_tokens=split)
        # other work between the runs changes what the caches and the
        # other workgroups hold when the next run starts
        torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        runs.append((o, lse))
    same_bits(runs, f"decode fp8={fp8} split={split}")


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_repeats_bit_exact(causal):
    """bf16 prefill in the B4 H32 T1024 D128 shape."""
    require_gpu()
    inp = wl.workload(wl.PREFILL_CAUSAL)
    q, k, v = (dev(inp[x]) for x in ("q", "k", "v"))
    runs = []
    for i in range(REPEATS):
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], device="cuda")
        attn.attn_prefill(q, k, v, o, lse, causal=causal, scale=1.0 / math.sqrt(128))
        torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        runs.append((o, lse))
    same_bits(runs, f"prefill causal={causal}")


def test_cascade_repeats_bit_exact():
    """Shared-prefix stage (prefix 4096) + suffix decode + merge, 16 requests."""
    require_gpu()
    c = wl.cascade_inputs(16, 32, 128, "bf16", 402)
    q, kp, vp = dev(c["q"]), dev(c["k_pages"]), dev(c["v_pages"])
    pp, st, sl = dev(c["prefix_pages"]), dev(c["suffix_table"]), dev(c["suffix_lens"])
    maxlen = int(c["suffix_lens"].max())
    runs = []
    for i in range(REPEATS):
        o_p, o_s = torch.empty_like(q), torch.empty_like(q)
        l_p, l_s = (torch.empty(q.shape[:2], device="cuda") for _ in range(2))
        attn.attn_decode_shared_prefix(q, kp, vp, pp, c["prefix_len"], o_p, l_p, scale=c["scale"])
        attn.attn_decode_paged(q, kp, vp, st, sl, o_s, l_s, max_kv_len=maxlen, scale=c["scale"])
        attn.attn_merge_states(o_p, l_p, o_s, l_s)
        torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        runs.append((o_p, l_p))
    same_bits(runs, "cascade")
