"""attn_decode_paged_noalloc (the decode entry point that allocates nothing:
its split partials live in the library's fixed per-GPU device array)
against attn_decode_paged with a caller workspace, through the C ABI.

Both run the same kernels with the same split plan, so the outputs must be
bit-identical; the oracle checks the result to the bf16 tolerance as well.
Two calls in a row, the second on a smaller input, show that a call does
not depend on what an earlier call left in the shared array."""
import numpy as np
import pytest
import torch

import oracle
from attention_tiled_fmha_amd import attn
from attention_tiled_fmha_amd import workloads as wl
from gpu_util import assert_close, dev, empty_like_out, host, require_gpu

pytestmark = pytest.mark.gpu


def both(d, o_dtype):
    q = dev(d["q"])
    kp, vp, bt, kl = dev(d["k_pages"]), dev(d["v_pages"]), dev(d["block_table"]), dev(d["kv_lens"])
    L = int(d["kv_lens"].max(initial=0))
    B, Hq, D = q.shape
    assert attn.attn_decode_workspace_bytes(B, Hq, d["Hkv"], D, L) > 0, "the case must use splits"
    out = []
    for fn in ("ws", "noalloc"):
        o = empty_like_out(q.shape, o_dtype)
        lse = torch.full(q.shape[:2], float("nan"), device="cuda")
        if fn == "ws":
            attn.attn_decode_paged(q, kp, vp, bt, kl, o, lse, max_kv_len=L, scale=d["scale"])
        else:
            attn.attn_decode_paged_noalloc(q, kp, vp, bt, kl, o, lse, max_kv_len=L,
                                           scale=d["scale"])
        torch.cuda.synchronize()
        out.append((host(o), host(lse)))
    return out


def test_noalloc_matches_workspace_entry_two_calls():
    require_gpu()
    big = wl.paged_decode_inputs(8, 32, 8, 128, "bf16", 81, lengths=[4096, 3000, 17, 1, 2500,
                                                                    4000, 1024, 0])
    small = wl.paged_decode_inputs(3, 8, 8, 64, "bf16", 82, lengths=[900, 33, 1500])
    for d, o_dtype in ((big, "bf16"), (small, "f32")):
        (o_ws, l_ws), (o_na, l_na) = both(d, o_dtype)
        assert np.array_equal(o_ws, o_na, equal_nan=True), "O differs from attn_decode_paged"
        assert np.array_equal(l_ws, l_na, equal_nan=True), "lse differs from attn_decode_paged"
        ro, rl = oracle.decode_paged(d["q"], d["k_pages"], d["v_pages"], d["block_table"],
                                     d["kv_lens"], d["scale"])
        assert_close(o_na, ro, "bf16", "O")
        assert_close(l_na, rl, "bf16", "lse")


def test_noalloc_rejects_plans_beyond_its_array():
    """B128 Hq32 D128 at 32768 tokens plans ~135 MB of partials: refused with
    ATTN_E_SCRATCH before anything is launched."""
    require_gpu()
    B, Hq, Hkv, D, L = 128, 32, 8, 128, 32768
    assert attn.attn_decode_workspace_bytes(B, Hq, Hkv, D, L) > attn.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    pages = torch.zeros((1, Hkv, 16, D), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((B, L // 16), dtype=torch.int32, device="cuda")
    kl = torch.zeros((B,), dtype=torch.int32, device="cuda")
    o = torch.zeros_like(q)
    with pytest.raises(attn.AttnError) as e:
        attn.attn_decode_paged_noalloc(q, pages, pages, bt, kl, o, None, max_kv_len=L)
    assert e.value.status == 7
