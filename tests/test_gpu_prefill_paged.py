"""GPU parity of prefill against a paged cache (chunked prefill) with the
fp64 oracle, through the C ABI: each sequence's last Tq positions attend its
kv_lens[b] cached keys through the block table, causal with the diagonal at
kv_lens[b] - Tq."""
import numpy as np
import pytest
import torch

import oracle
from attention_tiled_fmha_amd import attn
from attention_tiled_fmha_amd import workloads as wl
from gpu_util import assert_close, dev, host, require_gpu

pytestmark = pytest.mark.gpu


def run(d, causal):
    q = dev(d["q"])
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), device="cuda")
    attn.attn_prefill_paged(q, dev(d["k_pages"]), dev(d["v_pages"]), dev(d["block_table"]),
                            dev(d["kv_lens"]), o, lse, causal=causal, scale=d["scale"])
    torch.cuda.synchronize()
    return host(o), host(lse)


@pytest.mark.parametrize("B,Hq,Hkv,Tq,lengths,D", [
    (2, 4, 4, 37, [37, 100], 128),          # whole sequence as the chunk; ragged
    (3, 8, 2, 128, [128, 419, 700], 128),   # GQA, tile-aligned chunk
    (2, 4, 1, 300, [300, 1000], 64),        # two query tiles, D = 64
    (2, 2, 2, 1, [513, 16], 128),           # one-token chunk
    (3, 4, 2, 64, [20, 64, 0], 128),        # sequences shorter than the chunk, one empty
    (1, 32, 8, 256, [4099], 128),           # long context, ragged last page
])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_paged(B, Hq, Hkv, Tq, lengths, D, causal):
    require_gpu()
    d = wl.paged_prefill_inputs(B, Hq, Hkv, Tq, D, "bf16", 500 + B * Tq + D, lengths=lengths)
    o, lse = run(d, causal)
    ro, rl = oracle.prefill_paged(d["q"], d["k_pages"], d["v_pages"], d["block_table"],
                                  d["kv_lens"], causal, d["scale"])
    assert_close(o, ro, "bf16", "paged prefill O")
    assert_close(lse, rl, "bf16", "paged prefill lse")


def test_prefill_paged_equals_dense_prefill():
    """With every sequence the same length and its pages laid out in order,
    the paged instantiation reads the same values in the same order as the
    dense kernel: identical bits (bottom-right causal, Tq < Tk)."""
    require_gpu()
    B, Hq, Hkv, Tq, L, D = 2, 8, 2, 200, 333, 128
    d = wl.paged_prefill_inputs(B, Hq, Hkv, Tq, D, "bf16", 611, lengths=[L, L], permute=False,
                                tail_garbage=False)
    npg = -(-L // 16)
    # dense K/V [B, Hkv, L, D] from the pages of each sequence
    kd = np.stack([np.concatenate([d["k_pages"][d["block_table"][b, p]] for p in range(npg)],
                                  axis=1)[:, :L] for b in range(B)])
    vd = np.stack([np.concatenate([d["v_pages"][d["block_table"][b, p]] for p in range(npg)],
                                  axis=1)[:, :L] for b in range(B)])
    for causal in (True, False):
        o_p, l_p = run(d, causal)
        q = dev(d["q"])
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], device="cuda")
        attn.attn_prefill(q, dev(kd), dev(vd), o, lse, causal=causal, scale=d["scale"])
        torch.cuda.synchronize()
        assert np.array_equal(host(o), o_p), f"causal={causal}: O differs from dense prefill"
        assert np.array_equal(host(lse), l_p), f"causal={causal}: lse differs from dense prefill"


def test_prefill_paged_chunk512_sampled():
    """The bench shape (B4 Hq32 Hkv8 D128, 512-token chunk, kv_len U[2048,
    8192]) on sampled heads against the oracle."""
    require_gpu()
    d = wl.paged_prefill_inputs(4, 32, 8, 512, 128, "bf16", 1009, length_range=(2048, 8192))
    o, lse = run(d, True)
    # kv head 3 and its four query heads; every sequence
    heads = slice(12, 16)
    ro, rl = oracle.prefill_paged(d["q"][:, heads], d["k_pages"][:, 3:4], d["v_pages"][:, 3:4],
                                  d["block_table"], d["kv_lens"], True, d["scale"])
    assert_close(o[:, heads], ro, "bf16", "chunk O")
    assert_close(lse[:, heads], rl, "bf16", "chunk lse")


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_paged_paired_tiles(causal):
    """B4 Hq32 Hkv8 D128 with a 1000-token chunk: eight 128-row query tiles
    per (b, h), the last holding 104 rows, 1024 in all, so workgroups take
    tiles p and 7 - p; one sequence (600 tokens) is shorter than the chunk,
    so its first 400 rows see no key.  Two kv heads and their query heads,
    every sequence, against the oracle."""
    require_gpu()
    d = wl.paged_prefill_inputs(4, 32, 8, 1000, 128, "bf16", 1213 + int(causal),
                                lengths=[1000, 1700, 3000, 600])
    o, lse = run(d, causal)
    for kvh in (0, 5):
        heads = slice(4 * kvh, 4 * kvh + 4)
        ro, rl = oracle.prefill_paged(d["q"][:, heads], d["k_pages"][:, kvh:kvh + 1],
                                      d["v_pages"][:, kvh:kvh + 1], d["block_table"],
                                      d["kv_lens"], causal, d["scale"])
        assert_close(o[:, heads], ro, "bf16", f"O (kv head {kvh})")
        assert_close(lse[:, heads], rl, "bf16", f"lse (kv head {kvh})")
