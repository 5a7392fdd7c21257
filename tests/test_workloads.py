"""The seeded input generators (CPU only)."""
import numpy as np
import torch

from attention_tiled_fmha_amd import workloads as wl


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * s
                        for s in (1e-30, 1e-3, 1.0, 1e3, 1e30)])
    # ties: values exactly halfway between two bf16 numbers
    ties = (np.arange(1, 5000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.array([0.0, -0.0, np.inf, -np.inf], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wl.bf16_bits(x), ref)
    back = wl.bf16_to_f32(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_generation_is_deterministic_and_chunk_independent():
    a = wl.normal(wl.generator(5), (3, 1 << 21), "bf16")
    b = wl.normal(wl.generator(5), (3, 1 << 21), "bf16")
    assert np.array_equal(a, b)
    f = wl.bf16_to_f32(a)
    assert abs(f.mean()) < 5e-3 and abs(f.std() - 1) < 5e-3


def test_paged_layout():
    d = wl.paged_decode_inputs(5, 4, 2, 8, "bf16", 3, lengths=[1, 16, 17, 40, 100])
    npages = wl.pages_for(d["kv_lens"])
    used = np.concatenate([d["block_table"][b, :n] for b, n in enumerate(npages)])
    # every physical page is used by exactly one logical page
    assert sorted(used.tolist()) == list(range(d["k_pages"].shape[0]))
    assert d["k_pages"].shape == (int(npages.sum()), 2, 16, 8)
    # tail slots carry the sentinels
    pg = d["block_table"][2, 1]
    assert np.all(wl.bf16_to_f32(d["v_pages"][pg, :, 1:]) == wl.TAIL_V)


def test_workload_shapes():
    w1 = wl.workload(wl.PREFILL_F32)
    assert w1["q"].shape == (1, 1, 128, 64) and w1["q"].dtype == np.float32
    c = wl.cascade_inputs(4, 2, 8, "bf16", 9, prefix_len=64, suffix_range=(1, 33))
    assert len(c["prefix_pages"]) == 4
    n = wl.pages_for(c["suffix_lens"])
    suffix_used = np.concatenate([c["suffix_table"][r, :n[r]] for r in range(4)])
    assert set(c["prefix_pages"].tolist()).isdisjoint(suffix_used.tolist())
    assert len(set(suffix_used.tolist())) == len(suffix_used)
