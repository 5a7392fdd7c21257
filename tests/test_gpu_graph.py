"""Replay of captured decode steps (HIP graphs) against eager launches.

Graph replay as the xhh.club summary ("fast attention kernels and operator
fusion", section on torch.compile and CUDA Graphs) describes it: a recorded
sequence of GPU work resubmitted with one CPU call, for repeated small decode
steps, valid while addresses and shapes stay fixed.

Every call of the library is asynchronous on the caller's stream, allocates
nothing when the caller passes the workspace, never synchronises and issues
no memset; the split plan is made on the host from the host-side bound
max_kv_len.  A decode step can therefore be captured once and replayed while
the device-side inputs (queries, kv_lens within the bound, block tables,
cache contents) change between replays.  Each replay here follows eager work
of the program's own (new inputs written, a device synchronisation) and is
compared with the eager launch of the same calls on the same inputs: the
same kernels in the same plan, so bit-identical."""
import numpy as np
import pytest
import torch

import oracle
from attention_tiled_fmha_amd import attn
from attention_tiled_fmha_amd import workloads as wl
from gpu_util import assert_close, dev, host, require_gpu

pytestmark = pytest.mark.gpu


def capture(step):
    """Capture step() into a graph, after one warm-up run on a side stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def test_graph_replay_split_decode():
    """Paged decode with forced splits (decode kernel + combine kernel) over a
    GQA cache, replayed with new queries and shorter kv_lens each time."""
    require_gpu()
    d = wl.paged_decode_inputs(8, 16, 4, 128, "bf16", 4101, length_range=(100, 3000))
    gen = wl.generator(4102)
    B, Hq, D = d["B"], d["Hq"], d["D"]
    maxlen = int(d["kv_lens"].max())
    q = dev(d["q"])
    kp, vp, bt = dev(d["k_pages"]), dev(d["v_pages"]), dev(d["block_table"])
    kl = dev(d["kv_lens"])
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), device="cuda")
    split = 256
    ws = torch.empty(attn.attn_decode_workspace_bytes(B, Hq, d["Hkv"], D, maxlen, split),
                     dtype=torch.uint8, device="cuda")

    def step(o=o, lse=lse):
        attn.attn_decode_paged(q, kp, vp, bt, kl, o, lse, max_kv_len=maxlen, scale=d["scale"],
                               workspace=ws, split_tokens=split)

    g = capture(step)
    o_ref, lse_ref = torch.empty_like(o), torch.empty_like(lse)
    for rep in range(4):
        # eager work between replays: new queries, new lengths within the bound
        q_new = wl.normal(gen, (B, Hq, D), "bf16")
        lens = (d["kv_lens"] * gen.uniform(0.3, 1.0, size=B)).astype(np.int32)
        lens[rep % B] = 0 if rep == 2 else lens[rep % B]
        q.copy_(dev(q_new))
        kl.copy_(dev(lens))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        step(o_ref, lse_ref)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {rep}: O differs from the eager launch"
        assert torch.equal(lse, lse_ref), f"replay {rep}: lse differs from the eager launch"
    ro, rl = oracle.decode_paged(q_new, d["k_pages"], d["v_pages"], d["block_table"], lens,
                                 d["scale"])
    assert_close(host(o), ro, "bf16", "replayed O")
    assert_close(host(lse), rl, "bf16", "replayed lse")


def test_graph_replay_decode_gqa_full_size():
    """The GQA decode workload (B128 Hq32 Hkv8, L ~ logU[1024, 32768], 512-
    token chunks; more item slots than the persistent grid, so every
    workgroup walks several) captured once and replayed with new queries and
    lengths each time: every replay equals the eager launch."""
    require_gpu()
    d = wl.workload(wl.DECODE_GQA)
    gen = wl.generator(4103)
    B, Hq, D = d["B"], d["Hq"], d["D"]
    maxlen = int(d["kv_lens"].max())
    split = 512
    q = dev(d["q"])
    kp, vp, bt = dev(d["k_pages"]), dev(d["v_pages"]), dev(d["block_table"])
    kl = dev(d["kv_lens"])
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), device="cuda")
    ws = torch.empty(attn.attn_decode_workspace_bytes(B, Hq, d["Hkv"], D, maxlen, split),
                     dtype=torch.uint8, device="cuda")

    def step(o=o, lse=lse):
        attn.attn_decode_paged(q, kp, vp, bt, kl, o, lse, max_kv_len=maxlen, scale=d["scale"],
                               workspace=ws, split_tokens=split)

    g = capture(step)
    o_ref, lse_ref = torch.empty_like(o), torch.empty_like(lse)
    for rep in range(3):
        q_new = wl.normal(gen, (B, Hq, D), "bf16")
        lens = (d["kv_lens"] * gen.uniform(0.3, 1.0, size=B)).astype(np.int32)
        q.copy_(dev(q_new))
        kl.copy_(dev(lens))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        step(o_ref, lse_ref)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {rep}: O differs from the eager launch"
        assert torch.equal(lse, lse_ref), f"replay {rep}: lse differs from the eager launch"
    rows = [0, 57, 127]
    ro, rl = oracle.decode_paged(q_new[rows], d["k_pages"], d["v_pages"], d["block_table"][rows],
                                 lens[rows], d["scale"])
    assert_close(host(o)[rows], ro, "bf16", "replayed O")
    assert_close(host(lse)[rows], rl, "bf16", "replayed lse")


def test_graph_replay_cascade():
    """Prefix stage, suffix decode and merge captured as one graph, replayed
    with new queries and new suffix lengths."""
    require_gpu()
    c = wl.cascade_inputs(16, 8, 128, "bf16", 4103, prefix_len=1008, suffix_range=(50, 400))
    gen = wl.generator(4104)
    q = dev(c["q"])
    R, H, D = q.shape
    kp, vp = dev(c["k_pages"]), dev(c["v_pages"])
    pp, st, sl = dev(c["prefix_pages"]), dev(c["suffix_table"]), dev(c["suffix_lens"])
    maxlen = int(c["suffix_lens"].max())
    ws_p = torch.empty(max(1, attn.attn_shared_prefix_workspace_bytes(R, H, c["Hkv"], D,
                                                                          c["prefix_len"])),
                       dtype=torch.uint8, device="cuda")
    ws_s = torch.empty(max(1, attn.attn_decode_workspace_bytes(R, H, c["Hkv"], D, maxlen)),
                       dtype=torch.uint8, device="cuda")
    bufs = [[torch.empty_like(q), torch.empty((R, H), device="cuda"), torch.empty_like(q),
             torch.empty((R, H), device="cuda")] for _ in range(2)]

    def step(b=bufs[0]):
        o_p, l_p, o_s, l_s = b
        attn.attn_decode_shared_prefix(q, kp, vp, pp, c["prefix_len"], o_p, l_p,
                                       scale=c["scale"], workspace=ws_p)
        attn.attn_decode_paged(q, kp, vp, st, sl, o_s, l_s, max_kv_len=maxlen, scale=c["scale"],
                               workspace=ws_s)
        attn.attn_merge_states(o_p, l_p, o_s, l_s)

    g = capture(step)
    for rep in range(3):
        q_new = wl.normal(gen, (R, H, D), "bf16")
        lens = np.maximum(1, (c["suffix_lens"] * gen.uniform(0.2, 1.0, size=R))).astype(np.int32)
        q.copy_(dev(q_new))
        sl.copy_(dev(lens))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        step(bufs[1])
        torch.cuda.synchronize()
        assert torch.equal(bufs[0][0], bufs[1][0]), f"replay {rep}: O differs from eager"
        assert torch.equal(bufs[0][1], bufs[1][1]), f"replay {rep}: lse differs from eager"
    rows = [0, 7, 15]
    ro, rl = oracle.cascade_decode(q_new[rows], c["k_pages"], c["v_pages"], c["prefix_pages"],
                                   c["prefix_len"], c["suffix_table"][rows], lens[rows],
                                   c["scale"])
    assert_close(host(bufs[0][0])[rows], ro, "bf16", "replayed cascade O")
    assert_close(host(bufs[0][1])[rows], rl, "bf16", "replayed cascade lse")


def test_graph_replay_flat_gemm():
    """The flat GEMM of a decode projection with k sliced across workgroups
    (main kernel + partial-sum reduction, workspace passed in), captured once
    and replayed with new activations each time; every replay equals the
    eager launch bit for bit and the oracle to the GEMM bound."""
    require_gpu()
    m, n, k = 12, 1000, 4096
    d = wl.flat_gemm_inputs(m, n, k, 4201)
    w = dev(d["w"])
    a = dev(d["a"])
    c = torch.empty((m, n), device="cuda")
    splits = 4
    ws = torch.empty(attn.attn_flat_gemm_workspace_bytes(m, n, k, splits), dtype=torch.uint8,
                     device="cuda")
    assert ws.numel() > 0

    def step():
        attn.attn_flat_gemm(a, w, c, splits=splits, workspace=ws)

    g = capture(step)
    gen = wl.generator(4202)
    for rep in range(3):
        a_np = wl.normal(gen, (m, k), "bf16")
        a.copy_(dev(a_np))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = c.clone()
        c.fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        assert torch.equal(got, c), f"replay {rep} differs from the eager launch"
        ref = oracle.flat_gemm(a_np, d["w"])
        bound = k * 2.0 ** -24 * oracle.flat_gemm(a_np & 0x7FFF, d["w"] & 0x7FFF)
        assert (np.abs(host(got) - ref) <= bound).all(), f"replay {rep} outside the bound"
