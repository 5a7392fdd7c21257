"""The HBM read-rate probe (a measurement aid, not part of the attention
path) through the C ABI: it reads the blocks its order names, every one of
them, and clamps order entries into range.  Its XOR sink is written only
when one lane's words XOR to a fixed value, so a block holding that value in
lane 0's first word (every other byte zero) shows that the block was read."""
import numpy as np
import pytest
import torch

from attention_tiled_fmha_amd import attn
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9
BLK = 4096


def read(n_blocks, marked, order):
    buf = torch.zeros(n_blocks * BLK // 4, dtype=torch.int32, device="cuda")
    if marked is not None:
        buf[marked * BLK // 4] = np.int32(np.uint32(MAGIC).view(np.int32))
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = None if order is None else torch.tensor(order, dtype=torch.int32, device="cuda")
    attn.attn_probe_hbm_read(buf.view(torch.uint8), o, sink)
    torch.cuda.synchronize()
    return int(np.int32(sink.item()).view(np.uint32))


@pytest.mark.parametrize("n_blocks", [1, 7, 4096 + 3])
def test_every_block_is_read(n_blocks):
    require_gpu()
    rng = np.random.default_rng(n_blocks)
    for marked in sorted({0, n_blocks // 2, n_blocks - 1}):
        assert read(n_blocks, marked, None) == MAGIC
        perm = rng.permutation(n_blocks).tolist()
        assert read(n_blocks, marked, perm) == MAGIC
    assert read(n_blocks, None, None) == 0        # nothing matches: the sink is left alone


def test_order_selects_the_blocks():
    require_gpu()
    n = 16
    # a walk that visits block 3 only (every entry 3) misses a mark in block 5
    assert read(n, 5, [3] * n) == 0
    assert read(n, 3, [3] * n) == MAGIC
    # entries outside [0, n) are clamped to 0 and n - 1
    assert read(n, 0, [-7] * n) == MAGIC
    assert read(n, n - 1, [n + 100] * n) == MAGIC
