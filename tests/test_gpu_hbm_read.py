"""moe_hbm_read, the streaming read that measures the HBM read ceiling (MI355X).

The kernel XORs every word it reads and writes the sink only when a lane's
XOR equals one constant, so: a single 16-byte element holding that constant
must reach the sink (the load happened and was not dropped), and a large
buffer whose words cancel in every lane must leave the sink untouched.
"""
import pytest
import torch

import sparse_moe_layer_gemm_amd as moe
from tests.gpu_harness import log

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9


def test_single_element_reaches_sink():
    log("[hbm_read] one 16-byte element")
    buf = torch.tensor([MAGIC - (1 << 32), 0, 0, 0], dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_hbm_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == MAGIC


def test_large_buffer_reads_all_and_leaves_sink():
    log("[hbm_read] 256 MiB of ones")
    buf = torch.ones(64 << 20, dtype=torch.int32, device="cuda")  # each 16 B: 1^1^1^1 = 0
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_hbm_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


def test_ragged_size():
    log("[hbm_read] ragged element count")
    buf = torch.zeros(4 * (2048 * 256 * 8 + 77), dtype=torch.int32, device="cuda")
    buf[-4] = MAGIC - (1 << 32)  # the last element, read by the tail loop
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_hbm_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == MAGIC
