"""The HBM read probe (a measurement helper) runs and leaves its buffer alone."""
import pytest
import torch

import routed_expert_ffn_topk_amd as moe
from moe_cases import need_gpu, say

pytestmark = pytest.mark.gpu


def test_read_probe_runs_and_reads_only():
    need_gpu()
    say("read probe")
    buf = torch.arange(1 << 20, dtype=torch.int32, device="cuda")   # 4 MiB
    ref = buf.clone()
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    moe.moe_ffn_read_probe(buf, sink)
    moe.moe_ffn_read_probe(buf[: (1 << 20) - 4], sink)   # ragged tail: not a multiple of 8 loads
    torch.cuda.synchronize()
    assert torch.equal(buf, ref)
    assert sink[1:].tolist() == [7, 7, 7]     # at most the first word may be written
    assert sink[0].item() in (7, 1)
