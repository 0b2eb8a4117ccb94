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


def test_launch_probe_chain_runs():
    """The launch-gap probe enqueues n empty kernels; the chain completes and
    a launch costs microseconds, not milliseconds."""
    need_gpu()
    say("launch probe")
    stream = torch.cuda.current_stream()
    moe.moe_ffn_launch_probe(10, stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    moe.moe_ffn_launch_probe(200, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 200
    assert 0.0 < us < 100.0, us
    moe.moe_ffn_launch_probe(0, stream)
