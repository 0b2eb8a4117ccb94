"""The debug build: libmoe_ffn_debug.so is the library compiled with the
kernels' device bounds checks (every index of a weight row, a gathered token
row, an h or y row is checked before its access; a failed check is recorded
and the access skipped).  On every product it must compute the same layer as
the release build, bit for bit, and record no failed check."""
import contextlib
import os

import numpy as np
import pytest
import torch

import routed_expert_ffn_topk_amd as moe
import workloads
from moe_cases import need_gpu, random_case, say

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(moe.__file__)
BUILDS = {"release": os.path.join(HERE, "libmoe_ffn.so"),
          "debug": os.path.join(HERE, "libmoe_ffn_debug.so")}


@contextlib.contextmanager
def library(path):
    saved = (moe._lib, moe.LIB_PATH)
    moe._lib, moe.LIB_PATH = None, path
    try:
        yield moe.lib()
    finally:
        moe._lib, moe.LIB_PATH = saved


def both_builds(run):
    """run() under each build; returns the outputs, after checking that the
    debug build reports no failed check (and the release build none either:
    it has none to report)."""
    outs = {}
    for name, path in BUILDS.items():
        with library(path):
            moe.moe_ffn_device_check()                      # clear older records
            outs[name] = run()
            enabled, where = moe.moe_ffn_device_check()
            assert enabled == (name == "debug"), name
            assert where == 0, f"{name}: device check failed at file {where // 100000}, line {where % 100000}"
    return outs


@pytest.mark.parametrize("T,H,I,E,k", [
    (16, 256, 512, 8, 2),      # decode-sized: index in the gate/up prologue
    (1, 128, 128, 1, 1),
    (40, 128, 256, 2, 1),      # 17-32 tokens per expert: the wide chunks
    (100, 256, 256, 4, 2),     # > 64 tokens: the tiled product takes the experts
    (600, 128, 128, 64, 1),    # > 512 slots: the stand-alone index kernel
])
def test_debug_build_bf16_matches_release(T, H, I, E, k):
    need_gpu()
    say(f"debug build bf16 T={T} H={H} I={I} E={E} k={k}")
    case = random_case(T * 7 + E, T, H, I, E, k)
    if T == 16:                       # dropped and repeated expert ids
        case.ids[0, 0] = -1
        case.ids[3, :] = case.ids[3, 0]

    def run():
        x, ids, w = case.device_inputs()
        out = moe.moe_ffn_forward(x, ids, w, case.Wg, case.Wu, case.Wd)
        torch.cuda.synchronize()
        return workloads.bf16_bits(out)
    outs = both_builds(run)
    assert np.array_equal(outs["release"], outs["debug"])


def test_debug_build_quantised_and_attention_match_release():
    need_gpu()
    say("debug build int8 / int4 / attention")
    rng = np.random.default_rng(5)
    T, H, I, E, k = 12, 256, 384, 8, 2
    x = workloads.bits_to_bf16(workloads.bf16_bits(
        torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16))).cuda()
    ids = torch.from_numpy(np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
                           .astype(np.int32)).cuda()
    w = torch.from_numpy(rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)).cuda()
    draw = lambda *s: torch.from_numpy((rng.standard_normal(s) * 0.02).astype(np.float32))  # noqa: E731
    q8 = [workloads.quantize_groupwise(draw(E, I, H)), workloads.quantize_groupwise(draw(E, I, H)),
          workloads.quantize_groupwise(draw(E, H, I))]
    q8 = [t.cuda() for pair in q8 for t in pair]
    q4 = [workloads.quantize_groupwise(draw(E, I, H), 128, 7),
          workloads.quantize_groupwise(draw(E, I, H), 128, 7),
          workloads.quantize_groupwise(draw(E, H, I), 128, 7)]
    q4 = [t.cuda() for Q, S in q4 for t in (workloads.pack_int4(Q), S)]
    qa = torch.from_numpy(rng.standard_normal((3, 8, 64)).astype(np.float32)).to(torch.bfloat16).cuda()
    kv = [torch.from_numpy(rng.standard_normal((3, 2, 300, 64)).astype(np.float32)).to(torch.bfloat16).cuda()
          for _ in range(2)]
    lens = torch.tensor([300, 17, 0], dtype=torch.int32).cuda()

    def run():
        o8 = moe.moe_ffn_forward_int8(x, ids, w, *q8)
        o4 = moe.moe_ffn_forward_int4(x, ids, w, *q4)
        oa = moe.moe_attn_decode(qa, kv[0], kv[1], lens)
        torch.cuda.synchronize()
        return [workloads.bf16_bits(o) for o in (o8, o4, oa)]
    outs = both_builds(run)
    for a, b in zip(outs["release"], outs["debug"]):
        assert np.array_equal(a, b)
