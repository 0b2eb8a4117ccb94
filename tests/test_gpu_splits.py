"""Every K split of both grouped products, for both weight formats, against
the oracle.  The kernels choose the split on the device; the test hook
moe_ffn_set_split forces each one, on shapes whose K parts are ragged (the
last part shorter, or empty) and with more than 16 tokens per expert."""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_ffn_topk_amd as moe
import workloads
from moe_cases import (TOL_BF16, TOL_INT8, assert_close, assert_close_scaled, need_gpu,
                       random_case, say)

pytestmark = pytest.mark.gpu

SPLITS = [(1, 1), (2, 2), (4, 4), (1, 4), (4, 2)]


@pytest.fixture(autouse=True)
def _restore_device_choice():
    yield
    if torch.cuda.is_available():
        moe.moe_ffn_set_split(0, 0)


@pytest.mark.parametrize("T,H,I,E,k", [
    (13, 320, 288, 6, 3),      # K steps 10 / 9: parts 3,3,3,1 and 3,3,3,0 at S = 4
    (16, 1024, 512, 8, 2),     # several LDS slabs per part
    (40, 128, 96, 2, 1),       # 20 tokens per expert: one wide chunk
    (56, 256, 160, 2, 1),      # 28 tokens per expert: one wide chunk, several slabs
])
def test_bf16_every_split_matches_oracle(T, H, I, E, k):
    need_gpu()
    case = random_case(7 * T + H + I + E, T, H, I, E, k, std=0.08)
    ref = case.oracle()
    x, ids, w = case.device_inputs()
    outs = []
    for gu, dn in SPLITS:
        say(f"bf16 T={T} H={H} I={I} E={E} k={k} split gate/up {gu} down {dn}")
        moe.moe_ffn_set_split(gu, dn)
        out = moe.moe_ffn_forward(x, ids, w, case.Wg, case.Wu, case.Wd)
        torch.cuda.synchronize()
        got = workloads.bf16_bits(out)
        assert_close(got, ref, TOL_BF16, what=f"out, split {gu}/{dn}")
        assert_close_scaled(got, ref, 1e-2, what=f"out, split {gu}/{dn}")
        outs.append(got)
    # the split changes only the FP32 summation order
    for o in outs[1:]:
        assert (o == outs[0]).mean() >= 0.9


def int8_case(seed, T, H, I, E, k):
    rng = np.random.default_rng(seed)
    x = workloads.bf16_bits(torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32))
                            .to(torch.bfloat16))
    draw = lambda N, K: torch.from_numpy((rng.standard_normal((E, N, K)) * 0.05)  # noqa: E731
                                         .astype(np.float32))
    Q = []
    for N, K in ((I, H), (I, H), (H, I)):
        Q.extend(workloads.quantize_groupwise(draw(N, K)))
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    return x, ids, w, Q


@pytest.mark.parametrize("T,H,I,E,k", [
    (13, 384, 640, 4, 2),      # 3 / 5 scale groups: parts 1,1,1,0 and 2,2,1,0 at S = 4
    (16, 1024, 384, 64, 8),    # many experts, one or two tokens each
    (40, 256, 128, 2, 1),      # 20 tokens per expert: two token chunks
])
def test_int8_every_split_matches_oracle(T, H, I, E, k):
    need_gpu()
    x, ids, w, Q = int8_case(11 * T + H + I + E, T, H, I, E, k)
    Qg, Sg, Qu, Su, Qd, Sd = Q
    ref = oracle.moe_ffn_int8(x, ids, w, Qg.numpy(), Sg.numpy(), Qu.numpy(), Su.numpy(),
                              Qd.numpy(), Sd.numpy(), E=E)
    dev = [t.cuda() for t in (Qg, Sg, Qu, Su, Qd, Sd)]
    xd = workloads.bits_to_bf16(x).cuda()
    idd, wd = torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
    for gu, dn in SPLITS:
        say(f"int8 T={T} H={H} I={I} E={E} k={k} split gate/up {gu} down {dn}")
        moe.moe_ffn_set_split(gu, dn)
        out = moe.moe_ffn_forward_int8(xd, idd, wd, *dev)
        torch.cuda.synchronize()
        got = workloads.bf16_bits(out)
        assert_close(got, ref, TOL_INT8, what=f"out, split {gu}/{dn}")
        assert_close_scaled(got, ref, 2e-2, what=f"out, split {gu}/{dn}")
