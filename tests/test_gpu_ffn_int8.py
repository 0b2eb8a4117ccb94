"""GPU parity of the INT8 group-quantised FFN layer against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_ffn_topk_amd as moe
import workloads
from moe_cases import TOL_INT8, assert_close, assert_close_scaled, need_gpu, say

pytestmark = pytest.mark.gpu


def int8_case(seed, T, H, I, E, k, std=0.05, ids=None):
    rng = np.random.default_rng(seed)
    x = workloads.bf16_bits(torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32))
                            .to(torch.bfloat16))
    draw = lambda N, K: torch.from_numpy((rng.standard_normal((E, N, K)) * std)  # noqa: E731
                                         .astype(np.float32))
    Qg, Sg = workloads.quantize_groupwise(draw(I, H))
    Qu, Su = workloads.quantize_groupwise(draw(I, H))
    Qd, Sd = workloads.quantize_groupwise(draw(H, I))
    if ids is None:
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    return x, ids, w, (Qg, Sg, Qu, Su, Qd, Sd)


def run_both(x, ids, w, Q, E):
    T, H = x.shape
    Qg, Sg, Qu, Su, Qd, Sd = Q
    I = Qg.shape[1]
    k = ids.shape[1]
    dev = [t.cuda() for t in (Qg, Sg, Qu, Su, Qd, Sd)]
    ws = moe.alloc_workspace(T, H, I, E, k)
    out = moe.moe_ffn_forward_int8(workloads.bits_to_bf16(x).cuda(), torch.from_numpy(ids).cuda(),
                                   torch.from_numpy(w).cuda(), *dev, workspace=ws)
    torch.cuda.synchronize()
    got = workloads.bf16_bits(out)
    ref = oracle.moe_ffn_int8(x, ids, w, Qg.numpy(), Sg.numpy(), Qu.numpy(), Su.numpy(),
                              Qd.numpy(), Sd.numpy(), E=E)
    return got, ref


@pytest.mark.parametrize("T,H,I,E,k", [
    (16, 256, 512, 8, 2), (5, 384, 640, 4, 2), (1, 128, 128, 1, 1), (13, 512, 256, 16, 4),
    (40, 128, 256, 2, 1), (16, 1024, 384, 64, 8), (24, 128, 256, 1024, 4),
    (150, 128, 256, 2, 1),     # ~75 tokens per expert: several 16-token chunks each
])
def test_int8_layer_matches_oracle(T, H, I, E, k):
    need_gpu()
    x, ids, w, Q = int8_case(T + H + I + E, T, H, I, E, k)
    say(f"int8 T={T} H={H} I={I} E={E} k={k}")
    got, ref = run_both(x, ids, w, Q, E)
    assert_close(got, ref, TOL_INT8)
    assert_close_scaled(got, ref, 2e-2)


def test_int8_dropped_ids():
    need_gpu()
    T, E, k = 8, 4, 2
    ids = np.random.default_rng(3).integers(0, E, size=(T, k)).astype(np.int32)
    ids[0, 1] = -5
    x, ids, w, Q = int8_case(4, T, 256, 256, E, k, ids=ids)
    say("int8 dropped ids")
    got, ref = run_both(x, ids, w, Q, E)
    assert_close(got, ref, TOL_INT8)
