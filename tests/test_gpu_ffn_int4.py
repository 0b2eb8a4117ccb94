"""GPU parity of the INT4 group-quantised FFN layer against the oracle.

The INT4 layer computes the INT8 layer's definition (group sums scaled per
128 K) on integer weights in [-7, 7]; only the storage differs (two
offset-binary nibbles per byte), so the oracle is the INT8 one, fed the
unpacked values.  The packed bytes come from workloads.pack_int4.
"""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_ffn_topk_amd as moe
import workloads
from moe_cases import TOL_INT8, assert_close, assert_close_scaled, need_gpu, say

pytestmark = pytest.mark.gpu


def int4_case(seed, T, H, I, E, k, std=0.05, ids=None, qvals=None):
    rng = np.random.default_rng(seed)
    x = workloads.bf16_bits(torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32))
                            .to(torch.bfloat16))
    draw = lambda N, K: torch.from_numpy((rng.standard_normal((E, N, K)) * std)  # noqa: E731
                                         .astype(np.float32))
    Q = []
    for N, K in ((I, H), (I, H), (H, I)):
        q, s = workloads.quantize_groupwise(draw(N, K), 128, 7)
        if qvals is not None:                      # e.g. the extreme codes -8 and 7
            q = torch.from_numpy(rng.choice(qvals, size=q.shape).astype(np.int8))
        Q += [q, s]
    if ids is None:
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    return x, ids, w, tuple(Q)


def run_both(x, ids, w, Q, E):
    T, H = x.shape
    Qg, Sg, Qu, Su, Qd, Sd = Q
    I = Qg.shape[1]
    k = ids.shape[1]
    dev = [t.cuda() for t in (workloads.pack_int4(Qg), Sg, workloads.pack_int4(Qu), Su,
                              workloads.pack_int4(Qd), Sd)]
    ws = moe.alloc_workspace(T, H, I, E, k)
    out = moe.moe_ffn_forward_int4(workloads.bits_to_bf16(x).cuda(), torch.from_numpy(ids).cuda(),
                                   torch.from_numpy(w).cuda(), *dev, workspace=ws)
    torch.cuda.synchronize()
    got = workloads.bf16_bits(out)
    ref = oracle.moe_ffn_int8(x, ids, w, Qg.numpy(), Sg.numpy(), Qu.numpy(), Su.numpy(),
                              Qd.numpy(), Sd.numpy(), E=E)
    return got, ref


@pytest.mark.parametrize("T,H,I,E,k", [
    (16, 256, 512, 8, 2), (5, 384, 640, 4, 2), (1, 128, 128, 1, 1), (13, 512, 256, 16, 4),
    (40, 128, 256, 2, 1), (16, 1024, 384, 64, 8), (100, 256, 128, 3, 2),
])
def test_int4_layer_matches_oracle(T, H, I, E, k):
    need_gpu()
    x, ids, w, Q = int4_case(T + H + I + E, T, H, I, E, k)
    say(f"int4 T={T} H={H} I={I} E={E} k={k}")
    got, ref = run_both(x, ids, w, Q, E)
    assert_close(got, ref, TOL_INT8)
    assert_close_scaled(got, ref, 2e-2)


def test_int4_extreme_codes():
    """Every nibble at the ends of the range (-8 -> 0x0, 7 -> 0xF): the
    offset-binary decode and the bias correction at their limits."""
    need_gpu()
    x, ids, w, Q = int4_case(31, 9, 256, 256, 4, 2, qvals=[-8, 7])
    say("int4 extreme codes")
    got, ref = run_both(x, ids, w, Q, 4)
    assert_close(got, ref, TOL_INT8)
    assert_close_scaled(got, ref, 2e-2)


def test_int4_dropped_ids_and_every_split():
    need_gpu()
    T, E, k = 8, 4, 2
    ids = np.random.default_rng(3).integers(0, E, size=(T, k)).astype(np.int32)
    ids[0, 1] = -5
    x, ids, w, Q = int4_case(4, T, 512, 384, E, k, ids=ids)
    for gu in (1, 2, 4):
        for dn in (1, 2, 4):
            moe.moe_ffn_set_split(gu, dn)
            try:
                say(f"int4 dropped ids, split {gu}/{dn}")
                got, ref = run_both(x, ids, w, Q, E)
            finally:
                moe.moe_ffn_set_split(0, 0)
            assert_close(got, ref, TOL_INT8)
            assert_close_scaled(got, ref, 2e-2)


@pytest.mark.parametrize("m", [1, 16])
def test_int4_full_size_sampled_rows(m):
    need_gpu()
    name = f"mixtral8x7b_int4_m{m}"
    say(f"full-size int4 {name}")
    wl = workloads.WORKLOADS[name]
    xb = workloads.bf16_bits(workloads.gen_x(wl))
    ids, w = oracle.route_topk(workloads.gen_logits(wl).numpy(), wl.k)
    Qg, Sg, Qu, Su, Qd, Sd = workloads.gen_weights_int4(wl, "cuda")
    ws = moe.alloc_workspace(wl.T, wl.H, wl.I, wl.E, wl.k)
    out = moe.moe_ffn_forward_int4(workloads.bits_to_bf16(xb).cuda(), torch.from_numpy(ids).cuda(),
                                   torch.from_numpy(w).cuda(), workloads.pack_int4(Qg), Sg,
                                   workloads.pack_int4(Qu), Su, workloads.pack_int4(Qd),
                                   Sd, workspace=ws)
    torch.cuda.synchronize()
    got = workloads.bf16_bits(out)
    rows = np.array(sorted({0, wl.T - 1, wl.T // 2}))
    need = sorted(set(ids[rows].reshape(-1).tolist()))
    host = [{e: t[e].cpu().numpy() for e in need} for t in (Qg, Sg, Qu, Su, Qd, Sd)]
    ref = oracle.moe_ffn_int8(xb[rows], ids[rows], w[rows], *(h.get for h in host), E=wl.E)
    assert_close(got[rows], ref, TOL_INT8, what=f"{name} rows {rows.tolist()}")
