"""GPU parity of the residual-split layer (moe_ffn_forward_resplit) against
the oracle (oracle.moe_ffn_resplit).

Critical experts run gate/up as W^Q + W^R (two INT4 sets) and down from the
INT8 copy, the others W^Q and the INT4 down copy; the flags are mixed in
every case.  Tolerance as for the quantised layers (2e-2 x max(1, |ref|),
and 2e-2 x max(|ref|, rms(ref))): both sides compute the same grouped FP32
sums in different orders.  With no critical expert the layer is the INT4
layer, bit for bit when both use the same K split.
"""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_ffn_topk_amd as moe
import workloads
from moe_cases import TOL_INT8, assert_close, assert_close_scaled, need_gpu, say

pytestmark = pytest.mark.gpu


def resplit_case(seed, T, H, I, E, k, std=0.05, ids=None, crit=None):
    rng = np.random.default_rng(seed)
    x = workloads.bf16_bits(torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32))
                            .to(torch.bfloat16))
    draw = lambda N, K: torch.from_numpy((rng.standard_normal((E, N, K)) * std)  # noqa: E731
                                         .astype(np.float32))
    t = {}
    for n in ("g", "u"):
        q, s, r, sr = workloads.quantize_residual_split(draw(I, H), 128, 7)
        t["Q" + n], t["S" + n], t["R" + n], t["SR" + n] = q, s, r, sr
    wd = draw(H, I)
    t["Qd_lo"], t["Sd_lo"] = workloads.quantize_groupwise(wd, 128, 7)
    t["Qd_hi"], t["Sd_hi"] = workloads.quantize_groupwise(wd, 128, 127)
    if ids is None:
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    if crit is None:
        crit = (rng.random(E) < 0.5).astype(np.uint8)
        crit[0], crit[-1] = 1, 0 if E > 1 else 1
    return x, ids, w, t, np.asarray(crit, np.uint8)


def device_args(t, crit):
    p4 = workloads.pack_int4
    return [a.cuda() for a in (p4(t["Qg"]), t["Sg"], p4(t["Rg"]), t["SRg"],
                               p4(t["Qu"]), t["Su"], p4(t["Ru"]), t["SRu"],
                               p4(t["Qd_lo"]), t["Sd_lo"], t["Qd_hi"], t["Sd_hi"],
                               torch.from_numpy(crit))]


def run_gpu(x, ids, w, t, crit):
    T, H = x.shape
    E, I = t["Qg"].shape[0], t["Qg"].shape[1]
    ws = moe.alloc_workspace(T, H, I, E, ids.shape[1])
    out = moe.moe_ffn_forward_resplit(workloads.bits_to_bf16(x).cuda(),
                                      torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(),
                                      *device_args(t, crit), workspace=ws)
    torch.cuda.synchronize()
    return workloads.bf16_bits(out)


def run_oracle(x, ids, w, t, crit):
    n = {k: v.numpy() for k, v in t.items()}
    return oracle.moe_ffn_resplit(x, ids, w, n["Qg"], n["Sg"], n["Rg"], n["SRg"], n["Qu"],
                                  n["Su"], n["Ru"], n["SRu"], n["Qd_lo"], n["Sd_lo"], n["Qd_hi"],
                                  n["Sd_hi"], crit, E=len(crit))


@pytest.mark.parametrize("T,H,I,E,k", [
    (16, 256, 512, 8, 2), (5, 384, 640, 4, 2), (1, 128, 128, 2, 1), (13, 512, 256, 16, 4),
    (40, 128, 256, 2, 1), (16, 1024, 384, 64, 8), (100, 256, 128, 3, 2),
])
def test_resplit_layer_matches_oracle(T, H, I, E, k):
    need_gpu()
    x, ids, w, t, crit = resplit_case(T * 3 + H + I + E, T, H, I, E, k)
    say(f"resplit T={T} H={H} I={I} E={E} k={k} critical={crit.tolist()}")
    got = run_gpu(x, ids, w, t, crit)
    ref = run_oracle(x, ids, w, t, crit)
    assert_close(got, ref, TOL_INT8)
    assert_close_scaled(got, ref, 2e-2)


@pytest.mark.parametrize("flag", [0, 1])
def test_resplit_all_one_precision(flag):
    need_gpu()
    E = 4
    x, ids, w, t, crit = resplit_case(60 + flag, 12, 256, 384, E, 2, crit=[flag] * E)
    say(f"resplit every expert critical={flag}")
    got = run_gpu(x, ids, w, t, crit)
    ref = run_oracle(x, ids, w, t, crit)
    assert_close(got, ref, TOL_INT8)
    assert_close_scaled(got, ref, 2e-2)


def test_resplit_without_critical_experts_is_the_int4_layer():
    """No expert critical: the same INT4 arithmetic as moe_ffn_forward_int4;
    with the K split forced equal on both, the same bits."""
    need_gpu()
    E = 6
    x, ids, w, t, crit = resplit_case(70, 9, 384, 256, E, 2, crit=[0] * E)
    p4 = workloads.pack_int4
    for split in (1, 2, 4):
        moe.moe_ffn_set_split(split, split)
        try:
            say(f"resplit vs int4, split {split}")
            a = run_gpu(x, ids, w, t, crit)
            b = moe.moe_ffn_forward_int4(
                workloads.bits_to_bf16(x).cuda(), torch.from_numpy(ids).cuda(),
                torch.from_numpy(w).cuda(), p4(t["Qg"]).cuda(), t["Sg"].cuda(),
                p4(t["Qu"]).cuda(), t["Su"].cuda(), p4(t["Qd_lo"]).cuda(),
                t["Sd_lo"].cuda())
            torch.cuda.synchronize()
        finally:
            moe.moe_ffn_set_split(0, 0)
        assert np.array_equal(a, workloads.bf16_bits(b)), f"split {split}"


def test_resplit_dropped_ids_duplicates_and_every_split():
    need_gpu()
    T, E, k = 10, 4, 3
    rng = np.random.default_rng(8)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)      # duplicates
    ids[0, 1] = -5
    ids[4, 2] = E
    x, ids, w, t, crit = resplit_case(9, T, 512, 384, E, k, ids=ids, crit=[1, 0, 1, 0])
    ref = run_oracle(x, ids, w, t, crit)
    for gu in (1, 2, 4):
        for dn in (1, 2, 4):
            moe.moe_ffn_set_split(gu, dn)
            try:
                say(f"resplit dropped ids, split {gu}/{dn}")
                got = run_gpu(x, ids, w, t, crit)
            finally:
                moe.moe_ffn_set_split(0, 0)
            assert_close(got, ref, TOL_INT8)
            assert_close_scaled(got, ref, 2e-2)


@pytest.mark.parametrize("m", [1, 16])
def test_resplit_full_size_sampled_rows(m):
    """Mixtral-8x7B expert shape, forced routing (every expert m tokens),
    half the experts critical: the whole layer on the GPU, the oracle on
    three tokens."""
    need_gpu()
    wl = workloads.WORKLOADS[f"mixtral8x7b_int4_m{m}"]
    say(f"full-size resplit m={m}")
    xb = workloads.bf16_bits(workloads.gen_x(wl))
    ids, w = oracle.route_topk(workloads.gen_logits(wl).numpy(), wl.k)
    crit = workloads.gen_critical(wl)
    tens = workloads.gen_weights_resplit(wl, "cuda")
    names = ("Qg", "Sg", "Rg", "SRg", "Qu", "Su", "Ru", "SRu", "Qd_lo", "Sd_lo", "Qd_hi", "Sd_hi")
    t = dict(zip(names, tens))
    ws = moe.alloc_workspace(wl.T, wl.H, wl.I, wl.E, wl.k)
    out = moe.moe_ffn_forward_resplit(workloads.bits_to_bf16(xb).cuda(),
                                      torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(),
                                      *device_args(t, crit), workspace=ws)
    torch.cuda.synchronize()
    got = workloads.bf16_bits(out)
    rows = np.array(sorted({0, wl.T - 1, wl.T // 2}))
    need = sorted(set(ids[rows].reshape(-1).tolist()))
    host = {n: {e: t[n][e].cpu().numpy() for e in need} for n in names}
    ref = oracle.moe_ffn_resplit(xb[rows], ids[rows], w[rows],
                                 *(host[n].get for n in names), crit, E=wl.E)
    assert_close(got[rows], ref, TOL_INT8, what=f"resplit m={m} rows {rows.tolist()}")
    assert crit.any() and not crit.all()
