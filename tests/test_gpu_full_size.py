"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: the whole batch runs on the GPU, and the oracle recomputes a
sample of token rows (every output element of those rows) one by one.  The
gather index is compared in full, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_ffn_topk_amd as moe
import workloads
from moe_cases import (TOL_BF16, TOL_INT8, assert_close, check_lists, need_gpu,
                       read_workspace, say, workload_case)

pytestmark = pytest.mark.gpu

FULL = ["mixtral8x7b_m1", "mixtral8x7b_m2", "mixtral8x7b_m4", "mixtral8x7b_m8",
        "mixtral8x7b_m16", "mixtral8x7b_t64", "deepseekv3_t16", "deepseekv3_zipf_t16",
        "mixtral8x22b_t1", "mixtral8x22b_t4", "mixtral8x22b_t16", "qwen3_235b_t1",
        "qwen3_235b_t4", "qwen3_235b_t16",
        # prefill-sized batches: the tiled product takes the experts
        "mixtral8x7b_t512", "mixtral8x7b_t2048", "qwen3_235b_t2048", "deepseekv3_t4096"]


def sample_rows(T, n=3, seed=0):
    rng = np.random.default_rng(seed)
    rows = {0, T - 1} | set(rng.choice(T, size=min(n, T), replace=False).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", FULL)
def test_full_size_bf16_sampled_rows(name):
    need_gpu()
    say(f"full-size bf16 {name}")
    wl, case = workload_case(name)
    x, ids, w = case.device_inputs()
    ws = moe.alloc_workspace(wl.T, wl.H, wl.I, wl.E, wl.k)
    out = moe.moe_ffn_forward(x, ids, w, case.Wg, case.Wu, case.Wd, workspace=ws)
    torch.cuda.synchronize()
    got = workloads.bf16_bits(out)
    assert np.isfinite(oracle.bf16_bits_to_f32(got)).all()
    r = read_workspace(ws, moe.moe_ffn_workspace_layout(wl.T, wl.H, wl.I, wl.E, wl.k),
                       wl.T, wl.H, wl.I, wl.E, wl.k)
    p = oracle.permute(case.ids, wl.E)
    assert np.array_equal(r["offsets"], p["offsets"])
    assert np.array_equal(r["sorted_slot"], p["sorted_slot"])
    check_lists(r, p, wl.T)
    rows = sample_rows(wl.T)
    ref = case.oracle(rows=rows)
    assert_close(got[rows], ref, TOL_BF16, what=f"{name} rows {rows.tolist()}")
    del case, out, ws
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m", [1, 2, 4, 8, 16])
def test_full_size_int8_sampled_rows(m):
    need_gpu()
    name = f"mixtral8x7b_int8_m{m}"
    say(f"full-size int8 {name}")
    wl = workloads.WORKLOADS[name]
    xb = workloads.bf16_bits(workloads.gen_x(wl))
    ids, w = oracle.route_topk(workloads.gen_logits(wl).numpy(), wl.k)
    Q = workloads.gen_weights_int8(wl, "cuda")
    ws = moe.alloc_workspace(wl.T, wl.H, wl.I, wl.E, wl.k)
    Qg, Sg, Qu, Su, Qd, Sd = Q
    out = moe.moe_ffn_forward_int8(workloads.bits_to_bf16(xb).cuda(), torch.from_numpy(ids).cuda(),
                                   torch.from_numpy(w).cuda(), Qg, Sg, Qu, Su, Qd, Sd,
                                   workspace=ws)
    torch.cuda.synchronize()
    got = workloads.bf16_bits(out)
    rows = sample_rows(wl.T)
    need = sorted(set(ids[rows].reshape(-1).tolist()))
    host = [{e: t[e].cpu().numpy() for e in need} for t in Q]
    ref = oracle.moe_ffn_int8(xb[rows], ids[rows], w[rows], *(h.get for h in host), E=wl.E)
    assert_close(got[rows], ref, TOL_INT8, what=f"{name} rows {rows.tolist()}")
    del Q, out, ws
    torch.cuda.empty_cache()
