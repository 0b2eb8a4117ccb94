"""GPU parity: router ids and gather index bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_ffn_topk_amd as moe
import workloads
from moe_cases import (TOL_BF16, assert_close, assert_close_scaled, check_lists, need_gpu,
                       random_case, read_workspace, say)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,E,k,kind", [
    (16, 8, 2, "normal"), (16, 256, 8, "normal"), (1, 128, 8, "normal"), (37, 64, 64, "normal"),
    (33, 8, 2, "ties"), (16, 256, 8, "ties"), (5, 1024, 8, "normal"), (9, 1, 1, "normal"),
    (64, 200, 3, "ties"), (7, 65, 5, "masked"),
])
def test_route_matches_oracle(T, E, k, kind):
    need_gpu()
    rng = np.random.default_rng(T * 1000 + E + k)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if kind == "ties":
        lg = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    if kind == "masked":
        keep = rng.random((T, E)) < 0.2
        keep[np.arange(T)[:, None], np.arange(k)[None, :]] = True
        lg = np.where(keep, lg, -np.inf).astype(np.float32)
    say(f"route T={T} E={E} k={k} {kind}")
    ids, w = moe.moe_route_topk(torch.from_numpy(lg).cuda(), k)
    torch.cuda.synchronize()
    rid, rw = oracle.route_topk(lg, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_route_workload_recipes(name):
    need_gpu()
    wl = workloads.WORKLOADS[name]
    lg = workloads.gen_logits(wl).numpy()
    say(f"route workload {name}")
    ids, w = moe.moe_route_topk(torch.from_numpy(lg).cuda(), wl.k)
    torch.cuda.synchronize()
    rid, rw = oracle.route_topk(lg, wl.k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-5, atol=1e-7)


def test_route_empty_batch():
    need_gpu()
    ids, w = moe.moe_route_topk(torch.zeros(0, 8, device="cuda"), 2)
    assert ids.shape == (0, 2)


@pytest.mark.parametrize("T,E,k,bad", [(16, 8, 2, 0), (16, 256, 8, 0), (40, 3, 2, 0),
                                       (300, 7, 3, 0), (16, 8, 2, 5), (1, 128, 8, 0),
                                       (24, 1024, 4, 3),
                                       # one expert for every slot, two experts, all
                                       # slots dropped, several chunks of 256 slots
                                       (512, 1, 1, 0), (256, 2, 2, 0), (128, 64, 4, 7),
                                       (171, 64, 3, 2), (4, 8, 2, 8),
                                       # the gate/up product builds the index itself up
                                       # to 256 slots over 256 experts: both limits
                                       # exactly, and one past each
                                       (32, 256, 8, 0), (32, 256, 8, 4), (257, 8, 1, 0),
                                       (8, 257, 4, 1)])
def test_gather_index_matches_oracle(T, E, k, bad):
    need_gpu()
    rng = np.random.default_rng(T + 7 * E + bad)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)   # duplicates allowed
    if bad:
        pos = rng.choice(T * k, size=bad, replace=False)
        ids.reshape(-1)[pos] = rng.choice([-1, E, E + 5, -100], size=bad)
    H, I = 64, 64
    case = random_case(1, T, H, I, E, k, ids=ids)
    x, tid, tw = case.device_inputs()
    ws = moe.alloc_workspace(T, H, I, E, k)
    say(f"gather index T={T} E={E} k={k} bad={bad}")
    moe.moe_ffn_forward(x, tid, tw, case.Wg, case.Wu, case.Wd, workspace=ws)
    code, dropped = moe.moe_ffn_check_status(ws)
    r = read_workspace(ws, moe.moe_ffn_workspace_layout(T, H, I, E, k), T, H, I, E, k)
    p = oracle.permute(ids, E)
    assert np.array_equal(r["counts"], p["counts"])
    assert np.array_equal(r["offsets"], p["offsets"])
    check_lists(r, p, T)
    n = p["offsets"][E]
    assert np.array_equal(r["sorted_slot"][:n], p["sorted_slot"])
    assert dropped == p["n_invalid"] == bad
    assert code == (moe.MOE_FFN_ERR_BAD_IDS if bad else moe.MOE_FFN_OK)


# Router and gather index fused into one kernel (T*k <= 4096 slots), and the
# two-kernel path above that: ids and the gather index bit-exact against the
# oracle's router and permutation, weights within FP32 rounding, and the layer
# output against the oracle layer on those ids.
@pytest.mark.parametrize("T,H,I,E,k,kind", [
    (16, 256, 512, 8, 2, "normal"),      # the Tiny layer's shape
    (16, 64, 96, 256, 8, "normal"),      # DeepSeek-V3 routing shape
    (16, 64, 96, 256, 8, "zipf"),
    (1, 64, 64, 128, 8, "normal"),       # Qwen3-235B at one token
    (33, 64, 64, 8, 2, "ties"),
    (64, 32, 64, 64, 64, "normal"),      # k = 64: every lane of the wave chooses
    (5, 64, 64, 1024, 8, "masked"),
    (9, 32, 32, 1, 1, "normal"),
    (64, 32, 64, 256, 8, "normal"),      # 512 slots, 16384 logits: router and index in one
                                         # kernel at both of its limits (logits staged in LDS)
    (64, 32, 64, 257, 8, "normal"),      # 16448 logits: past the LDS staging of the logits
    (65, 32, 64, 16, 8, "normal"),       # 65 tokens: past the one-kernel router and index
    (512, 32, 64, 64, 8, "normal"),      # 4096 slots: the largest fused batch
    (600, 32, 64, 64, 8, "ties"),        # 4800 slots: router kernel, then the sort
])
def test_forward_logits_matches_oracle(T, H, I, E, k, kind):
    need_gpu()
    rng = np.random.default_rng(1000 * T + 7 * E + k)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if kind == "ties":
        lg = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    if kind == "zipf":
        p = (rng.permutation(E) + 1.0) ** -1.1
        lg = (lg + np.log(p / p.sum())[None, :]).astype(np.float32)
    if kind == "masked":
        keep = rng.random((T, E)) < 0.02
        keep[np.arange(T)[:, None], rng.integers(0, E, size=(T, k))] = True
        keep[:, :k] = True
        lg = np.where(keep, lg, -np.inf).astype(np.float32)
    rid, rw = oracle.route_topk(lg, k)
    case = random_case(T + E, T, H, I, E, k, ids=rid, w=rw)
    x, _, _ = case.device_inputs()
    ws = moe.alloc_workspace(T, H, I, E, k)
    say(f"forward_logits T={T} H={H} I={I} E={E} k={k} {kind}")
    out, ids, w = moe.moe_ffn_forward_logits(x, torch.from_numpy(lg).cuda(), k, case.Wg,
                                             case.Wu, case.Wd, workspace=ws)
    code, dropped = moe.moe_ffn_check_status(ws)
    assert code == moe.MOE_FFN_OK and dropped == 0
    assert np.array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-5, atol=1e-7)
    r = read_workspace(ws, moe.moe_ffn_workspace_layout(T, H, I, E, k), T, H, I, E, k)
    p = oracle.permute(rid, E)
    assert np.array_equal(r["counts"], p["counts"])
    assert np.array_equal(r["offsets"], p["offsets"])
    check_lists(r, p, T)
    assert np.array_equal(r["sorted_slot"][: p["offsets"][E]], p["sorted_slot"])
    # the oracle layer on the oracle's routing weights (the GPU's are equal
    # to them within FP32 rounding)
    ref = case.oracle()
    got = workloads.bf16_bits(out)
    assert_close(got, ref, TOL_BF16)
    assert_close_scaled(got, ref, 1e-2)


@pytest.mark.parametrize("name", ["tiny", "deepseekv3_zipf_t16", "qwen3_235b_t4"])
def test_forward_logits_equals_two_step_layer(name):
    """The logits entry point (router and gather index in one kernel) gives
    bit-identical output to moe_route_topk followed by moe_ffn_forward, whose
    gate/up product builds the gather index itself at these batch sizes."""
    need_gpu()
    wl = workloads.WORKLOADS[name]
    if wl.H > 1024:    # the real expert shapes, shrunk: routing is what differs here
        wl = workloads.Workload(**{**wl.__dict__, "H": 256, "I": 128})
    lg = workloads.gen_logits(wl).cuda()
    x = workloads.gen_x(wl).cuda()
    Wg, Wu, Wd = workloads.gen_weights(wl, "cuda")
    say(f"forward_logits vs two-step {name}")
    out, ids, w = moe.moe_ffn_forward_logits(x, lg, wl.k, Wg, Wu, Wd)
    ids2, w2 = moe.moe_route_topk(lg, wl.k)
    out2 = moe.moe_ffn_forward(x, ids2, w2, Wg, Wu, Wd)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2)
    assert torch.equal(w, w2)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
