"""GPU parity: router ids and gather index bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_ffn_topk_amd as moe
import workloads
from moe_cases import need_gpu, random_case, read_workspace, say

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
                                       (171, 64, 3, 2), (4, 8, 2, 8)])
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
    assert r["n_active"] == p["n_active"]
    assert np.array_equal(r["active"], p["active"])
    n = p["offsets"][E]
    assert np.array_equal(r["sorted_slot"][:n], p["sorted_slot"])
    assert dropped == p["n_invalid"] == bad
    assert code == (moe.MOE_FFN_ERR_BAD_IDS if bad else moe.MOE_FFN_OK)
