"""GPU parity of the tiled (many-token) expert product against the oracle.

In batches of more than 64 tokens, experts with more than 32 tokens take the
tiled product and the others the small-m product, in the same call.  Shapes
the oracle finishes in seconds that still span several row and token tiles,
ragged token tiles, partial row tiles (N not a multiple of 128), the
shortest K (one pipeline stage), a mix of experts on both sides of the
split, duplicate and dropped ids, and many tokens on one expert.
"""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_ffn_topk_amd as moe
import workloads
from moe_cases import (TOL_BF16, assert_close, assert_close_scaled, check_lists, need_gpu,
                       random_case, read_workspace, say)

pytestmark = pytest.mark.gpu


def skewed_ids(rng, T, E, k, s=1.5):
    """Distinct experts per token, expert e drawn with probability ~ (e+1)^-s."""
    p = (np.arange(E) + 1.0) ** -s
    p /= p.sum()
    return np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


def run_and_check(case, what):
    x, ids, w = case.device_inputs()
    ws = moe.alloc_workspace(case.T, case.H, case.I, case.E, case.k)
    say(what)
    out = moe.moe_ffn_forward(x, ids, w, case.Wg, case.Wu, case.Wd, workspace=ws)
    torch.cuda.synchronize()
    got = workloads.bf16_bits(out)
    r = read_workspace(ws, moe.moe_ffn_workspace_layout(case.T, case.H, case.I, case.E, case.k),
                       case.T, case.H, case.I, case.E, case.k)
    p = oracle.permute(case.ids, case.E)
    assert np.array_equal(r["offsets"], p["offsets"])
    assert np.array_equal(r["sorted_slot"][: p["offsets"][case.E]], p["sorted_slot"])
    check_lists(r, p, case.T)
    ref = case.oracle(aux=True)
    assert_close(got, ref["out"], TOL_BF16, what=what)
    assert_close_scaled(got, ref["out"], 1e-2, what=what)
    # h of every listed slot: nearly all bit-equal, all within 1% of scale
    n = p["offsets"][case.E]
    h = np.zeros_like(ref["h"])
    h[r["sorted_slot"][:n]] = r["h"][:n]
    keep = case.ids.reshape(-1) >= 0
    keep &= case.ids.reshape(-1) < case.E
    assert (h[keep] == ref["h"][keep]).mean() >= 0.99
    assert_close_scaled(h[keep], ref["h"][keep], 1e-2, what="h")
    # y of every slot: the sum of the K-part planes for tiled experts, plane 0
    # for the others
    flat = case.ids.reshape(-1)
    tiled = np.zeros(flat.shape, bool)
    tiled[keep] = r["counts"][flat[keep]] > 32
    y = np.where(tiled[:, None], r["y_planes"].sum(0, dtype=np.float64), r["y_planes"][0])
    assert_close_scaled(y[keep], ref["y"][keep], 1e-2, what="y")
    return r


@pytest.mark.parametrize("T,H,I,E,k", [
    (65, 128, 256, 2, 1),      # smallest tiled batch: two experts of ~32 tokens
    (130, 256, 384, 4, 2),     # ~65 tokens/expert: one full, one partial token tile
    (300, 256, 320, 8, 2),     # I = 320: the last gate/up row tile is half full
    (517, 288, 256, 3, 2),     # ~345 tokens/expert: two token tiles, ragged; K = 288
    (129, 32, 32, 1, 1),       # K = 32 (one stage), N = 32 (a quarter row tile)
    (400, 64, 1024, 2, 2),     # long down K, short gate/up K
    (1000, 96, 160, 2, 1),     # 500 tokens/expert: the register-staged gate/up; N = 160
])
def test_tiled_layer_matches_oracle(T, H, I, E, k):
    need_gpu()
    case = random_case(T * 7 + H + I + E, T, H, I, E, k, std=0.08)
    r = run_and_check(case, f"tiled T={T} H={H} I={I} E={E} k={k}")
    assert r["n_large"] >= 1



def test_tiled_and_small_experts_in_one_call():
    """Skewed routing: some experts above 32 tokens (tiled), some below
    (small-m), some idle."""
    need_gpu()
    rng = np.random.default_rng(11)
    T, H, I, E, k = 200, 128, 160, 16, 4
    ids = skewed_ids(rng, T, E, k)
    case = random_case(12, T, H, I, E, k, std=0.08, ids=ids)
    r = run_and_check(case, "tiled + small-m experts")
    assert r["n_large"] >= 1 and r["n_active"] >= 1


def test_tiled_duplicate_and_dropped_ids():
    need_gpu()
    rng = np.random.default_rng(5)
    T, H, I, E, k = 256, 64, 96, 4, 3
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)          # duplicates
    pos = rng.choice(T * k, size=20, replace=False)
    ids.reshape(-1)[pos] = rng.choice([-1, E, E + 3], size=20)       # dropped
    case = random_case(6, T, H, I, E, k, std=0.08, ids=ids)
    r = run_and_check(case, "tiled dup/drop")
    assert r["n_dropped"] == 20 and r["n_large"] >= 1


def test_tiled_even_token_tiles():
    """Experts of 257, 513 and 530 tokens: their 16-token blocks are split
    evenly over 2, 3 and 3 token tiles (8 + 9, 11 + 11 + 11 and 11 + 11 + 12
    blocks), the last tile ending inside a block; next to a small-m expert
    and an idle one."""
    need_gpu()
    counts = [257, 0, 513, 20, 530]
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    ids = np.random.default_rng(4).permutation(ids).reshape(-1, 1)
    T, H, I, E, k = ids.shape[0], 64, 96, len(counts), 1
    case = random_case(21, T, H, I, E, k, std=0.08, ids=ids)
    r = run_and_check(case, "tiled even token tiles 257/513/530")
    assert r["n_large"] == 3 and r["n_active"] == 1


def test_tiled_one_expert_many_tokens():
    need_gpu()
    T, H, I, E, k = 1000, 64, 128, 4, 1
    ids = np.full((T, 1), 2, dtype=np.int32)
    case = random_case(9, T, H, I, E, k, std=0.08, ids=ids)
    r = run_and_check(case, "tiled one expert, 1000 tokens")
    assert r["n_large"] == 1 and r["n_active"] == 0


def test_tiled_from_logits_matches_two_step():
    """The logits entry point takes the router + sort path for prefill-sized
    batches and reaches the same bits as moe_route_topk + moe_ffn_forward."""
    need_gpu()
    wl = workloads.Workload("prefill", H=256, I=384, E=16, k=2, T=300)
    lg = workloads.gen_logits(wl).cuda()
    x = workloads.gen_x(wl).cuda()
    Wg, Wu, Wd = workloads.gen_weights(wl, "cuda")
    say("tiled from logits vs two-step")
    out, ids, w = moe.moe_ffn_forward_logits(x, lg, wl.k, Wg, Wu, Wd)
    ids2, w2 = moe.moe_route_topk(lg, wl.k)
    out2 = moe.moe_ffn_forward(x, ids2, w2, Wg, Wu, Wd)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(w, w2)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
