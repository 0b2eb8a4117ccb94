"""Helpers for the GPU parity tests: build cases, run both sides, compare.

Inputs come from ``workloads.py`` (seeded) or are drawn here with numpy; the
expected values come only from ``oracle``.  The comparison bar for BF16
outputs is |gpu - ref| <= 1e-2 * max(1, |ref|) per element (2e-2 for the
INT8 variant); integer results (routing ids, gather index) must be equal.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

TOL_BF16 = 1e-2
TOL_INT8 = 2e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(msg: str):
    """Name the case on stdout before a GPU step (flushed)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def f32(bits: np.ndarray) -> np.ndarray:
    return oracle.bf16_bits_to_f32(bits)


def assert_close(gpu_bits: np.ndarray, ref_bits: np.ndarray, tol: float, what: str = "out"):
    g = f32(gpu_bits).astype(np.float64)
    r = f32(ref_bits).astype(np.float64)
    assert g.shape == r.shape
    bad = np.abs(g - r) > tol * np.maximum(1.0, np.abs(r))
    assert not np.isnan(g).any(), f"{what}: NaN in GPU result"
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements outside tolerance; "
                             f"first at {tuple(i)}: gpu={g[tuple(i)]} ref={r[tuple(i)]}")


def assert_close_scaled(gpu_bits: np.ndarray, ref_bits: np.ndarray, rel: float,
                        what: str = "out"):
    """A bar that also bites when outputs are far below 1 in magnitude:
    |gpu - ref| <= rel * max(|ref|, rms(ref)).  Differences in FP32 summation
    order are ~1e-6 relative to the terms summed, so values produced by
    cancellation (|ref| << rms) may differ by many ulps and still be right;
    the rms floor accepts those and nothing else."""
    g = f32(gpu_bits).astype(np.float64)
    r = f32(ref_bits).astype(np.float64)
    scale = np.sqrt(np.mean(r * r)) if r.size else 0.0
    bad = np.abs(g - r) > rel * np.maximum(np.abs(r), scale)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements beyond {rel} x "
                             f"max(|ref|, rms={scale:.3g}); first at {tuple(i)}: "
                             f"gpu={g[tuple(i)]} ref={r[tuple(i)]}")


def ulp_diff_bf16(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in BF16 units in the last place (same-sign values)."""
    a = a_bits.astype(np.int32)
    b = b_bits.astype(np.int32)
    ka = np.where(a & 0x8000, -(a & 0x7FFF), a)
    kb = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(ka - kb)


class Case:
    """A layer invocation held both on the device and (lazily) on the host."""

    def __init__(self, x_bits, ids, w, Wg, Wu, Wd, E):
        self.x_bits = np.ascontiguousarray(x_bits, np.uint16)
        self.ids = np.ascontiguousarray(ids, np.int32)
        self.w = np.ascontiguousarray(w, np.float32)
        self.Wg, self.Wu, self.Wd = Wg, Wu, Wd    # device tensors [E,...]
        self.E = E
        self.T, self.H = self.x_bits.shape
        self.I = Wg.shape[1]
        self.k = self.ids.shape[1]

    @classmethod
    def from_numpy(cls, x_bits, ids, w, Wg_list, Wu_list, Wd_list):
        dev = lambda L: torch.stack([workloads.bits_to_bf16(a) for a in L]).cuda()  # noqa: E731
        return cls(x_bits, ids, w, dev(Wg_list), dev(Wu_list), dev(Wd_list), len(Wg_list))

    def device_inputs(self):
        x = workloads.bits_to_bf16(self.x_bits).cuda()
        return x, torch.from_numpy(self.ids).cuda(), torch.from_numpy(self.w).cuda()

    def host_expert(self, W, e):
        return workloads.bf16_bits(W[e])

    def oracle(self, rows=None, aux=False):
        rows = np.arange(self.T) if rows is None else np.asarray(rows)
        cache = {}

        def get(W, tag):
            def f(e):
                key = (tag, e)
                if key not in cache:
                    cache[key] = self.host_expert(W, e)
                return cache[key]
            return f
        return oracle.moe_ffn_bf16(self.x_bits[rows], self.ids[rows], self.w[rows],
                                   get(self.Wg, "g"), get(self.Wu, "u"), get(self.Wd, "d"),
                                   E=self.E, aux=aux)


def random_case(seed, T, H, I, E, k, std=0.05, ids=None, w=None):
    """Small case with numpy-drawn inputs; distinct experts per token unless
    ``ids`` is given."""
    rng = np.random.default_rng(seed)
    x = workloads.bf16_bits(torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32))
                            .to(torch.bfloat16))
    mk = lambda N, K: workloads.bf16_bits(  # noqa: E731
        torch.from_numpy((rng.standard_normal((N, K)) * std).astype(np.float32)).to(torch.bfloat16))
    Wg = [mk(I, H) for _ in range(E)]
    Wu = [mk(I, H) for _ in range(E)]
    Wd = [mk(H, I) for _ in range(E)]
    if ids is None:
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    if w is None:
        w = rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    return Case.from_numpy(x, ids, w, Wg, Wu, Wd)


def workload_case(name: str, device="cuda"):
    """Full workload from the registry: x and routing (oracle router on the
    seeded logits) on the host, weights drawn on ``device``."""
    wl = workloads.WORKLOADS[name]
    x = workloads.bf16_bits(workloads.gen_x(wl))
    ids, w = oracle.route_topk(workloads.gen_logits(wl).numpy(), wl.k)
    Wg, Wu, Wd = workloads.gen_weights(wl, device)
    return wl, Case(x, ids, w, Wg, Wu, Wd, wl.E)


# The layer hands experts with more than TILED_MIN_TOKENS tokens to the
# tiled product when the batch has more than TILED_MIN_BATCH tokens and BF16
# weights (the workspace's `large` list); every other active expert goes to
# the small-m product (`active`).
TILED_MIN_BATCH = 64
TILED_MIN_TOKENS = 32


def expected_lists(p: dict, T: int, int8: bool = False):
    """(active, large) lists the gather index must produce, from the oracle's
    permutation ``p``."""
    act = p["active"]
    if int8 or T <= TILED_MIN_BATCH:
        return act, act[:0]
    big = p["counts"][act] > TILED_MIN_TOKENS
    return act[~big], act[big]


def check_lists(r: dict, p: dict, T: int, int8: bool = False):
    small, large = expected_lists(p, T, int8)
    assert r["n_active"] == len(small)
    assert np.array_equal(r["active"], small)
    assert r["n_large"] == len(large)
    assert np.array_equal(r["large"], large)


def read_workspace(ws: torch.Tensor, L: dict, T: int, H: int, I: int, E: int, k: int):
    """Host copies of the workspace regions after a forward call."""
    b = ws.cpu().numpy()
    S = T * k
    i32 = lambda off, n: b[off:off + 4 * n].view(np.int32).copy()  # noqa: E731
    meta = i32(L["meta"], 8)
    return {
        "n_active": int(meta[0]),
        "n_dropped": int(meta[1]),
        "counts": i32(L["counts"], E),
        "offsets": i32(L["offsets"], E + 1),
        "active": i32(L["active"], E)[: meta[0]],
        "n_large": int(meta[2]),
        "large": i32(L["large"], E)[: meta[2]],
        "sorted_slot": i32(L["sorted_slot"], S),
        "h": b[L["h"]:L["h"] + S * I * 2].view(np.uint16).reshape(S, I).copy(),
        "y": b[L["y"]:L["y"] + S * H * 4].view(np.float32).reshape(S, H).copy(),
        # every K-part plane of y (the tiled down product's partial sums)
        "y_planes": b[L["y"]:L["y"] + L["y_parts"] * S * H * 4].view(np.float32)
        .reshape(L["y_parts"], S, H).copy(),
    }
