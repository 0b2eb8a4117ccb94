"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test ties one oracle routine to a fact the HiNa-MoE paper (arXiv
2610.05123) or plain mathematics fixes: a library routine that computes the
same thing a different way (torch's BF16 cast, numpy's stable sort, a torch
float32 matmul), a float64 brute force of a differently structured form,
closed forms on specially built weights, and invariants the definition
implies.  ``test_oracle_mutants.py`` plants mistakes in copies of the oracle
and checks that this file catches every one.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# --------------------------------------------------------------------------
# helpers local to the pins (none of them is the oracle's code)
# --------------------------------------------------------------------------

def rand_bf16(rng, shape, std=1.0):
    return workloads.bf16_bits(torch.from_numpy(
        (rng.standard_normal(shape) * std).astype(np.float32)).to(torch.bfloat16))


def f32(bits):
    return workloads.bits_to_bf16(bits).float().numpy()


def bf16_round_f64(a):
    """Nearest BF16 of a float64 array, as float64 (torch's cast)."""
    return torch.from_numpy(np.asarray(a, dtype=np.float64)).float().to(
        torch.bfloat16).double().numpy()


def dense_fp64(x, ids, w, Wg, Wu, Wd):
    """Dense float64 form: out_t = sum_e c_{t,e} FFN_e(x_t) over ALL experts,
    with c_{t,e} = sum_j w_{t,j} [ids_{t,j} = e] and h rounded to BF16."""
    x = f32(x).astype(np.float64)
    E = len(Wg)
    T = x.shape[0]
    C = np.zeros((T, E))
    for t in range(T):
        for j in range(ids.shape[1]):
            e = ids[t, j]
            if 0 <= e < E:
                C[t, e] += w[t, j]
    out = np.zeros((T, f32(Wd[0]).shape[0]))
    for e in range(E):
        g = x @ f32(Wg[e]).astype(np.float64).T
        u = x @ f32(Wu[e]).astype(np.float64).T
        h = bf16_round_f64(g / (1.0 + np.exp(-g)) * u)
        out += C[:, e:e + 1] * (h @ f32(Wd[e]).astype(np.float64).T)
    return out


def small_case(seed=0, T=7, H=64, I=96, E=5, k=2, std=0.2):
    rng = np.random.default_rng(seed)
    x = rand_bf16(rng, (T, H))
    Wg = [rand_bf16(rng, (I, H), std) for _ in range(E)]
    Wu = [rand_bf16(rng, (I, H), std) for _ in range(E)]
    Wd = [rand_bf16(rng, (H, I), std) for _ in range(E)]
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    return x, ids, w, Wg, Wu, Wd


# --------------------------------------------------------------------------
# BF16 rounding vs torch's cast (a library routine)
# --------------------------------------------------------------------------

def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 1, 0x007fffff, 0x00800000, 0x3f800000,
                        0x3f808000, 0x3f818000, 0x3f807fff, 0x3f808001,
                        0x7f7fffff, 0xff7fffff, 0x7f800000, 0xff800000,
                        0x7f7f8000, 0x477f8000, 0x00008000, 0x00018000],
                       dtype=np.uint32)
    ties = (rng.integers(0, 2**16, size=1 << 16, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    bits = np.concatenate([bits, special, ties])
    a = bits.view(np.float32)
    finite = np.isfinite(a) | np.isinf(a)
    mine = oracle.f32_to_bf16_bits(a)
    ref = workloads.bf16_bits(torch.from_numpy(a.copy()).to(torch.bfloat16))
    assert np.array_equal(mine[finite], ref[finite])
    nan = ~finite
    assert np.all(np.isnan(f32(mine[nan])))


def test_bf16_widen_is_exact():
    rng = np.random.default_rng(2)
    b = rng.integers(0, 2**16, size=1 << 16, dtype=np.uint64).astype(np.uint16)
    ref = workloads.bits_to_bf16(b).float().numpy()
    got = oracle.bf16_bits_to_f32(b)
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok].view(np.uint32), ref[ok].view(np.uint32))


# --------------------------------------------------------------------------
# Routing (top-k of a softmax gate)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("E,k", [(8, 2), (256, 8), (128, 8), (5, 5), (7, 1)])
def test_route_ids_match_full_stable_sort(E, k):
    rng = np.random.default_rng(E * 31 + k)
    T = 33
    # integer-valued logits force many exact ties
    logits = rng.integers(-3, 4, size=(T, E)).astype(np.float32)
    logits[::2] = rng.standard_normal((logits[::2].shape)).astype(np.float32)
    ids, w = oracle.route_topk(logits, k)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))[:k]
        assert np.array_equal(ids[t], order)


@pytest.mark.parametrize("E,k", [(8, 2), (256, 8), (128, 8)])
def test_route_weights_are_softmax_over_kept_logits(E, k):
    # renormalising the k kept probabilities of a softmax over all E experts
    # equals a softmax over the k kept logits alone (the common denominator
    # cancels) -- a closed form that never forms the full softmax.
    rng = np.random.default_rng(E + k)
    T = 40
    logits = (rng.standard_normal((T, E)) * 3).astype(np.float32)
    ids, w = oracle.route_topk(logits, k)
    for t in range(T):
        kept = logits[t, ids[t]].astype(np.float64)
        ref = np.exp(kept - kept.max())
        ref /= ref.sum()
        np.testing.assert_allclose(w[t], ref, rtol=1e-6, atol=1e-7)
        assert np.all(np.diff(w[t]) <= 0)
        assert len(set(ids[t].tolist())) == k


def test_route_shift_invariance_and_masked_logits():
    rng = np.random.default_rng(5)
    T, E, k = 16, 8, 2
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids0, w0 = oracle.route_topk(lg, k)
    ids1, w1 = oracle.route_topk(lg + np.float32(0.5), k)
    assert np.array_equal(ids0, ids1)
    np.testing.assert_allclose(w0, w1, rtol=1e-6)
    # the "forced" recipe: only experts 2t, 2t+1 (mod 8) finite -> exactly those
    wl = workloads.Workload("f", H=64, I=64, E=8, k=2, T=16, routing="forced")
    ids, w = oracle.route_topk(workloads.gen_logits(wl).numpy(), 2)
    for t in range(16):
        assert set(ids[t].tolist()) == {(2 * t) % 8, (2 * t + 1) % 8}
    assert np.all(np.bincount(ids.reshape(-1), minlength=8) == 4)


def test_route_zipf_recipe_is_skewed():
    wl = workloads.WORKLOADS["deepseekv3_zipf_t16"]
    ids, _ = oracle.route_topk(workloads.gen_logits(wl).numpy(), wl.k)
    counts = np.bincount(ids.reshape(-1), minlength=wl.E)
    wl_u = workloads.WORKLOADS["deepseekv3_t16"]
    ids_u, _ = oracle.route_topk(workloads.gen_logits(wl_u).numpy(), wl_u.k)
    counts_u = np.bincount(ids_u.reshape(-1), minlength=wl_u.E)
    assert counts.max() > counts_u.max()
    assert (counts > 0).sum() < (counts_u > 0).sum()


# --------------------------------------------------------------------------
# Gather index (per-expert slot lists)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,k,E", [(16, 2, 8), (16, 8, 256), (1, 8, 128), (0, 2, 8),
                                   (300, 3, 7)])
def test_permute_matches_stable_argsort(T, k, E):
    rng = np.random.default_rng(T * 7 + E)
    ids = rng.integers(-2, E + 2, size=(T, k)).astype(np.int32)
    p = oracle.permute(ids, E)
    flat = ids.reshape(-1)
    valid = np.nonzero((flat >= 0) & (flat < E))[0]
    order = valid[np.argsort(flat[valid], kind="stable")]
    assert np.array_equal(p["sorted_slot"], order)
    assert np.array_equal(p["counts"], np.bincount(flat[valid], minlength=E))
    assert np.array_equal(p["offsets"], np.concatenate([[0], np.cumsum(p["counts"])]))
    assert np.array_equal(p["active"], np.nonzero(p["counts"])[0])
    assert p["n_invalid"] == flat.size - valid.size


# --------------------------------------------------------------------------
# The FFN layer
# --------------------------------------------------------------------------

def test_ffn_matches_dense_fp64_bruteforce():
    x, ids, w, Wg, Wu, Wd = small_case()
    r = oracle.moe_ffn_bf16(x, ids, w, Wg, Wu, Wd, E=len(Wg), aux=True)
    ref = dense_fp64(x, ids, w, Wg, Wu, Wd)
    err = np.abs(r["out_f32"] - ref) / np.maximum(1.0, np.abs(ref))
    assert err.max() < 2e-3, err.max()
    assert np.array_equal(r["out"], oracle.f32_to_bf16_bits(r["out_f32"]))
    assert np.abs(ref).max() > 0.5  # the case is not trivially small


def test_ffn_duplicate_ids_and_dropped_slots():
    x, ids, w, Wg, Wu, Wd = small_case(seed=3, T=6, E=4, k=3)
    ids[0] = [1, 1, 2]          # duplicate: expert 1 counted twice
    ids[1] = [0, -1, 3]         # dropped slot
    ids[2] = [4, 7, 2]          # two dropped slots (E = 4)
    r = oracle.moe_ffn_bf16(x, ids, w, Wg, Wu, Wd, E=4, aux=True)
    ref = dense_fp64(x, ids, w, Wg, Wu, Wd)
    err = np.abs(r["out_f32"] - ref) / np.maximum(1.0, np.abs(ref))
    assert err.max() < 2e-3
    assert np.all(r["h"][1 * 3 + 1] == 0) and np.all(r["y"][2 * 3 + 1] == 0)


@pytest.mark.parametrize("zero", ["gate", "up", "w"])
def test_ffn_closed_form_zero(zero):
    x, ids, w, Wg, Wu, Wd = small_case(seed=4)
    if zero == "gate":
        Wg = [np.zeros_like(a) for a in Wg]
    elif zero == "up":
        Wu = [np.zeros_like(a) for a in Wu]
    else:
        w = np.zeros_like(w)
    out = oracle.moe_ffn_bf16(x, ids, w, Wg, Wu, Wd, E=len(Wg))
    assert np.all(f32(out) == 0.0)


def test_ffn_closed_form_permutation_experts():
    """W_gate[e], W_up[e] are permutation matrices and W_down[e] a scaled one.

    Then g_i = x[pi_e(i)], u_i = x[sig_e(i)], h_i = bf16(silu(g_i) u_i),
    y_n = s_e h[rho_e(n)], out_n = bf16(sum_j w_j s_{e_j} h^{e_j}[rho_{e_j}(n)]).
    A transposed operand (pi -> pi^-1), swapped gate/up, a wrong expert, a
    wrong weight or a wrong slot all change the result by O(1).
    """
    rng = np.random.default_rng(9)
    T, D, E, k = 9, 64, 4, 2
    x = rand_bf16(rng, (T, D), 1.5)
    one = np.uint16(0x3F80)
    perms = [[rng.permutation(D) for _ in range(3)] for _ in range(E)]
    scales = [0.5, 2.0, -1.0, 0.25]
    Wg, Wu, Wd = [], [], []
    for e in range(E):
        pi, sig, rho = perms[e]
        g = np.zeros((D, D), np.uint16); g[np.arange(D), pi] = one
        u = np.zeros((D, D), np.uint16); u[np.arange(D), sig] = one
        d = np.zeros((D, D), np.uint16)
        d[np.arange(D), rho] = workloads.bf16_bits(torch.tensor([scales[e]]).to(torch.bfloat16))[0]
        Wg.append(g); Wu.append(u); Wd.append(d)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    got = oracle.moe_ffn_bf16(x, ids, w, Wg, Wu, Wd, E=E, aux=True)
    xf = f32(x).astype(np.float64)
    ref = np.zeros((T, D))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            pi, sig, rho = perms[e]
            gi = xf[t, pi]
            h = bf16_round_f64(gi / (1.0 + np.exp(-gi)) * xf[t, sig])
            ref[t] += w[t, j] * scales[e] * h[rho]
            hgot = f32(got["h"][t * k + j]).astype(np.float64)
            # silu in float32 vs float64 may move h by at most one BF16 ulp
            assert np.all(np.abs(hgot - h) <= np.abs(h) * 2.0**-7 + 1e-30)
    err = np.abs(got["out_f32"] - ref) / np.maximum(1.0, np.abs(ref))
    assert err.max() < 1e-2
    assert np.abs(ref).max() > 0.5


def test_ffn_single_expert_equals_dense_swiglu_torch():
    """k = 1, weight 1, one expert: the layer is a dense SwiGLU FFN, computed
    here with torch float32 matmuls and h rounded to BF16 at the same point."""
    rng = np.random.default_rng(11)
    T, H, I = 12, 96, 160
    x = rand_bf16(rng, (T, H))
    Wg, Wu, Wd = rand_bf16(rng, (I, H), 0.15), rand_bf16(rng, (I, H), 0.15), rand_bf16(rng, (H, I), 0.15)
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    got = oracle.moe_ffn_bf16(x, ids, w, [Wg], [Wu], [Wd], E=1, aux=True)
    tx, tg, tu, td = (workloads.bits_to_bf16(a).float() for a in (x, Wg, Wu, Wd))
    h = (torch.nn.functional.silu(tx @ tg.T) * (tx @ tu.T)).to(torch.bfloat16).float()
    ref = (h @ td.T).numpy()
    err = np.abs(got["out_f32"] - ref) / np.maximum(1.0, np.abs(ref))
    assert err.max() < 1e-3


def test_ffn_linear_in_topk_w():
    x, ids, w, Wg, Wu, Wd = small_case(seed=12)
    base = oracle.moe_ffn_bf16(x, ids, w, Wg, Wu, Wd, E=5, aux=True)
    dbl = oracle.moe_ffn_bf16(x, ids, 2 * w, Wg, Wu, Wd, E=5, aux=True)
    # scaling by two is exact in binary floating point, before and after rounding
    assert np.array_equal(dbl["out_f32"], 2 * base["out_f32"])
    w1 = (w * np.float32(0.375)).astype(np.float32)
    w2 = (w - w1).astype(np.float32)
    a = oracle.moe_ffn_bf16(x, ids, w1, Wg, Wu, Wd, E=5, aux=True)["out_f32"]
    b = oracle.moe_ffn_bf16(x, ids, w2, Wg, Wu, Wd, E=5, aux=True)["out_f32"]
    np.testing.assert_allclose(a + b, base["out_f32"], rtol=1e-5, atol=1e-5)


def test_ffn_token_permutation_invariance():
    x, ids, w, Wg, Wu, Wd = small_case(seed=13, T=11)
    perm = np.random.default_rng(0).permutation(11)
    a = oracle.moe_ffn_bf16(x, ids, w, Wg, Wu, Wd, E=5)
    b = oracle.moe_ffn_bf16(x[perm], ids[perm], w[perm], Wg, Wu, Wd, E=5)
    assert np.array_equal(a[perm], b)


def test_ffn_expert_relabelling_invariance():
    x, ids, w, Wg, Wu, Wd = small_case(seed=14)
    lab = np.array([3, 0, 4, 1, 2])          # new id of old expert e
    inv = np.argsort(lab)
    a = oracle.moe_ffn_bf16(x, ids, w, Wg, Wu, Wd, E=5)
    b = oracle.moe_ffn_bf16(x, lab[ids].astype(np.int32), w,
                            [Wg[i] for i in inv], [Wu[i] for i in inv],
                            [Wd[i] for i in inv], E=5)
    assert np.array_equal(a, b)


def test_ffn_slot_order_within_token_only_reorders_the_sum():
    x, ids, w, Wg, Wu, Wd = small_case(seed=15, k=3)
    a = oracle.moe_ffn_bf16(x, ids, w, Wg, Wu, Wd, E=5, aux=True)["out_f32"]
    b = oracle.moe_ffn_bf16(x, ids[:, ::-1].copy(), w[:, ::-1].copy(), Wg, Wu, Wd,
                            E=5, aux=True)["out_f32"]
    np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-6)


def test_expert_ffn_single_token_entry_matches_layer():
    x, ids, w, Wg, Wu, Wd = small_case(seed=16, T=2, k=1)
    w[:] = 1.0
    lay = oracle.moe_ffn_bf16(x, ids, w, Wg, Wu, Wd, E=5, aux=True)
    e = ids[0, 0]
    h, y = oracle.expert_ffn_bf16(x[0], Wg[e], Wu[e], Wd[e])
    assert np.array_equal(h, lay["h"][0]) and np.array_equal(y, lay["y"][0])


# --------------------------------------------------------------------------
# INT8 group-quantised variant
# --------------------------------------------------------------------------

def int8_case(seed=20, T=5, H=256, I=384, E=3, k=2, group=128):
    rng = np.random.default_rng(seed)
    x = rand_bf16(rng, (T, H))
    mk = lambda N, K: workloads.quantize_groupwise(  # noqa: E731
        torch.from_numpy((rng.standard_normal((N, K)) * 0.05).astype(np.float32)), group)
    Qg, Sg, Qu, Su, Qd, Sd = [], [], [], [], [], []
    for _ in range(E):
        q, s = mk(I, H); Qg.append(q.numpy()); Sg.append(s.numpy())
        q, s = mk(I, H); Qu.append(q.numpy()); Su.append(s.numpy())
        q, s = mk(H, I); Qd.append(q.numpy()); Sd.append(s.numpy())
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    return x, ids, w, Qg, Sg, Qu, Su, Qd, Sd


def _dequant_f64(q, s, group):
    return (q.astype(np.float64).reshape(q.shape[0], -1, group)
            * s.astype(np.float64)[..., None]).reshape(q.shape)


def test_int8_grouped_form_matches_dequantised_dense_fp64():
    x, ids, w, Qg, Sg, Qu, Su, Qd, Sd = int8_case()
    r = oracle.moe_ffn_int8(x, ids, w, Qg, Sg, Qu, Su, Qd, Sd, E=3, aux=True)
    xf = f32(x).astype(np.float64)
    ref = np.zeros((x.shape[0], 256))
    for t in range(x.shape[0]):
        for j in range(ids.shape[1]):
            e = ids[t, j]
            g = _dequant_f64(Qg[e], Sg[e], 128) @ xf[t]
            u = _dequant_f64(Qu[e], Su[e], 128) @ xf[t]
            h = bf16_round_f64(g / (1 + np.exp(-g)) * u)
            ref[t] += w[t, j] * (_dequant_f64(Qd[e], Sd[e], 128) @ h)
    err = np.abs(r["out_f32"] - ref) / np.maximum(1.0, np.abs(ref))
    assert err.max() < 2e-3
    assert np.abs(ref).max() > 0.2


def test_int8_power_of_two_scales_equal_bf16_path():
    """With power-of-two scales q*s is exact in BF16, so the INT8 layer must
    agree with the BF16 layer fed the dequantised weights (only the FP32
    summation grouping differs)."""
    x, ids, w, Qg, Sg, Qu, Su, Qd, Sd = int8_case(seed=21)
    p2 = lambda s: np.float32(2.0) ** np.round(np.log2(s)).astype(np.float32)  # noqa: E731
    Sg, Su, Sd = [p2(s) for s in Sg], [p2(s) for s in Su], [p2(s) for s in Sd]
    deq = lambda q, s: oracle.f32_to_bf16_bits(  # noqa: E731
        _dequant_f64(q, s, 128).astype(np.float32))
    a = oracle.moe_ffn_int8(x, ids, w, Qg, Sg, Qu, Su, Qd, Sd, E=3, aux=True)
    b = oracle.moe_ffn_bf16(x, ids, w, [deq(q, s) for q, s in zip(Qg, Sg)],
                            [deq(q, s) for q, s in zip(Qu, Su)],
                            [deq(q, s) for q, s in zip(Qd, Sd)], E=3, aux=True)
    err = np.abs(a["out_f32"] - b["out_f32"]) / np.maximum(1.0, np.abs(b["out_f32"]))
    assert err.max() < 1e-3
    assert (a["h"] == b["h"]).mean() > 0.99


def test_int8_quantiser_invariants():
    rng = np.random.default_rng(22)
    w = torch.from_numpy((rng.standard_normal((64, 512)) * 0.02).astype(np.float32))
    w[3, 128:256] = 0.0
    q, s = workloads.quantize_groupwise(w, 128)
    q = q.numpy().astype(np.int32); s = s.numpy(); wn = w.numpy()
    assert np.abs(q).max() <= 127
    assert np.all(s[3, 1] == 0) and np.all(q[3, 128:256] == 0)
    grp = np.abs(wn.reshape(64, 4, 128)).argmax(-1)
    qq = q.reshape(64, 4, 128)
    for r in range(64):
        for g in range(4):
            if s[r, g] > 0:
                assert abs(qq[r, g, grp[r, g]]) == 127
    err = np.abs(wn.reshape(64, 4, 128) - qq * s[..., None])
    assert np.all(err <= s[..., None] * 0.5 * (1 + 1e-6) + 1e-12)


def test_int4_quantiser_and_packing():
    """INT4 (the INT8 definition on values in [-7, 7], stored as two
    offset-binary nibbles per byte): quantiser range and extremes, packing
    layout (element 2i low nibble), exact round trip."""
    rng = np.random.default_rng(23)
    w = torch.from_numpy((rng.standard_normal((32, 256)) * 0.02).astype(np.float32))
    q, s = workloads.quantize_groupwise(w, 128, 7)
    qn, sn = q.numpy().astype(np.int32), s.numpy()
    assert np.abs(qn).max() <= 7
    grp = np.abs(w.numpy().reshape(32, 2, 128)).argmax(-1)
    for r in range(32):
        for g in range(2):
            assert abs(qn.reshape(32, 2, 128)[r, g, grp[r, g]]) == 7
    np.testing.assert_allclose(sn, np.abs(w.numpy()).reshape(32, 2, 128).max(-1) / 7, rtol=1e-6)
    p = workloads.pack_int4(q).numpy()
    assert p.shape == (32, 128) and p.dtype == np.uint8
    assert np.array_equal(p & 0xF, (qn[:, 0::2] + 8).astype(np.uint8))
    assert np.array_equal(p >> 4, (qn[:, 1::2] + 8).astype(np.uint8))
    every = torch.arange(-8, 8, dtype=torch.int8).repeat(4).reshape(2, 32)
    assert torch.equal(workloads.unpack_int4(workloads.pack_int4(every)), every)
