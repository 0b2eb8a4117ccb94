"""Pins of the residual-split oracle (oracle.moe_ffn_resplit; RapidMoE,
"Residual-Split Representation" and "GLU Architecture Adoption") against
things other than itself: the INT8-definition oracle it must reduce to when
no expert is critical or the residual is zero, a float64 dense brute force
over the dequantised weights, the quantiser's error bound, the per-expert
selection of precision, and the accuracy the residual buys.  CPU only.
"""
import numpy as np
import torch

import oracle
import workloads


def rand_bf16(rng, shape, std=1.0):
    return workloads.bf16_bits(torch.from_numpy(
        (rng.standard_normal(shape) * std).astype(np.float32)).to(torch.bfloat16))


def f32(bits):
    return workloads.bits_to_bf16(bits).float().numpy()


def bf16_round_f64(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64)).float().to(
        torch.bfloat16).double().numpy()


def deq_f64(q, s, group=128):
    q = np.asarray(q).astype(np.float64)
    return (q.reshape(q.shape[0], -1, group) * np.asarray(s, np.float64)[..., None]).reshape(q.shape)


def case(seed=40, T=6, H=256, I=384, E=4, k=2, std=0.05):
    """Weights as float32 draws, their residual split (gate/up), the low
    (INT4) and high (INT8) copies of down, tokens and routing."""
    rng = np.random.default_rng(seed)
    x = rand_bf16(rng, (T, H))
    W = {n: [torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32))
             for _ in range(E)]
         for n, shape in (("g", (I, H)), ("u", (I, H)), ("d", (H, I)))}
    t = {}
    for n in ("g", "u"):
        parts = [workloads.quantize_residual_split(w, 128, 7) for w in W[n]]
        for i, key in enumerate(("Q", "S", "R", "SR")):
            t[key + n] = [p[i].numpy() for p in parts]
    lo = [workloads.quantize_groupwise(w, 128, 7) for w in W["d"]]
    hi = [workloads.quantize_groupwise(w, 128, 127) for w in W["d"]]
    t["Qd_lo"], t["Sd_lo"] = [q.numpy() for q, _ in lo], [s.numpy() for _, s in lo]
    t["Qd_hi"], t["Sd_hi"] = [q.numpy() for q, _ in hi], [s.numpy() for _, s in hi]
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    return x, ids, w, t, W


def run(x, ids, w, t, crit, **kw):
    return oracle.moe_ffn_resplit(x, ids, w, t["Qg"], t["Sg"], t["Rg"], t["SRg"], t["Qu"],
                                  t["Su"], t["Ru"], t["SRu"], t["Qd_lo"], t["Sd_lo"],
                                  t["Qd_hi"], t["Sd_hi"], np.asarray(crit, np.uint8),
                                  E=len(t["Qg"]), **kw)


def test_no_critical_expert_is_the_int4_layer():
    """Every expert in low precision: gate/up from W^Q alone and the low down
    copy, i.e. the INT8-definition layer fed those integers, bit for bit."""
    x, ids, w, t, _ = case()
    a = run(x, ids, w, t, [0, 0, 0, 0], aux=True)
    b = oracle.moe_ffn_int8(x, ids, w, t["Qg"], t["Sg"], t["Qu"], t["Su"], t["Qd_lo"],
                            t["Sd_lo"], E=4, aux=True)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["h"], b["h"])


def test_zero_residual_and_equal_down_copies_is_the_int4_layer():
    """Every expert critical, but W^R = 0 (scales 0) and the high down copy
    equal to the low one: x W^Q + 0 is x W^Q exactly."""
    x, ids, w, t, _ = case(seed=41)
    t = dict(t)
    t["Rg"] = [np.zeros_like(r) for r in t["Rg"]]
    t["SRg"] = [np.zeros_like(s) for s in t["SRg"]]
    t["Ru"] = [np.zeros_like(r) for r in t["Ru"]]
    t["SRu"] = [np.zeros_like(s) for s in t["SRu"]]
    t["Qd_hi"], t["Sd_hi"] = t["Qd_lo"], t["Sd_lo"]
    a = run(x, ids, w, t, [1, 1, 1, 1])
    b = oracle.moe_ffn_int8(x, ids, w, t["Qg"], t["Sg"], t["Qu"], t["Su"], t["Qd_lo"],
                            t["Sd_lo"], E=4)
    assert np.array_equal(a, b)


def test_matches_dequantised_dense_fp64():
    """float64 brute force on the dequantised weights: W^Q + W^R and the high
    down copy for critical experts, W^Q and the low copy for the others."""
    x, ids, w, t, _ = case(seed=42, T=7, E=4)
    crit = np.array([1, 0, 1, 0], np.uint8)
    r = run(x, ids, w, t, crit, aux=True)
    xf = f32(x).astype(np.float64)
    ref = np.zeros((x.shape[0], xf.shape[1]))
    for tt in range(x.shape[0]):
        for j in range(ids.shape[1]):
            e = ids[tt, j]
            Wg = deq_f64(t["Qg"][e], t["Sg"][e])
            Wu = deq_f64(t["Qu"][e], t["Su"][e])
            if crit[e]:
                Wg = Wg + deq_f64(t["Rg"][e], t["SRg"][e])
                Wu = Wu + deq_f64(t["Ru"][e], t["SRu"][e])
                Wd = deq_f64(t["Qd_hi"][e], t["Sd_hi"][e])
            else:
                Wd = deq_f64(t["Qd_lo"][e], t["Sd_lo"][e])
            g, u = Wg @ xf[tt], Wu @ xf[tt]
            h = bf16_round_f64(g / (1 + np.exp(-g)) * u)
            ref[tt] += w[tt, j] * (Wd @ h)
    err = np.abs(r["out_f32"] - ref) / np.maximum(1.0, np.abs(ref))
    assert err.max() < 2e-3
    assert np.abs(ref).max() > 0.2


def test_precision_is_chosen_per_expert():
    """With one slot per token, each token's output equals the all-critical
    layer's where its expert is critical and the all-low layer's elsewhere,
    bit for bit."""
    x, ids, w, t, _ = case(seed=43, T=12, E=4, k=1)
    ids[:, 0] = np.arange(12) % 4
    crit = np.array([0, 1, 1, 0], np.uint8)
    mixed = run(x, ids, w, t, crit)
    hi = run(x, ids, w, t, [1, 1, 1, 1])
    lo = run(x, ids, w, t, [0, 0, 0, 0])
    for tt in range(12):
        ref = hi if crit[ids[tt, 0]] else lo
        assert np.array_equal(mixed[tt], ref[tt]), tt
    assert not np.array_equal(hi, lo)


def test_residual_split_error_bound():
    """|W - (q s + r sr)| <= sr / 2 elementwise (round to nearest of the
    residual), against |W - q s| <= s / 2 for W^Q alone; the residual's
    scale is at most 1/14 of the first stage's, so the split cuts the
    worst-case error at least sevenfold."""
    rng = np.random.default_rng(44)
    w = torch.from_numpy((rng.standard_normal((16, 512)) * 0.05).astype(np.float32))
    q, s, r, sr = workloads.quantize_residual_split(w, 128, 7)
    wd = w.double().numpy()
    e1 = np.abs(wd - deq_f64(q.numpy(), s.numpy()))
    e2 = np.abs(wd - deq_f64(q.numpy(), s.numpy()) - deq_f64(r.numpy(), sr.numpy()))
    b1 = np.repeat(s.double().numpy(), 128, axis=1) / 2
    b2 = np.repeat(sr.double().numpy(), 128, axis=1) / 2
    assert np.all(e1 <= b1 * (1 + 1e-5) + 1e-9)
    assert np.all(e2 <= b2 * (1 + 1e-5) + 1e-9)
    assert np.all(sr.numpy() <= s.numpy() / 14 * (1 + 1e-5) + 1e-12)
    assert e2.max() < e1.max() / 7


def test_high_precision_is_closer_to_the_bf16_layer():
    """The critical (W^Q + W^R, INT8 down) layer lands closer to the layer on
    the unquantised weights than the low-precision one, by a wide margin."""
    x, ids, w, t, W = case(seed=45, T=8)
    bits = lambda a: workloads.bf16_bits(a.to(torch.bfloat16))  # noqa: E731
    ref = oracle.moe_ffn_bf16(x, ids, w, [bits(a) for a in W["g"]], [bits(a) for a in W["u"]],
                              [bits(a) for a in W["d"]], E=4, aux=True)["out_f32"]
    hi = run(x, ids, w, t, [1, 1, 1, 1], aux=True)["out_f32"]
    lo = run(x, ids, w, t, [0, 0, 0, 0], aux=True)["out_f32"]
    e_hi = np.sqrt(np.mean((hi - ref) ** 2))
    e_lo = np.sqrt(np.mean((lo - ref) ** 2))
    assert e_hi < e_lo / 4, (e_hi, e_lo)


def test_dropped_slots_and_missing_tables():
    """A slot naming no expert contributes nothing; the residual tables of a
    non-critical expert are never needed (None is accepted)."""
    x, ids, w, t, _ = case(seed=46, T=5, E=4)
    ids[0, 1] = -1
    ids[3, 0] = 4
    t = dict(t)
    crit = np.array([1, 0, 0, 0], np.uint8)
    for key in ("Rg", "SRg", "Ru", "SRu", "Qd_hi", "Sd_hi"):
        t[key] = [t[key][0]] + [None] * 3
    r = run(x, ids, w, t, crit, aux=True)
    assert not r["h"][1].any() and not r["y"][6].any()
    keep = ids.copy()
    keep[0, 1], keep[3, 0] = ids[0, 0], ids[3, 1]
    w2 = w.copy()
    w2[0, 1] = 0.0
    w2[3, 0] = 0.0
    r2 = run(x, keep, w2, t, crit, aux=True)
    assert np.allclose(r["out_f32"], r2["out_f32"], rtol=0, atol=1e-6)
