"""Pins of the decode-attention oracle (HiNa-MoE §6.1: grouped-query SDPA
in decoding) against things other than itself: a float64 brute force, torch's
CPU scaled-dot-product attention, closed forms (one position, equal keys,
zero scale, values per KV head), exact invariants (doubling the values),
and permutation invariance.  CPU only.
"""
import numpy as np
import pytest
import torch

import oracle


def bits(a):
    return oracle.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def f32(b):
    return oracle.bf16_bits_to_f32(b).astype(np.float64)


def draw(rng, B, h_q, h_kv, d, max_len, lens=None, kv_std=1.0):
    q = bits(rng.standard_normal((B, h_q, d)))
    k = bits(rng.standard_normal((B, h_kv, max_len, d)) * kv_std)
    v = bits(rng.standard_normal((B, h_kv, max_len, d)))
    if lens is None:
        lens = rng.integers(0, max_len + 1, size=B)
    return q, k, v, np.asarray(lens, dtype=np.int32)


def brute_force(q, k, v, lens, scale=None):
    """float64, one query head at a time, straight from the definition."""
    qf, kf, vf = f32(q), f32(k), f32(v)
    B, h_q, d = qf.shape
    h_kv = kf.shape[1]
    g = h_q // h_kv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.zeros((B, h_q, d))
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        for h in range(h_q):
            j = h // g
            s = scale * (kf[b, j, :n] @ qf[b, h])
            p = np.exp(s - s.max())
            out[b, h] = (p / p.sum()) @ vf[b, j, :n]
    return out


def close(got_bits, ref, rms_v, what=""):
    """BF16 rounding of the output (2^-9 relative) plus FP32 summation."""
    got = f32(got_bits)
    bad = np.abs(got - ref) > 2.0 ** -8 * np.abs(ref) + 1e-4 * rms_v
    assert not bad.any(), f"{what}: {bad.sum()} elements off; first {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("B,h_q,h_kv,d,max_len", [
    (3, 8, 2, 64, 40), (2, 32, 4, 128, 130), (2, 28, 4, 32, 17), (1, 16, 1, 96, 64),
    (4, 4, 4, 32, 9), (2, 32, 8, 128, 200),
])
def test_attn_matches_float64_brute_force(B, h_q, h_kv, d, max_len):
    rng = np.random.default_rng(B * 100 + h_q + d)
    q, k, v, lens = draw(rng, B, h_q, h_kv, d, max_len)
    lens[0] = max_len
    got = oracle.attn_decode(q, k, v, lens)
    close(got, brute_force(q, k, v, lens), 1.0, "brute force")


def test_attn_matches_torch_sdpa():
    """Library special case: torch's CPU SDPA in float32 with the KV heads
    repeated for their query groups and the invalid positions masked."""
    rng = np.random.default_rng(3)
    B, h_q, h_kv, d, max_len = 3, 32, 4, 128, 96
    q, k, v, lens = draw(rng, B, h_q, h_kv, d, max_len, lens=[96, 1, 50])
    g = h_q // h_kv
    qt = torch.from_numpy(f32(q)).float()[:, :, None, :]                 # [B, h_q, 1, d]
    kt = torch.from_numpy(f32(k)).float().repeat_interleave(g, dim=1)    # [B, h_q, L, d]
    vt = torch.from_numpy(f32(v)).float().repeat_interleave(g, dim=1)
    mask = torch.arange(max_len)[None, None, None, :] < torch.from_numpy(lens)[:, None, None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    close(oracle.attn_decode(q, k, v, lens), ref[:, :, 0, :].double().numpy(), 1.0, "sdpa")


def test_attn_single_position_returns_that_value_exactly():
    rng = np.random.default_rng(4)
    q, k, v, _ = draw(rng, 2, 8, 2, 64, 5)
    lens = np.array([1, 1], np.int32)
    got = oracle.attn_decode(q, k, v, lens)
    for h in range(8):
        assert np.array_equal(got[:, h], v[:, h // 4, 0])


def test_attn_empty_sequence_gives_zeros():
    rng = np.random.default_rng(5)
    q, k, v, _ = draw(rng, 2, 4, 2, 32, 8)
    got = oracle.attn_decode(q, k, v, np.array([0, 8], np.int32))
    assert not got[0].any()
    assert got[1].any()


def test_attn_equal_keys_average_the_values():
    """Every key equal: uniform softmax, the output is the mean value."""
    rng = np.random.default_rng(6)
    B, h_q, h_kv, d, L = 2, 8, 2, 64, 33
    q, k, v, _ = draw(rng, B, h_q, h_kv, d, L)
    k[:] = k[:, :, :1, :]
    lens = np.array([33, 20], np.int32)
    ref = np.zeros((B, h_q, d))
    for b in range(B):
        for h in range(h_q):
            ref[b, h] = f32(v)[b, h // 4, : lens[b]].mean(axis=0)
    close(oracle.attn_decode(q, k, v, lens), ref, 1.0, "mean")


def test_attn_zero_scale_averages_the_values():
    """scale = 0: every score is 0 whatever q and k are."""
    rng = np.random.default_rng(7)
    q, k, v, lens = draw(rng, 2, 8, 4, 32, 25, lens=[25, 7])
    ref = np.stack([[f32(v)[b, h // 2, : lens[b]].mean(axis=0) for h in range(8)]
                    for b in range(2)])
    close(oracle.attn_decode(q, k, v, lens, scale=0.0), ref, 1.0, "zero scale")


def test_attn_query_head_reads_its_group_kv_head():
    """Values constant per KV head (= the head's index + 1): query head h
    must return h // (h_q / h_kv) + 1 exactly."""
    rng = np.random.default_rng(8)
    B, h_q, h_kv, d, L = 2, 12, 3, 32, 10
    q, k, v, _ = draw(rng, B, h_q, h_kv, d, L)
    for j in range(h_kv):
        v[:, j] = bits(np.full((B, L, d), j + 1.0))
    got = f32(oracle.attn_decode(q, k, v, np.array([10, 4], np.int32)))
    for h in range(h_q):
        assert np.all(got[:, h] == h // 4 + 1.0)


def test_attn_doubling_values_doubles_output_exactly():
    rng = np.random.default_rng(9)
    q, k, v, lens = draw(rng, 2, 8, 2, 64, 50, lens=[50, 13])
    a = oracle.attn_decode(q, k, v, lens)
    b = oracle.attn_decode(q, k, bits(f32(v) * 2.0), lens)
    assert np.array_equal(f32(b), 2.0 * f32(a))


def test_attn_sharp_query_selects_one_position():
    """One key aligned with the query and scaled up: the softmax puts
    essentially all weight on that position."""
    rng = np.random.default_rng(10)
    B, h_q, h_kv, d, L = 1, 4, 1, 64, 40
    q, k, v, _ = draw(rng, B, h_q, h_kv, d, L, kv_std=0.01)
    q[:] = q[:, :1]                       # every head asks the same question
    k[0, 0, 17] = bits(f32(q)[0, 0] * 4.0)
    got = f32(oracle.attn_decode(q, k, v, np.array([L], np.int32)))
    for h in range(h_q):
        np.testing.assert_allclose(got[0, h], f32(v)[0, 0, 17], rtol=1e-2, atol=1e-2)


def test_attn_position_permutation_invariance():
    rng = np.random.default_rng(11)
    B, h_q, h_kv, d, L = 2, 8, 2, 64, 60
    q, k, v, _ = draw(rng, B, h_q, h_kv, d, L)
    lens = np.array([60, 60], np.int32)
    perm = rng.permutation(L)
    a = oracle.attn_decode(q, k, v, lens)
    b = oracle.attn_decode(q, np.ascontiguousarray(k[:, :, perm]),
                           np.ascontiguousarray(v[:, :, perm]), lens)
    close(b, f32(a), 1.0, "permuted positions")
