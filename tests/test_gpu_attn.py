"""GPU parity of decode attention with grouped-query heads (moe_attn_decode)
against the oracle.

Small shapes that still span several 32-position tiles, several splits and
ragged lengths (0, 1, tile and split boundaries), every supported head
dimension and group size 1..16; the full-size workloads on sampled sequences
(every output of those sequences).  Tolerance: the GPU rounds the softmax
weights to BF16 for the value product (2^-9 relative per weight) and sums in
another order, so each output is held to 2e-2 x max(|ref|, rms(ref)); where
the result is exact in both (one position, an empty sequence) the bits must
match.
"""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_ffn_topk_amd as moe
import workloads
from moe_cases import assert_close_scaled, need_gpu, say

pytestmark = pytest.mark.gpu


def rnd_bits(rng, shape):
    return workloads.bf16_bits(torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
                               .to(torch.bfloat16))


def run(q, k, v, lens, scale=None):
    dev = lambda a: workloads.bits_to_bf16(a).cuda()  # noqa: E731
    out = moe.moe_attn_decode(dev(q), dev(k), dev(v), torch.from_numpy(lens).cuda(), scale=scale)
    torch.cuda.synchronize()
    return workloads.bf16_bits(out)


@pytest.mark.parametrize("B,h_q,h_kv,d,max_len,lens", [
    (3, 8, 2, 64, 300, [300, 129, 31]),
    (4, 4, 4, 64, 200, [0, 1, 32, 33]),          # empty, one position, tile edges
    (2, 32, 4, 128, 1000, [1000, 517]),          # Qwen3-30B-A3B heads
    (2, 32, 8, 128, 640, [640, 128]),            # Mixtral-8x7B heads
    (1, 28, 4, 128, 5000, [4999]),               # Qwen2-57B-A14B heads (7 per group)
    (2, 16, 1, 256, 700, [700, 3]),              # group of 16, d = 256
    (5, 6, 3, 64, 257, [257, 256, 255, 128, 2]),
])
def test_attn_matches_oracle(B, h_q, h_kv, d, max_len, lens):
    need_gpu()
    rng = np.random.default_rng(B * 1000 + h_q + d + max_len)
    q = rnd_bits(rng, (B, h_q, d))
    k = rnd_bits(rng, (B, h_kv, max_len, d))
    v = rnd_bits(rng, (B, h_kv, max_len, d))
    lens = np.array(lens, np.int32)
    say(f"attn B={B} h_q={h_q} h_kv={h_kv} d={d} max_len={max_len} lens={lens.tolist()}")
    got = run(q, k, v, lens)
    ref = oracle.attn_decode(q, k, v, lens)
    for b in range(B):
        if lens[b] == 0:
            assert not got[b].any(), "empty sequence must give zeros"
        elif lens[b] == 1:
            assert np.array_equal(got[b], ref[b]), "one position must return its value"
        else:
            assert_close_scaled(got[b], ref[b], 2e-2, what=f"sequence {b}")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_attn_default_scale_chosen_by_the_library(d):
    """A score scale that is not positive (0, negative, NaN) selects 1/sqrt(d)
    inside the library: the output equals, bit for bit, a call that passes
    1/sqrt(d) (rounded from double to float) explicitly."""
    need_gpu()
    rng = np.random.default_rng(d)
    B, h_q, h_kv, L = 2, 8, 2, 300
    q = rnd_bits(rng, (B, h_q, d))
    k = rnd_bits(rng, (B, h_kv, L, d))
    v = rnd_bits(rng, (B, h_kv, L, d))
    lens = np.array([300, 77], np.int32)
    say(f"attn default scale d={d}")
    explicit = run(q, k, v, lens, scale=float(np.float32(1.0 / np.sqrt(d))))
    for s in (None, 0.0, -1.0, float("nan")):
        assert np.array_equal(run(q, k, v, lens, scale=s), explicit), f"scale={s}"


def test_attn_other_scale_and_clamped_lengths():
    need_gpu()
    rng = np.random.default_rng(77)
    B, h_q, h_kv, d, L = 3, 8, 2, 128, 150
    q, k, v = rnd_bits(rng, (B, h_q, d)), rnd_bits(rng, (B, h_kv, L, d)), rnd_bits(rng, (B, h_kv, L, d))
    say("attn scale 0.3, lengths clamped")
    got = run(q, k, v, np.array([150, -5, 10_000], np.int32), scale=0.3)
    ref = oracle.attn_decode(q, k, v, np.array([150, 0, 150], np.int32), scale=0.3)
    assert not got[1].any()
    for b in (0, 2):
        assert_close_scaled(got[b], ref[b], 2e-2, what=f"sequence {b}")


def test_attn_empty_batch_and_zero_capacity():
    need_gpu()
    q = torch.zeros(0, 8, 64, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(0, 2, 16, 64, dtype=torch.bfloat16, device="cuda")
    out = moe.moe_attn_decode(q, kv, kv, torch.zeros(0, dtype=torch.int32, device="cuda"))
    assert out.shape == (0, 8, 64)
    q = torch.ones(2, 8, 64, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(2, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    out = moe.moe_attn_decode(q, kv, kv, torch.zeros(2, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert not out.any()


@pytest.mark.parametrize("name", ["attn_qwen3_30b_b32_ragged", "attn_mixtral8x7b_b16_l16384",
                                  "attn_qwen2_57b_b16_l16384", "attn_qwen3_30b_b1_l32768"])
def test_attn_full_size_sampled_sequences(name):
    """The whole batch on the GPU, at the size the benchmark times; the oracle
    recomputes every output of a few sequences."""
    need_gpu()
    wl = workloads.ATTN_WORKLOADS[name]
    say(f"attn full size {name}")
    q = workloads.gen_attn_q(wl)
    lens = workloads.gen_attn_lens(wl)
    k, v = workloads.gen_attn_kv(wl, "cuda")
    out = moe.moe_attn_decode(q.cuda(), k, v, lens.cuda())
    torch.cuda.synchronize()
    got = workloads.bf16_bits(out)
    rows = sorted({0, wl.B - 1, wl.B // 2})
    ref = oracle.attn_decode(workloads.bf16_bits(q[rows]), workloads.bf16_bits(k[rows]),
                             workloads.bf16_bits(v[rows]), lens[rows].numpy())
    for i, b in enumerate(rows):
        assert_close_scaled(got[b], ref[i], 2e-2, what=f"{name} sequence {b}")
    del k, v, out
    torch.cuda.empty_cache()
