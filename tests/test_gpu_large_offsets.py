"""GPU parity where the gathered rows lie past element 2^32 of x (gate/up) or
of h (down).

A batch of 2^20 + 32 tokens, top-1 over two experts: every token but the
last 20 goes to expert 0, which the tiled product takes; the last 20 go to
expert 1, which the small-m product takes as one wide chunk (17-32 tokens).
With hidden 4096 those 20 tokens' rows of x start past element 2^32; with
intermediate 4096 their rows of h do (h rows are in gathered order, and
expert 1's come last).  Row offsets therefore have to be formed in 64 bits.
The oracle recomputes expert 1's 20 rows and two of expert 0's.  The layer
holds about 35 GB of device memory (x, out and the FP32 per-slot rows of the
larger case).
"""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_ffn_topk_amd as moe
import workloads
from moe_cases import TOL_BF16, assert_close, need_gpu, say

pytestmark = pytest.mark.gpu

T = (1 << 20) + 32
TAIL = 20           # expert 1's tokens: one wide chunk of the small-m product
E = 2


def need_free(nbytes: int):
    free, _ = torch.cuda.mem_get_info()
    if free < nbytes:
        pytest.skip(f"needs {nbytes >> 30} GiB of free device memory, {free >> 30} free")


def bf16_weights(rng, shape, std=0.05):
    return workloads.bf16_bits(torch.from_numpy(
        (rng.standard_normal(shape) * std).astype(np.float32)).to(torch.bfloat16))


@pytest.mark.parametrize("H,I", [(4096, 32), (32, 4096)])
def test_rows_past_element_2_32(H, I):
    need_gpu()
    # x, out, the FP32 per-slot rows and h, with room to spare
    need_free(T * H * 2 * 2 + T * H * 4 + T * I * 2 + (4 << 30))
    say(f"rows past element 2^32: T={T} H={H} I={I} E={E} top-1")
    assert (T - TAIL) * max(H, I) > 1 << 32
    rng = np.random.default_rng(7)
    Wg = [bf16_weights(rng, (I, H)) for _ in range(E)]
    Wu = [bf16_weights(rng, (I, H)) for _ in range(E)]
    Wd = [bf16_weights(rng, (H, I)) for _ in range(E)]
    dev = lambda W: torch.stack([workloads.bits_to_bf16(w) for w in W]).cuda()  # noqa: E731
    ids = np.zeros((T, 1), dtype=np.int32)
    ids[T - TAIL:] = 1
    w = rng.uniform(0.5, 1.0, size=(T, 1)).astype(np.float32)

    gen = torch.Generator(device="cuda").manual_seed(11)
    x = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    step = 1 << 16
    for a in range(0, T, step):
        b = min(T, a + step)
        x[a:b] = torch.randn(b - a, H, device="cuda", generator=gen).to(torch.bfloat16)
    out = moe.moe_ffn_forward(x, torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(),
                              dev(Wg), dev(Wu), dev(Wd))
    torch.cuda.synchronize()

    rows = np.array([0, T - TAIL - 1] + list(range(T - TAIL, T)))
    idx = torch.from_numpy(rows).cuda()
    got = workloads.bf16_bits(out.index_select(0, idx).cpu())
    xb = workloads.bf16_bits(x.index_select(0, idx).cpu())
    ref = oracle.moe_ffn_bf16(xb, ids[rows], w[rows], Wg, Wu, Wd, E=E)
    assert_close(got, ref, TOL_BF16, what=f"H={H} I={I} rows {rows.tolist()}")
    del x, out
    torch.cuda.empty_cache()


def test_combine_past_2_31_outputs():
    """2^22 + 64 tokens of hidden 4096: the combine's flat index over T * H / 8
    output chunks passes 2^31 (x and out are 34 GB each, the FP32 per-slot
    rows 69 GB); the last 20 tokens again form one wide chunk of expert 1."""
    need_gpu()
    T2, H, I = (1 << 22) + 64, 4096, 32
    need_free(2 * T2 * H * 2 + T2 * H * 4 + (8 << 30))
    say(f"combine past 2^31 outputs: T={T2} H={H} I={I} E={E} top-1")
    assert T2 * (H // 8) > 1 << 31
    rng = np.random.default_rng(8)
    Wg = [bf16_weights(rng, (I, H)) for _ in range(E)]
    Wu = [bf16_weights(rng, (I, H)) for _ in range(E)]
    Wd = [bf16_weights(rng, (H, I)) for _ in range(E)]
    dev = lambda W: torch.stack([workloads.bits_to_bf16(w) for w in W]).cuda()  # noqa: E731
    ids = np.zeros((T2, 1), dtype=np.int32)
    ids[T2 - TAIL:] = 1
    w = rng.uniform(0.5, 1.0, size=(T2, 1)).astype(np.float32)
    gen = torch.Generator(device="cuda").manual_seed(12)
    x = torch.empty(T2, H, dtype=torch.bfloat16, device="cuda")
    step = 1 << 16
    for a in range(0, T2, step):
        b = min(T2, a + step)
        x[a:b] = torch.randn(b - a, H, device="cuda", generator=gen).to(torch.bfloat16)
    out = moe.moe_ffn_forward(x, torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(),
                              dev(Wg), dev(Wu), dev(Wd))
    torch.cuda.synchronize()
    rows = np.array([0, 1 << 21, (1 << 22) - 1, T2 - TAIL - 1] + list(range(T2 - TAIL, T2)))
    idx = torch.from_numpy(rows).cuda()
    got = workloads.bf16_bits(out.index_select(0, idx).cpu())
    xb = workloads.bf16_bits(x.index_select(0, idx).cpu())
    ref = oracle.moe_ffn_bf16(xb, ids[rows], w[rows], Wg, Wu, Wd, E=E)
    assert_close(got, ref, TOL_BF16, what=f"T={T2} rows {rows.tolist()}")
    del x, out
    torch.cuda.empty_cache()
