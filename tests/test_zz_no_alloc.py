"""GPU test of moe_ffn_forward_noalloc, the entry point that allocates
nothing (its workspace is a device array the library holds): on calls in a
row, the second and third smaller than the first, its output equals
moe_ffn_forward's with a caller workspace bit for bit, and the routed rows
it computes match the oracle to the BF16 bar."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import routed_expert_ffn_topk_amd as moe
import workloads
from moe_cases import TOL_BF16, assert_close, need_gpu, say

pytestmark = pytest.mark.gpu


def _random_layer(T, H, I, E, k, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    logits = torch.randn(T, E, generator=g)
    W = [(torch.randn(*shape, generator=g) * 0.02).to(torch.bfloat16)
         for shape in ((E, I, H), (E, I, H), (E, H, I))]
    ids, w = oracle.route_topk(logits.numpy(), k)
    return x, ids, w, W


def _noalloc_c(x, ids, w, W, out):
    """Call the C entry point directly (ctypes), as a caller without torch would."""
    T, H = x.shape
    E, I, _ = W[0].shape
    k = ids.shape[1]
    rc = moe.lib().moe_ffn_forward_noalloc(
        x.data_ptr(), ids.data_ptr(), w.data_ptr(), W[0].data_ptr(), W[1].data_ptr(),
        W[2].data_ptr(), out.data_ptr(), T, H, I, E, k,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == moe.MOE_FFN_OK, moe.moe_ffn_status_string(rc)


def test_noalloc_matches_forward_on_calls_in_a_row():
    need_gpu()
    cases = [("mixtral8x7b_m16", None), ("mixtral8x7b_m1", None),
             ("random T=37 H=256 I=384 E=16 k=4", (37, 256, 384, 16, 4))]
    held = None
    for name, shape in cases:
        say(f"noalloc {name}")
        if shape is None:
            wl = workloads.WORKLOADS[name]
            x = workloads.gen_x(wl)
            ids, w = oracle.route_topk(workloads.gen_logits(wl).numpy(), wl.k)
            if held is None:
                held = list(workloads.gen_weights(wl, "cuda"))
            Wd = held
        else:
            x, ids, w, W = _random_layer(*shape, seed=7)
            Wd = [t.cuda() for t in W]
        xd, idsd, wd = x.cuda(), torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
        out_c = torch.full_like(xd, float("nan"))
        _noalloc_c(xd, idsd, wd, Wd, out_c)
        ref_dev = moe.moe_ffn_forward(xd, idsd, wd, *Wd)
        torch.cuda.synchronize()
        got = workloads.bf16_bits(out_c)
        assert np.array_equal(got, workloads.bf16_bits(ref_dev)), f"{name}: differs from moe_ffn_forward"
        # oracle check on sampled rows (whole rows)
        T = x.shape[0]
        rows = np.array(sorted({0, T // 2, T - 1}))
        need = sorted(set(ids[rows].reshape(-1).tolist()))
        host = [{e: workloads.bf16_bits(t[e].cpu()) for e in need} for t in Wd]
        ref = oracle.moe_ffn_bf16(workloads.bf16_bits(x)[rows], ids[rows], w[rows],
                                  *(h.get for h in host), E=Wd[0].shape[0])
        assert_close(got[rows], ref, TOL_BF16, what=f"{name} rows {rows.tolist()}")
    # the binding reaches the same entry point
    out_b = moe.moe_ffn_forward_noalloc(xd, idsd, wd, *Wd, out=torch.empty_like(xd))
    torch.cuda.synchronize()
    assert np.array_equal(workloads.bf16_bits(out_b), got)
