"""The layer captured in a HIP graph: every replay equals the eager result bit
for bit (the forward call enqueues kernels only, with no memset or host
synchronisation, so it can be captured; the gather index and the round
split are recomputed on the device at every replay)."""
import numpy as np
import pytest
import torch

import routed_expert_ffn_topk_amd as moe
import workloads
from moe_cases import need_gpu, say

pytestmark = pytest.mark.gpu


def _replays_match(call, outs, other_call, n_replays=3):
    # the inputs were produced on the default stream; the side stream does
    # not wait for it by itself
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for r in range(n_replays):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for o, ref_o in zip(outs, ref):
            assert torch.equal(o, ref_o), f"replay {r} differs from the eager result"
        other_call()                 # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["tiny", "qwen3_235b_t4", "mixtral8x7b_m16"])
def test_bf16_layer_graph_replays_match_eager(name):
    need_gpu()
    say(f"graph replay bf16 {name}")
    wl = workloads.WORKLOADS[name]
    x = workloads.gen_x(wl).cuda()
    ids, w = moe.moe_route_topk(workloads.gen_logits(wl).cuda(), wl.k)
    W = workloads.gen_weights(wl, "cuda")
    ws = moe.alloc_workspace(wl.T, wl.H, wl.I, wl.E, wl.k)
    out = torch.empty_like(x)
    # the eager work between replays reuses the workspace with other routing
    ids2 = torch.roll(ids, 1, dims=0)

    def call():
        moe.moe_ffn_forward(x, ids, w, *W, out=out, workspace=ws,
                            stream=torch.cuda.current_stream())

    def other():
        moe.moe_ffn_forward(x, ids2, w, *W, workspace=ws)

    _replays_match(call, [out], other)
    del W
    torch.cuda.empty_cache()


def test_int8_layer_graph_replays_match_eager():
    need_gpu()
    say("graph replay int8")
    rng = np.random.default_rng(5)
    T, H, I, E, k = 16, 512, 384, 8, 2
    x = workloads.bits_to_bf16(workloads.bf16_bits(
        torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16))).cuda()
    Q = []
    for N, K in ((I, H), (I, H), (H, I)):
        q, sc = workloads.quantize_groupwise(
            torch.from_numpy((rng.standard_normal((E, N, K)) * 0.05).astype(np.float32)))
        Q += [q.cuda(), sc.cuda()]
    ids = torch.from_numpy(np.stack([rng.choice(E, size=k, replace=False)
                                     for _ in range(T)]).astype(np.int32)).cuda()
    w = torch.from_numpy(rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)).cuda()
    ws = moe.alloc_workspace(T, H, I, E, k)
    out = torch.empty_like(x)

    def call():
        moe.moe_ffn_forward_int8(x, ids, w, *Q, out=out, workspace=ws,
                                 stream=torch.cuda.current_stream())

    def other():
        moe.moe_ffn_forward_int8(x, torch.flip(ids, dims=[1]).contiguous(), w, *Q, workspace=ws)

    _replays_match(call, [out], other)


@pytest.mark.parametrize("T", [16, 300])
def test_logits_layer_graph_replays_match_eager(T):
    """Router + gather index + layer from logits (fused decode kernel at 16
    tokens; router, sort and the tiled product at 300)."""
    need_gpu()
    say(f"graph replay logits layer T={T}")
    wl = workloads.Workload("g", H=256, I=384, E=16, k=2, T=T)
    x = workloads.gen_x(wl).cuda()
    lg = workloads.gen_logits(wl).cuda()
    W = workloads.gen_weights(wl, "cuda")
    ws = moe.alloc_workspace(wl.T, wl.H, wl.I, wl.E, wl.k)
    out = torch.empty_like(x)
    ids = torch.empty(T, wl.k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.k, dtype=torch.float32, device="cuda")
    lg2 = torch.flip(lg, dims=[0]).contiguous()

    def call():
        moe.moe_ffn_forward_logits(x, lg, wl.k, *W, out=out, topk_ids=ids, topk_w=w,
                                   workspace=ws, stream=torch.cuda.current_stream())

    def other():
        moe.moe_ffn_forward_logits(x, lg2, wl.k, *W, workspace=ws)

    _replays_match(call, [out, ids, w], other)


def test_int4_layer_graph_replays_match_eager():
    need_gpu()
    say("graph replay int4")
    rng = np.random.default_rng(6)
    T, H, I, E, k = 16, 512, 384, 8, 2
    x = workloads.bits_to_bf16(workloads.bf16_bits(
        torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16))).cuda()
    P = []
    for N, K in ((I, H), (I, H), (H, I)):
        q, sc = workloads.quantize_groupwise(
            torch.from_numpy((rng.standard_normal((E, N, K)) * 0.05).astype(np.float32)), 128, 7)
        P += [workloads.pack_int4(q).cuda(), sc.cuda()]
    ids = torch.from_numpy(np.stack([rng.choice(E, size=k, replace=False)
                                     for _ in range(T)]).astype(np.int32)).cuda()
    w = torch.from_numpy(rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)).cuda()
    ws = moe.alloc_workspace(T, H, I, E, k)
    out = torch.empty_like(x)

    def call():
        moe.moe_ffn_forward_int4(x, ids, w, *P, out=out, workspace=ws,
                                 stream=torch.cuda.current_stream())

    def other():
        moe.moe_ffn_forward_int4(x, torch.flip(ids, dims=[1]).contiguous(), w, *P, workspace=ws)

    _replays_match(call, [out], other)


def test_resplit_layer_graph_replays_match_eager():
    need_gpu()
    say("graph replay residual split")
    rng = np.random.default_rng(7)
    T, H, I, E, k = 12, 384, 256, 6, 2
    x = workloads.bits_to_bf16(workloads.bf16_bits(
        torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16))).cuda()
    p4 = workloads.pack_int4
    draw = lambda N, K: torch.from_numpy(  # noqa: E731
        (rng.standard_normal((E, N, K)) * 0.05).astype(np.float32))
    P = []
    for N, K in ((I, H), (I, H)):
        q, s, r, sr = workloads.quantize_residual_split(draw(N, K), 128, 7)
        P += [p4(q).cuda(), s.cuda(), p4(r).cuda(), sr.cuda()]
    wd = draw(H, I)
    ql, sl = workloads.quantize_groupwise(wd, 128, 7)
    qh, sh = workloads.quantize_groupwise(wd, 128, 127)
    P += [p4(ql).cuda(), sl.cuda(), qh.cuda(), sh.cuda(),
          torch.tensor([1, 0, 1, 1, 0, 0], dtype=torch.uint8).cuda()]
    ids = torch.from_numpy(np.stack([rng.choice(E, size=k, replace=False)
                                     for _ in range(T)]).astype(np.int32)).cuda()
    w = torch.from_numpy(rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)).cuda()
    ws = moe.alloc_workspace(T, H, I, E, k)
    out = torch.empty_like(x)

    def call():
        moe.moe_ffn_forward_resplit(x, ids, w, *P, out=out, workspace=ws,
                                    stream=torch.cuda.current_stream())

    def other():
        moe.moe_ffn_forward_resplit(x, torch.flip(ids, dims=[1]).contiguous(), w, *P,
                                    workspace=ws)

    _replays_match(call, [out], other)


def test_attn_graph_replays_match_eager():
    need_gpu()
    say("graph replay attention")
    wl = workloads.ATTN_WORKLOADS["attn_tiny"]
    q = workloads.gen_attn_q(wl).cuda()
    lens = workloads.gen_attn_lens(wl).cuda()
    k, v = workloads.gen_attn_kv(wl, "cuda")
    ws = torch.empty(moe.moe_attn_decode_workspace_bytes(wl.B, wl.h_q, wl.h_kv, wl.d,
                                                         wl.max_len),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lens2 = torch.flip(lens, dims=[0]).contiguous()

    def call():
        moe.moe_attn_decode(q, k, v, lens, out=out, workspace=ws,
                            stream=torch.cuda.current_stream())

    def other():
        moe.moe_attn_decode(q, k, v, lens2, workspace=ws)

    _replays_match(call, [out], other)
