"""Seeded synthetic workloads for the routed-expert MoE FFN.

This module only draws inputs: token activations, router logits and expert
weights at the expert shapes of the models the HiNa-MoE paper measures
(arXiv 2610.05123, §7.3 and Table 3), plus the INT8 group quantisation of
those weights that the INT8 variant takes as input (§8.1).  It holds none of
the FFN's arithmetic (no routing, gathering, projection or combine); both the
CPU oracle and the HIP library receive what it returns.

Recipe (all draws are seeded; BF16 values are float32 draws rounded to
nearest-even by torch's dtype cast):
  * x [T,H] ~ N(0,1) in BF16, drawn on the CPU.
  * router logits [T,E] ~ N(0,1) float32, drawn on the CPU, then shaped by
    the routing recipe:
      - "uniform": used as drawn;
      - "forced" : token t may only pick experts 2t mod E and 2t+1 mod E (all
        other logits set to -inf), so with E = 8 and top-2 every expert gets
        exactly T/4 tokens;
      - "zipf"   : ln p_e is added to every logit, p_e proportional to
        r_e^-s, r a seeded permutation of 1..E (skewed expert popularity).
  * expert weights ~ N(0, 0.02): W_gate, W_up [E][I][H] and W_down [E][H][I],
    row-major BF16, drawn expert by expert on the device that will hold them
    (one seeded torch generator per (tensor, expert)).
  * INT8 weights: the float32 draws above, quantised symmetrically per group
    of 128 consecutive K elements of a row: s = max|w| / 127 (float32),
    q = clamp(round_half_even(w / s), -127, 127); an all-zero group gets
    s = 0 and q = 0.
  * INT4 weights: the same with s = max|w| / 7 and q in [-7, 7], stored two
    per byte as offset-binary nibbles (q + 8): K element 2i in the low
    nibble of byte i, element 2i + 1 in the high nibble (a storage layout
    only; the arithmetic is the INT8 variant's, on values of q in [-7, 7]).
"""
from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np
import torch

TAG_X, TAG_LOGITS, TAG_WG, TAG_WU, TAG_WD, TAG_ZIPF = range(6)
TAG_Q, TAG_K, TAG_V, TAG_LENS = range(6, 10)
TAG_CRIT = 10
WEIGHT_STD = 0.02


@dataclass(frozen=True)
class Workload:
    """One MoE FFN layer invocation: shapes, routing recipe and seed."""
    name: str
    H: int           # hidden size (model dimension)
    I: int           # expert intermediate size
    E: int           # number of routed experts
    k: int           # experts per token (top-k)
    T: int           # tokens in the decode batch
    routing: str = "uniform"   # "uniform" | "forced" | "zipf"
    zipf_s: float = 0.0
    int8: bool = False
    int4: bool = False
    resplit: bool = False      # residual-split INT4 gate/up, INT4 / INT8 down copies
    group: int = 128
    seed: int = 0

    def with_tokens(self, T: int) -> "Workload":
        return replace(self, T=T, name=f"{self.name.split('@')[0]}@T{T}")


def _registry() -> Dict[str, Workload]:
    w = {}
    w["tiny"] = Workload("tiny", H=256, I=512, E=8, k=2, T=16)
    for m in (1, 2, 4, 8, 16):
        w[f"mixtral8x7b_m{m}"] = Workload(f"mixtral8x7b_m{m}", H=4096, I=14336,
                                          E=8, k=2, T=4 * m, routing="forced")
        w[f"mixtral8x7b_int8_m{m}"] = Workload(f"mixtral8x7b_int8_m{m}", H=4096,
                                               I=14336, E=8, k=2, T=4 * m,
                                               routing="forced", int8=True)
        w[f"mixtral8x7b_int4_m{m}"] = Workload(f"mixtral8x7b_int4_m{m}", H=4096,
                                               I=14336, E=8, k=2, T=4 * m,
                                               routing="forced", int4=True)
        w[f"mixtral8x7b_resplit_m{m}"] = Workload(f"mixtral8x7b_resplit_m{m}", H=4096,
                                                  I=14336, E=8, k=2, T=4 * m,
                                                  routing="forced", resplit=True)
    w["deepseekv3_t16"] = Workload("deepseekv3_t16", H=7168, I=2048, E=256, k=8, T=16)
    w["deepseekv3_zipf_t16"] = Workload("deepseekv3_zipf_t16", H=7168, I=2048,
                                        E=256, k=8, T=16, routing="zipf", zipf_s=1.1)
    for T in (1, 4, 16):
        w[f"mixtral8x22b_t{T}"] = Workload(f"mixtral8x22b_t{T}", H=6144, I=16384,
                                           E=8, k=2, T=T)
        w[f"qwen3_235b_t{T}"] = Workload(f"qwen3_235b_t{T}", H=4096, I=1536,
                                         E=128, k=8, T=T)
    # the largest decode batch of the small-m product at the Mixtral-8x7B
    # shape with N(0,1) router logits: about 16 tokens per expert, some 17-32
    w["mixtral8x7b_t64"] = Workload("mixtral8x7b_t64", H=4096, I=14336, E=8, k=2, T=64)
    # prefill-sized batches (many tokens per expert) at the same expert shapes
    for T in (512, 2048):
        w[f"mixtral8x7b_t{T}"] = Workload(f"mixtral8x7b_t{T}", H=4096, I=14336,
                                          E=8, k=2, T=T)
    w["qwen3_235b_t2048"] = Workload("qwen3_235b_t2048", H=4096, I=1536, E=128, k=8, T=2048)
    w["deepseekv3_t4096"] = Workload("deepseekv3_t4096", H=7168, I=2048, E=256, k=8, T=4096)
    return w


WORKLOADS: Dict[str, Workload] = _registry()


def seed_for(seed: int, tag: int, index: int = 0) -> int:
    """Independent 63-bit seed for (workload seed, tensor tag, index)."""
    st = np.random.SeedSequence([seed, tag, index]).generate_state(1, np.uint64)[0]
    return int(st) & ((1 << 63) - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def gen_x(wl: Workload) -> torch.Tensor:
    """Token activations [T, H], BF16, CPU."""
    g = _gen("cpu", seed_for(wl.seed, TAG_X))
    return torch.randn(wl.T, wl.H, generator=g, dtype=torch.float32).to(torch.bfloat16)


def gen_logits(wl: Workload) -> torch.Tensor:
    """Router logits [T, E], float32, CPU, shaped by the routing recipe."""
    g = _gen("cpu", seed_for(wl.seed, TAG_LOGITS))
    lg = torch.randn(wl.T, wl.E, generator=g, dtype=torch.float32)
    if wl.routing == "uniform":
        return lg
    if wl.routing == "forced":
        allowed = torch.zeros(wl.T, wl.E, dtype=torch.bool)
        t = torch.arange(wl.T)
        allowed[t, (2 * t) % wl.E] = True
        allowed[t, (2 * t + 1) % wl.E] = True
        return torch.where(allowed, lg, torch.full_like(lg, float("-inf")))
    if wl.routing == "zipf":
        rng = np.random.default_rng(seed_for(wl.seed, TAG_ZIPF))
        rank = rng.permutation(wl.E) + 1
        p = rank.astype(np.float64) ** (-wl.zipf_s)
        logp = np.log(p / p.sum())
        return (lg.double() + torch.from_numpy(logp)[None, :]).float()
    raise ValueError(f"unknown routing recipe {wl.routing!r}")


def _draw(wl: Workload, tag: int, e: int, N: int, K: int, device) -> torch.Tensor:
    g = _gen(device, seed_for(wl.seed, tag, e))
    return torch.randn(N, K, generator=g, device=device, dtype=torch.float32) * WEIGHT_STD


def gen_weights(wl: Workload, device="cpu", experts: Optional[list] = None):
    """BF16 expert weights (W_gate [E,I,H], W_up [E,I,H], W_down [E,H,I]).

    ``experts`` limits the draw to those experts (the others stay zero); by
    default every expert is drawn.
    """
    ex = range(wl.E) if experts is None else experts
    Wg = torch.zeros(wl.E, wl.I, wl.H, dtype=torch.bfloat16, device=device)
    Wu = torch.zeros(wl.E, wl.I, wl.H, dtype=torch.bfloat16, device=device)
    Wd = torch.zeros(wl.E, wl.H, wl.I, dtype=torch.bfloat16, device=device)
    for e in ex:
        Wg[e] = _draw(wl, TAG_WG, e, wl.I, wl.H, device).to(torch.bfloat16)
        Wu[e] = _draw(wl, TAG_WU, e, wl.I, wl.H, device).to(torch.bfloat16)
        Wd[e] = _draw(wl, TAG_WD, e, wl.H, wl.I, device).to(torch.bfloat16)
    return Wg, Wu, Wd


def quantize_groupwise(w: torch.Tensor, group: int = 128, qmax: int = 127):
    """Symmetric per-group quantisation along the last dim of ``w`` to
    integers in [-qmax, qmax] (127: INT8, 7: INT4).

    Returns (q int8 with w's shape, s float32 of shape [..., K/group]).
    """
    *lead, K = w.shape
    assert K % group == 0
    wg = w.float().reshape(*lead, K // group, group)
    s = wg.abs().amax(dim=-1) / float(qmax)
    safe = torch.where(s > 0, s, torch.ones_like(s))
    q = torch.round(wg / safe[..., None]).clamp_(-qmax, qmax)
    q = torch.where((s > 0)[..., None], q, torch.zeros_like(q))
    return q.to(torch.int8).reshape(*lead, K), s.contiguous()


def gen_weights_int8(wl: Workload, device="cpu", experts: Optional[list] = None):
    """INT8 expert weights with per-group scales:
    (Qg [E,I,H], Sg [E,I,H/g], Qu, Su, Qd [E,H,I], Sd [E,H,I/g])."""
    ex = range(wl.E) if experts is None else experts
    gsz = wl.group
    Qg = torch.zeros(wl.E, wl.I, wl.H, dtype=torch.int8, device=device)
    Qu = torch.zeros(wl.E, wl.I, wl.H, dtype=torch.int8, device=device)
    Qd = torch.zeros(wl.E, wl.H, wl.I, dtype=torch.int8, device=device)
    Sg = torch.zeros(wl.E, wl.I, wl.H // gsz, dtype=torch.float32, device=device)
    Su = torch.zeros(wl.E, wl.I, wl.H // gsz, dtype=torch.float32, device=device)
    Sd = torch.zeros(wl.E, wl.H, wl.I // gsz, dtype=torch.float32, device=device)
    for e in ex:
        Qg[e], Sg[e] = quantize_groupwise(_draw(wl, TAG_WG, e, wl.I, wl.H, device), gsz)
        Qu[e], Su[e] = quantize_groupwise(_draw(wl, TAG_WU, e, wl.I, wl.H, device), gsz)
        Qd[e], Sd[e] = quantize_groupwise(_draw(wl, TAG_WD, e, wl.H, wl.I, device), gsz)
    return Qg, Sg, Qu, Su, Qd, Sd


def pack_int4(q: torch.Tensor) -> torch.Tensor:
    """INT4 values (int8 tensor in [-8, 7], last dim even) -> uint8 with two
    offset-binary nibbles per byte: element 2i in the low nibble, 2i + 1 in
    the high one.  A storage layout only."""
    u = (q.to(torch.int16) + 8).to(torch.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).contiguous()


def unpack_int4(p: torch.Tensor) -> torch.Tensor:
    """Inverse of pack_int4: uint8 [..., K/2] -> int8 [..., K] in [-8, 7]."""
    lo = (p & 0xF).to(torch.int16) - 8
    hi = (p >> 4).to(torch.int16) - 8
    return torch.stack([lo, hi], dim=-1).reshape(*p.shape[:-1], 2 * p.shape[-1]).to(torch.int8)


def gen_weights_int4(wl: Workload, device="cpu", experts: Optional[list] = None):
    """INT4 expert weights with per-group scales, unpacked (as int8 values in
    [-7, 7], the oracle's input): (Qg, Sg, Qu, Su, Qd, Sd) shaped like
    gen_weights_int8's.  pack_int4 gives the stored form."""
    ex = range(wl.E) if experts is None else experts
    gsz = wl.group
    Qg = torch.zeros(wl.E, wl.I, wl.H, dtype=torch.int8, device=device)
    Qu = torch.zeros(wl.E, wl.I, wl.H, dtype=torch.int8, device=device)
    Qd = torch.zeros(wl.E, wl.H, wl.I, dtype=torch.int8, device=device)
    Sg = torch.zeros(wl.E, wl.I, wl.H // gsz, dtype=torch.float32, device=device)
    Su = torch.zeros(wl.E, wl.I, wl.H // gsz, dtype=torch.float32, device=device)
    Sd = torch.zeros(wl.E, wl.H, wl.I // gsz, dtype=torch.float32, device=device)
    for e in ex:
        Qg[e], Sg[e] = quantize_groupwise(_draw(wl, TAG_WG, e, wl.I, wl.H, device), gsz, 7)
        Qu[e], Su[e] = quantize_groupwise(_draw(wl, TAG_WU, e, wl.I, wl.H, device), gsz, 7)
        Qd[e], Sd[e] = quantize_groupwise(_draw(wl, TAG_WD, e, wl.H, wl.I, device), gsz, 7)
    return Qg, Sg, Qu, Su, Qd, Sd


def quantize_residual_split(w: torch.Tensor, group: int = 128, qmax: int = 7):
    """Two-stage group-wise quantisation: q, s = quantize(w); the residual
    w - q*s (FP32) quantised the same way gives r, sr.  Returns (q, s, r, sr);
    q*s + r*sr is the high-precision weight, q*s the low-precision one."""
    q, s = quantize_groupwise(w, group, qmax)
    *lead, K = w.shape
    deq = (q.float().reshape(*lead, K // group, group) * s[..., None]).reshape(*lead, K)
    r, sr = quantize_groupwise(w.float() - deq, group, qmax)
    return q, s, r, sr


def gen_weights_resplit(wl: Workload, device="cpu", experts: Optional[list] = None):
    """Residual-split expert weights, unpacked (int8 values):
    (Qg, Sg, Rg, SRg, Qu, Su, Ru, SRu, Qd_lo, Sd_lo, Qd_hi, Sd_hi): INT4 W^Q
    and INT4 residual W^R of gate and up, an INT4 (low) and an INT8 (high)
    copy of down, each with row-major group scales [.., N, K/group]."""
    ex = range(wl.E) if experts is None else experts
    gsz = wl.group
    z8 = lambda N, K: torch.zeros(wl.E, N, K, dtype=torch.int8, device=device)  # noqa: E731
    zs = lambda N, K: torch.zeros(wl.E, N, K // gsz, dtype=torch.float32, device=device)  # noqa: E731
    out = [z8(wl.I, wl.H), zs(wl.I, wl.H), z8(wl.I, wl.H), zs(wl.I, wl.H),
           z8(wl.I, wl.H), zs(wl.I, wl.H), z8(wl.I, wl.H), zs(wl.I, wl.H),
           z8(wl.H, wl.I), zs(wl.H, wl.I), z8(wl.H, wl.I), zs(wl.H, wl.I)]
    for e in ex:
        for base, tag in ((0, TAG_WG), (4, TAG_WU)):
            q, s_, r, sr = quantize_residual_split(_draw(wl, tag, e, wl.I, wl.H, device), gsz, 7)
            out[base][e], out[base + 1][e], out[base + 2][e], out[base + 3][e] = q, s_, r, sr
        wd = _draw(wl, TAG_WD, e, wl.H, wl.I, device)
        out[8][e], out[9][e] = quantize_groupwise(wd, gsz, 7)
        out[10][e], out[11][e] = quantize_groupwise(wd, gsz, 127)
    return tuple(out)


def gen_critical(wl: Workload, frac: float = 0.5) -> np.ndarray:
    """Seeded per-expert precision flags: about ``frac`` of the experts
    critical (1), the rest 0."""
    rng = np.random.default_rng([wl.seed, TAG_CRIT])
    return (rng.random(wl.E) < frac).astype(np.uint8)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """BF16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_bf16(a: np.ndarray) -> torch.Tensor:
    """numpy uint16 bit patterns -> BF16 CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def weight_bytes_per_expert(wl: Workload, critical: bool = True) -> int:
    """Bytes of one expert's three weight matrices (plus scales for INT8 and
    INT4).  Residual split: what one expert of the given precision reads
    (critical: W^Q and W^R of gate/up and the INT8 down copy; otherwise W^Q
    and the INT4 down copy)."""
    n = 3 * wl.H * wl.I
    sc = (wl.H * wl.I // wl.group) * 4
    if wl.resplit:
        if critical:
            return 2 * wl.H * wl.I + 4 * sc + wl.H * wl.I + sc
        return n // 2 + 3 * sc
    if wl.int8:
        return n + 3 * (wl.H * wl.I // wl.group) * 4
    if wl.int4:
        return n // 2 + 3 * (wl.H * wl.I // wl.group) * 4
    return 2 * n


# --------------------------------------------------------------------------
# Decode attention with grouped-query heads (HiNa-MoE §6.1): g = h_q / h_kv
# consecutive query heads read the same KV head; the KV cache holds, per sequence
# and KV head, a [max_len][d] matrix of which the first len positions are
# valid.  Head layouts of the models the pages decode with (Qwen3-30B-A3B:
# 32 query heads over 4 KV heads; Mixtral-8x7B: 32 over 8; Qwen2-57B-A14B:
# 28 over 4; head dimension 128).
#   * q [B][h_q][d], k / v [B][h_kv][max_len][d] ~ N(0,1) in BF16 (k and v
#     drawn on the device that holds them, one seeded generator per
#     (tensor, sequence)).
#   * lens: "full" (every sequence max_len long) or "ragged" (uniform in
#     [1, max_len], seeded).
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class AttnWorkload:
    name: str
    B: int           # sequences in the decode batch
    h_q: int         # query heads
    h_kv: int        # KV heads (h_q / h_kv query heads share one)
    d: int           # head dimension
    max_len: int     # KV cache capacity per sequence
    lens: str = "full"    # "full" | "ragged"
    seed: int = 0


def _attn_registry() -> Dict[str, AttnWorkload]:
    w = {}
    w["attn_tiny"] = AttnWorkload("attn_tiny", B=3, h_q=8, h_kv=2, d=64, max_len=300,
                                  lens="ragged")
    for B, L in ((1, 32768), (32, 32768)):
        w[f"attn_qwen3_30b_b{B}_l{L}"] = AttnWorkload(f"attn_qwen3_30b_b{B}_l{L}", B=B,
                                                      h_q=32, h_kv=4, d=128, max_len=L)
    w["attn_qwen3_30b_b32_ragged"] = AttnWorkload("attn_qwen3_30b_b32_ragged", B=32, h_q=32,
                                                  h_kv=4, d=128, max_len=32768,
                                                  lens="ragged")
    w["attn_mixtral8x7b_b16_l16384"] = AttnWorkload("attn_mixtral8x7b_b16_l16384", B=16,
                                                    h_q=32, h_kv=8, d=128, max_len=16384)
    w["attn_qwen2_57b_b16_l16384"] = AttnWorkload("attn_qwen2_57b_b16_l16384", B=16, h_q=28,
                                                  h_kv=4, d=128, max_len=16384)
    return w


ATTN_WORKLOADS: Dict[str, AttnWorkload] = _attn_registry()


def gen_attn_q(wl: AttnWorkload) -> torch.Tensor:
    """Query vectors [B, h_q, d], BF16, CPU."""
    g = _gen("cpu", seed_for(wl.seed, TAG_Q))
    return torch.randn(wl.B, wl.h_q, wl.d, generator=g, dtype=torch.float32).to(torch.bfloat16)


def gen_attn_lens(wl: AttnWorkload) -> torch.Tensor:
    """Valid positions per sequence [B], int32, CPU."""
    if wl.lens == "full":
        return torch.full((wl.B,), wl.max_len, dtype=torch.int32)
    if wl.lens == "ragged":
        rng = np.random.default_rng(seed_for(wl.seed, TAG_LENS))
        return torch.from_numpy(rng.integers(1, wl.max_len + 1, size=wl.B).astype(np.int32))
    raise ValueError(f"unknown length recipe {wl.lens!r}")


def gen_attn_kv(wl: AttnWorkload, device="cpu", sequences: Optional[list] = None):
    """KV cache (k, v), each [B, h_kv, max_len, d] BF16.  ``sequences`` limits
    the draw to those sequences (the others stay zero)."""
    seqs = range(wl.B) if sequences is None else sequences
    shape = (wl.B, wl.h_kv, wl.max_len, wl.d)
    k = torch.zeros(shape, dtype=torch.bfloat16, device=device)
    v = torch.zeros(shape, dtype=torch.bfloat16, device=device)
    for b in seqs:
        for t, tag in ((k, TAG_K), (v, TAG_V)):
            g = _gen(device, seed_for(wl.seed, tag, b))
            t[b] = torch.randn(shape[1:], generator=g, device=device,
                               dtype=torch.float32).to(torch.bfloat16)
    return k, v


def attn_kv_bytes(wl: AttnWorkload, lens) -> int:
    """K and V bytes the valid positions of a batch occupy."""
    return int(sum(int(n) for n in lens)) * wl.h_kv * wl.d * 2 * 2
