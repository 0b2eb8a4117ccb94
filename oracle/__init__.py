"""CPU oracle for the routed-expert MoE FFN -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``routed_expert_ffn_topk_amd``) and never imports it; both receive the same
seeded inputs from ``workloads.py``.

This module only marshals numpy arrays into the plain C routines of
``moe_oracle.c`` (routing, gather index, per-token FFN, INT8 FFN, BF16
rounding).  See the header of that file for the passages of the HiNa-MoE paper
each routine follows and for the readings taken where the paper is silent.

BF16 arrays are carried as ``numpy.uint16`` bit patterns.
"""
import ctypes
import os
from typing import Callable, Optional, Sequence, Union

import numpy as np

from . import build as _build

_LIB = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
_vpp = ctypes.POINTER(ctypes.c_void_p)


def lib() -> ctypes.CDLL:
    """Load liboracle.so, building it first only if it does not exist.

    ``ORACLE_LIB`` names another build of moe_oracle.c to load instead; the
    mutation test uses it to run the pins against oracles with planted
    mistakes.
    """
    global _LIB
    if _LIB is None:
        path = os.environ.get("ORACLE_LIB", _build.LIB)
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_set_num_threads.restype = None
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16_array.restype = None
        L.oracle_f32_to_bf16_array.argtypes = [_f32p, _u16p, ctypes.c_int64]
        L.oracle_route_topk.restype = ctypes.c_int
        L.oracle_route_topk.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_int32, _i32p, _f32p]
        L.oracle_permute.restype = ctypes.c_int64
        L.oracle_permute.argtypes = [_i32p, ctypes.c_int64, ctypes.c_int32,
                                     _i32p, _i32p, _i32p, _i32p, _i32p]
        L.oracle_expert_ffn_bf16.restype = None
        L.oracle_expert_ffn_bf16.argtypes = [_u16p, _u16p, _u16p, _u16p,
                                             ctypes.c_int64, ctypes.c_int64,
                                             _u16p, _f32p]
        L.oracle_moe_ffn_bf16.restype = ctypes.c_int
        L.oracle_moe_ffn_bf16.argtypes = [
            _u16p, _i32p, _f32p, _vpp, _vpp, _vpp, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
            _u16p, _f32p, _u16p, _f32p]
        L.oracle_attn_decode.restype = ctypes.c_int
        L.oracle_attn_decode.argtypes = [_u16p, _u16p, _u16p, _i32p, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_float, _u16p]
        L.oracle_moe_ffn_int8.restype = ctypes.c_int
        L.oracle_moe_ffn_int8.argtypes = [
            _u16p, _i32p, _f32p, _vpp, _vpp, _vpp, _vpp, _vpp, _vpp,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int32, ctypes.c_int32, _u16p, _f32p, _u16p, _f32p]
        L.oracle_route_grouped.restype = ctypes.c_int
        L.oracle_route_grouped.argtypes = [_f32p, _f32p, ctypes.c_int64, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_float, _i32p, _f32p]
        L.oracle_moe_ffn_resplit.restype = ctypes.c_int
        L.oracle_moe_ffn_resplit.argtypes = [
            _u16p, _i32p, _f32p] + [_vpp] * 12 + [
            ctypes.POINTER(ctypes.c_uint8), ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _u16p, _f32p, _u16p, _f32p]
        _LIB = L
    return _LIB


def num_threads() -> int:
    """OpenMP threads the oracle's loops use."""
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Set the OpenMP threads of the oracle's loops (results do not depend on
    it: only independent outputs are split between threads)."""
    lib().oracle_set_num_threads(int(n))


def _ptr(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _opt(a: Optional[np.ndarray], ctype):
    return None if a is None else _ptr(a, ctype)


# --------------------------------------------------------------------------
# BF16 helpers (the oracle's own rounding routine).
# --------------------------------------------------------------------------

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns to float32 (exact: append 16 zero bits)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to BF16 bit patterns, nearest-even, via the C routine."""
    src = np.ascontiguousarray(a, dtype=np.float32)
    dst = np.empty(src.shape, dtype=np.uint16)
    lib().oracle_f32_to_bf16_array(_ptr(src, ctypes.c_float),
                                   _ptr(dst, ctypes.c_uint16), src.size)
    return dst


# --------------------------------------------------------------------------
# Routing and gather index.
# --------------------------------------------------------------------------

def route_topk(logits: np.ndarray, k: int):
    """Top-k routing of ``logits`` [T, E] float32 -> (ids [T,k] int32, w [T,k] f32)."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    rc = lib().oracle_route_topk(_ptr(lg, ctypes.c_float), T, E, k,
                                 _ptr(ids, ctypes.c_int32), _ptr(w, ctypes.c_float))
    if rc != 0:
        raise ValueError(f"oracle_route_topk failed ({rc})")
    return ids, w


def route_grouped(logits: np.ndarray, k: int, n_group: int, topk_group: int,
                  bias: Optional[np.ndarray] = None, scale: float = 1.0):
    """Grouped sigmoid router (see oracle_route_grouped): logits [T, E]
    float32, optional selection bias [E] -> (ids [T, k] int32, w [T, k]
    float32)."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    rc = lib().oracle_route_grouped(_ptr(lg, ctypes.c_float), _opt(b, ctypes.c_float), T, E,
                                    n_group, topk_group, k, scale, _ptr(ids, ctypes.c_int32),
                                    _ptr(w, ctypes.c_float))
    if rc != 0:
        raise ValueError(f"oracle_route_grouped failed ({rc})")
    return ids, w


def permute(topk_ids: np.ndarray, E: int) -> dict:
    """Per-expert slot lists (stable by slot) for ids [T, k]."""
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32).reshape(-1)
    n = ids.size
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    sorted_slot = np.full(max(n, 1), -1, dtype=np.int32)
    active = np.full(E, -1, dtype=np.int32)
    n_active = ctypes.c_int32(0)
    n_invalid = lib().oracle_permute(
        _ptr(ids, ctypes.c_int32), n, E, _ptr(counts, ctypes.c_int32),
        _ptr(offsets, ctypes.c_int32), _ptr(sorted_slot, ctypes.c_int32),
        _ptr(active, ctypes.c_int32), ctypes.byref(n_active))
    na = n_active.value
    return {
        "counts": counts,
        "offsets": offsets,
        "sorted_slot": sorted_slot[: offsets[E]].copy(),
        "active": active[:na].copy(),
        "n_active": na,
        "n_invalid": int(n_invalid),
    }


# --------------------------------------------------------------------------
# The FFN layer.
# --------------------------------------------------------------------------

WeightTable = Union[Sequence[Optional[np.ndarray]], Callable[[int], np.ndarray]]


def _table(src: WeightTable, needed, E: int, dtype, keep: list):
    """Pointer table with an entry for each needed expert, NULL elsewhere."""
    arr = (ctypes.c_void_p * E)()
    for e in needed:
        a = src(e) if callable(src) else src[e]
        if a is None:
            continue
        a = np.ascontiguousarray(a, dtype=dtype)
        keep.append(a)
        arr[e] = a.ctypes.data
    return arr


def _needed(ids: np.ndarray, E: int):
    v = ids.reshape(-1)
    return sorted(set(int(e) for e in v if 0 <= e < E))


def moe_ffn_bf16(x: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray,
                 W_gate: WeightTable, W_up: WeightTable, W_down: WeightTable,
                 E: int, aux: bool = False):
    """Routed-expert FFN layer, BF16 weights.

    x [T,H] uint16 (bf16 bits); ids [T,k] int32; w [T,k] float32;
    W_gate/W_up: per-expert [I,H] uint16; W_down: per-expert [H,I] uint16,
    given as a sequence indexed by expert or a callable e -> array (called only
    for experts that a valid slot names).  Returns out [T,H] uint16, or with
    ``aux`` a dict that also holds out_f32 [T,H], h [T*k,I] uint16 and
    y [T*k,H] float32.
    """
    x = np.ascontiguousarray(x, dtype=np.uint16)
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    T, H = x.shape
    k = ids.shape[1] if ids.ndim == 2 else 1
    keep: list = []
    need = _needed(ids, E)
    tg = _table(W_gate, need, E, np.uint16, keep)
    tu = _table(W_up, need, E, np.uint16, keep)
    td = _table(W_down, need, E, np.uint16, keep)
    if need:
        I = keep[0].shape[0]
    elif not callable(W_gate) and len(W_gate) and W_gate[0] is not None:
        I = np.asarray(W_gate[0]).shape[0]
    else:
        I = 1
    out = np.empty((T, H), dtype=np.uint16)
    out_f32 = np.empty((T, H), dtype=np.float32) if aux else None
    h = np.empty((T * k, I), dtype=np.uint16) if aux else None
    y = np.empty((T * k, H), dtype=np.float32) if aux else None
    rc = lib().oracle_moe_ffn_bf16(
        _ptr(x, ctypes.c_uint16), _ptr(ids, ctypes.c_int32), _ptr(w, ctypes.c_float),
        ctypes.cast(tg, _vpp), ctypes.cast(tu, _vpp), ctypes.cast(td, _vpp),
        T, H, I, E, k, _ptr(out, ctypes.c_uint16), _opt(out_f32, ctypes.c_float),
        _opt(h, ctypes.c_uint16), _opt(y, ctypes.c_float))
    if rc != 0:
        raise ValueError(f"oracle_moe_ffn_bf16 failed ({rc})")
    if aux:
        return {"out": out, "out_f32": out_f32, "h": h, "y": y}
    return out


def moe_ffn_int8(x: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray,
                 Q_gate: WeightTable, S_gate: WeightTable, Q_up: WeightTable,
                 S_up: WeightTable, Q_down: WeightTable, S_down: WeightTable,
                 E: int, group: int = 128, aux: bool = False):
    """Routed-expert FFN layer, INT8 weights with one FP32 scale per group.

    Q_gate/Q_up: per-expert [I,H] int8 with S_gate/S_up [I,H/group] float32;
    Q_down: per-expert [H,I] int8 with S_down [H,I/group] float32.
    """
    x = np.ascontiguousarray(x, dtype=np.uint16)
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    T, H = x.shape
    k = ids.shape[1]
    keep: list = []
    need = _needed(ids, E)
    qg = _table(Q_gate, need, E, np.int8, keep)
    I = keep[0].shape[0] if need else 1
    sg = _table(S_gate, need, E, np.float32, keep)
    qu = _table(Q_up, need, E, np.int8, keep)
    su = _table(S_up, need, E, np.float32, keep)
    qd = _table(Q_down, need, E, np.int8, keep)
    sd = _table(S_down, need, E, np.float32, keep)
    out = np.empty((T, H), dtype=np.uint16)
    out_f32 = np.empty((T, H), dtype=np.float32) if aux else None
    h = np.empty((T * k, I), dtype=np.uint16) if aux else None
    y = np.empty((T * k, H), dtype=np.float32) if aux else None
    c = lambda t: ctypes.cast(t, _vpp)  # noqa: E731
    rc = lib().oracle_moe_ffn_int8(
        _ptr(x, ctypes.c_uint16), _ptr(ids, ctypes.c_int32), _ptr(w, ctypes.c_float),
        c(qg), c(sg), c(qu), c(su), c(qd), c(sd), group, T, H, I, E, k,
        _ptr(out, ctypes.c_uint16), _opt(out_f32, ctypes.c_float),
        _opt(h, ctypes.c_uint16), _opt(y, ctypes.c_float))
    if rc != 0:
        raise ValueError(f"oracle_moe_ffn_int8 failed ({rc})")
    if aux:
        return {"out": out, "out_f32": out_f32, "h": h, "y": y}
    return out


def moe_ffn_resplit(x: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray,
                    Q_gate: WeightTable, S_gate: WeightTable, R_gate: WeightTable,
                    SR_gate: WeightTable, Q_up: WeightTable, S_up: WeightTable,
                    R_up: WeightTable, SR_up: WeightTable, Q_down_lo: WeightTable,
                    S_down_lo: WeightTable, Q_down_hi: WeightTable, S_down_hi: WeightTable,
                    critical: np.ndarray, E: int, group: int = 128, aux: bool = False):
    """Routed-expert FFN layer with residual-split low-bit weights.

    Q_* / R_*: per-expert int8 arrays of the quantised weight and of the
    quantised residual ([I,H] for gate/up), S_* / SR_* their group scales
    ([I,H/group] float32); Q_down_lo / Q_down_hi: the low- and
    high-precision copies of down ([H,I]) with their scales; critical [E]:
    nonzero for the experts that run in high precision.  Only the tables a
    valid slot needs are read (a callable table is called for those alone).
    """
    x = np.ascontiguousarray(x, dtype=np.uint16)
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    crit = np.ascontiguousarray(critical, dtype=np.uint8)
    assert crit.shape == (E,)
    T, H = x.shape
    k = ids.shape[1]
    keep: list = []
    need = _needed(ids, E)
    hi = [e for e in need if crit[e]]
    lo = [e for e in need if not crit[e]]
    qg = _table(Q_gate, need, E, np.int8, keep)
    I = keep[0].shape[0] if need else 1
    tabs = [qg, _table(S_gate, need, E, np.float32, keep),
            _table(R_gate, hi, E, np.int8, keep), _table(SR_gate, hi, E, np.float32, keep),
            _table(Q_up, need, E, np.int8, keep), _table(S_up, need, E, np.float32, keep),
            _table(R_up, hi, E, np.int8, keep), _table(SR_up, hi, E, np.float32, keep),
            _table(Q_down_lo, lo, E, np.int8, keep), _table(S_down_lo, lo, E, np.float32, keep),
            _table(Q_down_hi, hi, E, np.int8, keep), _table(S_down_hi, hi, E, np.float32, keep)]
    out = np.empty((T, H), dtype=np.uint16)
    out_f32 = np.empty((T, H), dtype=np.float32) if aux else None
    h = np.empty((T * k, I), dtype=np.uint16) if aux else None
    y = np.empty((T * k, H), dtype=np.float32) if aux else None
    rc = lib().oracle_moe_ffn_resplit(
        _ptr(x, ctypes.c_uint16), _ptr(ids, ctypes.c_int32), _ptr(w, ctypes.c_float),
        *[ctypes.cast(t, _vpp) for t in tabs], _ptr(crit, ctypes.c_uint8), group, T, H, I, E,
        k, _ptr(out, ctypes.c_uint16), _opt(out_f32, ctypes.c_float),
        _opt(h, ctypes.c_uint16), _opt(y, ctypes.c_float))
    if rc != 0:
        raise ValueError(f"oracle_moe_ffn_resplit failed ({rc})")
    if aux:
        return {"out": out, "out_f32": out_f32, "h": h, "y": y}
    return out


def expert_ffn_bf16(x_row: np.ndarray, Wg: np.ndarray, Wu: np.ndarray,
                    Wd: np.ndarray):
    """One expert on one token: returns (h [I] uint16, y [H] float32)."""
    x_row = np.ascontiguousarray(x_row, dtype=np.uint16)
    Wg = np.ascontiguousarray(Wg, dtype=np.uint16)
    Wu = np.ascontiguousarray(Wu, dtype=np.uint16)
    Wd = np.ascontiguousarray(Wd, dtype=np.uint16)
    I, H = Wg.shape
    h = np.empty(I, dtype=np.uint16)
    y = np.empty(H, dtype=np.float32)
    lib().oracle_expert_ffn_bf16(_ptr(x_row, ctypes.c_uint16), _ptr(Wg, ctypes.c_uint16),
                                 _ptr(Wu, ctypes.c_uint16), _ptr(Wd, ctypes.c_uint16),
                                 H, I, _ptr(h, ctypes.c_uint16), _ptr(y, ctypes.c_float))
    return h, y


# --------------------------------------------------------------------------
# Decode attention with grouped-query heads.
# --------------------------------------------------------------------------

def attn_decode(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                lens: np.ndarray, scale: Optional[float] = None) -> np.ndarray:
    """Decode SDPA: q [B, h_q, d], k / v [B, h_kv, max_len, d] (BF16 bits),
    lens [B] int32 -> out [B, h_q, d] BF16 bits.  ``scale`` defaults to
    1/sqrt(d)."""
    qb = np.ascontiguousarray(q_bits, dtype=np.uint16)
    kb = np.ascontiguousarray(k_bits, dtype=np.uint16)
    vb = np.ascontiguousarray(v_bits, dtype=np.uint16)
    ln = np.ascontiguousarray(lens, dtype=np.int32)
    B, h_q, d = qb.shape
    _, h_kv, max_len, d2 = kb.shape
    assert d2 == d and vb.shape == kb.shape and ln.shape == (B,)
    if scale is None:
        scale = float(np.float32(1.0) / np.sqrt(np.float32(d)))
    out = np.empty((B, h_q, d), dtype=np.uint16)
    rc = lib().oracle_attn_decode(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16),
                                  _ptr(vb, ctypes.c_uint16), _ptr(ln, ctypes.c_int32), B, h_q,
                                  h_kv, d, max_len, scale, _ptr(out, ctypes.c_uint16))
    if rc != 0:
        raise ValueError(f"oracle_attn_decode failed ({rc})")
    return out
