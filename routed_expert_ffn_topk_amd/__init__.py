"""MI355X-native routed-expert MoE FFN: ctypes binding over libmoe_ffn.so.

The library (HIP kernels for gfx950 behind the C ABI in ``include/moe_ffn.h``)
implements the routed-expert feed-forward layer of MoE decoding from the
HiNa-MoE paper (arXiv 2610.05123, §4.1 FFN equation; §2.1 routing; §8.1 INT8
variant).  This module only marshals torch tensors (device memory) and the
current HIP stream into those C calls, with the same names; every step of
the computation runs in the library's kernels.  There is no fallback: if
``libmoe_ffn.so`` is missing, loading fails with an error.
"""
import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_FFN_DEBUG=1 loads the debug build, whose kernels check their indices
# (moe_ffn_device_check)
LIB_PATH = os.path.join(_HERE, "libmoe_ffn_debug.so" if os.environ.get("MOE_FFN_DEBUG", "0") not in
                        ("", "0") else "libmoe_ffn.so")

MOE_FFN_OK = 0
MOE_FFN_ERR_NULL_ARG = -1
MOE_FFN_ERR_BAD_SHAPE = -2
MOE_FFN_ERR_MISALIGNED = -3
MOE_FFN_ERR_ALIAS = -4
MOE_FFN_ERR_WORKSPACE = -5
MOE_FFN_ERR_HIP = -6
MOE_FFN_ERR_BAD_IDS = -7
MOE_FFN_MAX_EXPERTS = 1024
MOE_FFN_INT8_GROUP = 128
MOE_FFN_NOALLOC_WORKSPACE_BYTES = 32 << 20

LAYOUT_FIELDS = ("total_bytes", "meta", "counts", "offsets", "active", "large", "sorted_slot",
                 "h", "y", "y_parts")


class MoeFfnError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {moe_ffn_status_string(code)} ({code})")


class _Layout(ctypes.Structure):
    _fields_ = [(f, ctypes.c_size_t) for f in LAYOUT_FIELDS]


_lib = None
_c = ctypes
_i64, _i32, _vp, _sz = _c.c_int64, _c.c_int32, _c.c_void_p, _c.c_size_t


def lib() -> ctypes.CDLL:
    """Load libmoe_ffn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "routed_expert_ffn_topk_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_ffn_workspace_layout.restype = _c.c_int
        L.moe_ffn_workspace_layout.argtypes = [_i64, _i64, _i64, _i32, _i32, _c.POINTER(_Layout)]
        L.moe_ffn_workspace_bytes.restype = _sz
        L.moe_ffn_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32, _i32]
        L.moe_route_topk.restype = _c.c_int
        L.moe_route_topk.argtypes = [_vp, _i64, _i32, _i32, _vp, _vp, _vp]
        L.moe_ffn_forward.restype = _c.c_int
        L.moe_ffn_forward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                      _i32, _i32, _vp, _sz, _vp]
        L.moe_ffn_forward_noalloc.restype = _c.c_int
        L.moe_ffn_forward_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                              _i32, _i32, _vp]
        L.moe_ffn_forward_logits.restype = _c.c_int
        L.moe_ffn_forward_logits.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64,
                                             _i64, _i32, _i32, _vp, _sz, _vp]
        L.moe_ffn_forward_int4.restype = _c.c_int
        L.moe_ffn_forward_int4.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                           _vp, _i64, _i64, _i64, _i32, _i32, _vp, _sz, _vp]
        L.moe_route_grouped.restype = _c.c_int
        L.moe_route_grouped.argtypes = [_vp, _vp, _i64, _i32, _i32, _i32, _i32, _c.c_float, _vp,
                                        _vp, _vp]
        L.moe_ffn_forward_resplit.restype = _c.c_int
        L.moe_ffn_forward_resplit.argtypes = [_vp] * 16 + [_i32, _vp, _i64, _i64, _i64, _i32,
                                                           _i32, _vp, _sz, _vp]
        L.moe_attn_decode.restype = _c.c_int
        L.moe_attn_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                      _c.c_float, _vp, _sz, _vp]
        L.moe_attn_decode_workspace_bytes.restype = _sz
        L.moe_attn_decode_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32]
        L.moe_ffn_forward_int8.restype = _c.c_int
        L.moe_ffn_forward_int8.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                           _vp, _i64, _i64, _i64, _i32, _i32, _vp, _sz, _vp]
        L.moe_ffn_check_status.restype = _c.c_int
        L.moe_ffn_check_status.argtypes = [_vp, _vp, _c.POINTER(_i64)]
        L.moe_ffn_device_check.restype = _c.c_int
        L.moe_ffn_device_check.argtypes = [_c.POINTER(_i32)]
        L.moe_ffn_status_string.restype = _c.c_char_p
        L.moe_ffn_status_string.argtypes = [_c.c_int]
        L.moe_ffn_set_stage_events.restype = _c.c_int
        L.moe_ffn_set_stage_events.argtypes = [_c.POINTER(_vp), _i32]
        L.moe_ffn_set_split.restype = _c.c_int
        L.moe_ffn_set_split.argtypes = [_i32, _i32]
        L.moe_ffn_launch_probe.restype = _c.c_int
        L.moe_ffn_launch_probe.argtypes = [_i32, _vp]
        L.moe_ffn_read_probe.restype = _c.c_int
        L.moe_ffn_read_probe.argtypes = [_vp, _sz, _vp, _vp]
        _lib = L
    return _lib


def moe_ffn_status_string(code: int) -> str:
    return lib().moe_ffn_status_string(code).decode()


def _check(fn: str, code: int):
    if code != MOE_FFN_OK:
        raise MoeFfnError(fn, code)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str, dtype) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a device (cuda) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _check_shape(name: str, t: torch.Tensor, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")


def _layer_args(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                out: Optional[torch.Tensor]) -> Tuple[int, int, int]:
    """Sizes (T, H, top_k) of a layer call, after checking that x is [T, H],
    topk_ids and topk_w are [T, top_k] and out (if given) is [T, H]: the
    kernels index these tensors by those sizes."""
    if x.dim() != 2:
        raise ValueError(f"x must be [T, H], got {list(x.shape)}")
    T, H = x.shape
    if topk_ids.dim() != 2 or topk_ids.shape[0] != T:
        raise ValueError(f"topk_ids must be [T, top_k] with T = {T}, got {list(topk_ids.shape)}")
    top_k = topk_ids.shape[1]
    _check_shape("topk_w", topk_w, (T, top_k))
    if out is not None:
        _check_shape("out", out, (T, H))
    return T, H, top_k


def moe_ffn_workspace_layout(T: int, H: int, I: int, E: int, top_k: int) -> dict:
    L = _Layout()
    _check("moe_ffn_workspace_layout", lib().moe_ffn_workspace_layout(T, H, I, E, top_k, _c.byref(L)))
    return {f: int(getattr(L, f)) for f in LAYOUT_FIELDS}


def moe_ffn_workspace_bytes(T: int, H: int, I: int, E: int, top_k: int) -> int:
    return int(lib().moe_ffn_workspace_bytes(T, H, I, E, top_k))


def alloc_workspace(T: int, H: int, I: int, E: int, top_k: int, device=None) -> torch.Tensor:
    """Device byte buffer large enough for one forward call of these sizes."""
    n = moe_ffn_workspace_bytes(T, H, I, E, top_k)
    if n == 0:
        raise MoeFfnError("moe_ffn_workspace_bytes", MOE_FFN_ERR_BAD_SHAPE)
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def moe_route_topk(logits: torch.Tensor, top_k: int, topk_ids: Optional[torch.Tensor] = None,
                   topk_w: Optional[torch.Tensor] = None, stream=None
                   ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Top-k router on ``logits`` [T, E] float32 -> (ids [T,k] int32, w [T,k] float32)."""
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty(T, top_k, dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty(T, top_k, dtype=torch.float32, device=logits.device)
    _check_shape("topk_ids", topk_ids, (T, top_k))
    _check_shape("topk_w", topk_w, (T, top_k))
    _check("moe_route_topk", lib().moe_route_topk(
        _dev(logits, "logits", torch.float32), T, E, top_k,
        _dev(topk_ids, "topk_ids", torch.int32), _dev(topk_w, "topk_w", torch.float32),
        _stream(stream)))
    return topk_ids, topk_w


def moe_ffn_forward(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                    W_gate: torch.Tensor, W_up: torch.Tensor, W_down: torch.Tensor,
                    out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Routed-expert FFN layer with BF16 weights; returns ``out`` [T, H] bf16."""
    T, H, top_k = _layer_args(x, topk_ids, topk_w, out)
    E, I, H2 = W_gate.shape
    if H2 != H or tuple(W_up.shape) != (E, I, H) or tuple(W_down.shape) != (E, H, I):
        raise ValueError("weight shapes must be W_gate/W_up [E,I,H], W_down [E,H,I]")
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(T, H, I, E, top_k, x.device)
    _check("moe_ffn_forward", lib().moe_ffn_forward(
        _dev(x, "x", torch.bfloat16), _dev(topk_ids, "topk_ids", torch.int32),
        _dev(topk_w, "topk_w", torch.float32), _dev(W_gate, "W_gate", torch.bfloat16),
        _dev(W_up, "W_up", torch.bfloat16), _dev(W_down, "W_down", torch.bfloat16),
        _dev(out, "out", torch.bfloat16), T, H, I, E, top_k,
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream)))
    return out


def moe_ffn_forward_noalloc(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                            W_gate: torch.Tensor, W_up: torch.Tensor, W_down: torch.Tensor,
                            out: torch.Tensor, stream=None) -> torch.Tensor:
    """moe_ffn_forward with the library's own per-GPU workspace (no workspace
    argument; the C call allocates nothing, and ``out`` is the caller's).
    Calls that may overlap on one GPU race on that workspace."""
    T, H, top_k = _layer_args(x, topk_ids, topk_w, out)
    E, I, H2 = W_gate.shape
    if H2 != H or tuple(W_up.shape) != (E, I, H) or tuple(W_down.shape) != (E, H, I):
        raise ValueError("weight shapes must be W_gate/W_up [E,I,H], W_down [E,H,I]")
    _check("moe_ffn_forward_noalloc", lib().moe_ffn_forward_noalloc(
        _dev(x, "x", torch.bfloat16), _dev(topk_ids, "topk_ids", torch.int32),
        _dev(topk_w, "topk_w", torch.float32), _dev(W_gate, "W_gate", torch.bfloat16),
        _dev(W_up, "W_up", torch.bfloat16), _dev(W_down, "W_down", torch.bfloat16),
        _dev(out, "out", torch.bfloat16), T, H, I, E, top_k, _stream(stream)))
    return out


def moe_ffn_forward_logits(x: torch.Tensor, logits: torch.Tensor, top_k: int,
                           W_gate: torch.Tensor, W_up: torch.Tensor, W_down: torch.Tensor,
                           out: Optional[torch.Tensor] = None,
                           topk_ids: Optional[torch.Tensor] = None,
                           topk_w: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None
                           ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Routed-expert FFN layer from router logits [T, E] float32 (BF16
    weights); returns (out [T, H] bf16, topk_ids [T, k] int32, topk_w [T, k]
    float32)."""
    if x.dim() != 2:
        raise ValueError(f"x must be [T, H], got {list(x.shape)}")
    T, H = x.shape
    E, I, H2 = W_gate.shape
    if tuple(logits.shape) != (T, E):
        raise ValueError(f"logits must be [T, E] = [{T}, {E}], got {list(logits.shape)}")
    if out is not None:
        _check_shape("out", out, (T, H))
    if H2 != H or tuple(W_up.shape) != (E, I, H) or tuple(W_down.shape) != (E, H, I):
        raise ValueError("weight shapes must be W_gate/W_up [E,I,H], W_down [E,H,I]")
    if out is None:
        out = torch.empty_like(x)
    if topk_ids is None:
        topk_ids = torch.empty(T, top_k, dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty(T, top_k, dtype=torch.float32, device=x.device)
    if tuple(topk_ids.shape) != (T, top_k) or tuple(topk_w.shape) != (T, top_k):
        raise ValueError("topk_ids and topk_w must be [T, top_k]")
    if workspace is None:
        workspace = alloc_workspace(T, H, I, E, top_k, x.device)
    _check("moe_ffn_forward_logits", lib().moe_ffn_forward_logits(
        _dev(x, "x", torch.bfloat16), _dev(logits, "logits", torch.float32),
        _dev(topk_ids, "topk_ids", torch.int32), _dev(topk_w, "topk_w", torch.float32),
        _dev(W_gate, "W_gate", torch.bfloat16), _dev(W_up, "W_up", torch.bfloat16),
        _dev(W_down, "W_down", torch.bfloat16), _dev(out, "out", torch.bfloat16),
        T, H, I, E, top_k, _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(stream)))
    return out, topk_ids, topk_w


def moe_ffn_forward_int8(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                         Q_gate: torch.Tensor, S_gate: torch.Tensor, Q_up: torch.Tensor,
                         S_up: torch.Tensor, Q_down: torch.Tensor, S_down: torch.Tensor,
                         out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Routed-expert FFN layer with INT8 group-quantised weights; returns ``out``.

    Scales are row-major, one per 128 K of a row: S_gate/S_up [E, I, H/128],
    S_down [E, H, I/128] (the layout the quantiser produces)."""
    T, H, top_k = _layer_args(x, topk_ids, topk_w, out)
    E, I, H2 = Q_gate.shape
    if H2 != H:
        raise ValueError("weight shapes must be Q_gate/Q_up [E,I,H], Q_down [E,H,I]")
    G = 128
    if H % G or I % G:
        raise ValueError("H and I must be multiples of 128")
    for name, t, shape in (("Q_up", Q_up, (E, I, H)), ("Q_down", Q_down, (E, H, I)),
                           ("S_gate", S_gate, (E, I, H // G)), ("S_up", S_up, (E, I, H // G)),
                           ("S_down", S_down, (E, H, I // G))):
        _check_shape(name, t, shape)
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(T, H, I, E, top_k, x.device)
    _check("moe_ffn_forward_int8", lib().moe_ffn_forward_int8(
        _dev(x, "x", torch.bfloat16), _dev(topk_ids, "topk_ids", torch.int32),
        _dev(topk_w, "topk_w", torch.float32), _dev(Q_gate, "Q_gate", torch.int8),
        _dev(S_gate, "S_gate", torch.float32), _dev(Q_up, "Q_up", torch.int8),
        _dev(S_up, "S_up", torch.float32), _dev(Q_down, "Q_down", torch.int8),
        _dev(S_down, "S_down", torch.float32), G, _dev(out, "out", torch.bfloat16),
        T, H, I, E, top_k, _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(stream)))
    return out


def moe_ffn_forward_int4(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                         P_gate: torch.Tensor, S_gate: torch.Tensor, P_up: torch.Tensor,
                         S_up: torch.Tensor, P_down: torch.Tensor, S_down: torch.Tensor,
                         out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Routed-expert FFN layer with INT4 group-quantised weights, two
    offset-binary nibbles per byte (P_gate/P_up [E, I, H/2], P_down [E, H, I/2]
    uint8); scales row-major as for INT8.  Returns ``out``."""
    T, H, top_k = _layer_args(x, topk_ids, topk_w, out)
    E, I, H2 = P_gate.shape
    G = 128
    if 2 * H2 != H or H % G or I % G:
        raise ValueError("P_gate must be [E,I,H/2] with H and I multiples of 128")
    for name, t, shape in (("P_up", P_up, (E, I, H // 2)), ("P_down", P_down, (E, H, I // 2)),
                           ("S_gate", S_gate, (E, I, H // G)), ("S_up", S_up, (E, I, H // G)),
                           ("S_down", S_down, (E, H, I // G))):
        _check_shape(name, t, shape)
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(T, H, I, E, top_k, x.device)
    _check("moe_ffn_forward_int4", lib().moe_ffn_forward_int4(
        _dev(x, "x", torch.bfloat16), _dev(topk_ids, "topk_ids", torch.int32),
        _dev(topk_w, "topk_w", torch.float32), _dev(P_gate, "P_gate", torch.uint8),
        _dev(S_gate, "S_gate", torch.float32), _dev(P_up, "P_up", torch.uint8),
        _dev(S_up, "S_up", torch.float32), _dev(P_down, "P_down", torch.uint8),
        _dev(S_down, "S_down", torch.float32), G, _dev(out, "out", torch.bfloat16),
        T, H, I, E, top_k, _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(stream)))
    return out


def moe_route_grouped(logits: torch.Tensor, top_k: int, n_group: int, topk_group: int,
                      bias: Optional[torch.Tensor] = None, scale: float = 1.0,
                      topk_ids: Optional[torch.Tensor] = None,
                      topk_w: Optional[torch.Tensor] = None, stream=None):
    """Grouped sigmoid router: logits [T, E] float32 (device), optional
    selection bias [E] -> (topk_ids [T, top_k] int32, topk_w [T, top_k]
    float32)."""
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty(T, top_k, dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty(T, top_k, dtype=torch.float32, device=logits.device)
    if bias is not None and tuple(bias.shape) != (E,):
        raise ValueError(f"bias must be [{E}], got {list(bias.shape)}")
    _check_shape("topk_ids", topk_ids, (T, top_k))
    _check_shape("topk_w", topk_w, (T, top_k))
    _check("moe_route_grouped", lib().moe_route_grouped(
        _dev(logits, "logits", torch.float32),
        None if bias is None else _dev(bias, "bias", torch.float32), T, E, n_group,
        topk_group, top_k, float(scale), _dev(topk_ids, "topk_ids", torch.int32),
        _dev(topk_w, "topk_w", torch.float32), _stream(stream)))
    return topk_ids, topk_w


def moe_ffn_forward_resplit(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                            P_gate: torch.Tensor, S_gate: torch.Tensor, R_gate: torch.Tensor,
                            SR_gate: torch.Tensor, P_up: torch.Tensor, S_up: torch.Tensor,
                            R_up: torch.Tensor, SR_up: torch.Tensor, P_down_lo: torch.Tensor,
                            S_down_lo: torch.Tensor, Q_down_hi: torch.Tensor,
                            S_down_hi: torch.Tensor, critical: torch.Tensor,
                            out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Routed-expert FFN layer with residual-split weights: gate/up as INT4
    W^Q plus INT4 residual W^R (packed [E, I, H/2] uint8), down as an INT4
    ([E, H, I/2] uint8) and an INT8 ([E, H, I] int8) copy, scales row-major;
    experts with ``critical[e]`` (uint8 [E]) nonzero use W^Q + W^R and the
    INT8 down, the others W^Q and the INT4 down.  Returns ``out``."""
    T, H, top_k = _layer_args(x, topk_ids, topk_w, out)
    E, I, H2 = P_gate.shape
    G = 128
    if 2 * H2 != H or H % G or I % G:
        raise ValueError("P_gate must be [E,I,H/2] with H and I multiples of 128")
    shapes = {"R_gate": (R_gate, (E, I, H // 2)), "P_up": (P_up, (E, I, H // 2)),
              "R_up": (R_up, (E, I, H // 2)), "P_down_lo": (P_down_lo, (E, H, I // 2)),
              "Q_down_hi": (Q_down_hi, (E, H, I)), "S_gate": (S_gate, (E, I, H // G)),
              "SR_gate": (SR_gate, (E, I, H // G)), "S_up": (S_up, (E, I, H // G)),
              "SR_up": (SR_up, (E, I, H // G)), "S_down_lo": (S_down_lo, (E, H, I // G)),
              "S_down_hi": (S_down_hi, (E, H, I // G)), "critical": (critical, (E,))}
    for name, (t, shape) in shapes.items():
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(T, H, I, E, top_k, x.device)
    u8, f32 = torch.uint8, torch.float32
    _check("moe_ffn_forward_resplit", lib().moe_ffn_forward_resplit(
        _dev(x, "x", torch.bfloat16), _dev(topk_ids, "topk_ids", torch.int32),
        _dev(topk_w, "topk_w", f32), _dev(P_gate, "P_gate", u8), _dev(S_gate, "S_gate", f32),
        _dev(R_gate, "R_gate", u8), _dev(SR_gate, "SR_gate", f32), _dev(P_up, "P_up", u8),
        _dev(S_up, "S_up", f32), _dev(R_up, "R_up", u8), _dev(SR_up, "SR_up", f32),
        _dev(P_down_lo, "P_down_lo", u8), _dev(S_down_lo, "S_down_lo", f32),
        _dev(Q_down_hi, "Q_down_hi", torch.int8), _dev(S_down_hi, "S_down_hi", f32),
        _dev(critical, "critical", u8), G, _dev(out, "out", torch.bfloat16), T, H, I, E, top_k,
        _dev(workspace, "workspace", u8), workspace.numel(), _stream(stream)))
    return out


def moe_ffn_check_status(workspace: torch.Tensor, stream=None) -> Tuple[int, int]:
    """Synchronise ``stream`` and return (status, dropped slots) of the last call."""
    n = _i64(0)
    code = lib().moe_ffn_check_status(_dev(workspace, "workspace", torch.uint8),
                                      _stream(stream), _c.byref(n))
    return code, int(n.value)


def moe_ffn_device_check() -> Tuple[bool, int]:
    """Wait for the device; return (the library is the debug build, the first
    failed device bounds check since the last call as file * 100000 + line,
    or 0), clearing the record."""
    where = _i32(0)
    code = lib().moe_ffn_device_check(_c.byref(where))
    if code < 0:
        raise MoeFfnError("moe_ffn_device_check", code)
    return bool(code), int(where.value)


def moe_ffn_set_split(gate_up: int = 0, down: int = 0) -> None:
    """Test hook: force the K parts per row block (1, 2 or 4) of the gate/up
    and down products for this thread's later calls; 0 = chosen on the
    device."""
    _check("moe_ffn_set_split", lib().moe_ffn_set_split(gate_up, down))


def moe_ffn_read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Measurement helper: enqueue one streaming read of every byte of the
    device buffer ``buf`` (its byte size a multiple of 16); ``sink`` is a
    device int32 tensor of at least one element."""
    if not (buf.is_cuda and buf.is_contiguous()):
        raise ValueError("buf must be a contiguous device tensor")
    if not (sink.is_cuda and sink.dtype == torch.int32 and sink.numel() >= 1):
        raise ValueError("sink must be a device int32 tensor")
    _check("moe_ffn_read_probe", lib().moe_ffn_read_probe(
        buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), _stream(stream)))


def moe_ffn_launch_probe(n: int, stream=None) -> None:
    """Measurement helper: enqueue n launches of an empty kernel (the
    launch-gap probe)."""
    _check("moe_ffn_launch_probe", lib().moe_ffn_launch_probe(n, _stream(stream)))


def moe_ffn_set_stage_events(events) -> None:
    """Benchmark hook: the next forward call of this thread records the given
    HIP events (``torch.cuda.Event`` objects already recorded once, or raw
    handles) right after its kernels 0..len-1 (permute, gate/up, down,
    combine).  An empty list clears the setting."""
    handles = [e.cuda_event if hasattr(e, "cuda_event") else int(e) for e in events]
    arr = (_vp * max(1, len(handles)))(*handles)
    _check("moe_ffn_set_stage_events", lib().moe_ffn_set_stage_events(arr, len(handles)))


def moe_attn_decode_workspace_bytes(B: int, h_q: int, h_kv: int, d: int, max_len: int) -> int:
    return int(lib().moe_attn_decode_workspace_bytes(B, h_q, h_kv, d, max_len))


def moe_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    seq_lens: torch.Tensor, scale: Optional[float] = None,
                    out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Decode attention with grouped-query heads: q [B, h_q, d], k_cache /
    v_cache [B, h_kv, max_len, d] (bf16), seq_lens [B] int32 -> out [B, h_q, d]
    bf16.  ``scale`` defaults to 1/sqrt(d) (chosen by the library: None is
    passed as 0)."""
    B, h_q, d = q.shape
    B2, h_kv, max_len, d2 = k_cache.shape
    if B2 != B or d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache / v_cache must be [B, h_kv, max_len, d] matching q")
    if tuple(seq_lens.shape) != (B,):
        raise ValueError("seq_lens must be [B]")
    if out is not None:
        _check_shape("out", out, (B, h_q, d))
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        n = moe_attn_decode_workspace_bytes(B, h_q, h_kv, d, max_len)
        if n == 0:
            raise MoeFfnError("moe_attn_decode_workspace_bytes", MOE_FFN_ERR_BAD_SHAPE)
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    _check("moe_attn_decode", lib().moe_attn_decode(
        _dev(q, "q", torch.bfloat16), _dev(k_cache, "k_cache", torch.bfloat16),
        _dev(v_cache, "v_cache", torch.bfloat16), _dev(seq_lens, "seq_lens", torch.int32),
        _dev(out, "out", torch.bfloat16), B, h_q, h_kv, d, max_len,
        0.0 if scale is None else float(scale),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream)))
    return out
