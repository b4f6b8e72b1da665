"""ctypes binding of libmoe's C ABI (include/moe.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU (or None for
nullable arguments), passes their device pointers and the current HIP stream
to the library, and raises MoeError on a non-OK status.  Nothing here computes
any part of the layer, and there is no fallback: if libmoe.so is missing the
import fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_CALL_ROUTE, MOE_CALL_DISPATCH, MOE_CALL_FFN, MOE_CALL_COMBINE, MOE_CALL_LAYER = range(5)
MOE_COMBINE_FUSED, MOE_COMBINE_UNFUSED = 0, 1
MOE_DISPATCH_DTYPE, MOE_DISPATCH_MXFP8 = 0, 1
MOE_NUM_STAGE_EVENTS = 10
NOALLOC_SCRATCH_BYTES = 64 << 20
ABI_VERSION = 5
MOE_PLAN_GATE, MOE_PLAN_X_PERM = 1, 2

STAGE_NAMES = ["latent_down", "gate", "route", "permute", "gemm_gate_up", "gemm_down",
               "shared_expert", "combine", "latent_up"]

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


class MoeError(RuntimeError):
    def __init__(self, call: str, status: int):
        super().__init__(f"{call}: {status_string(status)} (status {status})")
        self.status = status


class MoeShape(ctypes.Structure):
    _fields_ = [("T", _i64), ("H", _i64), ("E", _i64), ("k", _i64), ("I", _i64), ("L", _i64),
                ("dtype", _i32), ("shared_I", _i32), ("capacity", _i64), ("dispatch", _i32),
                ("reserved", _i32)]


class MoeLayerWeights(ctypes.Structure):
    _fields_ = [("gate_w", _vp), ("gate_bias", _vp), ("w1", _vp), ("w3", _vp), ("w2", _vp),
                ("wd", _vp), ("wu", _vp), ("ws1", _vp), ("ws3", _vp), ("ws2", _vp),
                ("w1_scale", _vp), ("w3_scale", _vp)]


class MoeLayerAux(ctypes.Structure):
    _fields_ = [("topk_ids", _vp), ("topk_w", _vp), ("counts", _vp), ("offsets", _vp),
                ("row_token", _vp), ("token_row", _vp), ("x_perm", _vp), ("y_perm", _vp),
                ("z", _vp), ("out_latent", _vp), ("x_perm_scale", _vp)]


class MoePlan(ctypes.Structure):
    _fields_ = [("launches", _i32), ("decode_path", _i32), ("rows_gathered", _i32),
                ("gate_up_tile_m", _i32), ("gate_up_tile_n", _i32), ("gate_up_persistent", _i32),
                ("down_tile_m", _i32), ("down_tile_n", _i32), ("down_persistent", _i32),
                ("route_workgroups", _i32), ("gate_up_kernel", ctypes.c_char_p),
                ("down_kernel", ctypes.c_char_p)]


def _load() -> ctypes.CDLL:
    # torch ships its own libamdhip64.so.7; loading torch first makes libmoe bind
    # to that same HIP runtime instance, so torch's streams, events and
    # allocations are the library's too
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libmoe.so not built at {LIB_PATH}; run "
                          "`python -m routing_dispatch_expert_logits_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.moe_abi_version.restype = ctypes.c_int
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_workspace_bytes.argtypes = [P(MoeShape), ctypes.c_int]
    sz = ctypes.c_size_t
    lib.moe_layer_plan.argtypes = [P(MoeShape), ctypes.c_int, P(MoePlan)]
    lib.moe_layer_plan.restype = ctypes.c_int
    lib.moe_route_topk.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, P(MoeShape), _vp, sz, _vp]
    lib.moe_dispatch_permute.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, P(MoeShape), _vp, sz, _vp]
    lib.moe_grouped_ffn.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, P(MoeShape), _vp, sz,
                                    _vp]
    lib.moe_quantize_mxfp8.argtypes = [_vp, ctypes.c_int, _i64, _i64, _vp, _vp, _vp]
    lib.moe_combine.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int, P(MoeShape),
                                _vp, sz, _vp]
    lib.moe_layer_forward.argtypes = [P(MoeLayerWeights), _vp, _vp, _vp, ctypes.c_int,
                                      P(MoeShape), P(MoeLayerAux), P(_vp), _vp, sz, _vp]
    lib.moe_layer_forward_noalloc.argtypes = [P(MoeLayerWeights), _vp, _vp, _vp, ctypes.c_int,
                                              P(MoeShape), P(MoeLayerAux), P(_vp), _vp]
    for f in ("moe_route_topk", "moe_dispatch_permute", "moe_grouped_ffn", "moe_combine",
              "moe_layer_forward", "moe_quantize_mxfp8", "moe_layer_forward_noalloc"):
        getattr(lib, f).restype = ctypes.c_int
    v = lib.moe_abi_version()
    if v != ABI_VERSION:
        raise ImportError(f"libmoe ABI version {v}, binding expects {ABI_VERSION}")
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.moe_status_string(int(status)).decode()


def shape(T: int, H: int, E: int, k: int, I: int, L: int = 0, dtype: str = "bf16",
          shared_I: int = 0, capacity: int = 0, dispatch: str = "dtype") -> MoeShape:
    fmt = {"dtype": MOE_DISPATCH_DTYPE, "mxfp8": MOE_DISPATCH_MXFP8}[dispatch]
    return MoeShape(T, H, E, k, I, L, MOE_BF16 if dtype == "bf16" else MOE_F32, shared_I, capacity, fmt, 0)


def workspace_bytes(s: MoeShape, call: int) -> int:
    return int(lib.moe_workspace_bytes(ctypes.byref(s), call))


def layer_plan(s: MoeShape, gate: bool, x_perm: bool = False) -> dict:
    """The kernels moe_layer_forward runs for shape s (host-only query)."""
    p = MoePlan()
    flags = (MOE_PLAN_GATE if gate else 0) | (MOE_PLAN_X_PERM if x_perm else 0)
    _check("moe_layer_plan", lib.moe_layer_plan(ctypes.byref(s), flags, ctypes.byref(p)))
    d = {f: getattr(p, f) for f, _ in MoePlan._fields_}
    for f in ("gate_up_kernel", "down_kernel"):
        d[f] = d[f].decode()
    return d


def _p(t) -> Optional[int]:
    """Device pointer of a tensor (None stays NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _check(call: str, rc: int):
    if rc != MOE_OK:
        raise MoeError(call, rc)


def route_topk(x, gate_w, gate_bias, logits, topk_ids, topk_w, counts, offsets, s: MoeShape,
               ws, stream=None):
    _check("moe_route_topk", lib.moe_route_topk(
        _p(x), _p(gate_w), _p(gate_bias), _p(logits), _p(topk_ids), _p(topk_w), _p(counts),
        _p(offsets), ctypes.byref(s), _p(ws), _nbytes(ws), _stream(stream)))


def dispatch_permute(x, topk_ids, offsets, x_perm, row_token, token_row, s: MoeShape, ws,
                     stream=None, x_perm_scale=None):
    _check("moe_dispatch_permute", lib.moe_dispatch_permute(
        _p(x), _p(topk_ids), _p(offsets), _p(x_perm), _p(x_perm_scale), _p(row_token), _p(token_row),
        ctypes.byref(s), _p(ws), _nbytes(ws), _stream(stream)))


def grouped_ffn(x_perm, offsets, w1, w3, w2, y_perm, s: MoeShape, ws, stream=None, x_perm_scale=None,
                w1_scale=None, w3_scale=None):
    _check("moe_grouped_ffn", lib.moe_grouped_ffn(
        _p(x_perm), _p(x_perm_scale), _p(offsets), _p(w1), _p(w1_scale), _p(w3), _p(w3_scale), _p(w2),
        _p(y_perm), ctypes.byref(s), _p(ws), _nbytes(ws), _stream(stream)))


def quantize_mxfp8(src, q, scale, stream=None):
    """MXFP8 codes and scales of a [rows x cols] bf16 (int16 bit tensor) or fp32 tensor."""
    import torch
    src_dtype = MOE_F32 if src.dtype == torch.float32 else MOE_BF16
    cols = src.shape[-1]
    rows = src.numel() // cols if cols else 0
    _check("moe_quantize_mxfp8", lib.moe_quantize_mxfp8(
        _p(src), src_dtype, rows, cols, _p(q), _p(scale), _stream(stream)))


def combine(y_perm, token_row, topk_w, out, out_dtype: int, flags: int, s: MoeShape, ws,
            stream=None, shared_out=None):
    _check("moe_combine", lib.moe_combine(
        _p(y_perm), _p(token_row), _p(topk_w), _p(shared_out), _p(out), int(out_dtype), int(flags),
        ctypes.byref(s), _p(ws), _nbytes(ws), _stream(stream)))


def layer_forward(weights: dict, x, logits, out, out_dtype: int, s: MoeShape, ws, aux: dict = None,
                  stage_events=None, stream=None):
    """weights: gate_w, gate_bias, w1, w3, w2, wd, wu, ws1, ws3, ws2, w1_scale, w3_scale (tensors or None);
    aux: moe_layer_aux fields."""
    w = MoeLayerWeights(*[_p(weights.get(f)) for f, _ in MoeLayerWeights._fields_])
    a = MoeLayerAux(*[_p((aux or {}).get(f)) for f, _ in MoeLayerAux._fields_])
    ev = None
    if stage_events is not None:
        assert len(stage_events) == MOE_NUM_STAGE_EVENTS
        ev = (_vp * MOE_NUM_STAGE_EVENTS)(*[e.cuda_event if hasattr(e, "cuda_event") else e
                                            for e in stage_events])
    _check("moe_layer_forward", lib.moe_layer_forward(
        ctypes.byref(w), _p(x), _p(logits), _p(out), int(out_dtype), ctypes.byref(s),
        ctypes.byref(a), ev, _p(ws), _nbytes(ws), _stream(stream)))


def layer_forward_noalloc(weights: dict, x, logits, out, out_dtype: int, s: MoeShape, aux: dict = None,
                          stage_events=None, stream=None):
    """moe_layer_forward_noalloc: the layer forward with the library's own per-GPU scratch
    array as its workspace (no caller workspace)."""
    w = MoeLayerWeights(*[_p(weights.get(f)) for f, _ in MoeLayerWeights._fields_])
    a = MoeLayerAux(*[_p((aux or {}).get(f)) for f, _ in MoeLayerAux._fields_])
    ev = None
    if stage_events is not None:
        assert len(stage_events) == MOE_NUM_STAGE_EVENTS
        ev = (_vp * MOE_NUM_STAGE_EVENTS)(*[e.cuda_event if hasattr(e, "cuda_event") else e
                                            for e in stage_events])
    _check("moe_layer_forward_noalloc", lib.moe_layer_forward_noalloc(
        ctypes.byref(w), _p(x), _p(logits), _p(out), int(out_dtype), ctypes.byref(s), ctypes.byref(a), ev,
        _stream(stream)))
