"""The C-ABI library on the host: it loads, exports every declared call, sizes
workspaces, and rejects bad arguments before any GPU work (CPU only).

The calls below all fail host-side validation, so they return before any HIP
call; the fake pointers are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import pytest

from routing_dispatch_expert_logits_amd import binding as B
from workloads import FULL_CONFIGS, PARITY_CONFIGS

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")
FAKE = 0x10000  # aligned, never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("moe_route_topk", "moe_dispatch_permute", "moe_grouped_ffn", "moe_combine",
                 "moe_layer_forward", "moe_workspace_bytes", "moe_status_string", "moe_abi_version"):
        assert want in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(B.lib, name)


def test_abi_version_and_status_strings():
    assert B.lib.moe_abi_version() == B.ABI_VERSION
    for code in range(5):
        assert B.status_string(code).startswith("MOE_")
    assert "unknown" in B.status_string(99)


def _bytes(cfg, call):
    return B.workspace_bytes(B.shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.L, cfg.dtype, cfg.shared_I,
                                     cfg.capacity), call)


@pytest.mark.parametrize("cfg", list(FULL_CONFIGS.values()) + list(PARITY_CONFIGS.values()),
                         ids=lambda c: c.name)
def test_workspace_sizes(cfg):
    R, D, es = cfg.R, cfg.D, cfg.elem_bytes
    route = _bytes(cfg, B.MOE_CALL_ROUTE)
    assert route >= ((cfg.T + 15) // 16) * cfg.E * 4       # per 16-token ranking block counts
    assert _bytes(cfg, B.MOE_CALL_FFN) >= R * cfg.I * es
    assert _bytes(cfg, B.MOE_CALL_COMBINE) >= R * D * es
    layer = _bytes(cfg, B.MOE_CALL_LAYER)
    shared = cfg.T * (cfg.shared_I + cfg.H) * es if cfg.shared_I else 0  # shared expert A and Y
    assert layer >= R * D * es + R * cfg.I * es + shared
    # one permuted-row buffer serves both x_perm and y_perm
    assert layer < (2 * R * D * es + R * cfg.I * es + 2 * cfg.T * max(cfg.L, 1) * es + shared
                    + 64 * 1024 * 1024)


def test_invalid_shapes_have_no_workspace():
    bad = [B.shape(0, 128, 8, 2, 256), B.shape(4, 128, 8, 9, 256), B.shape(4, 128, 0, 1, 256),
           B.shape(4, 128, 2048, 2, 256), B.shape(4, 100, 8, 2, 256),   # bf16 needs D % 64
           B.shape(4, 128, 8, 2, 100), B.shape(4, 128, 128, 65, 256)]
    for s in bad:
        assert B.workspace_bytes(s, B.MOE_CALL_LAYER) == 0


def _route(s, ws_bytes=1 << 20, **over):
    args = dict(x=FAKE, gate_w=None, bias=None, logits=FAKE, ids=FAKE, w=FAKE, counts=FAKE,
                offsets=FAKE, ws=FAKE)
    args.update(over)
    return B.lib.moe_route_topk(args["x"], args["gate_w"], args["bias"], args["logits"], args["ids"],
                                args["w"], args["counts"], args["offsets"], ctypes.byref(s),
                                args["ws"], ws_bytes, None)


def test_route_rejects_bad_arguments_on_host():
    s = B.shape(64, 128, 8, 2, 256)
    assert _route(B.shape(0, 128, 8, 2, 256)) == B.MOE_ERR_INVALID_ARG
    assert _route(B.shape(64, 128, 8, 9, 256)) == B.MOE_ERR_INVALID_ARG       # k > E
    assert _route(B.shape(64, 128, 2000, 2, 256)) == B.MOE_ERR_UNSUPPORTED    # E > 1024
    assert _route(B.shape(64, 128, 200, 65, 256)) == B.MOE_ERR_UNSUPPORTED    # k > 64
    assert _route(s, logits=None) == B.MOE_ERR_INVALID_ARG
    assert _route(s, ids=FAKE + 4) == B.MOE_ERR_INVALID_ARG                   # misaligned
    assert _route(s, ws_bytes=16) == B.MOE_ERR_WORKSPACE
    assert _route(s, ws=None) == B.MOE_ERR_WORKSPACE
    bad = B.shape(64, 128, 8, 2, 256)
    bad.shared_I = -1
    assert _route(bad) == B.MOE_ERR_INVALID_ARG
    assert _route(B.shape(64, 128, 8, 2, 256, shared_I=96)) == B.MOE_ERR_UNSUPPORTED   # bf16: % 64
    assert _route(B.shape(64, 128, 8, 2, 256, L=64, shared_I=128)) == B.MOE_ERR_UNSUPPORTED  # latent
    assert _route(B.shape(64, 128, 8, 2, 256, capacity=-1)) == B.MOE_ERR_INVALID_ARG
    bad = B.shape(64, 128, 8, 2, 256)
    bad.dtype = 7
    assert _route(bad) == B.MOE_ERR_INVALID_ARG
    bad = B.shape(64, 128, 8, 2, 256)
    bad.dispatch = 5
    assert _route(bad) == B.MOE_ERR_INVALID_ARG
    assert _route(B.shape(64, 128, 8, 2, 256, dtype="f32", dispatch="mxfp8")) == B.MOE_ERR_UNSUPPORTED
    assert _route(B.shape(64, 192, 8, 2, 256, dispatch="mxfp8")) == B.MOE_ERR_UNSUPPORTED  # D % 128
    assert _route(B.shape(64, 256, 8, 2, 256, dispatch="mxfp8"), ws_bytes=0) == B.MOE_ERR_WORKSPACE  # accepted


def test_other_calls_reject_bad_arguments_on_host():
    s = B.shape(64, 128, 8, 2, 256)
    L = B.lib
    assert L.moe_dispatch_permute(FAKE, FAKE, FAKE, None, None, FAKE, FAKE, ctypes.byref(s), FAKE, 1 << 20,
                                  None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_dispatch_permute(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, ctypes.byref(s), FAKE, 0,
                                  None) == B.MOE_ERR_WORKSPACE
    # a scale buffer is MXFP8-only
    assert L.moe_dispatch_permute(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(s), FAKE, 1 << 20,
                                  None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_grouped_ffn(FAKE, None, FAKE, FAKE, None, FAKE, None, None, FAKE, ctypes.byref(s), FAKE,
                             1 << 30, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_grouped_ffn(FAKE, None, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, ctypes.byref(s), FAKE, 8,
                             None) == B.MOE_ERR_WORKSPACE
    mx = B.shape(64, 128, 8, 2, 256, dispatch="mxfp8")
    assert L.moe_grouped_ffn(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(mx), FAKE,
                             1 << 30, None) == B.MOE_ERR_INVALID_ARG            # MXFP8 rows need scales
    assert L.moe_dispatch_permute(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, ctypes.byref(mx), FAKE, 1 << 20,
                                  None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_mxfp8(FAKE, B.MOE_BF16, 4, 48, FAKE, FAKE, None) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_quantize_mxfp8(FAKE, 9, 4, 64, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_mxfp8(FAKE, B.MOE_BF16, 4, 64, FAKE + 4, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_mxfp8(None, B.MOE_BF16, 0, 64, None, None, None) == B.MOE_OK   # nothing to do
    assert L.moe_combine(FAKE, FAKE, FAKE, None, FAKE, 5, 0, ctypes.byref(s), FAKE, 1 << 30,
                         None) == B.MOE_ERR_INVALID_ARG                     # out dtype
    assert L.moe_combine(FAKE, FAKE, FAKE, None, FAKE, 0, 3, ctypes.byref(s), FAKE, 1 << 30,
                         None) == B.MOE_ERR_INVALID_ARG                     # flags
    assert L.moe_combine(FAKE, FAKE, FAKE, FAKE + 4, FAKE, 0, 0, ctypes.byref(s), FAKE, 1 << 30,
                         None) == B.MOE_ERR_INVALID_ARG                     # misaligned shared_out
    assert L.moe_combine(FAKE, FAKE, FAKE, None, FAKE, 0, B.MOE_COMBINE_UNFUSED, ctypes.byref(s), FAKE,
                         8, None) == B.MOE_ERR_WORKSPACE
    w = B.MoeLayerWeights(None, None, FAKE, FAKE, FAKE, None, None, None, None, None)
    aux = B.MoeLayerAux()
    # no gate weight and no given logits
    assert L.moe_layer_forward(ctypes.byref(w), FAKE, None, FAKE, 0, ctypes.byref(s), ctypes.byref(aux),
                               None, FAKE, 1 << 30, None) == B.MOE_ERR_INVALID_ARG
    # latent layer without projections
    sl = B.shape(64, 128, 8, 2, 256, L=64)
    assert L.moe_layer_forward(ctypes.byref(w), FAKE, FAKE, FAKE, 0, ctypes.byref(sl), ctypes.byref(aux),
                               None, FAKE, 1 << 30, None) == B.MOE_ERR_INVALID_ARG
    aux.x_perm = FAKE + 8
    assert L.moe_layer_forward(ctypes.byref(w), FAKE, FAKE, FAKE, 0, ctypes.byref(s), ctypes.byref(aux),
                               None, FAKE, 1 << 30, None) == B.MOE_ERR_INVALID_ARG
    aux.x_perm = None
    assert L.moe_layer_forward(ctypes.byref(w), FAKE, FAKE, FAKE, 0, ctypes.byref(s), ctypes.byref(aux),
                               None, FAKE, 1024, None) == B.MOE_ERR_WORKSPACE
    assert L.moe_layer_forward(None, FAKE, FAKE, FAKE, 0, ctypes.byref(s), ctypes.byref(aux),
                               None, FAKE, 1 << 30, None) == B.MOE_ERR_INVALID_ARG
    # shared expert declared without its weights
    ss = B.shape(64, 128, 8, 2, 256, shared_I=128)
    assert L.moe_layer_forward(ctypes.byref(w), FAKE, FAKE, FAKE, 0, ctypes.byref(ss), ctypes.byref(aux),
                               None, FAKE, 1 << 30, None) == B.MOE_ERR_INVALID_ARG


def test_layer_plan_names_the_kernels_of_each_layer():
    """The host-only plan query reports the decision moe_layer_forward takes."""
    want = {  # layer: (decode path, rows gathered, gate/up kernel, down kernel, launches)
        "qwen3_30b_a3b_shaped": (0, 1, "k_gemm_wsp<128, 128, 2,", "k_gemm_wsp<128, 256, 1,", 7),
        "deepseek_r1_shaped": (0, 1, "k_gemm_wsp<128, 128, 2,", "k_gemm_wsp<128, 256, 1,", 7),
        "latent_moe": (0, 1, "k_gemm_wsp<128, 128, 2,", "k_gemm_wsp<256, 128, 1,", 9),
        "k3_shaped_decode_t8": (1, 1, "k_gemm_decode<2, 2,", "k_down_combine<16,", 3),
        "k3_shaped_decode": (1, 1, "k_gemm_decode<2, 2,", "k_down_combine<16,", 3),
        "tiny_f32": (0, 0, "k_gemm_simt<float, 2,", "k_gemm_simt<float, 1,", 6),
    }
    for name, (dec, gath, gu, dn, n) in want.items():
        c = FULL_CONFIGS[name]
        p = B.layer_plan(B.shape(c.T, c.H, c.E, c.k, c.I, c.L, c.dtype, c.shared_I, c.capacity),
                         c.gate == "computed")
        assert (p["decode_path"], p["rows_gathered"], p["gate_up_kernel"], p["down_kernel"],
                p["launches"]) == (dec, gath, gu, dn, n), name
    # asking for the permuted copy turns the gathered dataflow off (one more launch on
    # the decode path, the same count elsewhere: the permutation writes the rows)
    c = FULL_CONFIGS["qwen3_30b_a3b_shaped"]
    s = B.shape(c.T, c.H, c.E, c.k, c.I)
    assert B.layer_plan(s, True, x_perm=True)["rows_gathered"] == 0
    with pytest.raises(B.MoeError):
        B.layer_plan(B.shape(0, 128, 8, 2, 256), True)
    assert B.lib.moe_layer_plan(ctypes.byref(s), 8, None) == B.MOE_ERR_INVALID_ARG
    # decode-scale steps (T <= 128) route in one launch: one workgroup while
    # ceil(T / 16) * k * ceil(E / 64) <= 640, else ceil(T / 4) of them; 3 launches, 4 when
    # the Y columns do not fit the fused down GEMM + combine's LDS.  Past T = 128 the
    # general routing kernels add two
    for T, E, k, wgs in ((1, 8, 2, 1), (64, 1024, 8, 1), (8, 896, 16, 1), (128, 200, 8, 1),
                         (120, 700, 12, 30), (65, 896, 16, 17), (128, 896, 16, 32), (129, 64, 2, 0)):
        p = B.layer_plan(B.shape(T, 256, E, k, 128), False)
        fused = p["down_kernel"] == "k_down_combine<16,"
        assert p["decode_path"] == int(wgs > 0), (T, E, k)
        assert p["route_workgroups"] == wgs, (T, E, k)
        assert p["launches"] == (3 if fused else 4) + (0 if wgs else 2), (T, E, k)
    assert B.layer_plan(B.shape(4096, 256, 8, 2, 128), False)["route_workgroups"] == 0


def test_persistent_tile_table_fields_bound_the_expert_rows():
    """A persistent-GEMM table entry keeps an expert's m-tile index in 12 bits, so a
    layer in which one expert may hold more than 4096 m-tiles of rows (E = 1, k = 1,
    T > 4096 * 128) must take the one-workgroup-per-tile kernels instead."""
    at = B.layer_plan(B.shape(4096 * 128, 256, 1, 1, 128), False)
    assert at["gate_up_persistent"] == 1 and at["gate_up_kernel"] == "k_gemm_wsp<128, 128, 2,"
    over = B.layer_plan(B.shape(4096 * 128 + 1, 256, 1, 1, 128), False)
    assert over["gate_up_persistent"] == 0 and over["gate_up_kernel"] == "k_gemm_ws<128, 128, 2,"
    assert over["rows_gathered"] == 0            # gathering needs the persistent kernel
    assert over["down_persistent"] == 0
    # the down GEMM's 128 x 256 tiles meet the bound first (K >= 2048: the 256-row tiles
    # come next, with the same bound on 256-row m-tiles)
    at = B.layer_plan(B.shape(4096 * 256, 128, 1024, 1, 2048), False)
    assert at["down_kernel"] == "k_gemm_wsp<256, 128, 1," and at["down_persistent"] == 1
    over = B.layer_plan(B.shape(4096 * 256 + 256, 128, 1024, 1, 2048), False)
    assert over["down_kernel"] == "k_gemm_ws<256, 128, 1," and over["down_persistent"] == 0


def test_noalloc_rejects_before_any_gpu_work():
    """The allocation-free layer forward validates like moe_layer_forward, and a shape
    whose layer workspace exceeds the library's scratch array is MOE_ERR_WORKSPACE, all on
    the host before any HIP call."""
    L = B.lib
    w = B.MoeLayerWeights(None, None, FAKE, FAKE, FAKE, None, None, None, None, None)
    aux = B.MoeLayerAux()
    s = B.shape(64, 128, 8, 2, 256)
    assert L.moe_layer_forward_noalloc(ctypes.byref(w), FAKE, None, FAKE, 0, ctypes.byref(s),
                                       ctypes.byref(aux), None, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward_noalloc(ctypes.byref(w), FAKE, FAKE, FAKE, 0,
                                       ctypes.byref(B.shape(0, 128, 8, 2, 256)), ctypes.byref(aux), None,
                                       None) == B.MOE_ERR_INVALID_ARG
    c = FULL_CONFIGS["deepseek_r1_shaped"]
    big = B.shape(c.T, c.H, c.E, c.k, c.I)
    assert B.workspace_bytes(big, B.MOE_CALL_LAYER) > B.NOALLOC_SCRATCH_BYTES
    assert L.moe_layer_forward_noalloc(ctypes.byref(w), FAKE, FAKE, FAKE, 0, ctypes.byref(big),
                                       ctypes.byref(aux), None, None) == B.MOE_ERR_WORKSPACE
    # the decode-scale 896-expert top-16 step fits up to 256 tokens
    k3 = FULL_CONFIGS["k3_shaped_decode"]
    assert B.workspace_bytes(B.shape(256, k3.H, k3.E, k3.k, k3.I), B.MOE_CALL_LAYER) <= B.NOALLOC_SCRATCH_BYTES
