"""Helpers for the GPU parity tests: upload seeded inputs, run the C-ABI calls, read back.

bf16 tensors travel as their raw bits (int16 on the device, uint16 on the
host) so nothing is converted on the way.
"""
from __future__ import annotations

import numpy as np
import torch

from routing_dispatch_expert_logits_amd import binding as B

DEV = "cuda:0"


def dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor, bf16: bool = False) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if bf16 else a


def empty(shape, kind: str) -> torch.Tensor:
    dt = {"f32": torch.float32, "bf16": torch.int16, "i32": torch.int32, "u8": torch.uint8}[kind]
    return torch.empty(shape, dtype=dt, device=DEV)


def ws(s: B.MoeShape, call: int) -> torch.Tensor:
    n = max(B.workspace_bytes(s, call), 256)
    return torch.empty(n, dtype=torch.uint8, device=DEV)


def shape_of(cfg) -> B.MoeShape:
    return B.shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.L, cfg.dtype, cfg.shared_I, cfg.capacity,
                   cfg.dispatch)


def act_kind(cfg) -> str:
    return "f32" if cfg.dtype == "f32" else "bf16"


def rne_bf16_bits(f32: np.ndarray) -> np.ndarray:
    """Reference rounding of fp32 results to bf16 bits (torch's CPU conversion)."""
    return torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).bfloat16().view(
        torch.int16).numpy().view(np.uint16)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / RMS(ref)."""
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref))) / max(rms, 1e-300)


def check_permutation_valid(ids: np.ndarray, offsets: np.ndarray, row_token: np.ndarray,
                            token_row: np.ndarray):
    """Properties a correct expert-contiguous permutation of these ids has."""
    T, k = ids.shape
    R = T * k
    assert sorted(row_token.tolist()) == sorted(np.repeat(np.arange(T), k).tolist())
    flat = token_row.reshape(-1)
    assert sorted(flat.tolist()) == list(range(R))
    np.testing.assert_array_equal(row_token[flat], np.repeat(np.arange(T), k))
    E = len(offsets) - 1
    seg = np.searchsorted(offsets, flat, side="right") - 1
    np.testing.assert_array_equal(seg, ids.reshape(-1))
    for e in range(E):
        s = row_token[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(s) > 0)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """One bf16 unit in the last place at |v| (8 significant bits)."""
    return 2.0 ** (np.floor(np.log2(np.maximum(np.abs(v), 1e-30))) - 7)


def out_err_over_rms(got: np.ndarray, ref: np.ndarray, shared_ref=None) -> float:
    """max |got - ref| / RMS(ref).  With a shared expert, one bf16 ulp of its output
    is allowed per element first: both sides round that output to bf16 at the same
    point, an element near a rounding midpoint can land one ulp apart (fp32 sums vs
    exact ones), and the shared term enters with weight 1 instead of a routing
    weight, so the flip is not diluted."""
    err = np.abs(got - ref)
    if shared_ref is not None:
        err = np.maximum(err - bf16_ulp(shared_ref), 0.0)
    return float(err.max() / np.sqrt(np.mean(ref ** 2)))
