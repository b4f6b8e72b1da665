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


# Every buffer a test hands to the library as an output sits between two guard bands
# of poison bytes, and its own bytes start as poison too: after each test the bands
# must be intact (no write past either end of any output), and a region the library
# promises to leave alone (rows past offsets[E] under an expert capacity) must still
# hold poison.
GUARD_BYTES = 4096
POISON = 0xA5
_guarded = []


def empty(shape, kind: str) -> torch.Tensor:
    dt = {"f32": torch.float32, "bf16": torch.int16, "i32": torch.int32, "u8": torch.uint8}[kind]
    shape = tuple(shape) if isinstance(shape, (tuple, list)) else (shape,)
    n = int(np.prod(shape, dtype=np.int64)) * torch.empty((), dtype=dt).element_size()
    buf = torch.full((n + 2 * GUARD_BYTES,), POISON, dtype=torch.uint8, device=DEV)
    _guarded.append((buf, n))
    return buf[GUARD_BYTES:GUARD_BYTES + n].view(dt).view(shape)


def poison_of(kind: str):
    """The value a never-written element of an `empty` buffer holds."""
    return {"f32": np.frombuffer(bytes([POISON] * 4), np.float32)[0],
            "bf16": np.uint16(POISON * 0x101), "i32": np.frombuffer(bytes([POISON] * 4), np.int32)[0],
            "u8": np.uint8(POISON)}[kind]


def assert_poison(t: torch.Tensor, first_row: int):
    """Rows first_row.. of an `empty` buffer were never written (every byte still poison)."""
    raw = t[first_row:].detach().contiguous().view(torch.uint8).cpu().numpy()
    assert (raw == POISON).all(), f"rows from {first_row} on were written"


def check_guards():
    """Every guard band of the buffers `empty` handed out since the last check still
    holds poison (run after each test by the conftest fixture)."""
    if not _guarded:
        return
    torch.cuda.synchronize()
    bad = []
    for buf, n in _guarded:
        head = buf[:GUARD_BYTES]
        tail = buf[GUARD_BYTES + n:]
        if not bool((head == POISON).all()) or not bool((tail == POISON).all()):
            bad.append(n)
    _guarded.clear()
    assert not bad, f"writes past the end of {len(bad)} output buffer(s) of {bad[:4]} bytes"


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


def check_y_rows(bf16: bool, got: np.ndarray, ref_y: np.ndarray, inputs_rounded_apart: bool = False):
    """Expert outputs Y against the oracle's (got: bf16 bits or fp32 values).

    Both sides round A and Y to bf16 at the same points, but the fp32 sums run in
    different orders, so an A element near a rounding midpoint can land one ulp apart;
    that moves Y by ulp(a) * |w2| (about 1e-3 x RMS(Y) for |a| ~ 5 x RMS(a) at I = 256).
    Bound: every element within one bf16 ulp of Y plus 5e-3 x RMS(Y); at most 1e-4 of
    them beyond one ulp plus 1e-3 x RMS(Y).  fp32 layers: 1e-5 x RMS(Y).

    inputs_rounded_apart: the rows fed to the GPU's FFN are its own bf16 rounding of an
    upstream fp32 sum (the latent layer's Z), which may sit one ulp from the oracle's
    in some elements; each such element moves the exact A a little and so flips A's
    rounding far more often than the summation order does.  Then every element must be
    within the layer tolerance, 2e-2 x RMS(Y) (a wrong tile would be off by O(RMS))."""
    from oracle import decode
    if not bf16:
        assert rel_err(got, ref_y) <= 1e-5
        return
    y = decode(got)
    rms = float(np.sqrt(np.mean(ref_y ** 2)))
    err = np.abs(y - ref_y)
    if inputs_rounded_apart:
        worst = float(err.max()) / rms
        assert worst <= 2e-2, f"max |err| = {worst:.2e} x RMS(Y)"
        return
    ulp = bf16_ulp(ref_y)
    worst = float(np.max((err - ulp) / rms))
    assert not (err > ulp + 5e-3 * rms).any(), f"worst excess over 1 ulp: {worst:.2e} x RMS"
    frac = float(np.mean(err > ulp + 1e-3 * rms))
    assert frac <= 1e-4, f"{frac:.2e} of elements beyond 1 ulp + 1e-3 RMS (worst {worst:.2e})"
