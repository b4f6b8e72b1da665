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


U_F32 = 2.0 ** -24


def fp32_dot_slack(K: int, rms_rows: np.ndarray) -> np.ndarray:
    """How far the GPU's fp32 accumulation of a length-K dot product may land from the
    exact sum, for a row of results whose exact values have RMS `rms_rows`: the larger of
    8 sqrt(K) 2^-24 (eight times the random walk of K roundings of partial sums no larger
    than the row's RMS) and 2^-14 (room for a matrix instruction that sums its products
    more coarsely than fp32, as the fp8 one measurably does), times that RMS.  Either
    is far below half a bf16 ulp (2^-9 relative)."""
    return max(8.0 * np.sqrt(K) * U_F32, 2.0 ** -14) * rms_rows


def bf16_round_interval(v: np.ndarray, dv: np.ndarray):
    """The bf16 values (nearest even) that any value within dv of the exact v rounds to
    lie in [round(v - dv), round(v + dv)] (rounding is monotone)."""
    from oracle import round_bf16
    return round_bf16(v - dv), round_bf16(v + dv)


def _rms_rows(m: np.ndarray) -> np.ndarray:
    return np.sqrt(np.mean(m * m, axis=1, keepdims=True))


def expert_y_bound(x_rows, w1e, w3e, w2e, x_dev=None) -> np.ndarray:
    """Per-element bound on |Y_gpu - Y_oracle| for one bf16 expert's rows, derived from
    the arithmetic both sides perform: G = X W1^T and U = X W3^T as fp32 sums (within
    fp32_dot_slack of the exact ones, plus what an input deviation x_dev >= |X_gpu - X|
    moves them), A = bf16(SiLU(G) U) with SiLU from the hardware exp2 and reciprocal
    (a few fp32 ulps), Y = bf16(A W2^T) as an fp32 sum.  Each rounding to bf16 may land
    on any value between the roundings of the interval ends, so an A element near a
    rounding midpoint may take its neighbour (that moves Y by its bf16 spacing times
    |W2|), and Y itself may take its neighbour.  No statistics: every correct result is
    inside, and a missing K-step, tile or expert moves Y by percent of its RMS."""
    import oracle
    x = oracle.decode(x_rows)
    W1, W3, W2 = oracle.decode(w1e), oracle.decode(w3e), oracle.decode(w2e)
    K, I = x.shape[1], W1.shape[0]
    g, u = x @ W1.T, x @ W3.T
    dg, du = fp32_dot_slack(K, _rms_rows(g)), fp32_dot_slack(K, _rms_rows(u))
    if x_dev is not None:
        dg = dg + x_dev @ np.abs(W1).T
        du = du + x_dev @ np.abs(W3).T
    sg = oracle.silu(g)
    a = sg * u
    sig = 0.5 * (1.0 + np.tanh(0.5 * g))
    dsilu = sig * (1.0 + g * (1.0 - sig))             # d SiLU / dG, |.| <= 1.1
    da = np.abs(dsilu * u) * dg + (np.abs(sg) + 1.1 * dg) * du + 8 * U_F32 * np.abs(a)
    A = oracle.round_bf16(a)
    a_lo, a_hi = bf16_round_interval(a, da)
    dA = np.maximum(a_hi - A, A - a_lo)
    yex = A @ W2.T
    dy = dA @ np.abs(W2).T + fp32_dot_slack(I, _rms_rows(yex))
    Y = oracle.round_bf16(yex)
    y_lo, y_hi = bf16_round_interval(yex, dy)
    return np.maximum(y_hi - Y, Y - y_lo)


def check_y_rows(bf16: bool, got: np.ndarray, x_rows, w1e, w3e, w2e, x_dev=None):
    """One expert's outputs Y (got: bf16 bits, or fp32 values for fp32 layers) against the
    oracle's expert FFN on the same rows: bf16 within expert_y_bound per element, fp32
    within 1e-5 x RMS(Y)."""
    import oracle
    ref = oracle.expert_ffn_rows(x_rows, w1e, w3e, w2e, bf16)
    if not bf16:
        assert rel_err(got, ref) <= 1e-5
        return
    bound = expert_y_bound(x_rows, w1e, w3e, w2e, x_dev)
    err = np.abs(oracle.decode(got) - ref)
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    assert np.all(err <= bound), (f"{int(np.sum(err > bound))} of {err.size} Y elements outside the "
                                  f"derived bound (worst {worst:.2f}x)")


def check_grouped_y(bf16: bool, got: np.ndarray, x_perm, offsets, w1, w3, w2):
    """Every non-empty expert's rows of a grouped FFN output against the oracle (check_y_rows)."""
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            check_y_rows(bf16, got[lo:hi], x_perm[lo:hi], w1[e], w3[e], w2[e])


def latent_rows_and_dev(x_rows, wd):
    """The oracle's latent rows Z = bf16(X wd^T) of some tokens, and how far a correct
    GPU Z may be from them per element (its fp32 sum of H products within
    fp32_dot_slack of the exact one, then the same rounding)."""
    import oracle
    Z = oracle.latent_down(x_rows, wd, True)
    z = oracle.decode(x_rows) @ oracle.decode(wd).T
    z_lo, z_hi = bf16_round_interval(z, fp32_dot_slack(wd.shape[1], _rms_rows(z)))
    return Z, np.maximum(z_hi - Z, Z - z_lo)


def layer_out_bound(cfg, inp, ref) -> np.ndarray:
    """Per-element bound on |out_gpu - out_oracle| for a bf16 layer's fp32 output, derived
    from the arithmetic (no statistics): each routed term w_j Y_j may be off by
    w_j times its Y bound (expert_y_bound on the rows the expert received: token rows,
    or for latent layers the oracle's Z with the GPU Z's own derived deviation) plus the
    fp32 routing weight's difference from the oracle's (|dw| <= 1e-6) times |Y_j|; the
    shared expert's output by its own Y bound; the fp32 combine sums k + 1 terms (a few
    fp32 ulps of the sum of magnitudes).  For latent layers the combined row is rounded
    to bf16 (any value between the roundings of its interval ends) and multiplied by
    wu as an fp32 sum.  `ref` is oracle.layer_forward's result on the same inputs."""
    import oracle
    E, k = cfg.E, cfg.k
    rt, tr, offs, w = ref["row_token"], ref["token_row"], ref["offsets"], ref["weights"]
    if cfg.L:
        zs, zdev = latent_rows_and_dev(inp["x"], inp["wd"])
        src, dev_rows = zs, zdev
    else:
        src, dev_rows = inp["x"], None
    yb = np.zeros((int(offs[-1]), cfg.D))
    for e in range(E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi > lo:
            toks = rt[lo:hi]
            yb[lo:hi] = expert_y_bound(src[toks], inp["w1"][e], inp["w3"][e], inp["w2"][e],
                                       None if dev_rows is None else dev_rows[toks])
    Y = oracle.decode(ref["y_perm"]) if ref["y_perm"].dtype == np.uint16 else ref["y_perm"]
    bound = np.zeros((cfg.T, cfg.D))
    mag = np.zeros((cfg.T, cfg.D))
    for j in range(k):
        r = tr[:, j]
        kept = r >= 0
        rr = np.where(kept, r, 0)
        wj = np.where(kept, np.abs(w[:, j]), 0.0)[:, None]
        bound += wj * yb[rr] + np.where(kept, 1e-6, 0.0)[:, None] * np.abs(Y[rr])
        mag += wj * (np.abs(Y[rr]) + yb[rr])
    if "ws1" in inp:
        ysh = oracle.decode(ref["y_shared"]) if ref["y_shared"].dtype == np.uint16 else ref["y_shared"]
        shb = expert_y_bound(inp["x"], inp["ws1"], inp["ws3"], inp["ws2"])
        bound += shb
        mag += np.abs(ysh) + shb
    bound += 4 * (k + 1) * U_F32 * mag
    if cfg.L:
        oc = ref["out_combine"]
        OL = oracle.round_bf16(oc)
        lo_, hi_ = bf16_round_interval(oc, bound)
        dol = np.maximum(hi_ - OL, OL - lo_)
        WU = oracle.decode(inp["wu"])
        out = OL @ WU.T
        bound = dol @ np.abs(WU).T + fp32_dot_slack(cfg.L, _rms_rows(out))
    return bound


def check_layer_out(cfg, inp, ref, got_out: np.ndarray, keep: np.ndarray = None):
    """The layer's fp32 output against the oracle's on every element (of the tokens in
    `keep`): within layer_out_bound for bf16 layers, 1e-5 x RMS for fp32 layers."""
    ref_out = ref["out"]
    if keep is None:
        keep = np.ones(cfg.T, dtype=bool)
    assert not cfg.L, ("latent layers: the worst case of every Z element that may round either way "
                       "moving every G element makes this bound uninformative; their layer check is the "
                       "layer tolerance of 2e-2 x RMS(out)")
    if cfg.dtype != "bf16":
        assert rel_err(got_out[keep], ref_out[keep]) <= 1e-5
        return
    bound = layer_out_bound(cfg, inp, ref)[keep]
    err = np.abs(got_out[keep] - ref_out[keep])
    bad = err > bound
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} outputs outside the derived bound (worst {worst:.2f}x)"
