"""MXFP8 low-precision dispatch -- TEST INFRASTRUCTURE ONLY (part of the oracle).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or run anything here; the product path never does.

What the pages fix: the rows a device sends may travel in a narrower number format
with their scale factors alongside, the expert math may run in that format and the
results come back wide, and a fair comparison includes the conversion work, the
bytes of the scales and the change in the numbers ("Top-k multiplies traffic.
Locality subtracts it.", WideEP explainer); quantising
activations or weights is value-changing ("Three Parameter Counts...", table of
"Which optimizations need a task-level gate").

What they leave open (the format, the scale granularity, the rounding) is read
here as the OCP Microscaling (MX) v1.0 format MXFP8-E4M3, the format the gfx950
matrix cores take with per-block scales:

* element: OCP FP8 E4M3 -- 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
  subnormals, no infinities, S.1111.111 is NaN, largest magnitude 448;
* block: 32 consecutive elements along the contraction (K) axis share one
  E8M0 scale X = 2**(s - 127) (s = 0..254);
* conversion of a block V: X = 2**(floor(log2(max |V_i|)) - 8) (8 = largest
  exponent of E4M3), each P_i = V_i / X rounded to the nearest E4M3 value, ties
  to even, magnitudes beyond 448 saturated to 448.  An all-zero block takes the
  smallest scale (s = 0); the exponent is clamped to [-127, 127].

The expert FFN of an MXFP8 layer contracts the dequantised A and W1 / W3 exactly
(the hardware's products of E4M3 values and power-of-two scales are exact) and
from there follows the bf16 layer: SwiGLU intermediate and Y rounded to bf16,
the down projection in bf16.
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import decode, round_bf16, silu

E4M3_MAX = 448.0
E4M3_EMAX = 8          # largest unbiased exponent of a normal E4M3 value
MX_BLOCK = 32          # elements per shared scale
E8M0_BIAS = 127


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> float64 values (NaN for S.1111.111).

    Normal (exponent field f = 1..15): (-1)^S * 2^(f - 7) * (1 + m/8);
    subnormal (f = 0): (-1)^S * 2^-6 * m/8.
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    f = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(f == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(f - 7.0))
    mag = np.where((f == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Finite float64 values -> E4M3 codes: round to nearest, ties to even, saturate at 448.

    The sign is kept (also for values that round to zero, and -0.0 -> 0x80).
    A magnitude a >= 2^-6 is written a = 2^E * (1 + f) with f in [0, 1); the three
    mantissa bits are rint(8 f), and a carry (rint = 8) moves to the next binade.
    Below 2^-6 the value is a multiple of 2^-9: the code is rint(a / 2^-9), where 8
    lands exactly on the smallest normal's code.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode takes finite values")
    sign = np.signbit(v).astype(np.int64) << 7
    a = np.minimum(np.abs(v), E4M3_MAX)
    mant, e = np.frexp(a)                 # a = mant * 2^e, mant in [0.5, 1)
    E = e.astype(np.int64) - 1            # a = 2^E * (2 mant), 2 mant in [1, 2)
    q = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)
    carry = q == 8
    E = np.where(carry, E + 1, E)
    q = np.where(carry, 0, q)
    normal_code = ((E + 7) << 3) | q
    sub_code = np.rint(a * 2.0 ** 9).astype(np.int64)
    code = np.where(a >= 2.0 ** -6, normal_code, sub_code)
    return (code | sign).astype(np.uint8)


def mx_quantize(v: np.ndarray, block: int = MX_BLOCK):
    """[..., K] values -> (E4M3 codes [..., K] uint8, E8M0 scales [..., K/block] uint8).

    One scale per `block` consecutive elements of the last axis; see the module
    text for the conversion rule.
    """
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    if K % block:
        raise ValueError("last axis must be a multiple of the block")
    b = v.reshape(v.shape[:-1] + (K // block, block))
    amax = np.abs(b).max(axis=-1)
    _, e = np.frexp(amax)                     # floor(log2 amax) = e - 1 for amax > 0
    shared = np.where(amax > 0, e.astype(np.int64) - 1 - E4M3_EMAX, -E8M0_BIAS)
    shared = np.clip(shared, -E8M0_BIAS, E8M0_BIAS)
    codes = e4m3_encode(b / np.exp2(shared.astype(np.float64))[..., None])
    return codes.reshape(v.shape), (shared + E8M0_BIAS).astype(np.uint8)


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, block: int = MX_BLOCK) -> np.ndarray:
    """E4M3 codes [..., K] and E8M0 scales [..., K/block] -> float64 values."""
    vals = e4m3_decode(codes)
    K = vals.shape[-1]
    b = vals.reshape(vals.shape[:-1] + (K // block, block))
    x = np.exp2(np.asarray(scales).astype(np.float64) - E8M0_BIAS)
    return (b * x[..., None]).reshape(vals.shape)


def expert_ffn_rows_mx(xq: np.ndarray, xs: np.ndarray, w1q: np.ndarray, w1s: np.ndarray,
                       w3q: np.ndarray, w3s: np.ndarray, w2e: np.ndarray, parts: bool = False):
    """One expert's SwiGLU FFN with MXFP8 rows and gate/up weights.

    G = A W1^T and U = A W3^T on the dequantised operands, exact; then as the bf16
    layer: the intermediate SiLU(G) * U and the output (intermediate) W2^T are
    rounded to bf16.  w1q / w3q [I x D] with scales [I x D/32]; xq [rows x D] with
    scales [rows x D/32]; w2e [D x I] bf16.  With parts=True also returns the
    intermediates {"x", "w1", "w3", "g", "u", "a"} (dequantised operands, exact G and
    U, rounded A).
    """
    x = mx_dequantize(xq, xs)
    w1 = mx_dequantize(w1q, w1s)
    w3 = mx_dequantize(w3q, w3s)
    g = x @ w1.T
    u = x @ w3.T
    a = round_bf16(silu(g) * u)
    y = round_bf16(a @ decode(w2e).T)
    if parts:
        return y, {"x": x, "w1": w1, "w3": w3, "g": g, "u": u, "a": a}
    return y


def grouped_expert_ffn_mx(xq: np.ndarray, xs: np.ndarray, offsets: np.ndarray, w1q, w1s, w3q, w3s,
                          w2: np.ndarray, parts: bool = False):
    """Expert e runs expert_ffn_rows_mx on rows [offsets[e], offsets[e+1]).  With
    parts=True also returns, per expert with rows, (e, lo, hi, intermediates)."""
    E = len(offsets) - 1
    y = np.zeros((int(offsets[-1]), w2.shape[1]), dtype=np.float64)
    pieces = []
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            r = expert_ffn_rows_mx(xq[lo:hi], xs[lo:hi], w1q[e], w1s[e], w3q[e], w3s[e], w2[e], parts)
            if parts:
                y[lo:hi], pr = r
                pieces.append((e, lo, hi, pr))
            else:
                y[lo:hi] = r
    return (y, pieces) if parts else y


def dispatch_bytes_mx(rows: int, width: int) -> int:
    """Bytes of an MXFP8 dispatch of `rows` rows of `width` elements: one byte per
    element plus one scale byte per 32 elements (the scale metadata the pages ask
    to count)."""
    return rows * width + rows * (width // MX_BLOCK)
