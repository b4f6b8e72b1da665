"""Pins of the MXFP8 oracle (oracle.mxfp8) against things other than itself.

* E4M3 decoding and rounding against torch's own float8_e4m3fn conversion (an
  independent library routine), over every code and every bf16 bit pattern in range;
* closed forms: saturation, ties to even between neighbouring codes, a block worked
  by hand, power-of-two equivariance of the block scale, the error bound of the
  format;
* the MXFP8 expert FFN equals the (separately pinned) bf16 expert FFN whenever the
  operands are exactly representable, which fixes how codes and scales combine.
"""
import numpy as np
import pytest
import torch

from oracle import mxfp8 as M
from oracle import moe_oracle as O


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def torch_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


ALL = np.arange(256, dtype=np.uint8)
FINITE = ALL[(ALL & 0x7F) != 0x7F]


def test_decode_matches_torch_on_every_code():
    ours, ref = M.e4m3_decode(ALL), torch_decode(ALL).astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    assert np.nanmax(ours) == 448.0 and M.e4m3_decode(np.array([1]))[0] == 2.0 ** -9


def test_encode_matches_torch_on_all_bf16_patterns_in_range():
    bits = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    x = bits[np.isfinite(bits) & (np.abs(bits) <= 464.0)]   # torch saturates only up to 464
    np.testing.assert_array_equal(M.e4m3_encode(x.astype(np.float64)), torch_encode(x))


def test_encode_matches_torch_on_off_grid_fp32():
    r = np.random.default_rng(0)
    x = (r.standard_normal(200000) * np.exp2(r.integers(-14, 9, 200000))).astype(np.float32)
    x = x[np.abs(x) <= 464.0]
    np.testing.assert_array_equal(M.e4m3_encode(x.astype(np.float64)), torch_encode(x))


def test_encode_saturates_beyond_448():
    x = np.array([448.0, 450.0, 464.0, 464.5, 479.9, 480.0, 1e6, 3.4e38])
    np.testing.assert_array_equal(M.e4m3_encode(x), np.full(len(x), 0x7E, np.uint8))
    np.testing.assert_array_equal(M.e4m3_encode(-x), np.full(len(x), 0xFE, np.uint8))


def test_round_trip_and_ties_to_even():
    np.testing.assert_array_equal(M.e4m3_encode(M.e4m3_decode(FINITE)), FINITE)
    pos = np.arange(0, 0x7E, dtype=np.uint8)            # neighbours c, c + 1 up to 448
    lo, hi = M.e4m3_decode(pos), M.e4m3_decode(pos + 1)
    mid = (lo + hi) / 2
    even = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint8)
    np.testing.assert_array_equal(M.e4m3_encode(mid), even)
    np.testing.assert_array_equal(M.e4m3_encode(-mid), even | 0x80)
    # just off the midpoint goes to the nearer code
    np.testing.assert_array_equal(M.e4m3_encode(mid - (hi - lo) * 1e-3), pos)
    np.testing.assert_array_equal(M.e4m3_encode(mid + (hi - lo) * 1e-3), pos + 1)


def test_block_worked_by_hand():
    # amax 3 = 1.5 * 2^1: X = 2^(1 - 8) = 2^-7, scale code 127 - 7 = 120.
    # 1.0 * 2^7 = 128 = 2^7: field 7 + 7 = 14, mantissa 0 -> 0x70 = 112
    # -0.75 * 2^7 = -96 = -1.5 * 2^6: sign, field 13, mantissa 4 -> 0x80 | 0x6C = 236
    # 2^-9 * 2^7 = 2^-2: field 5, mantissa 0 -> 40
    # 3 * 2^7 = 384 = 1.5 * 2^8: field 15, mantissa 4 -> 124
    v = np.zeros((1, 32))
    v[0, :4] = [1.0, -0.75, 2.0 ** -9, 3.0]
    q, s = M.mx_quantize(v)
    assert s.tolist() == [[120]]
    assert q[0, :4].tolist() == [112, 236, 40, 124] and not q[0, 4:].any()
    # amax 1.9: X = 2^-8, 1.9 * 256 = 486.4 saturates to 448
    v2 = np.zeros((1, 32))
    v2[0, 0], v2[0, 1] = 1.9, -1.9
    q2, s2 = M.mx_quantize(v2)
    assert s2.tolist() == [[119]] and q2[0, :2].tolist() == [0x7E, 0xFE]
    # an all-zero block takes the smallest scale
    q3, s3 = M.mx_quantize(np.zeros((2, 64)))
    assert not q3.any() and s3.tolist() == [[0, 0], [0, 0]]


def test_scale_is_per_block_and_power_of_two_equivariant():
    r = np.random.default_rng(1)
    v = r.standard_normal((6, 128)) * np.exp2(r.integers(-8, 8, (6, 1)))
    q, s = M.mx_quantize(v)
    for j in (-5, 3, 11):
        qj, sj = M.mx_quantize(v * 2.0 ** j)
        np.testing.assert_array_equal(qj, q)
        np.testing.assert_array_equal(sj.astype(int), s.astype(int) + j)
    np.testing.assert_array_equal(M.mx_quantize(-v)[0], q ^ 0x80)
    w = v.copy()
    w[:, 32:64] *= 1000.0                       # one block changes; the others keep codes and scales
    qw, sw = M.mx_quantize(w)
    keep = np.r_[0:32, 64:128]
    np.testing.assert_array_equal(qw[:, keep], q[:, keep])
    np.testing.assert_array_equal(sw[:, [0, 2, 3]], s[:, [0, 2, 3]])


def test_error_bound_of_the_format():
    r = np.random.default_rng(2)
    v = r.standard_normal((64, 256)) * np.exp2(r.integers(-20, 20, (64, 8))).repeat(32, axis=1)
    q, s = M.mx_quantize(v)
    d = M.mx_dequantize(q, s)
    X = np.exp2(s.astype(float) - 127).repeat(32, axis=1)
    a = np.abs(v)
    _, e = np.frexp(np.maximum(a, 1e-300))
    half_ulp = np.maximum(np.exp2(e - 1.0 - 4.0), 2.0 ** -10 * X)  # 3 mantissa bits / subnormal step
    sat = a > 448 * X
    assert np.all(np.abs(d - v)[~sat] <= half_ulp[~sat] * (1 + 1e-12))
    np.testing.assert_array_equal(np.abs(d[sat]), 448 * X[sat])
    assert np.all(a[sat] < 512 * X[sat])          # only the top of a block can saturate


def _representable(r, shape):
    """Values n * 2^j (|n| <= 14, one |n| >= 8 per block of 32): MX quantisation is exact."""
    n = r.integers(-14, 15, shape)
    blocks = n.reshape(shape[:-1] + (shape[-1] // 32, 32))
    blocks[..., 0] = np.where(r.integers(0, 2, blocks.shape[:-1]) == 1, 1, -1) * r.integers(8, 15, blocks.shape[:-1])
    j = r.integers(-12, -3, blocks.shape[:-1] + (1,))
    return (blocks * np.exp2(j)).reshape(shape)


def _to_bf16_bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_exact_operands_quantise_losslessly():
    r = np.random.default_rng(3)
    v = _representable(r, (10, 96))
    q, s = M.mx_quantize(v)
    np.testing.assert_array_equal(M.mx_dequantize(q, s), v)


def test_mx_ffn_equals_bf16_ffn_on_exact_operands():
    r = np.random.default_rng(4)
    D, I, rows = 64, 96, 7
    x = _representable(r, (rows, D))
    w1 = _representable(r, (I, D))
    w3 = _representable(r, (I, D))
    w2 = _to_bf16_bits(r.standard_normal((D, I)) * 0.05)
    xq, xs = M.mx_quantize(x)
    w1q, w1s = M.mx_quantize(w1)
    w3q, w3s = M.mx_quantize(w3)
    got = M.expert_ffn_rows_mx(xq, xs, w1q, w1s, w3q, w3s, w2)
    ref = O.expert_ffn_rows(_to_bf16_bits(x), _to_bf16_bits(w1), _to_bf16_bits(w3), w2, True)
    np.testing.assert_array_equal(got, ref)
    # swapping the two scale blocks of a row changes the result (scales are per block)
    bad = w1s.copy()
    bad[:, [0, 1]] = bad[:, [1, 0]]
    if not np.array_equal(bad, w1s):
        assert not np.array_equal(M.expert_ffn_rows_mx(xq, xs, w1q, bad, w3q, w3s, w2), ref)


def test_layer_forward_mxfp8_equals_per_expert_definition():
    from workloads import PARITY_CONFIGS, generator as gen
    cfg = PARITY_CONFIGS["small_bf16_zipf"]
    inp = gen.layer_inputs(cfg)
    res = O.layer_forward(inp, k=cfg.k, E=cfg.E, bf16=True, dispatch="mxfp8")
    base = O.layer_forward(inp, k=cfg.k, E=cfg.E, bf16=True)
    np.testing.assert_array_equal(res["ids"], base["ids"])      # routing does not see the format
    # token-by-token definition: out[t] = sum_j w[t, j] * FFN_mx_{ids[t, j]}(quantised x_t)
    x = O.decode(inp["x"])
    t = 5
    ref = np.zeros(cfg.H)
    for j in range(cfg.k):
        e = res["ids"][t, j]
        xq, xs = M.mx_quantize(x[t:t + 1])
        w1q, w1s = M.mx_quantize(O.decode(inp["w1"][e]))
        w3q, w3s = M.mx_quantize(O.decode(inp["w3"][e]))
        ref += res["weights"][t, j] * M.expert_ffn_rows_mx(xq, xs, w1q, w1s, w3q, w3s, inp["w2"][e])[0]
    np.testing.assert_allclose(res["out"][t], ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    # the value change is visible but small next to the output
    rel = np.abs(res["out"] - base["out"]).max() / np.sqrt(np.mean(base["out"] ** 2))
    assert 1e-4 < rel < 0.5
    assert M.dispatch_bytes_mx(cfg.R, cfg.D) == cfg.R * cfg.D * 33 // 32


def test_planted_mistakes_fail():
    """Plausible oracle mistakes fail the comparisons the pins above make."""
    # bias 8 (the gfx942 FNUZ layout) instead of 7
    fnuz = M.e4m3_decode(FINITE) / 2
    assert not np.array_equal(fnuz, torch_decode(FINITE).astype(np.float64))
    # truncation instead of round to nearest: the largest code not above |x|
    x = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    x = x[np.isfinite(x) & (x >= 0) & (x <= 448.0)].astype(np.float64)
    table = M.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    trunc = (np.searchsorted(table, x, side="right") - 1).astype(np.uint8)
    assert not np.array_equal(trunc, torch_encode(x.astype(np.float32)))
    # scale from the block mean instead of the block maximum
    v = np.zeros((1, 32))
    v[0, 0], v[0, 1] = 3.0, 0.5
    _, e = np.frexp(np.abs(v).mean())
    assert M.mx_quantize(v)[1][0, 0] != e - 1 - 8 + 127
