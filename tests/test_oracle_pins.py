"""Pins of the CPU oracle against things other than itself (CPU only).

Each test fixes one oracle function with a library routine on a special case,
brute force on tiny inputs, a closed form, an invariant, or a worked number
printed on the pages (tests/golden/pages_worked_numbers.json).  The pins are
chosen so that a dropped term, a wrong sign or index, or a transposed operand
in the oracle fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import PARITY_CONFIGS, TINY_F32, generator as gen

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "pages_worked_numbers.json")))


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ element formats

def test_decode_known_bf16_bits():
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x0000, 0x8000, 0x4049], dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.decode(bits), ref)
    assert oracle.decode(bits)[0] == 1.0 and oracle.decode(bits)[1] == -2.0


def test_round_bf16_matches_torch_on_fp32_values():
    a = _rng(1).standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    ref = torch.from_numpy(a).bfloat16().double().numpy()
    np.testing.assert_array_equal(oracle.round_bf16(a.astype(np.float64)), ref)


def test_round_bf16_ties_to_even():
    u = 2.0 ** -8
    cases = {1 + u: 1.0, 1 + 3 * u: 1 + 4 * u, -(1 + u): -1.0, 1 + 1.5 * u: 1 + 2 * u,
             0.0: 0.0, 3.0: 3.0}
    for x, want in cases.items():
        assert oracle.round_bf16(np.array([x]))[0] == want, x


def test_round_bf16_agrees_with_generator_rounding():
    # two independent implementations (frexp/rint here, bit arithmetic in the generator)
    a = _rng(2).standard_normal(100_000).astype(np.float32) * np.float32(0.02)
    np.testing.assert_array_equal(oracle.decode(gen.f32_to_bf16_bits(a)),
                                  oracle.round_bf16(a.astype(np.float64)))


# ------------------------------------------------------------------ a1 gate

def test_gate_logits_brute_force():
    r = _rng(3)
    x = r.standard_normal((5, 7)).astype(np.float32)
    wg = r.standard_normal((4, 7)).astype(np.float32)     # stored [E x H]
    b = r.standard_normal(4).astype(np.float32)
    got = oracle.gate_logits(x, wg, b)
    for t in range(5):
        for e in range(4):
            want = math.fsum(float(x[t, h]) * float(wg[e, h]) for h in range(7)) + float(b[e])
            assert abs(got[t, e] - want) <= 1e-12 * (1 + abs(want))
    np.testing.assert_allclose(oracle.gate_logits(x, wg), got - b.astype(np.float64), rtol=0,
                               atol=1e-12)


def test_router_scores_fp32_add():
    r = _rng(4)
    lg = r.standard_normal((6, 5)).astype(np.float32)
    b = r.standard_normal(5).astype(np.float32)
    np.testing.assert_array_equal(oracle.router_scores(lg, None), lg)
    ref = (torch.from_numpy(lg) + torch.from_numpy(b)[None, :]).numpy()
    got = oracle.router_scores(lg, b)
    assert got.dtype == np.float32
    np.testing.assert_array_equal(got, ref)


# ------------------------------------------------------------------ a2 top-k

def _brute_topk(s, k):
    E = len(s)
    return sorted(range(E), key=lambda e: (-float(s[e]), e))[:k]


@pytest.mark.parametrize("T,E,k", [(50, 8, 2), (40, 16, 5), (30, 7, 7), (60, 12, 1)])
def test_topk_matches_stable_argsort_and_brute_force(T, E, k):
    r = _rng(T * E + k)
    # integer-valued scores: many ties
    s = r.integers(-3, 4, size=(T, E)).astype(np.float32)
    got = oracle.topk_ids(s, k)
    lib = np.argsort(-s.astype(np.float64), axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(got, lib)
    for t in range(T):
        assert got[t].tolist() == _brute_topk(s[t], k)


def test_topk_special_cases():
    T, E, k = 9, 10, 4
    same = np.full((T, E), 0.25, dtype=np.float32)
    np.testing.assert_array_equal(oracle.topk_ids(same, k), np.tile(np.arange(k), (T, 1)))
    s = _rng(5).standard_normal((T, E)).astype(np.float32)
    np.testing.assert_array_equal(oracle.topk_ids(s, 1)[:, 0], np.argmax(s, axis=1))
    full = oracle.topk_ids(s, E)
    np.testing.assert_array_equal(full, np.argsort(-s, axis=1, kind="stable"))
    # -0.0 ranks equal to +0.0: ties go to the lower index either way
    z = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], dtype=np.float32)
    np.testing.assert_array_equal(oracle.topk_ids(z, 2), [[0, 1], [0, 1]])
    # -inf scores are selectable when nothing larger remains
    ninf = np.array([[-np.inf, 1.0, -np.inf, -np.inf]], dtype=np.float32)
    np.testing.assert_array_equal(oracle.topk_ids(ninf, 3), [[1, 0, 2]])


def test_topk_ids_distinct_per_token():
    s = _rng(6).standard_normal((200, 32)).astype(np.float32)
    ids = oracle.topk_ids(s, 8)
    for row in ids:
        assert len(set(row.tolist())) == 8


# ------------------------------------------------------------------ a2 weights

def test_routing_weights_properties():
    r = _rng(7)
    s = (r.standard_normal((100, 16)) * 2).astype(np.float32)
    ids = oracle.topk_ids(s, 4)
    w = oracle.routing_weights(s, ids)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 1e-17)                 # non-increasing along j
    # closed form: selected-only softmax (the full denominator cancels)
    sel = np.take_along_axis(s.astype(np.float64), ids.astype(np.int64), axis=1)
    ez = np.exp(sel - sel.max(axis=1, keepdims=True))
    np.testing.assert_allclose(w, ez / ez.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)
    # invariant to adding a constant per token
    shift = (s.astype(np.float64) + 37.0)
    np.testing.assert_allclose(oracle.routing_weights(shift, ids), w, rtol=1e-12, atol=0)


def test_routing_weights_k_equals_e_is_softmax():
    s = _rng(8).standard_normal((20, 9)).astype(np.float32)
    ids = oracle.topk_ids(s, 9)
    w = oracle.routing_weights(s, ids)
    ref = torch.softmax(torch.from_numpy(s).double(), dim=1).numpy()
    np.testing.assert_allclose(w, np.take_along_axis(ref, ids.astype(np.int64), axis=1),
                               rtol=1e-13, atol=0)


# ------------------------------------------------------------------ a3 counts / offsets

def test_counts_and_offsets_match_library():
    s = _rng(9).standard_normal((333, 24)).astype(np.float32)
    ids = oracle.topk_ids(s, 6)
    c = oracle.expert_counts(ids, 24)
    np.testing.assert_array_equal(c, np.bincount(ids.ravel(), minlength=24))
    off = oracle.segment_offsets(c)
    np.testing.assert_array_equal(off[1:], np.cumsum(np.bincount(ids.ravel(), minlength=24)))
    assert off[0] == 0 and off[-1] == 333 * 6


def test_counts_are_assignments_golden():
    g = GOLDEN["top2_rows_per_token"]
    T, E = 41, 5
    s = _rng(10).standard_normal((T, E)).astype(np.float32)
    ids = oracle.topk_ids(s, g["k"])
    assert oracle.expert_counts(ids, E).sum() == g["rows_per_token"] * T
    g16 = GOLDEN["top16_payloads_per_token"]
    s = _rng(11).standard_normal((3, 64)).astype(np.float32)
    assert oracle.expert_counts(oracle.topk_ids(s, g16["k"]), 64).sum() == 3 * g16["payloads_out"]


def test_all_ties_counts():
    T, E, k = 17, 6, 3
    ids = oracle.topk_ids(np.zeros((T, E), dtype=np.float32), k)
    np.testing.assert_array_equal(oracle.expert_counts(ids, E), [T] * k + [0] * (E - k))


# ------------------------------------------------------------------ a4 permutation

@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (37, 16, 4), (1, 5, 5), (20, 1, 1)])
def test_permutation_stable_sort_and_inverse(T, E, k):
    s = _rng(12 + T).integers(-2, 3, size=(T, E)).astype(np.float32)
    ids = oracle.topk_ids(s, k)
    rt, tr = oracle.permutation(ids, E)
    lib = np.argsort(ids.ravel(), kind="stable")
    np.testing.assert_array_equal(rt, lib // k)
    flat = np.empty(T * k, dtype=np.int64)
    flat[lib] = np.arange(T * k)
    np.testing.assert_array_equal(tr.ravel(), flat)
    np.testing.assert_array_equal(tr.ravel()[lib], np.arange(T * k))     # inverse
    off = oracle.segment_offsets(oracle.expert_counts(ids, E))
    for e in range(E):
        seg = rt[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)                          # ascending tokens
        assert all(e in ids[t] for t in seg.tolist())


def test_permute_then_unpermute_is_identity_bitwise():
    cfg = TINY_F32
    x = gen.activations(cfg)
    ids = oracle.topk_ids(gen.drawn_logits(cfg), cfg.k)
    rt, tr = oracle.permutation(ids, cfg.E)
    xp = oracle.gather_rows(x, rt)
    for t in range(cfg.T):
        for j in range(cfg.k):
            assert xp[tr[t, j]].tobytes() == x[t].tobytes()
    xb = gen.f32_to_bf16_bits(x)
    xpb = oracle.gather_rows(xb, rt)
    assert xpb.dtype == np.uint16
    np.testing.assert_array_equal(xpb[tr[:, 1]], xb)


def test_dispatch_bytes_golden():
    g = GOLDEN["halving_topk_halves_dispatch"]
    T, H = 4096, 2048
    b8 = oracle.dispatch_bytes(T, g["k_before"], H, 2)
    b4 = oracle.dispatch_bytes(T, g["k_after"], H, 2)
    assert b4 / b8 == g["bytes_ratio"]
    # equals the bytes of the real permuted buffer (no padding on one device)
    cfg = TINY_F32
    ids = oracle.topk_ids(gen.drawn_logits(cfg), cfg.k)
    xp = oracle.gather_rows(gen.activations(cfg), oracle.permutation(ids, cfg.E)[0])
    assert xp.nbytes == oracle.dispatch_bytes(cfg.T, cfg.k, cfg.H, 4)
    # latent dispatch width vs full width (latent layer shape)
    assert oracle.dispatch_bytes(4096, 8, 2048, 2) * 7168 == oracle.dispatch_bytes(4096, 8, 7168, 2) * 2048


# ------------------------------------------------------------------ a5 experts

def test_silu_matches_torch():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(),
                               rtol=1e-14, atol=1e-300)


def _torch_swiglu(x, w1, w3, w2):
    F = torch.nn.functional
    X = torch.from_numpy(x).double()
    return F.linear(F.silu(F.linear(X, torch.from_numpy(w1).double())) *
                    F.linear(X, torch.from_numpy(w3).double()),
                    torch.from_numpy(w2).double()).numpy()


def test_one_expert_top1_is_plain_swiglu():
    r = _rng(13)
    T, H, I = 11, 12, 20
    x = r.standard_normal((T, H)).astype(np.float32)
    w1, w3 = (r.standard_normal((1, I, H)) * 0.3).astype(np.float32), (r.standard_normal((1, I, H)) * 0.3).astype(np.float32)
    w2 = (r.standard_normal((1, H, I)) * 0.3).astype(np.float32)
    inp = {"x": x, "logits": r.standard_normal((T, 1)).astype(np.float32), "w1": w1, "w3": w3, "w2": w2}
    res = oracle.layer_forward(inp, k=1, E=1, bf16=False)
    np.testing.assert_allclose(res["out"], _torch_swiglu(x, w1[0], w3[0], w2[0]), rtol=1e-12, atol=1e-12)


def test_sparse_layer_equals_masked_dense_brute_force():
    r = _rng(14)
    T, H, E, k, I = 23, 10, 6, 3, 14
    x = r.standard_normal((T, H)).astype(np.float32)
    w1 = (r.standard_normal((E, I, H)) * 0.3).astype(np.float32)
    w3 = (r.standard_normal((E, I, H)) * 0.3).astype(np.float32)
    w2 = (r.standard_normal((E, H, I)) * 0.3).astype(np.float32)
    lg = r.standard_normal((T, E)).astype(np.float32)
    res = oracle.layer_forward({"x": x, "logits": lg, "w1": w1, "w3": w3, "w2": w2}, k=k, E=E, bf16=False)
    # dense: every expert on every token, then mask with the top-k weights
    p = np.exp(lg.astype(np.float64) - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    mask = np.zeros((T, E))
    for t in range(T):
        top = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:k]
        mask[t, top] = p[t, top] / p[t, top].sum()
    dense = sum(mask[:, e:e + 1] * _torch_swiglu(x, w1[e], w3[e], w2[e]) for e in range(E))
    np.testing.assert_allclose(res["out"], dense, rtol=1e-11, atol=1e-12)


def test_identical_experts_and_zero_up_branch():
    r = _rng(15)
    T, H, E, k, I = 19, 8, 5, 2, 12
    x = r.standard_normal((T, H)).astype(np.float32)
    one1 = (r.standard_normal((I, H)) * 0.3).astype(np.float32)
    one3 = (r.standard_normal((I, H)) * 0.3).astype(np.float32)
    one2 = (r.standard_normal((H, I)) * 0.3).astype(np.float32)
    w1, w3, w2 = (np.stack([m] * E) for m in (one1, one3, one2))
    lg = r.standard_normal((T, E)).astype(np.float32)
    res = oracle.layer_forward({"x": x, "logits": lg, "w1": w1, "w3": w3, "w2": w2}, k=k, E=E, bf16=False)
    np.testing.assert_allclose(res["out"], _torch_swiglu(x, one1, one3, one2), rtol=1e-12, atol=1e-13)
    res0 = oracle.layer_forward({"x": x, "logits": lg, "w1": w1, "w3": np.zeros_like(w3), "w2": w2},
                                k=k, E=E, bf16=False)
    assert np.all(res0["out"] == 0.0)


def test_empty_experts_weights_never_read():
    r = _rng(16)
    T, H, E, k, I = 9, 8, 12, 2, 8
    x = r.standard_normal((T, H)).astype(np.float32)
    lg = r.standard_normal((T, E)).astype(np.float32)
    lg[:, 6:] = -50.0                                            # experts 6.. never chosen
    w1 = (r.standard_normal((E, I, H)) * 0.3).astype(np.float32)
    w3 = (r.standard_normal((E, I, H)) * 0.3).astype(np.float32)
    w2 = (r.standard_normal((E, H, I)) * 0.3).astype(np.float32)
    base = oracle.layer_forward({"x": x, "logits": lg, "w1": w1, "w3": w3, "w2": w2}, k=k, E=E, bf16=False)
    for w in (w1, w3, w2):
        w[6:] = np.nan
    pois = oracle.layer_forward({"x": x, "logits": lg, "w1": w1, "w3": w3, "w2": w2}, k=k, E=E, bf16=False)
    assert np.isfinite(pois["out"]).all()
    np.testing.assert_array_equal(pois["out"], base["out"])


def test_bf16_rounding_points_are_bf16():
    cfg = PARITY_CONFIGS["small_bf16_zipf"]
    inp = gen.layer_inputs(cfg)
    res = oracle.layer_forward(inp, k=cfg.k, E=cfg.E, bf16=True)
    y = res["y_perm"]
    np.testing.assert_array_equal(oracle.round_bf16(y), y)
    # Y lies within half a bf16 ulp of the unrounded product of the (rounded) A
    e = int(np.argmax(res["counts"]))
    lo, hi = int(res["offsets"][e]), int(res["offsets"][e + 1])
    xr = res["x_perm"][lo:hi]
    a = oracle.round_bf16(oracle.silu(xr @ oracle.decode(inp["w1"][e]).T) * (xr @ oracle.decode(inp["w3"][e]).T))
    yr = a @ oracle.decode(inp["w2"][e]).T
    ulp = 2.0 ** (np.floor(np.log2(np.abs(yr) + 1e-300)) - 7)
    assert np.all(np.abs(y[lo:hi] - yr) <= 0.5 * ulp + 1e-300)


# ------------------------------------------------------------------ a6 combine

def test_combine_of_token_major_rows_is_weight_sum():
    r = _rng(17)
    T, E, k, D = 31, 9, 3, 6
    s = r.standard_normal((T, E)).astype(np.float32)
    ids = oracle.topk_ids(s, k)
    w = oracle.routing_weights(s, ids)
    rt, tr = oracle.permutation(ids, E)
    V = r.standard_normal((T, D))
    out = oracle.combine(V[rt], tr, w)          # every assignment of t carries V[t]
    np.testing.assert_allclose(out, V * w.sum(axis=1, keepdims=True), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(out, V, rtol=1e-14, atol=1e-15)
    # brute force on one token
    t = 4
    want = sum(w[t, j] * V[rt][tr[t, j]] for j in range(k))
    np.testing.assert_allclose(out[t], want, rtol=1e-15, atol=0)


# ------------------------------------------------------------------ a7 latent

def test_latent_identity_projections_reduce_to_plain_layer():
    cfg = PARITY_CONFIGS["small_latent"]
    r = _rng(18)
    H = 16
    T, E, k, I = 21, cfg.E, cfg.k, 24
    x = gen.f32_to_bf16_bits(r.standard_normal((T, H)).astype(np.float32))
    w1 = gen.f32_to_bf16_bits((r.standard_normal((E, I, H)) * 0.2).astype(np.float32))
    w3 = gen.f32_to_bf16_bits((r.standard_normal((E, I, H)) * 0.2).astype(np.float32))
    w2 = gen.f32_to_bf16_bits((r.standard_normal((E, H, I)) * 0.2).astype(np.float32))
    lg = r.standard_normal((T, E)).astype(np.float32)
    eye = gen.f32_to_bf16_bits(np.eye(H, dtype=np.float32))
    base = oracle.layer_forward({"x": x, "logits": lg, "w1": w1, "w3": w3, "w2": w2}, k=k, E=E, bf16=True)
    lat = oracle.layer_forward({"x": x, "logits": lg, "w1": w1, "w3": w3, "w2": w2, "wd": eye, "wu": eye},
                               k=k, E=E, bf16=True)
    np.testing.assert_array_equal(lat["z"], oracle.decode(x))
    np.testing.assert_array_equal(lat["out"], oracle.round_bf16(base["out"]))
    # down-projection is the transposed storage: Z = X Wd with wd stored [L x H]
    wd = gen.f32_to_bf16_bits((r.standard_normal((5, H)) * 0.2).astype(np.float32))
    np.testing.assert_array_equal(oracle.latent_down(x, wd, bf16=False),
                                  torch.nn.functional.linear(torch.from_numpy(oracle.decode(x)),
                                                             torch.from_numpy(oracle.decode(wd))).numpy())


# ------------------------------------------------------------------ measurements

def test_skew_and_p95():
    assert oracle.load_skew(np.array([4, 0, 0, 0]), T=2, k=2) == 4.0
    assert oracle.load_skew(np.array([2, 2, 2, 2]), T=4, k=2) == 1.0
    v = list(range(1, 21))
    assert oracle.p95_nearest_rank(v) == 19
    assert oracle.p95_nearest_rank(list(range(100, 0, -1))) == 95
    vals = _rng(19).random(37)
    assert oracle.p95_nearest_rank(vals) == np.percentile(vals, 95, method="inverted_cdf")


def test_routing_margins():
    s = np.array([[3.0, 1.0, 2.5, 0.0], [1.0, 1.0, 0.0, 0.0]])
    np.testing.assert_allclose(oracle.routing_margins(s, 2), [0.5, 0.0])


def test_context_numbers_golden():
    g = GOLDEN
    k3 = g["k3_active_fraction"]
    assert round(100 * k3["active"] / k3["experts"], 1) == k3["fraction_percent_approx"]
    assert k3["experts"] - k3["active"] == k3["idle"]
    ep = g["k3_ep64_experts_per_rank"]
    assert ep["experts"] // ep["ranks"] == ep["per_rank"]
    assert g["r1_ep8_experts_per_gpu"]["experts"] // g["r1_ep8_experts_per_gpu"]["gpus"] == 32
    assert g["r1_ep64_experts_per_gpu"]["experts"] // g["r1_ep64_experts_per_gpu"]["gpus"] == 4
    c = g["r1_ep8_cold_share"]
    assert 100 * (c["local_experts"] - c["max_active_local"]) / c["local_experts"] == c["cold_percent"]
    q = g["qwen3_30b_resident_bytes"]
    b = q["params"] * q["bytes_per_param"]
    assert b / 1e9 == q["gb_decimal"] and round(b / 2 ** 30, 1) == q["gib"]


# ------------------------------------------------------------------ planted mistakes

def test_pins_catch_planted_mistakes():
    """The brute-force pin must reject an oracle with a transposed operand or dropped term."""
    r = _rng(20)
    T, H, E, k, I = 7, 6, 4, 2, 6
    x = r.standard_normal((T, H)).astype(np.float32)
    w1 = (r.standard_normal((E, I, H)) * 0.3).astype(np.float32)
    w3 = (r.standard_normal((E, I, H)) * 0.3).astype(np.float32)
    w2 = (r.standard_normal((E, H, I)) * 0.3).astype(np.float32)
    good = oracle.expert_ffn_rows(x, w1[0], w3[0], w2[0], bf16=False)
    ref = _torch_swiglu(x, w1[0], w3[0], w2[0])
    np.testing.assert_allclose(good, ref, rtol=1e-12, atol=1e-13)
    # planted: up and gate branches swapped / up branch dropped
    swapped = oracle.expert_ffn_rows(x, w3[0], w1[0], w2[0], bf16=False)
    assert not np.allclose(swapped, ref, rtol=1e-6, atol=1e-6)
    dropped = (oracle.silu(x @ w1[0].T.astype(np.float64))) @ w2[0].T.astype(np.float64)
    assert not np.allclose(dropped, ref, rtol=1e-6, atol=1e-6)
    # planted: ties broken toward the higher index
    s = np.array([[1.0, 1.0, 0.0]], dtype=np.float32)
    assert oracle.topk_ids(s, 1)[0, 0] == 0
    assert np.argsort(-s[0], kind="stable")[0] == 0 and np.argsort(s[0])[::-1][0] != 0


def test_token_outputs_match_whole_layer():
    """The sampled-token evaluation (full-size layers) equals the whole-layer oracle's rows."""
    for name in ("small_bf16_zipf", "small_latent"):
        cfg = PARITY_CONFIGS[name]
        inp = gen.layer_inputs(cfg)
        ref = oracle.layer_forward(inp, k=cfg.k, E=cfg.E, bf16=True)
        tok = np.array([0, 3, 7, 11, cfg.T - 1])
        ew = {e: (inp["w1"][e], inp["w3"][e], inp["w2"][e]) for e in range(cfg.E)}
        z = ref["z"][tok] if cfg.L else None
        got = oracle.token_outputs(inp, tok, ref["ids"][tok], ref["weights"][tok], ew, bf16=True, z=z)
        np.testing.assert_allclose(got, ref["out"][tok], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ shared expert

def test_shared_expert_is_swiglu_of_every_token():
    """The shared expert is the SwiGLU FFN on all T rows, independent of the routing."""
    r = _rng(30)
    T, H, Is = 13, 10, 18
    x = r.standard_normal((T, H)).astype(np.float32)
    ws1, ws3 = ((r.standard_normal((Is, H)) * 0.3).astype(np.float32) for _ in range(2))
    ws2 = (r.standard_normal((H, Is)) * 0.3).astype(np.float32)
    np.testing.assert_allclose(oracle.shared_expert_ffn(x, ws1, ws3, ws2, bf16=False),
                               _torch_swiglu(x, ws1, ws3, ws2), rtol=1e-12, atol=1e-13)


def test_shared_expert_enters_with_weight_one():
    """Two routed experts and the shared expert all equal to one FFN: the routing
    weights sum to 1, so the layer is exactly twice that FFN (a shared term scaled by
    a routing weight would give (1 + w) FFN instead)."""
    r = _rng(31)
    T, H, E, k, I = 17, 8, 2, 2, 12
    x = r.standard_normal((T, H)).astype(np.float32)
    f1 = (r.standard_normal((I, H)) * 0.3).astype(np.float32)
    f3 = (r.standard_normal((I, H)) * 0.3).astype(np.float32)
    f2 = (r.standard_normal((H, I)) * 0.3).astype(np.float32)
    inp = {"x": x, "logits": r.standard_normal((T, E)).astype(np.float32),
           "w1": np.stack([f1] * E), "w3": np.stack([f3] * E), "w2": np.stack([f2] * E),
           "ws1": f1, "ws3": f3, "ws2": f2}
    res = oracle.layer_forward(inp, k=k, E=E, bf16=False)
    ffn = _torch_swiglu(x, f1, f3, f2)
    np.testing.assert_allclose(res["out"], 2.0 * ffn, rtol=1e-12, atol=1e-13)
    # planted: the shared term weighted by the first routing weight
    wrong = oracle.combine(res["y_perm"], res["token_row"], res["weights"]) + \
        res["weights"][:, :1] * res["y_shared"]
    assert not np.allclose(wrong, 2.0 * ffn, rtol=1e-6, atol=1e-6)


def test_shared_expert_with_zero_up_branch_adds_nothing():
    cfg = PARITY_CONFIGS["shared_expert"]
    inp = gen.layer_inputs(cfg)
    plain = {n: v for n, v in inp.items() if n not in ("ws1", "ws3", "ws2")}
    zero = dict(inp, ws3=np.zeros_like(inp["ws3"]))
    a = oracle.layer_forward(zero, k=cfg.k, E=cfg.E, bf16=True)
    b = oracle.layer_forward(plain, k=cfg.k, E=cfg.E, bf16=True)
    np.testing.assert_array_equal(a["out"], b["out"])


def test_token_outputs_match_whole_layer_with_shared_expert():
    cfg = PARITY_CONFIGS["shared_expert"]
    inp = gen.layer_inputs(cfg)
    ref = oracle.layer_forward(inp, k=cfg.k, E=cfg.E, bf16=True)
    tok = np.array([0, 5, 99, cfg.T - 1])
    ew = {e: (inp["w1"][e], inp["w3"][e], inp["w2"][e]) for e in range(cfg.E)}
    got = oracle.token_outputs(inp, tok, ref["ids"][tok], ref["weights"][tok], ew, bf16=True)
    np.testing.assert_allclose(got, ref["out"][tok], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ expert capacity (dropping)

def test_capacity_worked_example():
    """Hand-worked: 4 tokens, 3 experts, k = 2, capacity 2 per expert."""
    ids = np.array([[0, 1], [0, 2], [0, 1], [1, 0]])
    rt, tr = oracle.permutation(ids, 3, capacity=2)
    # expert 0 keeps tokens 0, 1 (drops 2, 3); expert 1 keeps 0, 2 (drops 3); expert 2 keeps 1
    np.testing.assert_array_equal(rt, [0, 1, 0, 2, 1])
    np.testing.assert_array_equal(tr, [[0, 2], [1, 4], [-1, 3], [-1, -1]])
    r = oracle.route(np.array([[3., 2., 1.], [3., 1., 2.], [3., 2., 1.], [2., 3., 1.]], np.float32),
                     2, 3, capacity=2)
    np.testing.assert_array_equal(r["ids"], ids)
    np.testing.assert_array_equal(r["routed_counts"], [4, 3, 1])
    np.testing.assert_array_equal(r["counts"], [2, 2, 1])
    np.testing.assert_array_equal(r["offsets"], [0, 2, 4, 5])


@pytest.mark.parametrize("C", [1, 3, 7])
def test_capacity_keeps_each_experts_first_tokens(C):
    r = _rng(40 + C)
    T, E, k = 60, 9, 3
    ids = oracle.topk_ids(r.standard_normal((T, E)).astype(np.float32), k)
    rt, tr = oracle.permutation(ids, E, capacity=C)
    counts = oracle.expert_counts(ids, E)
    assert int((tr < 0).sum()) == int(np.maximum(counts - C, 0).sum())
    for e in range(E):
        toks = sorted(t for t in range(T) if e in ids[t])
        keep = set(toks[:C])
        for t in toks:
            j = int(np.nonzero(ids[t] == e)[0][0])
            assert (tr[t, j] >= 0) == (t in keep)
            if t in keep:
                assert rt[tr[t, j]] == t
    # kept rows are expert-contiguous and ascending inside each segment
    off = oracle.segment_offsets(np.minimum(counts, C))
    for e in range(E):
        seg = rt[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)


def test_capacity_above_max_count_changes_nothing():
    cfg = PARITY_CONFIGS["small_bf16_zipf"]
    inp = gen.layer_inputs(cfg)
    a = oracle.layer_forward(inp, k=cfg.k, E=cfg.E, bf16=True)
    b = oracle.layer_forward(inp, k=cfg.k, E=cfg.E, bf16=True, capacity=int(a["counts"].max()))
    for key in ("ids", "counts", "offsets", "row_token", "token_row", "out"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


def test_capacity_drops_only_the_dropped_terms():
    """Each token's output is the sum over its kept assignments only (brute force)."""
    cfg = PARITY_CONFIGS["small_bf16_zipf"]
    inp = gen.layer_inputs(cfg)
    C = 40
    full = oracle.layer_forward(inp, k=cfg.k, E=cfg.E, bf16=True)
    cap = oracle.layer_forward(inp, k=cfg.k, E=cfg.E, bf16=True, capacity=C)
    assert (cap["token_row"] < 0).any() and (cap["token_row"] >= 0).any()
    y_full = full["y_perm"]
    for t in range(cfg.T):
        want = np.zeros(cfg.D)
        for j in range(cfg.k):
            if cap["token_row"][t, j] >= 0:      # same expert row value with or without dropping
                want += full["weights"][t, j] * y_full[full["token_row"][t, j]]
        np.testing.assert_allclose(cap["out"][t], want, rtol=1e-12, atol=1e-14)
