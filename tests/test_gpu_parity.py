"""GPU parity of every stage against the CPU oracle on small seeded layers.

Each test feeds the same seeded inputs (workloads/) to the HIP path through the
C ABI and to the oracle, then compares element by element:

* integers (ids, counts, offsets, row_token, token_row) and the permuted rows:
  bit-exact;
* routing weights: |dw| <= 1e-6;
* gate logits: max |d| <= 1e-5 x RMS(logits);
* expert outputs Y: every element within a bound derived from the arithmetic
  (tests/gpu_util.expert_y_bound: both sides round A and Y to bf16 at the same
  points, but the GPU's fp32 sums may sit on the other side of a rounding
  midpoint); fp32 layers 1e-5 x RMS;
* layer output (fp32 result): max |d| <= 2e-2 x RMS(out) for bf16 layers (with a
  shared expert, after one bf16 ulp of its output per element, see
  out_err_over_rms), 1e-5 x RMS(out) for fp32 layers; the bf16 output is bitwise
  the round-to-nearest-even of the fp32 output.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import MoEConfig, PARITY_CONFIGS, generator as gen
from routing_dispatch_expert_logits_amd import binding as B
from tests.gpu_util import (dev, host, empty, ws, shape_of, act_kind, rne_bf16_bits, rel_err,
                            check_permutation_valid, out_err_over_rms, check_y_rows, check_grouped_y,
                            check_layer_out, assert_poison)

pytestmark = pytest.mark.gpu

CFGS = list(PARITY_CONFIGS.values())
IDS = [c.name for c in CFGS]


def _scores_input(cfg, step=0):
    """Seeded fp32 router logits given to moe_route_topk (and the bias, if any)."""
    lg = gen.drawn_logits(cfg, step)
    return lg, gen.zipf_bias(cfg)


def _route_gpu(cfg, logits, bias):
    s = shape_of(cfg)
    T, E, k = cfg.T, cfg.E, cfg.k
    ids, w = empty((T, k), "i32"), empty((T, k), "f32")
    counts, offs = empty((E,), "i32"), empty((E + 1,), "i32")
    B.route_topk(None, None, None if bias is None else dev(bias), dev(logits), ids, w, counts, offs,
                 s, ws(s, B.MOE_CALL_ROUTE))
    torch.cuda.synchronize()
    return host(ids), host(w), host(counts), host(offs)


def _check_route(cfg, logits, bias):
    ids, w, counts, offs = _route_gpu(cfg, logits, bias)
    ref = oracle.route(oracle.router_scores(logits, bias), cfg.k, cfg.E, cfg.capacity)
    np.testing.assert_array_equal(ids, ref["ids"])
    np.testing.assert_array_equal(counts, ref["counts"])
    np.testing.assert_array_equal(offs, ref["offsets"])
    assert np.max(np.abs(w - ref["weights"])) <= 1e-6
    return ref


@pytest.mark.parametrize("cfg", CFGS, ids=IDS)
def test_route_topk_bit_exact(cfg):
    lg, bias = _scores_input(cfg)
    _check_route(cfg, lg, bias)


@pytest.mark.parametrize("E,k", [(8, 2), (64, 8), (100, 7), (256, 8), (896, 16), (1024, 64), (5, 5)])
def test_route_ties_and_signed_zeros(E, k):
    """Integer-valued scores (heavy ties), -0.0 next to +0.0, and -inf entries."""
    T = 203
    r = np.random.default_rng(E * 1000 + k)
    lg = r.integers(-2, 3, size=(T, E)).astype(np.float32)
    lg[lg == 0] = np.where(r.random(int((lg == 0).sum())) < 0.5, -0.0, 0.0).astype(np.float32)
    lg[5, :] = 0.0
    lg[6, :] = -0.0
    lg[7, : E // 2] = -np.inf
    cfg = PARITY_CONFIGS["all_ties"].with_(T=T, E=E, k=k)
    _check_route(cfg, lg, None)


@pytest.mark.parametrize("E,k", [(256, 8), (300, 8), (700, 12), (896, 16), (1024, 16), (512, 32)])
def test_route_ties_at_threshold(E, k):
    """Integer scores from a range wide enough that ties sit at the k-th place but
    few entries reach it (the threshold ranking, not the rounds, orders them), plus
    tokens whose top entries are all one value (more than 64 reach the threshold,
    so those tokens are ranked in rounds), and a token of -inf with k finite entries."""
    T = 160
    r = np.random.default_rng(E * 31 + k)
    lg = r.integers(-40, 41, size=(T, E)).astype(np.float32)
    lg[10:20, :] = 3.0                          # all tied
    lg[20:30, : E // 2] = 7.0                   # half tied at the top
    lg[30, :] = -np.inf
    lg[30, E - k:] = 1.0                        # exactly k finite, at the highest indices
    lg[31, :] = r.integers(0, 2, size=E).astype(np.float32) * 0.5   # two values
    cfg = PARITY_CONFIGS["all_ties"].with_(T=T, E=E, k=k)
    _check_route(cfg, lg, None)


def test_p95_skew_from_gpu_counts():
    """The p95 of the max / mean expert-load skew over reseeded routing steps (the
    figure the bench reports, taken from the GPU's counts) equals the oracle's, on a
    layer whose router logits carry a Zipf bias."""
    cfg = PARITY_CONFIGS["decode_many_experts"].with_(T=512, capacity=0)
    bias = gen.zipf_bias(cfg)
    gpu, ref = [], []
    for step in range(8):
        lg = gen.drawn_logits(cfg, step)
        _, _, counts, _ = _route_gpu(cfg, lg, bias)
        r = oracle.route(oracle.router_scores(lg, bias), cfg.k, cfg.E)
        np.testing.assert_array_equal(counts, r["counts"])
        gpu.append(oracle.load_skew(counts, cfg.T, cfg.k))
        ref.append(oracle.load_skew(r["counts"], cfg.T, cfg.k))
    assert oracle.p95_nearest_rank(gpu) == oracle.p95_nearest_rank(ref)
    assert oracle.p95_nearest_rank(ref) > 2.0   # the bias makes the load uneven


@pytest.mark.parametrize("E,k", [(300, 8), (500, 9), (1024, 64)])
def test_route_many_tokens_wide(E, k):
    """More than 2048 tokens (over 128 ranking blocks, so every scan thread walks
    several batches of block counts) with wide expert sets: drawn scores with a
    block of exact ties."""
    T = 2100
    r = np.random.default_rng(E * 7 + k)
    lg = r.standard_normal((T, E)).astype(np.float32)
    lg[100:164, : E // 3] = 1.5
    cfg = PARITY_CONFIGS["all_ties"].with_(T=T, E=E, k=k)
    _check_route(cfg, lg, None)


@pytest.mark.parametrize("E,k,cap", [(256, 8, 0), (64, 4, 6000)])
def test_route_and_dispatch_max_tokens(E, k, cap):
    """131072 tokens (8192 ranking blocks, a million assignments): routing, the
    permutation and the permuted rows bit-exact, with and without an expert capacity
    that drops rows of the hot experts."""
    T, H = 1 << 17, 64
    r = np.random.default_rng(E + k)
    lg = (r.standard_normal((T, E)) - 0.6 * np.log1p(np.arange(E))).astype(np.float32)  # skewed
    cfg = PARITY_CONFIGS["all_ties"].with_(T=T, E=E, k=k, H=H, capacity=cap)
    ref = _check_route(cfg, lg, None)
    rt, tr = oracle.permutation(ref["ids"], E, cap)
    if cap:
        assert ref["routed_counts"].max() > cap        # something is dropped
    x = gen.draw(cfg, gen.TAG_X, 0, (T, H), 1.0)
    s = shape_of(cfg)
    R = T * k
    xp = empty((R, H), "bf16")
    row_token, token_row = empty((R,), "i32"), empty((T, k), "i32")
    B.dispatch_permute(dev(x), dev(ref["ids"].astype(np.int32)), dev(ref["offsets"].astype(np.int32)),
                       xp, row_token, token_row, s, ws(s, B.MOE_CALL_DISPATCH))
    torch.cuda.synchronize()
    n = len(rt)
    np.testing.assert_array_equal(host(row_token)[:n], rt)
    np.testing.assert_array_equal(host(token_row), tr)
    np.testing.assert_array_equal(host(xp, True)[:n], x[rt])
    if cap:  # rows from offsets[E] on are left untouched
        assert_poison(xp, n)
        assert_poison(row_token, n)


# Gates that take the 64-expert-wide wave tile (long K slices): ragged T and E, with
# split-K over 8 slices and with a bias
WIDE_GATES = [MoEConfig(name="gate64_ragged", T=130, H=8192, E=200, k=4, I=64, seed=51, gate="computed",
                        gate_std=None),
              MoEConfig(name="gate64_bias", T=70, H=8192, E=96, k=6, I=64, seed=52, gate="computed",
                        gate_std=None, zipf_s=1.1, zipf_alpha=1.0)]


@pytest.mark.parametrize("cfg", [c for c in CFGS if c.gate == "computed"] + WIDE_GATES,
                         ids=[c.name for c in CFGS if c.gate == "computed"] + [c.name for c in WIDE_GATES])
def test_gate_logits(cfg):
    inp = gen.layer_inputs(cfg, with_experts=False)
    s = shape_of(cfg)
    T, E, k = cfg.T, cfg.E, cfg.k
    logits = empty((T, E), "f32")
    ids, w = empty((T, k), "i32"), empty((T, k), "f32")
    counts, offs = empty((E,), "i32"), empty((E + 1,), "i32")
    bias = inp.get("bias")
    B.route_topk(dev(inp["x"]), dev(inp["gate_w"]), None if bias is None else dev(bias), logits,
                 ids, w, counts, offs, s, ws(s, B.MOE_CALL_ROUTE))
    torch.cuda.synchronize()
    ref = oracle.gate_logits(inp["x"], inp["gate_w"], bias)
    glg = host(logits)
    assert rel_err(glg, ref) <= 1e-5
    # routing given fp32 logits is bit-exact: the call ranked exactly the fp32 values it
    # wrote (bias included), so its ids, weights, counts and offsets are the oracle
    # router's on those values
    r = oracle.route(oracle.router_scores(glg, None), k, E)
    np.testing.assert_array_equal(host(ids), r["ids"])
    np.testing.assert_array_equal(host(counts), r["counts"])
    np.testing.assert_array_equal(host(offs), r["offsets"])
    assert np.max(np.abs(host(w) - r["weights"])) <= 1e-6


@pytest.mark.parametrize("cfg", CFGS, ids=IDS)
def test_dispatch_permute_bit_exact(cfg):
    lg, bias = _scores_input(cfg)
    ref = oracle.route(oracle.router_scores(lg, bias), cfg.k, cfg.E, cfg.capacity)
    rt, tr = oracle.permutation(ref["ids"], cfg.E, cfg.capacity)
    x = gen.activations(cfg)
    s = shape_of(cfg)
    R, D = cfg.R, cfg.H
    sc = s if not cfg.L else B.shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, 0, cfg.dtype, 0, cfg.capacity)
    x_perm = empty((R, D), act_kind(cfg))
    row_token, token_row = empty((R,), "i32"), empty((cfg.T, cfg.k), "i32")
    B.dispatch_permute(dev(x), dev(ref["ids"].astype(np.int32)), dev(ref["offsets"].astype(np.int32)),
                       x_perm, row_token, token_row, sc, ws(sc, B.MOE_CALL_DISPATCH))
    torch.cuda.synchronize()
    n = len(rt)                      # kept rows (all T*k without a capacity)
    np.testing.assert_array_equal(host(row_token)[:n], rt)
    np.testing.assert_array_equal(host(token_row), tr)
    xp = host(x_perm, bf16=cfg.dtype == "bf16")[:n]
    np.testing.assert_array_equal(xp, oracle.gather_rows(x, rt))
    if not cfg.capacity:
        assert xp.nbytes == oracle.dispatch_bytes(cfg.T, cfg.k, D, cfg.elem_bytes)
    else:  # rows from offsets[E] on are left untouched
        assert n < cfg.R
        assert_poison(x_perm, n)
        assert_poison(row_token, n)


def _ffn_inputs(cfg):
    lg, bias = _scores_input(cfg)
    ref = oracle.route(oracle.router_scores(lg, bias), cfg.k, cfg.E, cfg.capacity)
    rt, _ = oracle.permutation(ref["ids"], cfg.E, cfg.capacity)
    x = gen.draw(cfg, gen.TAG_X, 0, (cfg.T, cfg.D), cfg.x_std)
    return ref, oracle.gather_rows(x, rt)


@pytest.mark.parametrize("cfg", CFGS, ids=IDS)
def test_grouped_ffn(cfg):
    ref, xp = _ffn_inputs(cfg)
    wts = gen.expert_weights(cfg)
    s = shape_of(cfg)
    y = empty((cfg.R, cfg.D), act_kind(cfg))
    B.grouped_ffn(dev(xp), dev(ref["offsets"].astype(np.int32)), dev(wts["w1"]), dev(wts["w3"]),
                  dev(wts["w2"]), y, s, ws(s, B.MOE_CALL_FFN))
    torch.cuda.synchronize()
    bf = cfg.dtype == "bf16"
    check_grouped_y(bf, host(y, bf16=bf), xp, ref["offsets"], wts["w1"], wts["w3"], wts["w2"])


def test_grouped_ffn_never_reads_empty_experts():
    """Weights of experts with no rows are NaN: outputs stay finite and unchanged."""
    cfg = PARITY_CONFIGS["many_empty"]
    ref, xp = _ffn_inputs(cfg)
    wts = gen.expert_weights(cfg)
    s = shape_of(cfg)
    offs = dev(ref["offsets"].astype(np.int32))
    y0, y1 = empty((cfg.R, cfg.D), "bf16"), empty((cfg.R, cfg.D), "bf16")
    B.grouped_ffn(dev(xp), offs, dev(wts["w1"]), dev(wts["w3"]), dev(wts["w2"]), y0, s,
                  ws(s, B.MOE_CALL_FFN))
    empty_e = np.nonzero(ref["counts"] == 0)[0]
    assert len(empty_e) > cfg.E // 2
    nan = np.uint16(0x7FC0)
    for name in ("w1", "w3", "w2"):
        wts[name][empty_e] = nan
    B.grouped_ffn(dev(xp), offs, dev(wts["w1"]), dev(wts["w3"]), dev(wts["w2"]), y1, s,
                  ws(s, B.MOE_CALL_FFN))
    torch.cuda.synchronize()
    a, b = host(y0, True), host(y1, True)
    assert np.isfinite(oracle.decode(b)).all()
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("cfg", CFGS, ids=IDS)
def test_combine(cfg):
    lg, bias = _scores_input(cfg)
    ref = oracle.route(oracle.router_scores(lg, bias), cfg.k, cfg.E, cfg.capacity)
    _, tr = oracle.permutation(ref["ids"], cfg.E, cfg.capacity)
    w32 = ref["weights"].astype(np.float32)
    y = gen.stage_rows(cfg, cfg.R, cfg.D)
    s = shape_of(cfg)
    outs = {}
    for flags in (B.MOE_COMBINE_FUSED, B.MOE_COMBINE_UNFUSED):
        for od in (B.MOE_F32, B.MOE_BF16):
            o = empty((cfg.T, cfg.D), "f32" if od == B.MOE_F32 else "bf16")
            B.combine(dev(y), dev(tr.astype(np.int32)), dev(w32), o, od, flags, s,
                      ws(s, B.MOE_CALL_COMBINE))
            outs[(flags, od)] = o
    torch.cuda.synchronize()
    f32 = host(outs[(B.MOE_COMBINE_FUSED, B.MOE_F32)])
    ref_out = oracle.combine(y, tr, w32.astype(np.float64))
    assert rel_err(f32, ref_out) <= 1e-5
    np.testing.assert_array_equal(host(outs[(B.MOE_COMBINE_UNFUSED, B.MOE_F32)]), f32)
    bf = host(outs[(B.MOE_COMBINE_FUSED, B.MOE_BF16)], True)
    np.testing.assert_array_equal(bf, rne_bf16_bits(f32))
    np.testing.assert_array_equal(host(outs[(B.MOE_COMBINE_UNFUSED, B.MOE_BF16)], True), bf)


@pytest.mark.parametrize("cfg", [c for c in CFGS if c.L == 0], ids=[c.name for c in CFGS if c.L == 0])
def test_combine_with_shared_term(cfg):
    """A shared expert's output enters the combine with weight 1, after the k routed terms."""
    lg, bias = _scores_input(cfg)
    ref = oracle.route(oracle.router_scores(lg, bias), cfg.k, cfg.E, cfg.capacity)
    _, tr = oracle.permutation(ref["ids"], cfg.E, cfg.capacity)
    w32 = ref["weights"].astype(np.float32)
    y = gen.stage_rows(cfg, cfg.R, cfg.D)
    ysh = gen.stage_rows(cfg, cfg.T, cfg.D, index=1)
    s = shape_of(cfg)
    got = {}
    for flags in (B.MOE_COMBINE_FUSED, B.MOE_COMBINE_UNFUSED):
        o = empty((cfg.T, cfg.D), "f32")
        B.combine(dev(y), dev(tr.astype(np.int32)), dev(w32), o, B.MOE_F32, flags, s,
                  ws(s, B.MOE_CALL_COMBINE), shared_out=dev(ysh))
        got[flags] = o
    torch.cuda.synchronize()
    f32 = host(got[B.MOE_COMBINE_FUSED])
    assert rel_err(f32, oracle.combine(y, tr, w32.astype(np.float64), ysh)) <= 1e-5
    np.testing.assert_array_equal(host(got[B.MOE_COMBINE_UNFUSED]), f32)


# Rows whose last 64-lane column pass leaves fewer active lanes than k: every lane
# must still take part in the shuffles of the k row indices and weights.
NARROW = [MoEConfig(name="narrow_f32_k7", T=50, H=16, E=20, k=7, I=16, dtype="f32", seed=31,
                    gate="drawn"),
          MoEConfig(name="narrow_bf16_k9", T=33, H=64, E=12, k=9, I=64, seed=32, gate="drawn"),
          MoEConfig(name="split_tail_bf16_k16", T=256, H=1088, E=64, k=16, I=64, seed=33,
                    gate="drawn")]


@pytest.mark.parametrize("cfg", NARROW, ids=[c.name for c in NARROW])
def test_combine_rows_narrower_than_k(cfg):
    lg, bias = _scores_input(cfg)
    ref = oracle.route(oracle.router_scores(lg, bias), cfg.k, cfg.E)
    _, tr = oracle.permutation(ref["ids"], cfg.E)
    w32 = ref["weights"].astype(np.float32)
    y = gen.stage_rows(cfg, cfg.R, cfg.D)
    ysh = gen.stage_rows(cfg, cfg.T, cfg.D, index=1)
    s = shape_of(cfg)
    got = {}
    for flags in (B.MOE_COMBINE_FUSED, B.MOE_COMBINE_UNFUSED):
        o = empty((cfg.T, cfg.D), "f32")
        B.combine(dev(y), dev(tr.astype(np.int32)), dev(w32), o, B.MOE_F32, flags, s,
                  ws(s, B.MOE_CALL_COMBINE), shared_out=dev(ysh))
        got[flags] = o
    torch.cuda.synchronize()
    f32 = host(got[B.MOE_COMBINE_FUSED])
    assert rel_err(f32, oracle.combine(y, tr, w32.astype(np.float64), ysh)) <= 1e-5
    np.testing.assert_array_equal(host(got[B.MOE_COMBINE_UNFUSED]), f32)


# ------------------------------------------------------------------ whole layer

def run_layer(cfg, inp, out_dtype=B.MOE_F32, with_aux=True, workspace=None):
    """moe_layer_forward on uploaded inputs (in `workspace` if given); returns host copies
    of out and the aux buffers."""
    s = shape_of(cfg)
    T, E, k, R, D = cfg.T, cfg.E, cfg.k, cfg.R, cfg.D
    w = {n: dev(inp[n]) for n in ("gate_w", "w1", "w3", "w2", "wd", "wu", "ws1", "ws3", "ws2")
         if n in inp}
    if "bias" in inp:
        w["gate_bias"] = dev(inp["bias"])
    logits = dev(inp["logits"]) if "logits" in inp else empty((T, E), "f32")
    aux = {}
    if with_aux:
        aux = {"topk_ids": empty((T, k), "i32"), "topk_w": empty((T, k), "f32"),
               "counts": empty((E,), "i32"), "offsets": empty((E + 1,), "i32"),
               "row_token": empty((R,), "i32"), "token_row": empty((T, k), "i32"),
               "x_perm": empty((R, D), act_kind(cfg)), "y_perm": empty((R, D), act_kind(cfg))}
        if cfg.L:
            aux["z"] = empty((T, cfg.L), act_kind(cfg))
            aux["out_latent"] = empty((T, cfg.L), act_kind(cfg))
    out = empty((T, cfg.H), "f32" if out_dtype == B.MOE_F32 else "bf16")
    wsp = ws(s, B.MOE_CALL_LAYER) if workspace is None else workspace
    B.layer_forward(w, dev(inp["x"]), logits, out, out_dtype, s, wsp, aux)
    torch.cuda.synchronize()
    res = {"out": host(out, out_dtype == B.MOE_BF16), "logits": host(logits)}
    bf = cfg.dtype == "bf16"
    for n, t in aux.items():
        res[n] = host(t, bf and n in ("x_perm", "y_perm", "z", "out_latent"))
    return res


def unambiguous_tokens(scores_ref: np.ndarray, k: int, tol: float) -> np.ndarray:
    """Tokens whose top-k set cannot change under score perturbations below tol."""
    if k == scores_ref.shape[1]:
        return np.ones(scores_ref.shape[0], dtype=bool)
    srt = -np.sort(-scores_ref, axis=1)
    return (srt[:, k - 1] - srt[:, k]) > 2 * tol


# Layers on which correct arithmetic itself exceeds the layer tolerance
# max |err| <= 2e-2 x RMS(out): a float32 simulation of the kernels' arithmetic (fp32 sums
# in another order than the oracle's exact ones, the same bf16 rounding points) reaches
# 2.7e-2 on wsp_chunk_down, where one of its 16.8M outputs takes a Y element of magnitude
# 2.17 that rounded to the neighbouring bf16 value (one ulp, 1.6e-2) under a routing
# weight of 0.42.  These layers are held to the derived per-element bound alone.
RMS_TOL_FLOOR = {"wsp_chunk_down"}


@pytest.mark.parametrize("cfg", CFGS, ids=IDS)
def test_layer_forward(cfg):
    inp = gen.layer_inputs(cfg)
    bf = cfg.dtype == "bf16"
    got = run_layer(cfg, inp)
    ref = oracle.layer_forward(inp, k=cfg.k, E=cfg.E, bf16=bf, capacity=cfg.capacity)
    if "logits" in inp:   # given router output: routing must be bit-exact everywhere
        keep = np.ones(cfg.T, dtype=bool)
        np.testing.assert_array_equal(got["topk_ids"], ref["ids"])
        np.testing.assert_array_equal(got["counts"], ref["counts"])
        np.testing.assert_array_equal(got["offsets"], ref["offsets"])
        np.testing.assert_array_equal(got["row_token"][:len(ref["row_token"])], ref["row_token"])
        np.testing.assert_array_equal(got["token_row"], ref["token_row"])
    else:                 # computed logits: compare routing where the scores decide it uniquely
        assert not cfg.capacity, "capacity layers use given logits (dropping needs exact routing)"
        tol = 1e-5 * float(np.sqrt(np.mean(ref["logits"] ** 2)))
        assert rel_err(got["logits"], ref["logits"]) <= 1e-5
        keep = unambiguous_tokens(ref["logits"], cfg.k, tol)
        assert keep.mean() > 0.99
        np.testing.assert_array_equal(np.sort(got["topk_ids"][keep], axis=1),
                                      np.sort(ref["ids"][keep], axis=1))
        check_permutation_valid(got["topk_ids"], got["offsets"], got["row_token"], got["token_row"])
        np.testing.assert_array_equal(got["counts"], np.diff(got["offsets"]))
    tol = 2e-2 if bf else 1e-5
    if not cfg.L:   # every element within the bound derived from the arithmetic
        check_layer_out(cfg, inp, ref, got["out"], keep)
    if cfg.name not in RMS_TOL_FLOOR:   # the layer tolerance, 2e-2 x RMS(out) (1e-5 for fp32)
        ysh = ref["y_shared"][keep] if (bf and cfg.shared_I) else None
        assert out_err_over_rms(got["out"][keep], ref["out"][keep], ysh) <= tol
    # bf16 output is the RNE of the fp32 output of the same kernels
    got16 = run_layer(cfg, inp, out_dtype=B.MOE_BF16, with_aux=False)
    np.testing.assert_array_equal(got16["out"], rne_bf16_bits(got["out"]))


@pytest.mark.parametrize("T,E,k,wgs", [(8, 896, 16, 1), (40, 300, 8, 1), (100, 256, 8, 1), (24, 1024, 16, 1),
                                       (128, 896, 16, 32), (60, 1024, 16, 15), (100, 512, 32, 25),
                                       (17, 1000, 64, 5)])
def test_layer_decode_routing_ties(T, E, k, wgs):
    """The one-launch decode routing on wide expert sets, in one workgroup and over
    ceil(T / 4) workgroups (threshold ranking, and the rounds for tokens with heavy
    ties) with integer router logits: ids, counts, offsets and the row metadata
    bit-exact against the oracle, on two calls in a row, each in a workspace of
    random bytes."""
    cfg = PARITY_CONFIGS["decode_t100"].with_(T=T, E=E, k=k, H=128, I=64, zipf_s=None)
    s = shape_of(cfg)
    p = B.layer_plan(s, gate=False)
    assert (p["decode_path"], p["route_workgroups"]) == (1, wgs)
    inp = gen.layer_inputs(cfg)
    r = np.random.default_rng(T * E + k)
    lg = r.integers(-40, 41, size=(T, E)).astype(np.float32)
    lg[1, :] = 2.0                                # all tied: ranked in rounds
    lg[2, : E // 2] = 5.0
    lg[3, :] = -np.inf
    lg[3, E - k:] = 0.0                           # exactly k finite
    inp["logits"] = lg
    inp.pop("bias", None)
    ref = oracle.route(oracle.router_scores(lg, None), k, E)
    rt, tr = oracle.permutation(ref["ids"], E)
    # the workspace starts as random bytes each time: whatever the hand-over word holds
    # counts as zero unless it carries the call's own tag
    wsp = ws(s, B.MOE_CALL_LAYER)
    gen_t = torch.Generator(device="cuda:0").manual_seed(T * 7 + k)
    for _ in range(2):
        wsp.copy_(torch.randint(0, 256, wsp.shape, generator=gen_t, device="cuda:0", dtype=torch.uint8))
        got = run_layer(cfg, inp, workspace=wsp)
        np.testing.assert_array_equal(got["topk_ids"], ref["ids"])
        assert np.max(np.abs(got["topk_w"] - ref["weights"])) <= 1e-6
        np.testing.assert_array_equal(got["counts"], ref["counts"])
        np.testing.assert_array_equal(got["offsets"], ref["offsets"])
        np.testing.assert_array_equal(got["row_token"][:len(rt)], rt)
        np.testing.assert_array_equal(got["token_row"], tr)


@pytest.mark.parametrize("T,H,E,k,I,dtype", [(1000, 256, 16, 2, 192, "bf16"),   # persistent prefill tiles
                                              (600, 256, 4, 1, 2048, "bf16"),    # long-K down tiles
                                              (100, 256, 300, 4, 128, "bf16"),   # decode, one routing workgroup
                                              (128, 256, 896, 16, 128, "bf16"),  # decode, 32 routing workgroups
                                              (97, 96, 6, 3, 80, "f32")])
def test_layer_all_tokens_on_the_same_experts(T, H, E, k, I, dtype):
    """Every token picks the same k experts (the hottest possible skew): those experts
    hold T rows each, every other expert is empty.  Routing and the row metadata are
    bit-exact and every output element is within the derived bound."""
    cfg = PARITY_CONFIGS["decode_t100"].with_(T=T, H=H, E=E, k=k, I=I, dtype=dtype, zipf_s=None,
                                              seed=T + E + k)
    inp = gen.layer_inputs(cfg)
    r = np.random.default_rng(T * 3 + E)
    lg = r.standard_normal((T, E)).astype(np.float32)
    hot = r.choice(E, size=k, replace=False)
    lg[:, hot] = (10.0 + np.arange(k, dtype=np.float32))[None, :]   # same order for every token
    inp["logits"] = lg
    inp.pop("bias", None)
    got = run_layer(cfg, inp)
    bf = dtype == "bf16"
    ref = oracle.layer_forward(inp, k=k, E=E, bf16=bf, capacity=0)
    np.testing.assert_array_equal(got["topk_ids"], ref["ids"])
    assert set(np.unique(ref["ids"])) == set(hot.tolist())
    np.testing.assert_array_equal(got["counts"], ref["counts"])
    np.testing.assert_array_equal(got["offsets"], ref["offsets"])
    np.testing.assert_array_equal(got["row_token"][:len(ref["row_token"])], ref["row_token"])
    np.testing.assert_array_equal(got["token_row"], ref["token_row"])
    check_layer_out(cfg, inp, ref, got["out"], np.ones(T, dtype=bool))
    assert out_err_over_rms(got["out"], ref["out"], None) <= (2e-2 if bf else 1e-5)


@pytest.mark.parametrize("name", ["small_bf16_zipf", "small_latent", "tiny_f32"])
def test_layer_matches_separate_calls_and_is_deterministic(name):
    """Fusion is execution-only: routing, permutation and output bits equal the separate calls."""
    cfg = PARITY_CONFIGS[name]
    inp = gen.layer_inputs(cfg)
    a = run_layer(cfg, inp)
    b = run_layer(cfg, inp)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    # separate calls on the fused call's own logits
    lg = a["logits"]
    bias = None if cfg.gate == "computed" else inp.get("bias")
    ids, w, counts, offs = _route_gpu(cfg, lg, bias)
    np.testing.assert_array_equal(ids, a["topk_ids"])
    np.testing.assert_array_equal(w, a["topk_w"])
    np.testing.assert_array_equal(counts, a["counts"])
    np.testing.assert_array_equal(offs, a["offsets"])


GATHER_CFGS = ["small_bf16_zipf", "small_bf16_uniform", "wide_experts", "shared_expert", "capacity_prefill",
               "all_ties", "decode_many_experts", "decode_t128"]


@pytest.mark.parametrize("name", GATHER_CFGS)
def test_layer_gathered_rows_equal_permuted_copy(name):
    """Without aux x_perm the fused layer writes only the row metadata and its gate/up
    GEMM reads the token rows through row_token (persistent prefill tiles; decode tiles
    after the general routing or after the one-launch routing); the output bits equal
    those of the layer that writes the permuted copy, and its routing metadata is the
    same."""
    cfg = PARITY_CONFIGS[name]
    inp = gen.layer_inputs(cfg)
    a = run_layer(cfg, inp)
    b = run_layer(cfg, inp, with_aux=False)
    np.testing.assert_array_equal(b["out"], a["out"])
    s = shape_of(cfg)
    w = {n: dev(inp[n]) for n in ("gate_w", "w1", "w3", "w2", "ws1", "ws3", "ws2") if n in inp}
    if "bias" in inp:
        w["gate_bias"] = dev(inp["bias"])
    logits = dev(inp["logits"]) if "logits" in inp else empty((cfg.T, cfg.E), "f32")
    aux = {"row_token": empty((cfg.R,), "i32"), "token_row": empty((cfg.T, cfg.k), "i32"),
           "offsets": empty((cfg.E + 1,), "i32")}
    out = empty((cfg.T, cfg.H), "f32")
    B.layer_forward(w, dev(inp["x"]), logits, out, B.MOE_F32, s, ws(s, B.MOE_CALL_LAYER), aux)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), a["out"])
    n = int(a["offsets"][-1])
    np.testing.assert_array_equal(host(aux["row_token"])[:n], a["row_token"][:n])
    np.testing.assert_array_equal(host(aux["token_row"]), a["token_row"])


WIDE = ["wide_experts", "long_k_down", "wsp_chunk_gate_up", "wsp_chunk_down"]


@pytest.mark.parametrize("name", WIDE)
def test_layer_gathered_y_every_row(name):
    """The fused layer in the dataflow bench.py times (no permuted copy: the gate/up GEMM
    gathers the token rows through row_token) on layers that take the full-size layers'
    kernels: 16 and 64 n-tiles of 128, K = 2048 and 8192, the persistent 128 x 256 and
    256 x 128 down tiles, and XCD-chunk-only tile tables (more tiles than one table
    holds).  Every row of every expert's Y against the oracle, and the layer output on
    every token."""
    cfg = PARITY_CONFIGS[name]
    s = shape_of(cfg)
    plan = B.layer_plan(s, cfg.gate == "computed")
    assert plan["rows_gathered"] == 1 and plan["gate_up_persistent"] == 1
    inp = gen.layer_inputs(cfg)
    T, E, k, R, D = cfg.T, cfg.E, cfg.k, cfg.R, cfg.D
    w = {n: dev(inp[n]) for n in ("w1", "w3", "w2")}
    if "bias" in inp:
        w["gate_bias"] = dev(inp["bias"])
    aux = {"topk_ids": empty((T, k), "i32"), "topk_w": empty((T, k), "f32"),
           "offsets": empty((E + 1,), "i32"), "row_token": empty((R,), "i32"),
           "token_row": empty((T, k), "i32"), "y_perm": empty((R, D), "bf16")}
    out = empty((T, cfg.H), "f32")
    B.layer_forward(w, dev(inp["x"]), dev(inp["logits"]), out, B.MOE_F32, s, ws(s, B.MOE_CALL_LAYER), aux)
    torch.cuda.synchronize()
    ref = oracle.route(oracle.router_scores(inp["logits"], inp.get("bias")), k, E)
    rt, tr = oracle.permutation(ref["ids"], E)
    np.testing.assert_array_equal(host(aux["topk_ids"]), ref["ids"])
    np.testing.assert_array_equal(host(aux["offsets"]), ref["offsets"])
    np.testing.assert_array_equal(host(aux["row_token"]), rt)
    np.testing.assert_array_equal(host(aux["token_row"]), tr)
    xp = oracle.gather_rows(inp["x"], rt)
    check_grouped_y(True, host(aux["y_perm"], True), xp, ref["offsets"], inp["w1"], inp["w3"], inp["w2"])
    ref_l = oracle.layer_forward(inp, k=k, E=E, bf16=True)
    check_layer_out(cfg, inp, ref_l, host(out))
    if name not in RMS_TOL_FLOOR:
        assert out_err_over_rms(host(out), ref_l["out"]) <= 2e-2


def test_stage_events_skip_null_entries():
    """A stage-event array may leave entries NULL: only the others are recorded, and the
    layer's results do not depend on which are."""
    from bench import HipEvents
    cfg = PARITY_CONFIGS["small_bf16_zipf"]
    inp = gen.layer_inputs(cfg)
    s = shape_of(cfg)
    w = {n: dev(inp[n]) for n in ("gate_w", "w1", "w3", "w2")}
    x = dev(inp["x"])
    outs = []
    hip = HipEvents()
    full = hip.create(B.MOE_NUM_STAGE_EVENTS)
    pair = hip.create(2)
    g = B.STAGE_NAMES.index("gemm_gate_up")
    some = [None] * B.MOE_NUM_STAGE_EVENTS
    some[g], some[g + 1] = pair
    stream = torch.cuda.current_stream().cuda_stream
    for evs in (None, full, some):
        logits = empty((cfg.T, cfg.E), "f32")
        out = empty((cfg.T, cfg.H), "f32")
        B.layer_forward(w, x, logits, out, B.MOE_F32, s, ws(s, B.MOE_CALL_LAYER), stage_events=evs, stream=stream)
        torch.cuda.synchronize()
        outs.append(host(out))
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[0], outs[2])
    assert hip.elapsed_ms(pair[0], pair[1]) > 0
    assert hip.elapsed_ms(full[0], full[-1]) >= hip.elapsed_ms(full[g], full[g + 1]) > 0
    hip.destroy(full)
    hip.destroy(pair)


@pytest.mark.parametrize("name", ["shared_expert", "shared_expert_decode", "shared_expert_f32",
                                  "small_bf16_decode", "single_token", "many_empty", "decode_t100",
                                  "decode_t128", "decode_many_experts", "decode_many_experts_cap", "all_ties",
                                  "capacity_prefill", "capacity_decode", "capacity_f32"])
def test_layer_output_equals_separate_calls(name):
    """Fused layer == route, permute, grouped FFN, (the shared expert as a
    one-expert grouped FFN over all tokens,) and the combine, bit for bit: the
    fusion is execution-only.  Decode-scale layers (T <= 128 with 16-row tiles)
    take the one-launch routing (over several workgroups for decode_many_experts*),
    the gathering gate/up GEMM and the down GEMM fused with the combine in the fused
    call (its Y, written to aux.y_perm, has the bits of the separate down GEMM), the
    general kernels in the separate calls."""
    cfg = PARITY_CONFIGS[name]
    inp = gen.layer_inputs(cfg)
    a = run_layer(cfg, inp)
    T, H, k, R, D = cfg.T, cfg.H, cfg.k, cfg.R, cfg.D
    s = shape_of(cfg)
    bias = None if cfg.gate == "computed" else inp.get("bias")
    ids, w, counts, offs = _route_gpu(cfg, a["logits"], bias)
    np.testing.assert_array_equal(ids, a["topk_ids"])
    kind = act_kind(cfg)
    xp, rt, tr = empty((R, D), kind), empty((R,), "i32"), empty((T, k), "i32")
    B.dispatch_permute(dev(inp["x"]), dev(ids), dev(offs), xp, rt, tr, s, ws(s, B.MOE_CALL_DISPATCH))
    yp = empty((R, D), kind)
    B.grouped_ffn(xp, dev(offs), dev(inp["w1"]), dev(inp["w3"]), dev(inp["w2"]), yp, s,
                  ws(s, B.MOE_CALL_FFN))
    ysh = None
    if cfg.shared_I:
        s1 = B.shape(T, H, 1, 1, cfg.shared_I, 0, cfg.dtype)
        ysh = empty((T, H), kind)
        B.grouped_ffn(dev(inp["x"]), dev(np.array([0, T], dtype=np.int32)), dev(inp["ws1"]),
                      dev(inp["ws3"]), dev(inp["ws2"]), ysh, s1, ws(s1, B.MOE_CALL_FFN))
    out = empty((T, H), "f32")
    B.combine(yp, tr, dev(w), out, B.MOE_F32, B.MOE_COMBINE_FUSED, s, ws(s, B.MOE_CALL_COMBINE),
              shared_out=ysh)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), a["out"])
    kept = int(offs[-1])
    for n, t in (("x_perm", xp), ("row_token", rt), ("y_perm", yp)):
        np.testing.assert_array_equal(host(t, cfg.dtype == "bf16" and n in ("x_perm", "y_perm"))[:kept],
                                      a[n][:kept], err_msg=n)
    np.testing.assert_array_equal(host(tr), a["token_row"])
    if cfg.shared_I:  # and the shared expert alone matches the oracle's
        bf = cfg.dtype == "bf16"
        check_y_rows(bf, host(ysh, bf), inp["x"], inp["ws1"], inp["ws3"], inp["ws2"])


@pytest.mark.parametrize("name", ["small_bf16_decode", "decode_many_experts", "small_bf16_zipf"])
def test_layer_under_graph_capture(name):
    """The layer captured into a graph on a side stream (the library launches kernels
    only: no allocation, copy, memset or host synchronisation) replays with the output
    bits of the eager call, on every replay, with eager work and synchronisations
    between the replays."""
    cfg = PARITY_CONFIGS[name]
    inp = gen.layer_inputs(cfg)
    s = shape_of(cfg)
    w = {n: dev(inp[n]) for n in ("gate_w", "w1", "w3", "w2") if n in inp}
    if "bias" in inp:
        w["gate_bias"] = dev(inp["bias"])
    x = dev(inp["x"])
    logits = dev(inp["logits"]) if "logits" in inp else empty((cfg.T, cfg.E), "f32")
    ref = empty((cfg.T, cfg.H), "f32")
    B.layer_forward(w, x, logits, ref, B.MOE_F32, s, ws(s, B.MOE_CALL_LAYER))
    torch.cuda.synchronize()
    want = host(ref)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device="cuda:0")
    wsg = ws(s, B.MOE_CALL_LAYER)
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        B.layer_forward(w, x, logits, out, B.MOE_F32, s, wsg, stream=st.cuda_stream)
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), want)


def test_concurrent_layers_on_separate_streams():
    """Calls are re-entrant across distinct workspaces: different layers launched
    concurrently on separate streams (default priority) give the bits of serial runs,
    the decode routing over several workgroups (its hand-over word in each call's own
    workspace) among them."""
    cfgs = [PARITY_CONFIGS["small_bf16_zipf"], PARITY_CONFIGS["small_bf16_decode"].with_(dispatch="mxfp8"),
            PARITY_CONFIGS["decode_many_experts"]]
    setups = []
    for cfg in cfgs:
        inp = gen.layer_inputs(cfg)
        s = shape_of(cfg)
        w = {n: dev(inp[n]) for n in ("gate_w", "w1", "w3", "w2") if n in inp}
        if cfg.dispatch == "mxfp8":
            for n in ("w1", "w3"):
                q, sc = empty((cfg.E, cfg.I, cfg.D), "u8"), empty((cfg.E, cfg.I, cfg.D // 32), "u8")
                B.quantize_mxfp8(w[n], q, sc)
                w[n], w[n + "_scale"] = q, sc
        if "bias" in inp:
            w["gate_bias"] = dev(inp["bias"])
        logits = dev(inp["logits"]) if "logits" in inp else empty((cfg.T, cfg.E), "f32")
        setups.append((cfg, s, w, dev(inp["x"]), logits))
    torch.cuda.synchronize()

    def run(i, stream, reps):
        cfg, s, w, x, logits = setups[i]
        out = empty((cfg.T, cfg.H), "f32")
        wsp = ws(s, B.MOE_CALL_LAYER)
        torch.cuda.synchronize()  # the buffers' poison fill ran on the default stream
        for _ in range(reps):
            B.layer_forward(w, x, logits, out, B.MOE_F32, s, wsp, stream=stream)
        return out

    assert B.layer_plan(setups[2][1], gate=False)["route_workgroups"] > 1
    serial = [host(run(i, None, 1)) for i in range(len(cfgs))]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cfgs]
    outs = [run(i, streams[i], 20) for i in range(len(cfgs))]
    torch.cuda.synchronize()
    for i in range(len(cfgs)):
        np.testing.assert_array_equal(host(outs[i]), serial[i])
