"""GPU parity of the MXFP8 dispatch path (value-changing, opt-in) against the oracle.

* conversion kernel: E4M3 codes and E8M0 scales bit-exact (both sides take every
  rounding decision on the same exact quotient value / 2^k);
* dispatch: the quantised, permuted rows and their scales bit-exact, metadata exact;
* grouped FFN on the oracle's codes: every element of Y within a bound derived from
  the arithmetic (y_bound below);
* the whole layer with weights quantised on the GPU: routing and codes exact, every
  output element within that bound carried through the combine, and bit-equal to the
  separate calls.

The bound.  The products of E4M3 values and power-of-two scales are exact, but the
scaled fp8 matrix instruction sums a K-step's 128 products to about 2^-18 of their
absolute sum (measured: max 2^-18.1 of sum |p| on random 128-term dot products),
far coarser than fp32.  So G and U may be off by EPS * sum_k |x_k w_k| (EPS = 2^-16,
four times the measured worst), the intermediate A = bf16(SiLU(G) U) by one bf16 ulp
(its rounding can flip) plus |dA/dG| dG + |dA/dU| dU, and Y by its own ulp (twice,
for the flip) plus sum_i |w2_i| dA_i plus the fp32 sum of the down projection.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import mxfp8 as M
from workloads import MoEConfig, PARITY_CONFIGS, generator as gen
from routing_dispatch_expert_logits_amd import binding as B
from tests.gpu_util import dev, host, empty, ws, shape_of
from tests.test_gpu_parity import _scores_input

pytestmark = pytest.mark.gpu


def _mx(cfg):
    return cfg.with_(dispatch="mxfp8")


# bf16 layers whose dispatched width is a multiple of 128, plus a decode-scale layer
# above 128 tokens (16-row tiles through the general routing kernels)
MX_CFGS = [_mx(c) for c in PARITY_CONFIGS.values() if c.dtype == "bf16" and c.D % 128 == 0]
MX_CFGS.append(MoEConfig(name="mx_decode_general", T=130, H=256, E=64, k=4, I=128, seed=41,
                         gate="drawn", dispatch="mxfp8"))
MX_IDS = [c.name for c in MX_CFGS]


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).bfloat16().view(
        torch.int16).numpy().view(np.uint16)


def _quant_inputs(seed, rows, cols):
    """bf16 rows over a wide exponent range, with the blocks the rule treats specially."""
    r = np.random.default_rng(seed)
    nb = cols // 32
    v = r.standard_normal((rows, cols)) * np.exp2(r.integers(-120, 110, (rows, nb))).repeat(32, axis=1)
    v[0, :32] = 0.0                                   # all-zero block
    v[0, 32:64] = -0.0
    v[1, :32] = np.exp2(-130.0) * r.integers(-3, 4, 32)   # bf16 subnormals
    v[2, :32] = 1.9 * np.exp2(5.0) * np.sign(r.standard_normal(32))  # saturates (1.9 * 256)
    v[3, :32] = 3.0e38 * np.sign(r.standard_normal(32))  # near the top of bf16
    v[4, :32] = np.exp2(r.integers(-20, 3, 32).astype(float))  # one binade per element
    return _bf16_bits(v)


@pytest.mark.parametrize("rows,cols", [(1, 32), (37, 128), (333, 256), (64, 7168)])
def test_quantize_bf16_bit_exact(rows, cols):
    src = _quant_inputs(rows * 7 + cols, max(rows, 5), cols)[:rows]
    q, sc = empty((rows, cols), "u8"), empty((rows, cols // 32), "u8")
    B.quantize_mxfp8(dev(src), q, sc)
    torch.cuda.synchronize()
    rq, rs = M.mx_quantize(oracle.decode(src))
    np.testing.assert_array_equal(host(sc), rs)
    np.testing.assert_array_equal(host(q), rq)


def test_quantize_f32_bit_exact():
    r = np.random.default_rng(5)
    src = (r.standard_normal((50, 192)) * np.exp2(r.integers(-30, 30, (50, 1)))).astype(np.float32)
    q, sc = empty((50, 192), "u8"), empty((50, 6), "u8")
    B.quantize_mxfp8(dev(src), q, sc)
    torch.cuda.synchronize()
    rq, rs = M.mx_quantize(src.astype(np.float64))
    np.testing.assert_array_equal(host(sc), rs)
    np.testing.assert_array_equal(host(q), rq)


@pytest.mark.parametrize("cfg", MX_CFGS, ids=MX_IDS)
def test_dispatch_permute_mx_bit_exact(cfg):
    lg, bias = _scores_input(cfg)
    ref = oracle.route(oracle.router_scores(lg, bias), cfg.k, cfg.E, cfg.capacity)
    rt, tr = oracle.permutation(ref["ids"], cfg.E, cfg.capacity)
    x = gen.draw(cfg, gen.TAG_X, 0, (cfg.T, cfg.D), cfg.x_std)
    s = shape_of(cfg)
    R, D = cfg.R, cfg.D
    xp, xs = empty((R, D), "u8"), empty((R, D // 32), "u8")
    row_token, token_row = empty((R,), "i32"), empty((cfg.T, cfg.k), "i32")
    B.dispatch_permute(dev(x), dev(ref["ids"].astype(np.int32)), dev(ref["offsets"].astype(np.int32)),
                       xp, row_token, token_row, s, ws(s, B.MOE_CALL_DISPATCH), x_perm_scale=xs)
    torch.cuda.synchronize()
    n = len(rt)
    np.testing.assert_array_equal(host(row_token)[:n], rt)
    np.testing.assert_array_equal(host(token_row), tr)
    xq, xsc = M.mx_quantize(oracle.decode(x))
    np.testing.assert_array_equal(host(xp)[:n], xq[rt])
    np.testing.assert_array_equal(host(xs)[:n], xsc[rt])
    if not cfg.capacity:   # one byte per element plus one scale byte per 32
        assert host(xp).nbytes + host(xs).nbytes == M.dispatch_bytes_mx(cfg.R, D)


MFMA_F8_EPS = 2.0 ** -16


def _ulp(v):
    """One bf16 ulp at |v| (8 significant bits; at least the smallest subnormal)."""
    return 2.0 ** (np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126))) - 7)


def y_bound(y_ref, pieces, w2):
    """Per-element bound on |Y_gpu - Y_oracle| (module text) from the oracle's intermediates."""
    dy = np.zeros_like(y_ref)
    for e, lo, hi, p in pieces:
        g, u, a = p["g"], p["u"], p["a"]
        ax = np.abs(p["x"])
        dg = MFMA_F8_EPS * (ax @ np.abs(p["w1"]).T)
        du = MFMA_F8_EPS * (ax @ np.abs(p["w3"]).T)
        sig = 0.5 * (1.0 + np.tanh(0.5 * g))
        dsilu = sig * (1.0 + g * (1.0 - sig))           # d SiLU / dG, |.| <= 1.1
        da = _ulp(a) + np.abs(dsilu * u) * dg + np.abs(g * sig) * du + 1.1 * dg * du
        w2e = np.abs(oracle.decode(w2[e]))
        dy[lo:hi] = 2.0 * _ulp(y_ref[lo:hi]) + da @ w2e.T + 2.0 ** -20 * (np.abs(a) @ w2e.T)
    return dy


def _check_y_mx(got, ref_y, dy):
    err = np.abs(oracle.decode(got) - ref_y)
    worst = float(np.max(err / dy))
    assert worst <= 1.0, f"worst |dY| / bound = {worst:.3f}"
    return worst


def _weights_mx(wts):
    return {n: M.mx_quantize(oracle.decode(wts[n])) for n in ("w1", "w3")}


@pytest.mark.parametrize("cfg", MX_CFGS, ids=MX_IDS)
def test_grouped_ffn_mx(cfg):
    lg, bias = _scores_input(cfg)
    ref = oracle.route(oracle.router_scores(lg, bias), cfg.k, cfg.E, cfg.capacity)
    rt, _ = oracle.permutation(ref["ids"], cfg.E, cfg.capacity)
    x = gen.draw(cfg, gen.TAG_X, 0, (cfg.T, cfg.D), cfg.x_std)
    xq, xsc = M.mx_quantize(oracle.decode(x))
    xq, xsc = xq[rt], xsc[rt]
    wts = gen.expert_weights(cfg)
    wq = _weights_mx(wts)
    s = shape_of(cfg)
    y = empty((cfg.R, cfg.D), "bf16")
    B.grouped_ffn(dev(xq), dev(ref["offsets"].astype(np.int32)), dev(wq["w1"][0]), dev(wq["w3"][0]),
                  dev(wts["w2"]), y, s, ws(s, B.MOE_CALL_FFN), x_perm_scale=dev(xsc),
                  w1_scale=dev(wq["w1"][1]), w3_scale=dev(wq["w3"][1]))
    torch.cuda.synchronize()
    ref_y, pieces = M.grouped_expert_ffn_mx(xq, xsc, ref["offsets"], wq["w1"][0], wq["w1"][1], wq["w3"][0],
                                            wq["w3"][1], wts["w2"], parts=True)
    _check_y_mx(host(y, bf16=True)[:len(ref_y)], ref_y, y_bound(ref_y, pieces, wts["w2"]))


def run_layer_mx(cfg, inp, with_aux=True, out_dtype=B.MOE_F32):
    """moe_layer_forward with MXFP8 dispatch; W1 / W3 quantised on the GPU."""
    s = shape_of(cfg)
    T, E, k, R, D, I = cfg.T, cfg.E, cfg.k, cfg.R, cfg.D, cfg.I
    w = {n: dev(inp[n]) for n in ("gate_w", "w2", "wd", "wu", "ws1", "ws3", "ws2") if n in inp}
    res = {}
    for n in ("w1", "w3"):
        q, sc = empty((E, I, D), "u8"), empty((E, I, D // 32), "u8")
        B.quantize_mxfp8(dev(inp[n]), q, sc)
        w[n], w[n + "_scale"] = q, sc
    if "bias" in inp:
        w["gate_bias"] = dev(inp["bias"])
    logits = dev(inp["logits"]) if "logits" in inp else empty((T, E), "f32")
    aux = {}
    if with_aux:
        aux = {"topk_ids": empty((T, k), "i32"), "topk_w": empty((T, k), "f32"),
               "counts": empty((E,), "i32"), "offsets": empty((E + 1,), "i32"),
               "row_token": empty((R,), "i32"), "token_row": empty((T, k), "i32"),
               "x_perm": empty((R, D), "u8"), "x_perm_scale": empty((R, D // 32), "u8"),
               "y_perm": empty((R, D), "bf16")}
        if cfg.L:
            aux["z"] = empty((T, cfg.L), "bf16")
            aux["out_latent"] = empty((T, cfg.L), "bf16")
    out = empty((T, cfg.H), "f32" if out_dtype == B.MOE_F32 else "bf16")
    B.layer_forward(w, dev(inp["x"]), logits, out, out_dtype, s, ws(s, B.MOE_CALL_LAYER), aux)
    torch.cuda.synchronize()
    res["out"] = host(out, out_dtype == B.MOE_BF16)
    res["logits"] = host(logits)
    for n in ("w1", "w3"):
        res[n + "_q"], res[n + "_scale"] = host(w[n]), host(w[n + "_scale"])
    for n, t in aux.items():
        res[n] = host(t, n in ("y_perm", "z", "out_latent"))
    return res


@pytest.mark.parametrize("cfg", MX_CFGS, ids=MX_IDS)
def test_layer_forward_mx(cfg):
    check_layer_mx(cfg)


def check_layer_mx(cfg):
    """The MXFP8 layer against the oracle's: weight codes, routing and dispatched codes
    bit-exact (given logits), every output element within the derived bound."""
    inp = gen.layer_inputs(cfg)
    got = run_layer_mx(cfg, inp)
    ref = oracle.layer_forward(inp, k=cfg.k, E=cfg.E, bf16=True, capacity=cfg.capacity, dispatch="mxfp8")
    for n in ("w1", "w3"):       # the conversion kernel on the weights
        np.testing.assert_array_equal(got[n + "_scale"], ref[n + "_scale"])
        np.testing.assert_array_equal(got[n + "_q"], ref[n + "_q"])
    same = np.ones(cfg.T, dtype=bool)
    if cfg.L:
        # Z comes from a bf16 GEMM whose sums may put an element one ulp from the
        # oracle's, and then its codes differ too: codes and the bound are checked on
        # the tokens whose Z row matches bit for bit (most of them)
        same = np.all(got["z"] == _bf16_bits(ref["z"]), axis=1)
        assert same.mean() > 0.5, f"only {same.mean():.2f} of the Z rows match"
    if "logits" in inp:          # routing and the quantised dispatch bit-exact
        np.testing.assert_array_equal(got["topk_ids"], ref["ids"])
        np.testing.assert_array_equal(got["offsets"], ref["offsets"])
        n = len(ref["row_token"])
        np.testing.assert_array_equal(got["row_token"][:n], ref["row_token"])
        np.testing.assert_array_equal(got["token_row"], ref["token_row"])
        rows = same[ref["row_token"]]
        np.testing.assert_array_equal(got["x_perm"][:n][rows], ref["x_perm_q"][rows])
        np.testing.assert_array_equal(got["x_perm_scale"][:n][rows], ref["x_perm_scale"][rows])
        keep = np.ones(cfg.T, dtype=bool)
    else:                        # computed gate: compare where the exact logits decide routing
        from tests.test_gpu_parity import unambiguous_tokens
        tol = 1e-5 * float(np.sqrt(np.mean(ref["logits"] ** 2)))
        keep = unambiguous_tokens(ref["logits"], cfg.k, tol)
        assert keep.mean() > 0.99
        np.testing.assert_array_equal(np.sort(got["topk_ids"][keep], axis=1),
                                      np.sort(ref["ids"][keep], axis=1))
    keep = keep & same
    # the bound on Y carried through the combine's weights (fp32 sums); a shared
    # expert's bf16 term adds the bf16 path's allowance (one ulp of its output + 5e-3 x
    # its RMS); a latent layer rounds the combined rows to bf16 (one more ulp) and
    # spreads each over the H outputs of the up-projection
    dy = y_bound(ref["y_perm"], ref["ffn_parts"], inp["w2"])
    tr = ref["token_row"]
    dcomb = np.zeros((cfg.T, cfg.D))
    for j in range(cfg.k):
        r = tr[:, j]
        kept = r >= 0
        dcomb[kept] += ref["weights"][kept, j][:, None] * dy[r[kept]]
    if cfg.L:
        dcomb += _ulp(ref["out_combine"])
        dout = dcomb @ np.abs(oracle.decode(inp["wu"])).T
    else:
        dout = dcomb
    if cfg.shared_I:
        ysh = ref["y_shared"]
        dout = dout + _ulp(ysh) + 5e-3 * np.sqrt(np.mean(ysh ** 2))
    dout = dout + 2.0 ** -20 * np.abs(ref["out"]) + 1e-30
    err = np.abs(got["out"] - ref["out"])
    worst = float(np.max(err[keep] / dout[keep]))
    assert worst <= 1.0, f"worst |d out| / bound = {worst:.3f}"


@pytest.mark.parametrize("name", ["small_bf16_zipf", "small_bf16_decode", "wide_experts", "small_latent",
                                  "capacity_decode"])
def test_layer_mx_equals_separate_calls(name):
    """The fused MXFP8 layer equals route -> dispatch -> grouped FFN -> combine, bit for bit,
    and is deterministic; its value change against the bf16 layer is reported, not zero."""
    cfg = _mx(PARITY_CONFIGS[name])
    inp = gen.layer_inputs(cfg)
    a = run_layer_mx(cfg, inp)
    b = run_layer_mx(cfg, inp)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    s = shape_of(cfg)
    T, E, k, R, D = cfg.T, cfg.E, cfg.k, cfg.R, cfg.D
    ids, offs = dev(a["topk_ids"]), dev(a["offsets"])
    src = dev(inp["x"]) if not cfg.L else dev(a["z"])
    xp, xs = empty((R, D), "u8"), empty((R, D // 32), "u8")
    rt, tr = empty((R,), "i32"), empty((T, k), "i32")
    B.dispatch_permute(src, ids, offs, xp, rt, tr, s, ws(s, B.MOE_CALL_DISPATCH), x_perm_scale=xs)
    yp = empty((R, D), "bf16")
    B.grouped_ffn(xp, offs, dev(a["w1_q"]), dev(a["w3_q"]), dev(inp["w2"]), yp, s, ws(s, B.MOE_CALL_FFN),
                  x_perm_scale=xs, w1_scale=dev(a["w1_scale"]), w3_scale=dev(a["w3_scale"]))
    torch.cuda.synchronize()
    n = int(a["offsets"][-1])
    np.testing.assert_array_equal(host(xp)[:n], a["x_perm"][:n])
    np.testing.assert_array_equal(host(xs)[:n], a["x_perm_scale"][:n])
    np.testing.assert_array_equal(host(yp, True)[:n], a["y_perm"][:n])
    # the decode-scale fast path (no aux x_perm) gives the same output bits
    c = run_layer_mx(cfg, inp, with_aux=False)
    np.testing.assert_array_equal(c["out"], a["out"])
    # bf16 output = RNE of the fp32 output
    d = run_layer_mx(cfg, inp, with_aux=False, out_dtype=B.MOE_BF16)
    np.testing.assert_array_equal(d["out"], _bf16_bits(a["out"]))


# MXFP8 layers whose gate/up GEMM reads the token rows through row_token when the caller
# does not ask for the permuted codes: persistent prefill tiles (D / 2 >= 256 16-bit
# columns) and decode-scale tiles above 128 tokens (the general routing kernels)
MX_GATHER = [MoEConfig(name="mx_gather_prefill", T=300, H=512, E=16, k=4, I=192, seed=43,
                       gate="computed", gate_std=0.05, dispatch="mxfp8"),
             MoEConfig(name="mx_gather_prefill_ragged", T=517, H=640, E=24, k=6, I=320, seed=44,
                       gate="drawn", dispatch="mxfp8"),
             MoEConfig(name="mx_gather_decode", T=130, H=512, E=64, k=4, I=128, seed=45,
                       gate="drawn", dispatch="mxfp8")]


@pytest.mark.parametrize("cfg", MX_GATHER, ids=[c.name for c in MX_GATHER])
def test_layer_mx_gathered_rows(cfg):
    """Without aux x_perm the layer quantises the token rows once and gathers them; the
    output bits equal those of the layer that writes the permuted codes, which the oracle
    bounds."""
    inp = gen.layer_inputs(cfg)
    a = run_layer_mx(cfg, inp)
    b = run_layer_mx(cfg, inp, with_aux=False)
    np.testing.assert_array_equal(b["out"], a["out"])
    check_layer_mx(cfg)


# ------------------------------------------------------------------ full size, sampled tokens

FULL_MX = ["qwen3_30b_a3b_shaped", "k3_shaped_decode", "k3_shaped_decode_t8"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL_MX)
def test_layer_full_size_mx_sampled(name):
    """The full-size layer with MXFP8 dispatch in the launch configuration bench.py
    times: W1 / W3 codes of the sampled tokens' experts bit-exact against the oracle's
    conversion, and the fp32 output of sampled tokens within the derived bound."""
    from workloads import FULL_CONFIGS
    cfg = _mx(FULL_CONFIGS[name])
    print(f"\n[{name}] generating inputs", flush=True)
    inp = gen.layer_inputs(cfg)
    T, E, k, D, I = cfg.T, cfg.E, cfg.k, cfg.D, cfg.I
    assert not cfg.L and not cfg.shared_I
    s = shape_of(cfg)
    w = {n: dev(inp[n]) for n in ("gate_w", "w2") if n in inp}
    for n in ("w1", "w3"):
        q, sc = empty((E, I, D), "u8"), empty((E, I, D // 32), "u8")
        B.quantize_mxfp8(dev(inp[n]), q, sc)
        w[n], w[n + "_scale"] = q, sc
    if "bias" in inp:
        w["gate_bias"] = dev(inp["bias"])
    logits = dev(inp["logits"]) if "logits" in inp else empty((T, E), "f32")
    ids = empty((T, k), "i32")
    out32 = empty((T, cfg.H), "f32")
    print(f"[{name}] running the layer", flush=True)
    B.layer_forward(w, dev(inp["x"]), logits, out32, B.MOE_F32, s, ws(s, B.MOE_CALL_LAYER), {"topk_ids": ids})
    torch.cuda.synchronize()
    o32, gids = host(out32), host(ids)
    rng = np.random.default_rng(cfg.seed + 1)
    tok = np.sort(rng.choice(T, size=min(12, T), replace=False))
    if "logits" in inp:
        scores = oracle.router_scores(inp["logits"][tok], inp.get("bias"))
        keep = np.ones(len(tok), dtype=bool)
    else:
        lg_ref = oracle.gate_logits(inp["x"][tok], inp["gate_w"], inp.get("bias"))
        rms_l = float(np.sqrt(np.mean(lg_ref ** 2)))
        scores = lg_ref.astype(np.float32)
        srt = -np.sort(-lg_ref, axis=1)
        keep = (srt[:, k - 1] - srt[:, k]) > 2e-5 * rms_l
    r = oracle.route(scores, k, E)
    np.testing.assert_array_equal(np.sort(gids[tok][keep], 1), np.sort(r["ids"][keep], 1))
    tk, ids_k, wts_k = tok[keep], r["ids"][keep], r["weights"][keep]
    xq, xs = M.mx_quantize(oracle.decode(inp["x"][tk]))
    need = sorted(set(int(e) for e in ids_k.ravel()))
    print(f"[{name}] oracle on {len(tk)} sampled tokens, {len(need)} experts", flush=True)
    y, dy = {}, {}
    for e in need:
        wq = [M.mx_quantize(oracle.decode(inp[n][e])) for n in ("w1", "w3")]
        for n, (q, sc) in zip(("w1", "w3"), wq):   # the conversion kernel at full size
            np.testing.assert_array_equal(host(w[n + "_scale"][e]), sc)
            np.testing.assert_array_equal(host(w[n][e]), q)
        rows = [i for i in range(len(tk)) if e in ids_k[i]]
        ye, p = M.expert_ffn_rows_mx(xq[rows], xs[rows], wq[0][0], wq[0][1], wq[1][0], wq[1][1],
                                     inp["w2"][e], parts=True)
        de = y_bound(ye, [(e, 0, len(rows), p)], {e: inp["w2"][e]})
        for j, i in enumerate(rows):
            y[(i, e)], dy[(i, e)] = ye[j], de[j]
    ref = np.zeros((len(tk), cfg.H))
    dout = np.zeros((len(tk), cfg.H))
    for i in range(len(tk)):
        for j in range(k):
            e = int(ids_k[i, j])
            ref[i] += wts_k[i, j] * y[(i, e)]
            dout[i] += wts_k[i, j] * dy[(i, e)]
    dout += 2.0 ** -20 * np.abs(ref) + 1e-30
    ratio = float(np.max(np.abs(o32[tk] - ref) / dout))
    print(f"[{name}] worst |d out| / bound = {ratio:.3f}", flush=True)
    assert ratio <= 1.0
