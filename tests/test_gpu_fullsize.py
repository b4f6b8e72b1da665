"""GPU parity at the full layer sizes, in the launch configuration bench.py times.

* routing (ids, counts, offsets) on the full seeded fp32 logits: bit-exact over
  all T tokens;
* moe_layer_forward on the full layer, in the dataflow bench.py times (no permuted
  copy requested): ids, weights, counts and offsets over all T tokens against the
  oracle's router on the fp32 logits the layer ranked (bit-exact; weights within
  1e-6), the permutation bit-exact, the dispatch buffer exactly T*k*D*b bytes;
* every row of whole experts' outputs Y (the most loaded expert, one whose rows end
  in a ragged m-tile, one of median load and the least loaded one) against the
  oracle's expert FFN: these are the rows the full-size kernels and tile tables
  (XCD-chunk tables, 256-row long-K down tiles) produce;
* the fp32 output of sampled tokens against the oracle evaluated token by token
  (max |d| <= 2e-2 x RMS for bf16, 1e-5 x RMS for fp32), on tokens whose top-k
  set the scores fix beyond rounding;
* the bf16 output is the round-to-nearest-even of the fp32 output everywhere.

Full-size weights (up to 22.5 GB) are generated on the host once per module.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import FULL_CONFIGS, generator as gen
from routing_dispatch_expert_logits_amd import binding as B
from tests.gpu_util import (dev, host, empty, ws, shape_of, act_kind, rne_bf16_bits,
                            check_permutation_valid, out_err_over_rms, check_y_rows,
                            latent_rows_and_dev)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

NAMES = ["qwen3_30b_a3b_shaped", "k3_shaped_decode", "latent_moe", "deepseek_r1_shaped"]
N_SAMPLE = 12


@pytest.mark.parametrize("name", NAMES + ["tiny_f32"])
def test_route_full_size_bit_exact(name):
    cfg = FULL_CONFIGS[name]
    lg, bias = gen.drawn_logits(cfg), gen.zipf_bias(cfg)
    s = shape_of(cfg)
    ids, w = empty((cfg.T, cfg.k), "i32"), empty((cfg.T, cfg.k), "f32")
    counts, offs = empty((cfg.E,), "i32"), empty((cfg.E + 1,), "i32")
    B.route_topk(None, None, None if bias is None else dev(bias), dev(lg), ids, w, counts, offs, s,
                 ws(s, B.MOE_CALL_ROUTE))
    torch.cuda.synchronize()
    ref = oracle.route(oracle.router_scores(lg, bias), cfg.k, cfg.E)
    np.testing.assert_array_equal(host(ids), ref["ids"])
    np.testing.assert_array_equal(host(counts), ref["counts"])
    np.testing.assert_array_equal(host(offs), ref["offsets"])
    assert np.max(np.abs(host(w) - ref["weights"])) <= 1e-6


@pytest.mark.parametrize("name", NAMES + ["deepseek_r1_shaped_shared"])
def test_layer_full_size_sampled(name):
    cfg = FULL_CONFIGS[name]
    bf = cfg.dtype == "bf16"
    print(f"\n[{name}] generating inputs", flush=True)
    inp = gen.layer_inputs(cfg)
    s = shape_of(cfg)
    T, E, k, R, D = cfg.T, cfg.E, cfg.k, cfg.R, cfg.D
    w = {n: dev(inp[n]) for n in ("gate_w", "w1", "w3", "w2", "wd", "wu", "ws1", "ws3", "ws2")
         if n in inp}
    if "bias" in inp:
        w["gate_bias"] = dev(inp["bias"])
    x = dev(inp["x"])
    logits = dev(inp["logits"]) if "logits" in inp else empty((T, E), "f32")
    aux = {"topk_ids": empty((T, k), "i32"), "topk_w": empty((T, k), "f32"),
           "counts": empty((E,), "i32"), "offsets": empty((E + 1,), "i32"),
           "row_token": empty((R,), "i32"), "token_row": empty((T, k), "i32"),
           "y_perm": empty((R, D), act_kind(cfg))}
    if cfg.L:
        aux["z"] = empty((T, cfg.L), act_kind(cfg))
    wsp = ws(s, B.MOE_CALL_LAYER)
    out32 = empty((T, cfg.H), "f32")
    out16 = empty((T, cfg.H), "bf16")
    print(f"[{name}] running the layer", flush=True)
    B.layer_forward(w, x, logits, out32, B.MOE_F32, s, wsp, aux)
    B.layer_forward(w, x, logits, out16, B.MOE_BF16, s, wsp)
    torch.cuda.synchronize()
    got = {n: host(t, bf and n == "y_perm") for n, t in aux.items() if n != "z"}
    o32 = host(out32)
    # whole-size invariants
    assert got["counts"].sum() == T * k
    np.testing.assert_array_equal(got["counts"], np.diff(got["offsets"]))
    check_permutation_valid(got["topk_ids"], got["offsets"], got["row_token"], got["token_row"])
    # routing over all T tokens, given the fp32 scores the layer ranked: the logits it
    # wrote (computed gates, bias included) or the given logits plus the bias
    if "logits" in inp:
        scores_all = oracle.router_scores(inp["logits"], inp.get("bias"))
    else:
        scores_all = oracle.router_scores(host(logits), None)
    r_all = oracle.route(scores_all, k, E)
    np.testing.assert_array_equal(got["topk_ids"], r_all["ids"])
    np.testing.assert_array_equal(got["counts"], r_all["counts"])
    np.testing.assert_array_equal(got["offsets"], r_all["offsets"])
    assert np.max(np.abs(got["topk_w"] - r_all["weights"])) <= 1e-6
    # the row order is a function of the ids alone: bit-exact against the oracle's
    rt, tr = oracle.permutation(got["topk_ids"], E)
    np.testing.assert_array_equal(got["row_token"], rt)
    np.testing.assert_array_equal(got["token_row"], tr)
    assert R * D * cfg.elem_bytes == oracle.dispatch_bytes(T, k, D, cfg.elem_bytes)
    np.testing.assert_array_equal(host(out16, True), rne_bf16_bits(o32))
    # whole experts' Y rows against the oracle's expert FFN on the same input rows
    cnt = got["counts"]
    live = np.nonzero(cnt)[0]
    ragged = [e for e in live if cnt[e] % 128 and cnt[e] > 128]
    pick = {int(live[np.argmax(cnt[live])]), int(live[np.argmin(cnt[live])]),
            int(live[np.argsort(cnt[live])[len(live) // 2]])}
    if ragged:
        pick.add(int(ragged[len(ragged) // 2]))
    for e in sorted(pick):
        lo, hi = int(got["offsets"][e]), int(got["offsets"][e + 1])
        toks = rt[lo:hi]
        x_dev = None
        if cfg.L:   # the dispatched rows are the latent ones: the oracle's own Z of these tokens;
            # the layer's Z within the derived bound of it, which then widens the Y bound
            xr, x_dev = latent_rows_and_dev(inp["x"][toks], inp["wd"])
            zg = oracle.decode(host(aux["z"], True)[toks])
            assert np.all(np.abs(zg - xr) <= x_dev), "latent Z outside its derived bound"
        else:
            xr = inp["x"][toks]
        print(f"[{name}] expert {e}: {hi - lo} rows", flush=True)
        check_y_rows(bf, got["y_perm"][lo:hi], xr, inp["w1"][e], inp["w3"][e], inp["w2"][e], x_dev)
    # sampled tokens against the oracle
    rng = np.random.default_rng(cfg.seed)
    tok = np.sort(rng.choice(T, size=min(N_SAMPLE, T), replace=False))
    if "logits" in inp:
        scores = oracle.router_scores(inp["logits"][tok], inp.get("bias"))
        keep = np.ones(len(tok), dtype=bool)
    else:
        lg_ref = oracle.gate_logits(inp["x"][tok], inp["gate_w"], inp.get("bias"))
        g_lg = host(logits)[tok]
        rms_l = float(np.sqrt(np.mean(lg_ref ** 2)))
        assert float(np.max(np.abs(g_lg - lg_ref))) <= 1e-5 * rms_l
        scores = lg_ref.astype(np.float32)
        srt = -np.sort(-lg_ref, axis=1)
        keep = (srt[:, k - 1] - srt[:, k]) > 2e-5 * rms_l
    r = oracle.route(scores, k, E)
    np.testing.assert_array_equal(np.sort(got["topk_ids"][tok][keep], 1), np.sort(r["ids"][keep], 1))
    need = sorted(set(int(e) for e in r["ids"][keep].ravel()))
    ew = {e: (inp["w1"][e], inp["w3"][e], inp["w2"][e]) for e in need}
    z = oracle.latent_down(inp["x"][tok], inp["wd"], bf) if cfg.L else None
    print(f"[{name}] oracle on {keep.sum()} sampled tokens, {len(need)} experts", flush=True)
    ref_out = oracle.token_outputs(inp, tok[keep], r["ids"][keep], r["weights"][keep], ew, bf16=bf,
                                   z=None if z is None else z[keep])
    ysh = None
    if cfg.shared_I and bf:
        ysh = oracle.shared_expert_ffn(inp["x"][tok[keep]], inp["ws1"], inp["ws3"], inp["ws2"], bf)
    err = out_err_over_rms(o32[tok][keep], ref_out, ysh)
    print(f"[{name}] max|err|/RMS = {err:.3e}", flush=True)
    assert err <= (2e-2 if bf else 1e-5)
