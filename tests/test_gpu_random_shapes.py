"""GPU parity on seeded random small layers (shapes the fixed configs do not hit).

Each case draws T, H, E, k, I (within the library's limits: bf16 widths in
multiples of 64, fp32 widths in multiples of 4) and optionally a shared expert
and an expert capacity, routes on given logits (so routing, counts, offsets and
the permutation must be bit-exact) and compares the whole layer with the oracle
at the tolerances of test_gpu_parity.  Further cases draw latent layers, and
layers with MXFP8 dispatch (dispatched width a multiple of 128; checked against
the derived per-element bound of test_gpu_mxfp8).
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import MoEConfig, generator as gen
from routing_dispatch_expert_logits_amd import binding as B
from tests.gpu_util import dev, host, empty, ws, shape_of, out_err_over_rms

pytestmark = pytest.mark.gpu


def _case(i):
    r = np.random.default_rng(9000 + i)
    f32 = i % 5 == 4
    E = int(r.choice([1, 3, 8, 17, 40, 100, 257, 600]))
    k = int(r.integers(1, min(E, 9) + 1))
    T = int(r.choice([1, 7, 33, 64, 65, 130, 400, 1000]))
    if f32:
        H, I = int(r.integers(2, 40)) * 4, int(r.integers(2, 40)) * 4
    else:
        H, I = int(r.integers(1, 6)) * 64, int(r.integers(1, 6)) * 64
    shared = int(r.choice([0, 0, I])) if not f32 else int(r.choice([0, 8]))
    cap = int(r.choice([0, 0, max(1, T * k // (2 * E))]))
    return MoEConfig(name=f"rand{i}", T=T, H=H, E=E, k=k, I=I, dtype="f32" if f32 else "bf16",
                     seed=9000 + i, w_std=0.05 if f32 else 0.02, gate="drawn", gate_std=None,
                     zipf_s=1.1 if i % 3 == 0 else None, zipf_alpha=1.0, shared_I=shared, capacity=cap)


CASES = [_case(i) for i in range(24)]


@pytest.mark.parametrize("cfg", CASES, ids=[f"{c.name}-T{c.T}-E{c.E}-k{c.k}-H{c.H}-I{c.I}-s{c.shared_I}-c{c.capacity}-{c.dtype}"
                                            for c in CASES])
def test_random_layer(cfg):
    inp = gen.layer_inputs(cfg)
    T, E, k, R, D = cfg.T, cfg.E, cfg.k, cfg.R, cfg.D
    s = shape_of(cfg)
    w = {n: dev(inp[n]) for n in ("w1", "w3", "w2", "ws1", "ws3", "ws2") if n in inp}
    if "bias" in inp:
        w["gate_bias"] = dev(inp["bias"])
    aux = {"topk_ids": empty((T, k), "i32"), "topk_w": empty((T, k), "f32"),
           "counts": empty((E,), "i32"), "offsets": empty((E + 1,), "i32"),
           "row_token": empty((R,), "i32"), "token_row": empty((T, k), "i32")}
    out = empty((T, cfg.H), "f32")
    B.layer_forward(w, dev(inp["x"]), dev(inp["logits"]), out, B.MOE_F32, s, ws(s, B.MOE_CALL_LAYER), aux)
    torch.cuda.synchronize()
    bf = cfg.dtype == "bf16"
    ref = oracle.layer_forward(inp, k=k, E=E, bf16=bf, capacity=cfg.capacity)
    got = {n: host(t) for n, t in aux.items()}
    np.testing.assert_array_equal(got["topk_ids"], ref["ids"])
    assert np.max(np.abs(got["topk_w"] - ref["weights"])) <= 1e-6
    np.testing.assert_array_equal(got["counts"], ref["counts"])
    np.testing.assert_array_equal(got["offsets"], ref["offsets"])
    n = len(ref["row_token"])
    np.testing.assert_array_equal(got["row_token"][:n], ref["row_token"])
    np.testing.assert_array_equal(got["token_row"], ref["token_row"])
    ysh = ref.get("y_shared") if bf else None
    err = out_err_over_rms(host(out), ref["out"], ysh)
    assert err <= (2e-2 if bf else 1e-5), f"max|err|/RMS {err:.3e}"


def _latent_case(i):
    r = np.random.default_rng(9500 + i)
    E = int(r.choice([4, 16, 64, 300]))
    k = int(r.integers(1, min(E, 8) + 1))
    T = int(r.choice([5, 64, 100, 700]))
    H = int(r.integers(2, 8)) * 64
    L = int(r.integers(1, 5)) * 64
    I = int(r.integers(1, 5)) * 64
    cap = int(r.choice([0, max(1, T * k // (2 * E))]))
    return MoEConfig(name=f"lat{i}", T=T, H=H, L=L, E=E, k=k, I=I, seed=9500 + i, gate="drawn",
                     gate_std=None, zipf_s=1.1 if i % 2 else None, zipf_alpha=1.0, capacity=cap)


LATENT = [_latent_case(i) for i in range(8)]


@pytest.mark.parametrize("cfg", LATENT, ids=[f"{c.name}-T{c.T}-E{c.E}-k{c.k}-H{c.H}-L{c.L}-I{c.I}-c{c.capacity}"
                                             for c in LATENT])
def test_random_latent_layer(cfg):
    inp = gen.layer_inputs(cfg)
    T, E, k, R = cfg.T, cfg.E, cfg.k, cfg.R
    s = shape_of(cfg)
    w = {n: dev(inp[n]) for n in ("w1", "w3", "w2", "wd", "wu")}
    if "bias" in inp:
        w["gate_bias"] = dev(inp["bias"])
    aux = {"topk_ids": empty((T, k), "i32"), "offsets": empty((E + 1,), "i32"),
           "token_row": empty((T, k), "i32")}
    out = empty((T, cfg.H), "f32")
    B.layer_forward(w, dev(inp["x"]), dev(inp["logits"]), out, B.MOE_F32, s, ws(s, B.MOE_CALL_LAYER), aux)
    torch.cuda.synchronize()
    ref = oracle.layer_forward(inp, k=k, E=E, bf16=True, capacity=cfg.capacity)
    np.testing.assert_array_equal(host(aux["topk_ids"]), ref["ids"])
    np.testing.assert_array_equal(host(aux["offsets"]), ref["offsets"])
    np.testing.assert_array_equal(host(aux["token_row"]), ref["token_row"])
    assert out_err_over_rms(host(out), ref["out"]) <= 2e-2


def _mx_case(i):
    r = np.random.default_rng(9700 + i)
    E = int(r.choice([1, 6, 32, 100, 257]))
    k = int(r.integers(1, min(E, 9) + 1))
    T = int(r.choice([1, 9, 64, 65, 300, 900]))
    latent = i % 4 == 3
    H = int(r.integers(1, 5)) * 128
    L = int(r.integers(1, 3)) * 128 if latent else 0
    I = int(r.integers(1, 6)) * 64
    shared = 0 if latent else int(r.choice([0, 0, 128]))
    cap = int(r.choice([0, 0, max(1, T * k // (2 * E))]))
    return MoEConfig(name=f"mx{i}", T=T, H=H, L=L, E=E, k=k, I=I, seed=9700 + i, gate="drawn",
                     gate_std=None, zipf_s=1.2 if i % 3 == 0 else None, zipf_alpha=1.0,
                     shared_I=shared, capacity=cap, dispatch="mxfp8")


MX = [_mx_case(i) for i in range(16)]


@pytest.mark.parametrize("cfg", MX, ids=[f"{c.name}-T{c.T}-E{c.E}-k{c.k}-H{c.H}-L{c.L}-I{c.I}-s{c.shared_I}"
                                         f"-c{c.capacity}" for c in MX])
def test_random_mx_layer(cfg):
    from tests.test_gpu_mxfp8 import check_layer_mx
    check_layer_mx(cfg)
