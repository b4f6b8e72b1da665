"""CPU oracle of the routed-expert MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or run anything in this package.  The product
path (the HIP library and its Python binding) never touches it, and this
package imports nothing from the product path: the two share only the seeded
input generator in ``workloads/``.

It is a plain, slow, obviously correct restatement of what the layer
computes, in float64 numpy, one step per function, in the order of the
pipeline described on the WideEP explainer page ("The router writes a network
schedule"): scoring and top-k selection at the source, a tally per destination
and the reservation of places, a permutation of activations into
destination-contiguous rows with routing metadata, grouping by expert and the
expert matrix multiplies, and the combine that undoes the permutation and
applies the routing weights.

Where the pages leave a step open the plainest reading is taken (each one is
listed in the repository's design notes):

* scores: softmax over all E experts, keep the top k, renormalise the kept
  probabilities (the tiny fp32 layer's workload text); an optional per-expert
  bias is added to the logits used for both selection and weights;
* ties: equal scores are ordered by the lower expert index, and the k ids of a
  token are listed by descending score; -0.0 ranks equal to +0.0;
* the selection decision is taken on fp32 scores (the router precision);
* rows inside an expert's segment are in ascending token order;
* the expert FFN is SwiGLU: (SiLU(x W1) * (x W3)) W2, W1 the gate branch;
* bf16 layers keep the expert intermediate A, the expert output Y, the latent
  Z and the latent combine output in bf16 (round to nearest, ties to even);
  everything else is exact (fp64) here.

Parity pins: every function is checked in ``tests/test_oracle_pins.py``
against something other than itself (library routines on special cases,
brute force on tiny inputs, closed forms, invariants and the worked numbers
the pages print).
"""
from __future__ import annotations

import time
from typing import Dict, Optional

import numpy as np

# --------------------------------------------------------------------------------------
# element formats
# --------------------------------------------------------------------------------------


def decode(a: np.ndarray) -> np.ndarray:
    """Stored layer tensor -> float64.  uint16 arrays hold bf16 bit patterns."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even (returned as float64).

    bf16 keeps 8 significant bits.  Write x = m * 2**e with 0.5 <= |m| < 1
    (frexp), scale m to 8 integer bits, round half to even (rint) and scale
    back.  Values here are far from the bf16 subnormal and overflow ranges.
    """
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.rint(m * 256.0), e - 8)


def round_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 values to fp32 (IEEE round to nearest even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# --------------------------------------------------------------------------------------
# a1: gating scores
# --------------------------------------------------------------------------------------


def gate_logits(x: np.ndarray, gate_w: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Router logits[t, e] = sum_h X[t, h] * Wg[e, h] (+ bias[e]), exact in float64.

    The source rank scores every token against every expert (WideEP explainer,
    "The router writes a network schedule"; the gating network is replicated on
    every rank, research-vault claim IX2-0406).  ``gate_w`` is stored [E x H].
    """
    out = decode(x) @ decode(gate_w).T
    if bias is not None:
        out = out + decode(bias)[None, :]
    return out


def router_scores(logits_f32: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """fp32 scores used for selection and weights when the logits are given.

    With a bias the score is the fp32 sum logits + bias (one IEEE fp32 add).
    """
    s = np.asarray(logits_f32, dtype=np.float32)
    if bias is not None:
        s = (s + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    return s


# --------------------------------------------------------------------------------------
# a2: top-k selection and routing weights
# --------------------------------------------------------------------------------------


def topk_ids(scores: np.ndarray, k: int) -> np.ndarray:
    """Per token, the k experts with the largest scores, listed by descending score.

    Each token picks k distinct experts (WideEP explainer, "Sparse compute. Dense
    availability." and "The router writes a network schedule": one token becomes
    k expert assignments).  Selection is k rounds of: among experts not yet
    taken, the largest score, the lowest expert index on ties.  -0.0 and +0.0
    compare equal, as in IEEE arithmetic.
    """
    s = np.asarray(scores, dtype=np.float64)
    T, E = s.shape
    assert 1 <= k <= E
    taken = np.zeros((T, E), dtype=bool)
    ids = np.empty((T, k), dtype=np.int32)
    rows = np.arange(T)
    for j in range(k):
        cand = np.where(taken, -np.inf, s)
        best = cand.max(axis=1)
        hit = (cand == best[:, None]) & ~taken
        pick = hit.argmax(axis=1)            # first (lowest index) untaken expert at the max
        ids[:, j] = pick
        taken[rows, pick] = True
    return ids


def routing_weights(scores: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Softmax over all E experts, gathered at the selected ids and renormalised over k.

    The weights are applied by the source after the combine (WideEP explainer,
    "The router writes a network schedule").  Float64 throughout.
    """
    s = np.asarray(scores, dtype=np.float64)
    z = s - s.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    g = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    return g / g.sum(axis=1, keepdims=True)


def routing_margins(scores: np.ndarray, k: int) -> np.ndarray:
    """Per token, the smallest gap between consecutive scores among the k+1 largest.

    Not a step of the layer: tests use it to tell tokens whose routing is fixed by
    the scores alone from near-ties that rounding may decide either way.
    """
    s = -np.sort(-np.asarray(scores, dtype=np.float64), axis=1)
    top = s[:, : min(k + 1, s.shape[1])]
    if top.shape[1] < 2:
        return np.full(s.shape[0], np.inf)
    return np.min(top[:, :-1] - top[:, 1:], axis=1)


# --------------------------------------------------------------------------------------
# a3: counts per destination and slot offsets
# --------------------------------------------------------------------------------------


def expert_counts(ids: np.ndarray, E: int) -> np.ndarray:
    """counts[e] = number of (token, slot) assignments routed to expert e.

    Counts are assignments, not unique tokens: a top-k token adds k rows ("Three
    Parameter Counts...", section "What the utilization dashboard smooths
    away"); the dispatcher tallies the rows per destination ("The router writes a
    network schedule").
    """
    counts = np.zeros(E, dtype=np.int64)
    for e in range(E):
        counts[e] = int(np.count_nonzero(ids == e))
    return counts


def segment_offsets(counts: np.ndarray) -> np.ndarray:
    """offsets[0] = 0, offsets[e+1] = offsets[e] + counts[e]: each expert's slot range."""
    off = np.zeros(len(counts) + 1, dtype=np.int64)
    for e, c in enumerate(counts):
        off[e + 1] = off[e] + int(c)
    return off


# --------------------------------------------------------------------------------------
# a4: permutation into expert-contiguous rows + routing metadata
# --------------------------------------------------------------------------------------


def permutation(ids: np.ndarray, E: int, capacity: int = 0):
    """Expert-contiguous row order and its inverse.

    Expert e's segment holds, in ascending token order, every token that picked
    e.  Returns ``row_token[r]`` (source token of row r) and ``token_row[t, j]``
    (row holding token t's j-th assignment), the routing metadata attached to
    the permuted rows (WideEP explainer, "The router writes a network
    schedule").

    With ``capacity`` C > 0 an expert keeps only its first C assignments in that
    order; the later ones are dropped (``token_row`` = -1) and ``row_token`` holds
    the kept rows only.  Dropping is value-changing (WideEP explainer, "An
    imbalanced router creates a network hotspot"); C = 0 keeps everything.
    """
    T, k = ids.shape
    row_token = []
    token_row = np.full((T, k), -1, dtype=np.int64)
    for e in range(E):
        hit_t, hit_j = np.nonzero(ids == e)       # row-major scan: ascending token
        for n, (t, j) in enumerate(zip(hit_t.tolist(), hit_j.tolist())):
            if capacity and n >= capacity:
                break
            token_row[t, j] = len(row_token)
            row_token.append(t)
    if not capacity:
        assert len(row_token) == T * k
    return np.asarray(row_token, dtype=np.int64), token_row


def gather_rows(x: np.ndarray, row_token: np.ndarray) -> np.ndarray:
    """x_perm[r] = X[row_token[r]]: the dispatch payload, a plain copy of rows."""
    return np.asarray(x)[row_token]


def dispatch_bytes(T: int, k: int, width: int, elem_bytes: int) -> int:
    """Bytes of the permuted activation buffer: T * k * width * bytes per element.

    The pages give T x k x H x B as the dispatch payload (WideEP explainer, "Top-k
    multiplies traffic. Locality subtracts it."; an upper bound in "Three
    Parameter Counts...", "Halving top-k is a network change first").  On one
    GPU with an unpadded layout every assignment is local and the product is
    exact.
    """
    return int(T) * int(k) * int(width) * int(elem_bytes)


# --------------------------------------------------------------------------------------
# a5: grouped SwiGLU expert FFN
# --------------------------------------------------------------------------------------


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def expert_ffn_rows(x_rows: np.ndarray, w1e: np.ndarray, w3e: np.ndarray, w2e: np.ndarray,
                    bf16: bool) -> np.ndarray:
    """One expert's SwiGLU FFN on its rows: Y = (SiLU(X W1) * (X W3)) W2.

    Weights are stored output-major: w1e, w3e [I x D], w2e [D x I], so the math
    matrices are their transposes.  For bf16 layers the intermediate A and the
    output Y are rounded to bf16 (nearest even); sums are exact here.
    """
    xr = decode(x_rows)
    g = xr @ decode(w1e).T
    u = xr @ decode(w3e).T
    a = silu(g) * u
    if bf16:
        a = round_bf16(a)
    y = a @ decode(w2e).T
    if bf16:
        y = round_bf16(y)
    return y


def grouped_expert_ffn(x_perm: np.ndarray, offsets: np.ndarray, w1: np.ndarray, w3: np.ndarray,
                       w2: np.ndarray, bf16: bool) -> np.ndarray:
    """Expert e runs its FFN on rows [offsets[e], offsets[e+1]); an expert with no rows does nothing.

    The receiver groups rows by local expert and runs the expert matrix
    multiplies (WideEP explainer, "The router writes a network schedule"); a
    grouped GEMM gives an expert without rows nothing to do ("Three Parameter
    Counts...", "Which optimizations need a task-level gate").
    """
    E = len(offsets) - 1
    D = w2.shape[1]
    y = np.zeros((int(offsets[-1]), D), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            y[lo:hi] = expert_ffn_rows(x_perm[lo:hi], w1[e], w3[e], w2[e], bf16)
    return y


def shared_expert_ffn(x: np.ndarray, ws1: np.ndarray, ws3: np.ndarray, ws2: np.ndarray,
                      bf16: bool) -> np.ndarray:
    """The shared expert: a SwiGLU FFN that every token passes through, whatever
    the router picked ("Three Parameter Counts...", "What the utilization dashboard
    smooths away": shared experts of the DeepSeekMoE kind process every token
    whatever the router decides; it is one of the non-expert weights every rank replicates,
    research-vault claim IX2-0406).  The pages give no formula; it is read as an
    expert of the routed experts' form (and rounding points) with its own
    intermediate width, on all T rows of the full-width state.  ws1, ws3 are
    [Is x H], ws2 [H x Is].
    """
    return expert_ffn_rows(x, ws1, ws3, ws2, bf16)


# --------------------------------------------------------------------------------------
# a6: combine (unpermute + routing weights)
# --------------------------------------------------------------------------------------


def combine(y_perm: np.ndarray, token_row: np.ndarray, weights: np.ndarray,
            shared: Optional[np.ndarray] = None) -> np.ndarray:
    """out[t] = sum_j w[t, j] * Y[token_row[t, j]] (+ shared[t]), exact.

    The combine reverses the route, then the source unpermutes and applies the
    routing weights (WideEP explainer, "The router writes a network schedule").
    A shared expert's output, when present, enters with weight 1.  Assignments
    dropped by an expert capacity (token_row = -1) add nothing; the kept weights
    are not renormalised.
    """
    y = decode(y_perm) if y_perm.dtype == np.uint16 else np.asarray(y_perm, dtype=np.float64)
    T, k = token_row.shape
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for j in range(k):
        kept = token_row[:, j] >= 0               # dropped assignments (capacity) add nothing
        out[kept] += weights[kept, j:j + 1] * y[token_row[kept, j]]
    if shared is not None:
        out += decode(shared) if shared.dtype == np.uint16 else np.asarray(shared, dtype=np.float64)
    return out


# --------------------------------------------------------------------------------------
# a7: latent dispatch projections
# --------------------------------------------------------------------------------------


def latent_down(x: np.ndarray, wd: np.ndarray, bf16: bool) -> np.ndarray:
    """Z = X Wd: the reduced-width state that is dispatched ("Latent MoE": Definition).

    ``wd`` is stored [L x H]; Z is rounded to bf16 for bf16 layers.
    """
    z = decode(x) @ decode(wd).T
    return round_bf16(z) if bf16 else z


def latent_up(out_l: np.ndarray, wu: np.ndarray, bf16: bool) -> np.ndarray:
    """out = out_L Wu: restore the model width after the combine ("Latent MoE": Current Synthesis).

    ``wu`` is stored [H x L]; for bf16 layers the latent combine output is
    rounded to bf16 before the projection.
    """
    a = round_bf16(out_l) if bf16 else out_l
    return a @ decode(wu).T


# --------------------------------------------------------------------------------------
# whole layer
# --------------------------------------------------------------------------------------


def route(scores_f32: np.ndarray, k: int, E: int, capacity: int = 0) -> Dict[str, np.ndarray]:
    """a2 + a3 on given fp32 scores: ids, weights, counts, offsets.

    With an expert capacity C > 0 the slots allocated per expert are
    min(count, C): ``counts`` and ``offsets`` describe the kept rows, and
    ``routed_counts`` keeps the assignments before dropping.
    """
    ids = topk_ids(scores_f32, k)
    w = routing_weights(scores_f32, ids)
    routed = expert_counts(ids, E)
    counts = np.minimum(routed, capacity) if capacity else routed
    return {"ids": ids, "weights": w, "counts": counts, "offsets": segment_offsets(counts),
            "routed_counts": routed}


def layer_forward(inp: Dict[str, np.ndarray], *, k: int, E: int, bf16: bool, capacity: int = 0,
                  timers: Optional[Dict[str, float]] = None,
                  dispatch: str = "dtype") -> Dict[str, np.ndarray]:
    """The whole routed-expert layer forward on one device, every stage kept.

    ``inp`` holds x, then either logits (given router output) or gate_w, an
    optional bias, w1 / w3 / w2, wd / wu for latent layers and ws1 / ws3 / ws2
    for a shared expert (non-latent layers).  Given logits
    are routed on fp32(logits + bias); computed logits are exact here and
    rounded once to fp32 for the selection decision.  ``timers`` (optional)
    receives the wall-clock seconds of routing, permutation, expert FFN and
    combine (the stage timers of Three Parameter Counts, "What the utilization
    dashboard smooths away").  ``capacity`` C > 0 drops each expert's assignments
    beyond its first C (value-changing, see ``permutation``).  ``dispatch="mxfp8"``
    (bf16 layers) sends the dispatched rows as MXFP8 and runs the gate/up
    contraction on MXFP8 rows and weights (value-changing, see ``oracle.mxfp8``):
    each token row is quantised once (``x_q``, ``x_scale``), the permutation copies
    codes and scales, and W1 / W3 are quantised along their contraction axis.
    """
    clock = [time.perf_counter()]

    def lap(name):
        if timers is not None:
            now = time.perf_counter()
            timers[name] = timers.get(name, 0.0) + now - clock[0]
            clock[0] = now

    res: Dict[str, np.ndarray] = {}
    if "logits" in inp:
        scores = router_scores(inp["logits"], inp.get("bias"))
    else:
        lg = gate_logits(inp["x"], inp["gate_w"], inp.get("bias"))
        res["logits"] = lg
        scores = lg.astype(np.float32)
    res["scores"] = scores
    res.update(route(scores, k, E, capacity))
    lap("routing")
    rt, tr = permutation(res["ids"], E, capacity)
    res["row_token"], res["token_row"] = rt, tr
    if "wd" in inp:
        res["z"] = latent_down(inp["x"], inp["wd"], bf16)
        src = res["z"]
    else:
        src = decode(inp["x"])
    if dispatch == "mxfp8":
        from . import mxfp8
        assert bf16, "MXFP8 dispatch of bf16 layers"
        res["x_q"], res["x_scale"] = mxfp8.mx_quantize(src)
        res["x_perm_q"] = res["x_q"][rt]
        res["x_perm_scale"] = res["x_scale"][rt]
        lap("permutation")
        res["w1_q"], res["w1_scale"] = mxfp8.mx_quantize(decode(inp["w1"]))
        res["w3_q"], res["w3_scale"] = mxfp8.mx_quantize(decode(inp["w3"]))
        res["y_perm"], res["ffn_parts"] = mxfp8.grouped_expert_ffn_mx(
            res["x_perm_q"], res["x_perm_scale"], res["offsets"], res["w1_q"], res["w1_scale"], res["w3_q"],
            res["w3_scale"], inp["w2"], parts=True)
    else:
        assert dispatch == "dtype"
        res["x_perm"] = gather_rows(src, rt)
        lap("permutation")
        res["y_perm"] = grouped_expert_ffn(res["x_perm"], res["offsets"], inp["w1"], inp["w3"],
                                           inp["w2"], bf16)
    lap("expert_ffn")
    if "ws1" in inp:
        assert "wd" not in inp, "shared expert on non-latent layers only"
        res["y_shared"] = shared_expert_ffn(inp["x"], inp["ws1"], inp["ws3"], inp["ws2"], bf16)
    lap("shared_expert")
    res["out_combine"] = combine(res["y_perm"], tr, res["weights"], res.get("y_shared"))
    if "wu" in inp:
        res["out"] = latent_up(res["out_combine"], inp["wu"], bf16)
    else:
        res["out"] = res["out_combine"]
    lap("combine")
    return res


def token_outputs(inp: Dict[str, np.ndarray], tokens: np.ndarray, ids: np.ndarray,
                  weights: np.ndarray, expert_w: Dict[int, tuple], *, bf16: bool,
                  z: Optional[np.ndarray] = None) -> np.ndarray:
    """Layer output of selected tokens only: out[t] = sum_j w[t, j] * FFN_{ids[t, j]}(x_t)
    (+ the shared expert's FFN(x_t) when ``inp`` holds ws1 / ws3 / ws2).

    For full-size layers.  ``ids`` / ``weights`` are [len(tokens) x k] for the
    selected tokens, ``expert_w[e] = (w1e, w3e, w2e)`` for every expert they
    use, ``z`` the latent rows of the selected tokens (latent layers).  Each
    expert's FFN acts on rows independently, so it is evaluated once on all the
    selected rows routed to it.  Same rounding points as ``layer_forward``.
    """
    tokens = np.asarray(tokens)
    src = z if z is not None else decode(np.asarray(inp["x"])[tokens])
    n, k = ids.shape
    y = {}
    for e in sorted(set(int(v) for v in ids.ravel())):
        rows = [i for i in range(n) if e in ids[i]]
        w1e, w3e, w2e = expert_w[e]
        ye = expert_ffn_rows(src[rows], w1e, w3e, w2e, bf16)
        for r, i in enumerate(rows):
            y[(i, e)] = ye[r]
    out = np.zeros((n, src.shape[1]), dtype=np.float64)
    for j in range(k):
        for i in range(n):
            out[i] += weights[i, j] * y[(i, int(ids[i, j]))]
    if "ws1" in inp:
        out += shared_expert_ffn(np.asarray(inp["x"])[tokens], inp["ws1"], inp["ws3"], inp["ws2"], bf16)
    if "wu" in inp:
        out = latent_up(out, inp["wu"], bf16)
    return out


# --------------------------------------------------------------------------------------
# measurements the pages ask for
# --------------------------------------------------------------------------------------


def load_skew(counts: np.ndarray, T: int, k: int) -> float:
    """The largest per-expert load over the mean per-expert load (mean = T*k/E).

    "Three Parameter Counts...", "What the utilization dashboard smooths away".
    """
    E = len(counts)
    return float(np.max(counts)) / (T * k / E)


def p95_nearest_rank(values) -> float:
    """Nearest-rank 95th percentile: the ceil(0.95 n)-th smallest value."""
    v = sorted(float(x) for x in values)
    n = len(v)
    rank = int(np.ceil(0.95 * n))
    return v[max(rank, 1) - 1]
