"""Seeded input generator shared by the CPU oracle's tests and the GPU path.

Every tensor is drawn from its own numpy PCG64 stream keyed by
``SeedSequence([cfg.seed, tag, index])`` so that any single expert (or any
step's activations) can be regenerated on its own, independent of torch or
GPU versions.  Normals are drawn in fp32 and scaled; bf16 layers store the
round-to-nearest-even bf16 bit patterns as ``uint16`` (the GPU side views
them as ``torch.bfloat16``, the oracle decodes them itself).

This module draws inputs only: it computes no step of the MoE layer.

Storage orientation (the library's layout, output-major like a linear
layer's weight): gate_w [E x H], w1 / w3 [E x I x D], w2 [E x D x I],
wd [L x H], wu [H x L].
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Iterable, Optional

import numpy as np

from .configs import MoEConfig

TAG_X, TAG_GATE_W, TAG_BIAS_RANK, TAG_W1, TAG_W3, TAG_W2, TAG_WD, TAG_WU, TAG_LOGITS, TAG_Y = \
    1, 2, 3, 4, 5, 6, 7, 8, 9, 10
TAG_WS1, TAG_WS3, TAG_WS2 = 11, 12, 13


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def rng(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, index])))


def normal_f32(seed: int, tag: int, index: int, shape, std: float) -> np.ndarray:
    a = rng(seed, tag, index).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns uint16 bits.

    Input values are finite normals, so NaN handling is not needed here.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def draw(cfg: MoEConfig, tag: int, index: int, shape, std: float) -> np.ndarray:
    """A tensor in the layer's storage dtype: fp32 array or bf16 bits (uint16)."""
    a = normal_f32(cfg.seed, tag, index, shape, std)
    return a if cfg.dtype == "f32" else f32_to_bf16_bits(a)


def activations(cfg: MoEConfig, step: int = 0) -> np.ndarray:
    """X [T x H] in the storage dtype; each step reseeds the activations."""
    return draw(cfg, TAG_X, step, (cfg.T, cfg.H), cfg.x_std)


def drawn_logits(cfg: MoEConfig, step: int = 0) -> np.ndarray:
    """Router logits ~ N(0,1) fp32 [T x E] for layers whose router output is drawn."""
    if cfg.const_logits:
        return np.full((cfg.T, cfg.E), 0.5, dtype=np.float32)
    return normal_f32(cfg.seed, TAG_LOGITS, step, (cfg.T, cfg.E), 1.0)


def gate_weight(cfg: MoEConfig) -> np.ndarray:
    """Router weight, fp32 [E x H] (row e holds expert e's scoring vector)."""
    std = cfg.gate_std if cfg.gate_std is not None else 1.0 / np.sqrt(cfg.H)
    return normal_f32(cfg.seed, TAG_GATE_W, 0, (cfg.E, cfg.H), float(std))


def zipf_bias(cfg: MoEConfig) -> Optional[np.ndarray]:
    """Per-expert fp32 bias -alpha*s*ln(rank_e), rank a seeded permutation of 1..E."""
    if cfg.zipf_s is None:
        return None
    rank = rng(cfg.seed, TAG_BIAS_RANK, 0).permutation(cfg.E).astype(np.float64) + 1.0
    return (-cfg.zipf_alpha * cfg.zipf_s * np.log(rank)).astype(np.float32)


def _expert_mats(cfg: MoEConfig, e: int):
    D, I = cfg.D, cfg.I
    return (draw(cfg, TAG_W1, e, (I, D), cfg.w_std),
            draw(cfg, TAG_W3, e, (I, D), cfg.w_std),
            draw(cfg, TAG_W2, e, (D, I), cfg.w_std))


def expert_weights(cfg: MoEConfig, experts: Optional[Iterable[int]] = None,
                   threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """w1, w3 [n x I x D] and w2 [n x D x I] for the listed experts (all by default).

    Experts are independent streams, so they are drawn in parallel.
    """
    ex = list(range(cfg.E)) if experts is None else list(experts)
    dt = np.float32 if cfg.dtype == "f32" else np.uint16
    D, I = cfg.D, cfg.I
    w1 = np.empty((len(ex), I, D), dtype=dt)
    w3 = np.empty((len(ex), I, D), dtype=dt)
    w2 = np.empty((len(ex), D, I), dtype=dt)

    def fill(i_e):
        i, e = i_e
        a, b, c = _expert_mats(cfg, e)
        w1[i], w3[i], w2[i] = a, b, c

    with ThreadPoolExecutor(threads or _threads()) as pool:
        list(pool.map(fill, enumerate(ex)))
    return {"w1": w1, "w3": w3, "w2": w2, "experts": np.asarray(ex, dtype=np.int64)}


def shared_weights(cfg: MoEConfig) -> Dict[str, np.ndarray]:
    """Shared expert ws1, ws3 [Is x H] and ws2 [H x Is] (layers with shared_I > 0)."""
    assert cfg.shared_I > 0
    Is, H = cfg.shared_I, cfg.H
    return {"ws1": draw(cfg, TAG_WS1, 0, (Is, H), cfg.w_std),
            "ws3": draw(cfg, TAG_WS3, 0, (Is, H), cfg.w_std),
            "ws2": draw(cfg, TAG_WS2, 0, (H, Is), cfg.w_std)}


def latent_weights(cfg: MoEConfig) -> Dict[str, np.ndarray]:
    """Down projection wd [L x H] and up projection wu [H x L] (latent layers only)."""
    assert cfg.L > 0
    return {"wd": draw(cfg, TAG_WD, 0, (cfg.L, cfg.H), cfg.w_std),
            "wu": draw(cfg, TAG_WU, 0, (cfg.H, cfg.L), cfg.w_std)}


def layer_inputs(cfg: MoEConfig, step: int = 0, with_experts: bool = True) -> Dict[str, np.ndarray]:
    """Everything one forward of the layer consumes."""
    d: Dict[str, np.ndarray] = {"x": activations(cfg, step)}
    if cfg.gate == "drawn":
        d["logits"] = drawn_logits(cfg, step)
    else:
        d["gate_w"] = gate_weight(cfg)
    b = zipf_bias(cfg)
    if b is not None:
        d["bias"] = b
    if cfg.L:
        d.update(latent_weights(cfg))
    if with_experts:
        d.update({k: v for k, v in expert_weights(cfg).items() if k != "experts"})
        if cfg.shared_I:
            d.update(shared_weights(cfg))
    return d


def stage_rows(cfg: MoEConfig, rows: int, width: int, tag: int = TAG_Y, index: int = 0,
               std: float = 1.0) -> np.ndarray:
    """Generic seeded [rows x width] activation block (inputs of a single stage)."""
    return draw(cfg, tag, index, (rows, width), std)
