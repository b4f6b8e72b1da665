"""Seeded synthetic MoE-layer workloads.

The five full-size layers follow the model shapes the pages quote (128
experts / top-8 like Qwen3-30B-A3B, 256 / top-8 like DeepSeek-R1, 896 /
top-16 like Kimi K3 at decode scale, and a latent-dispatch layer) plus a
tiny fp32 layer.  The small ``PARITY_CONFIGS`` are cut-down layers the CPU
oracle finishes in seconds while still spanning several GEMM tiles, ragged
tails, empty experts and the degenerate routings (k = 1, k = E, E = 1,
T = 1, every token on the same experts).

Nothing here computes any step of the layer: a config is a bag of sizes,
seeds and value distributions.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                 # tokens in the step
    H: int                 # model hidden width
    E: int                 # routed experts
    k: int                 # experts selected per token
    I: int                 # expert FFN intermediate width
    L: int = 0             # latent dispatch width (0 = dispatch at H)
    dtype: str = "bf16"    # "bf16" (fp32 accumulate, fp32 router) or "f32"
    seed: int = 0
    x_std: float = 1.0     # activations ~ N(0, x_std^2)
    w_std: float = 0.02    # expert / projection weights ~ N(0, w_std^2)
    gate: str = "computed"  # "computed": logits = X.Wg (+bias); "drawn": logits ~ N(0,1) given
    gate_std: Optional[float] = 0.02   # Wg ~ N(0, gate_std^2); None means 1/sqrt(H)
    zipf_s: Optional[float] = None     # per-expert bias -alpha*s*ln(rank) when set
    zipf_alpha: float = 0.0
    const_logits: bool = False         # every router logit equal (all-tie routing)
    shared_I: int = 0                  # shared expert intermediate width (0 = none)
    capacity: int = 0                  # rows kept per expert (0 = no limit, nothing dropped)
    dispatch: str = "dtype"            # "dtype" or "mxfp8" (E4M3 rows + E8M0 scales per 32)

    @property
    def D(self) -> int:
        """Width of the dispatched rows (latent width when L > 0)."""
        return self.L if self.L else self.H

    @property
    def R(self) -> int:
        """Routed rows: every token yields exactly k assignments."""
        return self.T * self.k

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def has_bias(self) -> bool:
        return self.zipf_s is not None

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


# Scale of the log-Zipf expert bias.  The literal prior -s*ln(rank) makes the
# p95 max/mean expert-load ratio about 24 on the DeepSeek-R1-shaped layer; the
# workload asks for about 4.  The value below was chosen by
# workloads/calibrate_zipf.py (which runs the oracle's router on the seeded
# layer) and is frozen here; it only shapes the workload.
ZIPF_ALPHA = 0.25

TINY_F32 = MoEConfig(
    name="tiny_f32", T=64, H=128, E=8, k=2, I=256, dtype="f32", seed=101,
    x_std=1.0, w_std=0.05, gate="drawn", gate_std=None)

QWEN3_30B_A3B_SHAPED = MoEConfig(
    name="qwen3_30b_a3b_shaped", T=4096, H=2048, E=128, k=8, I=768, seed=202,
    gate="computed", gate_std=0.02)

DEEPSEEK_R1_SHAPED = MoEConfig(
    name="deepseek_r1_shaped", T=8192, H=7168, E=256, k=8, I=2048, seed=303,
    gate="computed", gate_std=0.02, zipf_s=1.1, zipf_alpha=ZIPF_ALPHA)

K3_SHAPED_DECODE = MoEConfig(
    name="k3_shaped_decode", T=128, H=4096, E=896, k=16, I=1024, seed=404,
    gate="drawn", gate_std=None, zipf_s=1.2, zipf_alpha=ZIPF_ALPHA)

LATENT_MOE = MoEConfig(
    name="latent_moe", T=4096, H=7168, L=2048, E=256, k=8, I=4096, seed=505,
    gate="computed", gate_std=None)

# the K3-shaped decode layer at a small step (8 tokens): the latency-bound regime
K3_SHAPED_DECODE_T8 = K3_SHAPED_DECODE.with_(name="k3_shaped_decode_t8", T=8, seed=406)

# DeepSeek-R1-shaped layer with its shared expert (one, of the routed experts' width)
DEEPSEEK_R1_SHAPED_SHARED = DEEPSEEK_R1_SHAPED.with_(name="deepseek_r1_shaped_shared", shared_I=2048)

FULL_CONFIGS = {c.name: c for c in (TINY_F32, QWEN3_30B_A3B_SHAPED, DEEPSEEK_R1_SHAPED,
                                    K3_SHAPED_DECODE, LATENT_MOE, DEEPSEEK_R1_SHAPED_SHARED,
                                    K3_SHAPED_DECODE_T8)}

# Cut-down layers for element-by-element parity (oracle runs in seconds).
PARITY_CONFIGS = {c.name: c for c in (
    TINY_F32,
    # several m-tiles for hot experts, ragged tails, empty experts
    MoEConfig(name="small_bf16_zipf", T=300, H=256, E=16, k=4, I=192, seed=11,
              gate="computed", gate_std=0.0625, zipf_s=1.1, zipf_alpha=1.0),
    MoEConfig(name="small_bf16_uniform", T=517, H=384, E=32, k=8, I=256, seed=12,
              gate="computed", gate_std=0.05),
    # decode-like: most experts get 0-3 rows
    MoEConfig(name="small_bf16_decode", T=24, H=512, E=96, k=6, I=128, seed=13,
              gate="drawn", gate_std=None, zipf_s=1.2, zipf_alpha=ZIPF_ALPHA),
    MoEConfig(name="small_latent", T=200, H=320, L=128, E=16, k=4, I=256, seed=14,
              gate="computed", gate_std=None),
    # decode-like steps of 65-128 tokens (the one-launch router's second token-mask word)
    MoEConfig(name="decode_t100", T=100, H=512, E=96, k=6, I=128, seed=35, gate="drawn",
              zipf_s=1.2, zipf_alpha=ZIPF_ALPHA),
    MoEConfig(name="decode_t128", T=128, H=1024, E=200, k=8, I=256, seed=36, gate="drawn",
              zipf_s=1.2, zipf_alpha=ZIPF_ALPHA),
    # decode-scale steps whose ranking is too much work for one workgroup (many experts,
    # large k, like the 896-expert top-16 step at T = 128): the general routing kernels,
    # then the decode tiles and the fused down GEMM + combine; one with an expert capacity
    MoEConfig(name="decode_many_experts", T=120, H=256, E=700, k=12, I=128, seed=38, gate="drawn",
              zipf_s=1.2, zipf_alpha=ZIPF_ALPHA),
    MoEConfig(name="decode_many_experts_cap", T=60, H=256, E=1024, k=16, I=128, seed=39,
              gate="drawn", zipf_s=1.2, zipf_alpha=ZIPF_ALPHA, capacity=3),
    # a decode-like latent layer: the fused down GEMM + combine writes the latent rows
    MoEConfig(name="decode_latent", T=24, H=320, L=128, E=96, k=4, I=256, seed=37, gate="computed",
              gate_std=None),
    # degenerate routings
    MoEConfig(name="one_expert", T=130, H=128, E=1, k=1, I=128, seed=15, gate="drawn"),
    MoEConfig(name="k_equals_e", T=70, H=128, E=8, k=8, I=64, seed=16, gate="drawn"),
    MoEConfig(name="single_token", T=1, H=192, E=12, k=3, I=64, seed=17, gate="drawn"),
    MoEConfig(name="all_ties", T=150, H=128, E=16, k=2, I=128, seed=18, gate="drawn",
              const_logits=True),
    MoEConfig(name="many_empty", T=5, H=128, E=64, k=2, I=64, seed=19, gate="drawn"),
    MoEConfig(name="small_f32_computed", T=97, H=96, E=6, k=3, I=80, dtype="f32",
              seed=20, w_std=0.05, gate="computed", gate_std=0.1),
    # more than 2048 tokens: 163 ranking blocks of 16 tokens
    MoEConfig(name="many_tokens", T=2600, H=128, E=40, k=3, I=128, seed=21, gate="drawn",
              zipf_s=1.1, zipf_alpha=0.5),
    # wide experts: 16 n-tiles of 128 in the gate/up GEMM and K = 2048 in the down GEMM
    # with at least 192 rows per expert on average (so the persistent 128 x 256 down
    # tiles), skewed counts spanning several m-tiles
    MoEConfig(name="wide_experts", T=400, H=256, E=4, k=2, I=2048, seed=22, gate="drawn",
              zipf_s=1.1, zipf_alpha=1.0),
    # long-K down GEMM (K = I = 2048) with fewer than 192 rows per expert on average:
    # the persistent 256 x 128 down tiles on the second m-tile table
    MoEConfig(name="long_k_down", T=400, H=256, E=16, k=4, I=2048, seed=29, gate="drawn",
              zipf_s=1.1, zipf_alpha=0.5),
    # more persistent-GEMM tiles than one LDS tile table holds (3520): each workgroup
    # decodes only its XCD's chunk and no tile is taken across XCDs.  Gate/up: 64
    # n-tiles x ~70 m-tiles; the down GEMM of this layer has ~70 tiles (whole table).
    # Top-8 of 16 with near-uniform weights and a wide intermediate, like the pages'
    # models, so the layer tolerance applies as it does to them.
    MoEConfig(name="wsp_chunk_gate_up", T=1024, H=256, E=16, k=8, I=8192, seed=30, gate="drawn"),
    # the same for the down GEMM on 128 x 256 tiles: ~260 m-tiles x 16 n-tiles
    MoEConfig(name="wsp_chunk_down", T=4096, H=4096, E=16, k=8, I=768, seed=34, gate="drawn"),
    # a shared expert next to the routed ones: 128-row tiles (T >= 48), 16-row
    # tiles (T < 48) and fp32
    MoEConfig(name="shared_expert", T=300, H=256, E=16, k=4, I=192, seed=23, gate="computed",
              gate_std=0.0625, zipf_s=1.1, zipf_alpha=1.0, shared_I=320),
    MoEConfig(name="shared_expert_decode", T=24, H=512, E=96, k=6, I=128, seed=24, gate="drawn",
              gate_std=None, zipf_s=1.2, zipf_alpha=ZIPF_ALPHA, shared_I=256),
    MoEConfig(name="shared_expert_f32", T=97, H=96, E=6, k=3, I=80, dtype="f32", seed=25,
              w_std=0.05, gate="computed", gate_std=0.1, shared_I=64),
    # expert capacity (value-changing dropping) on skewed routing: 128-row tiles,
    # the decode-scale path and fp32
    MoEConfig(name="capacity_prefill", T=300, H=256, E=16, k=4, I=192, seed=26, gate="drawn",
              zipf_s=1.1, zipf_alpha=1.0, capacity=60),
    MoEConfig(name="capacity_decode", T=24, H=512, E=96, k=6, I=128, seed=27, gate="drawn",
              zipf_s=1.2, zipf_alpha=1.0, capacity=2),
    MoEConfig(name="capacity_f32", T=97, H=96, E=6, k=3, I=80, dtype="f32", seed=28, w_std=0.05,
              gate="drawn", zipf_s=1.1, zipf_alpha=1.0, capacity=40),
)}
