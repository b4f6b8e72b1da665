"""Seeded synthetic inputs for the MoE layer (shared by the oracle's tests and the GPU path)."""
from .configs import (MoEConfig, FULL_CONFIGS, PARITY_CONFIGS, TINY_F32, QWEN3_30B_A3B_SHAPED,
                      DEEPSEEK_R1_SHAPED, K3_SHAPED_DECODE, LATENT_MOE, ZIPF_ALPHA)
from . import generator

__all__ = ["MoEConfig", "FULL_CONFIGS", "PARITY_CONFIGS", "TINY_F32", "QWEN3_30B_A3B_SHAPED",
           "DEEPSEEK_R1_SHAPED", "K3_SHAPED_DECODE", "LATENT_MOE", "ZIPF_ALPHA", "generator"]
