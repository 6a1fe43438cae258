"""The five synthetic workloads of the compressed-KV decode path.

Shapes follow Llama-3-8B attention (32 query heads, 8 KV heads, head_dim 128,
32 layers), the model that StiefAttention evaluates on (StiefAttention
technical summary, "Resultados Experimentais"), with ranks that are per layer
(StiefAttention, "Mecanismo Central" item 4) or per head (STAR-KV,
"Metodologia" section 1, hard thresholds at inference).

Every workload is synthetic and seeded; no model weights or datasets are
used. ``Config.scaled`` gives the same recipe at a smaller size for parity
cases that the float64 oracle finishes in seconds.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    cid: int                 # seed key of the workload (every random stream is keyed on it)
    name: str
    B: int                   # batch
    Hq: int                  # query heads
    Hkv: int                 # key/value heads
    d: int                   # head_dim
    n_layers: int = 1
    T: Optional[int] = None  # uniform cache length (None: ragged, see T_range)
    T_range: Optional[Tuple[int, int]] = None  # ragged lengths, inclusive bounds
    rank_mode: str = "uniform"   # uniform | per_head | per_layer_profile
    r_k: int = 0                 # uniform ranks
    r_v: int = 0
    rank_choices: Tuple[int, ...] = ()   # per_head draw set
    profile_moves: int = 0               # per_layer_profile: number of +16/-16 moves
    profile_step: int = 16
    profile_bounds: Tuple[int, int] = (16, 128)
    profile_start: int = 64
    in_dtype: str = "bf16"       # dtype of K, V rows handed to compression
    latent_dtype: str = "bf16"   # dtype of the latent cache
    n_outliers: int = 0          # key channels per (layer, KV head) scaled by outlier_scale
    outlier_scale: float = 8.0
    decode_steps: int = 0        # >0: append-then-attend steps after prefill of T tokens
    description: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def capacity(self) -> int:
        """Rows allocated per (batch, KV head) in the latent cache."""
        if self.T is not None:
            return self.T + self.decode_steps
        return self.T_range[1] + self.decode_steps

    def scaled(self, **changes) -> "Config":
        """Same recipe (seeds, distributions) at other sizes."""
        return dataclasses.replace(self, **changes)


CONFIGS = (
    Config(
        cid=0, name="single_head_f32", B=1, Hq=1, Hkv=1, d=128, T=2048,
        r_k=32, r_v=32, in_dtype="f32", latent_dtype="f32",
        description="single head, batch 1, T=2048, r=32/32, all fp32",
    ),
    Config(
        cid=1, name="llama3_8b_layer_32k", B=8, Hq=32, Hkv=8, d=128, T=32768,
        r_k=64, r_v=64, n_outliers=4,
        description="Llama-3-8B layer decode, B=8, T=32768, r=64/64 per KV head, bf16 latents",
    ),
    Config(
        cid=2, name="per_head_ranks_ragged", B=16, Hq=32, Hkv=8, d=128,
        T_range=(4096, 16384), rank_mode="per_head",
        rank_choices=(16, 32, 48, 64, 80, 96), n_outliers=4,
        description="per-head r_k, r_v from {16..96}, ragged T in [4096,16384], B=16, bf16",
    ),
    Config(
        cid=3, name="long_context_128k", B=2, Hq=32, Hkv=8, d=128, T=131072,
        r_k=48, r_v=80, n_outliers=4, decode_steps=64,
        description="prefill-compress 131072 tokens then 64 append+decode steps, B=2, r=48/80",
    ),
    Config(
        cid=4, name="llama3_8b_32_layers", B=32, Hq=32, Hkv=8, d=128, T=8192,
        n_layers=32, rank_mode="per_layer_profile", profile_moves=256, n_outliers=4,
        description="32 layers, B=32, T=8192, per-layer ranks with 50% latent budget",
    ),
)


SINGLE_HEAD_F32, LLAMA3_LAYER_32K, PER_HEAD_RAGGED, LONG_CONTEXT_128K, LLAMA3_32_LAYERS = CONFIGS

# The workloads by name.
WORKLOADS = {c.name: c for c in CONFIGS}
