"""The five decode workloads, by shape.

The workload shapes follow the pages' demo (a small random-init Qwen3 serving
60 prompts with up to 256 generated tokens: hysenlabs review of MinivLLM,
section on what main.py does) and the model families they name (Qwen3 and
Llama 3.2: miniVLLM docs, "Explore by topic"; tiny-vllm note, "Chi tiết").
The pages give no kernel shapes; every number here is a synthetic stand-in.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class Config:
    name: str
    dtype: str                # "fp32" | "fp16" | "bf16": storage type of q, k, v and the caches
    batch: int                # B: sequences in the decode batch (one new token each)
    num_heads: int            # Hq
    num_kv_heads: int         # Hkv
    head_dim: int             # D
    block_size: int           # bs: tokens per physical KV block
    lengths: str              # "fixed" | "uniform" | "lognormal" | "list"
    len_list: tuple = ()      # for "list"
    len_lo: int = 0           # inclusive bounds (uniform) or clip bounds (lognormal)
    len_hi: int = 0
    len_median: float = 0.0   # lognormal median
    len_sigma: float = 0.0    # lognormal sigma of the natural log
    pool_blocks: Optional[int] = None   # fixed pool size; None = ceil(1.25 * blocks needed)
    q_mult: float = 1.0       # q ~ N(0,1) * q_mult before rounding to dtype
    scale: Optional[float] = None       # None = 1/sqrt(D)
    prefix_group: int = 0     # >0: groups of this many consecutive sequences share prefix blocks
    prefix_tokens: int = 0    # tokens of the shared prefix (a multiple of block_size)
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)

    @property
    def max_len(self) -> int:
        if self.lengths == "list":
            return max(self.len_list)
        return self.len_hi

    @property
    def max_blocks_per_seq(self) -> int:
        return -(-self.max_len // self.block_size)

    @property
    def elem_bytes(self) -> int:
        return {"fp32": 4, "fp16": 2, "bf16": 2}[self.dtype]


CONFIGS = {
    "tiny_fp32": Config(
        name="tiny_fp32", dtype="fp32", batch=4, num_heads=4, num_kv_heads=2, head_dim=64,
        block_size=16, lengths="list", len_list=(1, 17, 33, 64), pool_blocks=32,
        scale=1.0 / 8.0, seed=1),
    "qwen3_0p6b_bf16": Config(
        name="qwen3_0p6b_bf16", dtype="bf16", batch=60, num_heads=16, num_kv_heads=8,
        head_dim=128, block_size=256, lengths="uniform", len_lo=32, len_hi=288,
        scale=1.0 / math.sqrt(128), seed=2),
    "llama32_1b_fp16": Config(
        name="llama32_1b_fp16", dtype="fp16", batch=64, num_heads=32, num_kv_heads=8,
        head_dim=64, block_size=16, lengths="uniform", len_lo=512, len_hi=4096, seed=3),
    "long_ctx_bf16": Config(
        name="long_ctx_bf16", dtype="bf16", batch=16, num_heads=32, num_kv_heads=8,
        head_dim=128, block_size=16, lengths="fixed", len_lo=32768, len_hi=32768,
        q_mult=2.0, seed=4),
    "skewed_prefix_bf16": Config(
        name="skewed_prefix_bf16", dtype="bf16", batch=256, num_heads=16, num_kv_heads=8,
        head_dim=128, block_size=16, lengths="lognormal", len_lo=1, len_hi=16384,
        len_median=1024.0, len_sigma=1.0, prefix_group=8, prefix_tokens=512, seed=5),
}

# Order in which the workloads are listed (smallest first).
CONFIG_ORDER = ["tiny_fp32", "qwen3_0p6b_bf16", "llama32_1b_fp16", "long_ctx_bf16",
                "skewed_prefix_bf16"]

# A further prefix-caching shape, for the shared-prefix option: 32 prompts of 4096 tokens, each
# sampled 8 times (groups of 8 sequences share the prompt's blocks), 1 to 512 tokens generated
# per sample. The distinct prompt K/V (0.54 GB) is larger than the 256 MB last-level cache.
CONFIGS["shared_prompt_bf16"] = Config(
    name="shared_prompt_bf16", dtype="bf16", batch=256, num_heads=16, num_kv_heads=8, head_dim=128,
    block_size=16, lengths="uniform", len_lo=4097, len_hi=4608, prefix_group=8, prefix_tokens=4096, seed=6)
EXTRA_CONFIGS = ["shared_prompt_bf16"]


def get_config(name: str) -> Config:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {CONFIG_ORDER + EXTRA_CONFIGS}") from None
