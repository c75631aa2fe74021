"""Workload shapes for block/page-sparse long-context decode attention.

Each workload names the shape of one decode step: batch, query and KV heads
(GQA ratio = num_q_heads / num_kv_heads), head dim, KV dtype, context length
L (the current token included), page size P, attention-sink length S, window
W, token budget and the page-summary mode.  The sizes follow the pages'
workloads: a Qwen3-8B layer (course module 14, section 14.1 KV arithmetic:
36 layers, 8 KV heads, head dim 128), a Llama-3-70B layer (self-indexing
attention page, "How much memory the KV cache eats": 80 layers, 8 KV heads,
head dim 128), the hybrid sink-256 + window + Quest scheme at 256K with
per-layer (window, budget) and refresh every 32 steps (hybrid sparse attention
page), and semantic blocks of about 2048 tokens with budget L/16 at 512K
(semantic-blocks page).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple

QUEST, MEAN, CENTROID, COMPRESSED = 0, 1, 2, 3
MODE_NAMES = {"quest": QUEST, "mean": MEAN, "centroid": CENTROID, "compressed": COMPRESSED}
F32, BF16 = 0, 1
DTYPE_NAMES = {"f32": F32, "bf16": BF16}


@dataclass(frozen=True)
class Layer:
    """Per-layer (window, token budget) of a full-attention layer."""

    window: int
    budget: int


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str  # "f32" | "bf16"
    context: int  # L: tokens in the cache, current token(s) included
    page_size: int
    sink: int
    window: int
    budget: int  # token budget of the selected pages; k = budget // page_size
    mode: str = "quest"
    q_rows: int = 1  # query rows per step (the last q_rows positions)
    seed: int = 0
    layers: Tuple[Layer, ...] = field(default_factory=tuple)  # multi-layer schedule
    steps: int = 0  # decode steps (multi-layer schedule)
    refresh: int = 0  # re-select every `refresh` steps (multi-layer schedule)
    block: int = 0  # tokens appended between two evictions (eviction workload)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def k_pages(self) -> int:
        return self.budget // self.page_size

    @property
    def max_pages(self) -> int:
        extra = self.steps if self.steps else 0
        return -(-(self.context + extra) // self.page_size)

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


# tiny fp32 case with one planted needle page
TINY = Workload(
    name="tiny-fp32-2k", batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64, dtype="f32",
    context=2048, page_size=16, sink=16, window=64, budget=128, seed=0,
)

# one Qwen3-8B-shaped layer, 32k context, budget L/16
QWEN3_8B = Workload(
    name="qwen3-8b-layer-32k", batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
    context=32768, page_size=16, sink=256, window=1024, budget=32768 // 16, seed=1,
)

# one Llama-3-70B-shaped layer, 128k context, GQA-8
LLAMA3_70B = Workload(
    name="llama3-70b-layer-128k", batch=4, num_q_heads=64, num_kv_heads=8, head_dim=128, dtype="bf16",
    context=131072, page_size=64, sink=256, window=4096, budget=131072 // 16, seed=2,
)

# hybrid model, 3 full-attention layers at 256k, 128 decode steps
HYBRID_256K = Workload(
    name="hybrid-3layer-256k", batch=4, num_q_heads=32, num_kv_heads=4, head_dim=128, dtype="bf16",
    context=262144, page_size=32, sink=256, window=2048, budget=8192, seed=3,
    layers=(Layer(2048, 8192), Layer(4096, 4096), Layer(1024, 16384)), steps=128, refresh=32,
)

# semantic blocks at 512K, 64-query chunk per step
SEMANTIC_512K = Workload(
    name="semantic-512k", batch=2, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="bf16",
    context=524288 + 64, page_size=2048, sink=0, window=64, budget=524288 // 16, mode="centroid",
    q_rows=64, seed=4,
)

# KeyDiff eviction: a Llama-3.1-8B-shaped layer whose cache holds an 8K-token
# budget plus one 2048-token block, evicted back to the budget (sink of 4)
KEYDIFF_8K = Workload(
    name="keydiff-llama3.1-8b-8k", batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
    context=8192 + 2048, page_size=16, sink=4, window=1, budget=8192, seed=5, block=2048,
)

# chunked sparse prefill of a 64K-token prompt over one semantic block index
# of the whole prompt: 128-row chunks whose window is the chunk itself,
# budget L/16 of each chunk's length
SEMANTIC_PREFILL_64K = Workload(
    name="semantic-prefill-64k", batch=2, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="bf16",
    context=65536 + 128, page_size=2048, sink=0, window=128, budget=65536 // 16, mode="centroid",
    q_rows=128, seed=6,
)

ALL = (TINY, QWEN3_8B, LLAMA3_70B, HYBRID_256K, SEMANTIC_512K, KEYDIFF_8K, SEMANTIC_PREFILL_64K)
BY_NAME = {w.name: w for w in ALL}
