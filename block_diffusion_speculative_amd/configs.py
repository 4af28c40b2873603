"""Named workloads for one DFlash draft-and-verify step.

Shapes only: no arithmetic of the method lives here.  The drafter structure
(fused target features injected into every layer's K/V, a B-slot block that
holds the last accepted token followed by mask tokens, a shared lm_head) is
the one described on the pages:

* "DFlash, Diffusion LLMs, dLLM, MTP and Speculative Decoding: A Deep
  Research Report", section "Key points" (KV injection into every draft
  layer, block_size 16, 5-8 draft layers);
* "Term: DFlash speculative decoding", section "DFlash: architecture and
  workflow" (anchor, one drafting pass, argmax verification, longest
  accepted prefix plus a fallback token).

The sizes themselves (Qwen3-8B-shaped drafter, the tiny fp32 case, the
batch-32 ragged case, long context and the larger shape with a block-size
sweep) are the workloads this library is measured and checked on.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Dims:
    """Drafter dimensions.  ``dtype`` is the storage type ("bf16" or "f32")."""

    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_layers: int
    intermediate: int
    vocab: int
    n_feat_layers: int
    block_size: int = 16
    rope_theta: float = 1e4
    rms_eps: float = 1e-6
    dtype: str = "bf16"

    @property
    def mask_id(self) -> int:
        # The mask token is the last id of the vocabulary; real tokens are
        # drawn from [0, vocab - 1) so they never collide with it.
        return self.vocab - 1

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def feat_dim(self) -> int:
        return self.n_feat_layers * self.hidden

    def with_block(self, block_size: int) -> "Dims":
        return replace(self, block_size=block_size)

    def param_count(self) -> dict:
        H, I, V, d = self.hidden, self.intermediate, self.vocab, self.head_dim
        per_layer = (self.qkv_rows * H + self.n_q_heads * d * H + 3 * I * H)
        return {
            "fc": H * self.feat_dim,
            "layers": self.n_layers * per_layer,
            "lm_head": V * H,
            "embed": V * H,
        }


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: dimensions, batch, context lengths and the
    per-step injection and acceptance distributions."""

    name: str
    dims: Dims
    batch: int
    ctx: Tuple[int, int]                 # inclusive range; lo == hi means fixed
    new_rows: Optional[Tuple[int, int]]  # seeded U{lo..hi} per sequence, or None
    mean_accept: float                   # target E[L] of the planted acceptance
    block_sizes: Tuple[int, ...] = (16,)
    geom_p: Optional[float] = None       # explicit geometric parameter, if given
    description: str = ""

    @property
    def max_ctx(self) -> int:
        return self.ctx[1]


QWEN3_8B_DRAFT = Dims(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
                      n_layers=5, intermediate=12288, vocab=151936,
                      n_feat_layers=5, dtype="bf16")

LARGER_DRAFT = Dims(hidden=5120, n_q_heads=40, n_kv_heads=8, head_dim=128,
                    n_layers=8, intermediate=17408, vocab=151936,
                    n_feat_layers=5, dtype="bf16")

# The target of the Qwen3-8B-shaped drafter: the drafter's layer type at
# Qwen3-8B's sizes (36 layers); its five feature layers feed the fc.
QWEN3_8B_TARGET = Dims(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
                       n_layers=36, intermediate=12288, vocab=151936,
                       n_feat_layers=5, dtype="bf16")

TINY_DRAFT = Dims(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                  n_layers=1, intermediate=512, vocab=1024, n_feat_layers=2,
                  dtype="f32")

WORKLOADS = {
    "tiny-f32": Workload(
        "tiny-f32", TINY_DRAFT, batch=1, ctx=(128, 128), new_rows=None,
        mean_accept=0.0, geom_p=0.12,
        description="tiny fp32 step: hidden 256, 4/2 heads, 1 layer, vocab 1024, ctx 128"),
    "qwen3-8b-b1": Workload(
        "qwen3-8b-b1", QWEN3_8B_DRAFT, batch=1, ctx=(2048, 2048), new_rows=None,
        mean_accept=7.8,
        description="Qwen3-8B-shaped drafter, bf16, batch 1, ctx 2048, B=16"),
    "qwen3-8b-b32": Workload(
        "qwen3-8b-b32", QWEN3_8B_DRAFT, batch=32, ctx=(512, 4096), new_rows=(1, 17),
        mean_accept=7.8,
        description="Qwen3-8B-shaped drafter, bf16, 32 sequences, ragged ctx 512..4096"),
    "qwen3-8b-long": Workload(
        "qwen3-8b-long", QWEN3_8B_DRAFT, batch=4, ctx=(16384, 16384), new_rows=None,
        mean_accept=7.8,
        description="Qwen3-8B-shaped drafter, bf16, batch 4, ctx 16384"),
    "larger-b8": Workload(
        "larger-b8", LARGER_DRAFT, batch=8, ctx=(8192, 8192), new_rows=None,
        mean_accept=7.8, block_sizes=(4, 8, 16),
        description="hidden 5120, 40/8 heads, 8 layers, batch 8, ctx 8192, B in {4,8,16}"),
}


def get(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError as exc:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from exc


def kv_capacity(max_ctx: int, max_new: int = 17, block: int = 16) -> int:
    """Cache capacity in positions: context plus one step of injection,
    rounded up to 32 (the key-step size of the bf16 cache layout)."""
    need = max_ctx + max_new + block
    return ((need + 31) // 32) * 32
