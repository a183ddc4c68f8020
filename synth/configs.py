"""Workload shapes used by tests and the benchmark.

Each workload is one attention layer of the shape named in its docstring field, with the
statistics of the hidden states h that feed it.  Nothing here computes any part of the
codec; it only names sizes.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    d_head: int
    decay: float                 # eigenvalues of Cov(h) proportional to i^-decay
    outlier_frac: float          # fraction of rows that are multivariate Student-t(3)
    calib_rows: int              # rows used to estimate the activation Gram matrix
    n_seg: int                   # 1 = one latent over all KV heads; n_kv_heads = one per head
    seg_rank: int                # latent rank per segment (before dropping 0-bit groups)
    group_size: int
    budget_bits: float           # bits per original element, fp16 group scales included
    fixed_width: Optional[int]   # if set, every group gets this width (no water-filling)
    energy: Optional[float]      # energy threshold whose rank is reported next to seg_rank
    dtype: str                   # "f32" or "bf16": x, W_down, q, W_up
    decode_batch: int
    decode_ctx: int
    encode_tokens: int
    stream_steps: int = 0        # 1-token appends per sequence after the prefill
    note: str = ""

    @property
    def n_orig(self) -> int:     # original elements per token per tensor per segment
        return self.n_kv_heads * self.d_head // self.n_seg

    @property
    def seg_cols(self) -> int:
        return self.n_kv_heads * self.d_head // self.n_seg


# Tiny single head, fp32.
TINY = Workload(
    name="tiny_f32_d512_h1_r16_g4_b2", d_model=512, n_q_heads=1, n_kv_heads=1, d_head=64,
    decay=1.5, outlier_frac=0.0, calib_rows=4096, n_seg=1, seg_rank=16, group_size=4,
    budget_bits=2.0, fixed_width=None, energy=None, dtype="f32",
    decode_batch=1, decode_ctx=256, encode_tokens=256,
    note="tiny single head, fp32")

# Llama-3.1-8B-shaped layer, 4 bits per element.
LLAMA8B_4BIT = Workload(
    name="llama8b_d4096_q32_kv8_r512_g16_b4", d_model=4096, n_q_heads=32, n_kv_heads=8,
    d_head=128, decay=1.2, outlier_frac=0.01, calib_rows=16384, n_seg=1, seg_rank=512,
    group_size=16, budget_bits=4.0, fixed_width=None, energy=None, dtype="bf16",
    decode_batch=16, decode_ctx=32768, encode_tokens=32768,
    note="Llama-3.1-8B-shaped layer, 4x vs bf16")

# Qwen2.5-7B-shaped layer, 2 bits per element.
QWEN7B_2BIT = Workload(
    name="qwen7b_d3584_q28_kv4_r384_g16_b2", d_model=3584, n_q_heads=28, n_kv_heads=4,
    d_head=128, decay=1.2, outlier_frac=0.01, calib_rows=16384, n_seg=1, seg_rank=384,
    group_size=16, budget_bits=2.0, fixed_width=None, energy=None, dtype="bf16",
    decode_batch=32, decode_ctx=16384, encode_tokens=16384,
    note="Qwen2.5-7B-shaped layer, 8x vs bf16")

# Long context at 4/3 bits per element.
LLAMA8B_LONG = Workload(
    name="llama8b_long_d4096_r512_g16_b1.33", d_model=4096, n_q_heads=32, n_kv_heads=8,
    d_head=128, decay=1.2, outlier_frac=0.01, calib_rows=16384, n_seg=1, seg_rank=512,
    group_size=16, budget_bits=4.0 / 3.0, fixed_width=None, energy=None, dtype="bf16",
    decode_batch=4, decode_ctx=131072, encode_tokens=131072, stream_steps=256,
    note="Llama-3.1-8B shapes, 12x vs bf16, 128k context, streaming appends")

# Aggressive per-head low rank.
PERHEAD_R6 = Workload(
    name="perhead_d5120_q40_kv8_r6_g2_w4", d_model=5120, n_q_heads=40, n_kv_heads=8,
    d_head=128, decay=3.0, outlier_frac=0.0, calib_rows=16384, n_seg=8, seg_rank=6,
    group_size=2, budget_bits=0.0, fixed_width=4, energy=0.95, dtype="bf16",
    decode_batch=64, decode_ctx=32768, encode_tokens=65536,
    note="per-head rank 6, 4-bit latent groups, about 28x vs bf16")

ALL = (TINY, LLAMA8B_4BIT, QWEN7B_2BIT, LLAMA8B_LONG, PERHEAD_R6)
BY_NAME = {w.name: w for w in ALL}
