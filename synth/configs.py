"""Workload definitions for the DFlash2 draft -> select -> verify step.

These are the synthetic stand-ins for the pages' workloads.  The pages
(NeMo AutoModel "Train a DFlash Drafter for Speculative Decoding",
§Key Config Fields; NeMo SpeechLM "DFlash speculative decoding with vLLM",
§DFlash2 inference) name the configuration fields -- target_layer_ids,
block_size, conv_kernel_size, selector_rank, selector_top_k, mask_token_id,
draft head shape -- but print no model, so every shape below is a seeded
synthetic workload.  This module holds sizes and distributions only: none of
the method's arithmetic lives here.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

WEIGHT_DTYPES = ("fp32", "bf16", "fp8")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int                   # seed component; fixed per workload
    batch: int
    block_size: int              # anchor + num_speculative_tokens
    hidden: int
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    num_taps: int                # len(target_layer_ids)
    tap_width: int
    ctx: Tuple[int, int]         # context length after append: fixed (a, a) or uniform [a, b]
    top_k: int
    rank: int
    weight_dtype: str            # "fp32" | "bf16" | "fp8"
    agree: Tuple[str, float]     # ("const", p) or ("decay", p0): p_k = p0 * exp(-(k-1)/gamma)
    decay_gamma: float = 7.0
    conv_kernel_size: int = 2
    conv_group_size: int = 0     # 0: static per-channel taps; > 0: dynamic taps per channel group
    cold: bool = False           # cache empty before the step: n_new = ctx (whole context appended)
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    input_embedding_scale: float = 1.0
    output_multiplier: float = 1.0
    final_logit_softcapping: float = 0.0
    sliding_window: int = 0
    spare_context: int = 0           # extra cache rows for multi-step decoding
    weight_std: float = 0.02
    gain_jitter: float = 0.0     # norm gains = 1 + N(0, gain_jitter^2); 0 -> exactly 1
    selector_active: bool = False
    selector_sigma_w: Optional[float] = None  # overrides the active-variant sigma

    # ---- derived sizes -------------------------------------------------
    @property
    def mask_token_id(self) -> int:
        return self.vocab - 1

    @property
    def act_dtype(self) -> str:
        return "fp32" if self.weight_dtype == "fp32" else "bf16"

    @property
    def param_dtype(self) -> str:
        """dtype of embedding, conv taps and norm gains (never fp8)."""
        return "fp32" if self.weight_dtype == "fp32" else "bf16"

    @property
    def qkv_rows(self) -> int:
        return (self.num_q_heads + 2 * self.num_kv_heads) * self.head_dim

    @property
    def max_context(self) -> int:
        # rows [ctx, ctx + block_size) hold the block's transient keys/values;
        # spare_context more rows let a decode loop grow the context; rounded
        # up to a multiple of 32 rows
        return (self.ctx[1] + self.spare_context + self.block_size + 31) // 32 * 32

    def abi_config(self) -> dict:
        """Field values of the C ABI's dflash2_config for this workload."""
        return dict(
            hidden=self.hidden, num_layers=self.num_layers, num_q_heads=self.num_q_heads,
            num_kv_heads=self.num_kv_heads, head_dim=self.head_dim, ffn=self.ffn,
            vocab=self.vocab, num_taps=self.num_taps, tap_width=self.tap_width,
            block_size=self.block_size, conv_kernel_size=self.conv_kernel_size,
            conv_group_size=self.conv_group_size,
            selector_top_k=self.top_k, selector_rank=self.rank, max_batch=self.batch,
            max_context=self.max_context, sliding_window=self.sliding_window,
            mask_token_id=self.mask_token_id, weight_dtype=self.weight_dtype,
            rms_eps=self.rms_eps, rope_theta=self.rope_theta,
            input_embedding_scale=self.input_embedding_scale,
            output_multiplier=self.output_multiplier,
            final_logit_softcapping=self.final_logit_softcapping)

    def agreement(self, pos: int) -> float:
        """Probability that the verifier agrees with the draft at block position pos (1-based)."""
        kind, p = self.agree
        if kind == "const":
            return p
        return p * math.exp(-(pos - 1) / self.decay_gamma)

    def selector_table_std(self) -> float:
        """Std of the per-token selector factor tables.

        The tables stand for embedding rows (N(0, w^2), width H) times a rank-r
        projection with entries N(0, sigma_w^2); their entries then have std
        w * sqrt(H) * sigma_w.  The literal workloads use sigma_w = w; the
        selector-active variants pick sigma_w so the pair term's spread matches
        the unary logit spread.
        """
        w = self.weight_std
        if self.selector_sigma_w is not None:
            sw = self.selector_sigma_w
        elif self.selector_active:
            sw = math.sqrt(w * math.sqrt(self.hidden) / math.sqrt(self.rank)) / (w * math.sqrt(self.hidden))
        else:
            sw = w
        return w * math.sqrt(self.hidden) * sw

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, in order.  Indices are seed components.
TINY_FP32 = Workload(
    name="tiny_fp32", index=0, batch=1, block_size=8, hidden=64, num_layers=1,
    num_q_heads=4, num_kv_heads=4, head_dim=16, ffn=256, vocab=512, num_taps=2,
    tap_width=64, ctx=(32, 32), top_k=4, rank=8, weight_dtype="fp32",
    agree=("const", 0.7), cold=True)

DENSE27B_BF16 = Workload(
    name="dense27b_bf16", index=1, batch=1, block_size=8, hidden=5120, num_layers=5,
    num_q_heads=40, num_kv_heads=8, head_dim=128, ffn=17408, vocab=151936,
    num_taps=5, tap_width=5120, ctx=(4096, 4096), top_k=16, rank=64,
    weight_dtype="bf16", agree=("const", 0.8))

BATCHED_BF16 = Workload(
    name="batched_bf16", index=2, batch=64, block_size=7, hidden=4096, num_layers=1,
    num_q_heads=32, num_kv_heads=8, head_dim=128, ffn=14336, vocab=131072,
    num_taps=3, tap_width=4096, ctx=(512, 2048), top_k=16, rank=32,
    weight_dtype="bf16", agree=("const", 0.75))

LONGBLOCK_BF16 = Workload(
    name="longblock_bf16", index=3, batch=16, block_size=16, hidden=4096, num_layers=2,
    num_q_heads=32, num_kv_heads=8, head_dim=128, ffn=14336, vocab=151936,
    num_taps=4, tap_width=4096, ctx=(8192, 8192), top_k=16, rank=64,
    weight_dtype="bf16", agree=("decay", 0.9), decay_gamma=7.0)

FP8_B256 = Workload(
    name="fp8_b256", index=4, batch=256, block_size=8, hidden=5120, num_layers=1,
    num_q_heads=40, num_kv_heads=8, head_dim=128, ffn=17408, vocab=151936,
    num_taps=5, tap_width=5120, ctx=(2048, 2048), top_k=16, rank=64,
    weight_dtype="fp8", agree=("const", 0.8))

WORKLOADS = {w.name: w for w in (TINY_FP32, DENSE27B_BF16, BATCHED_BF16, LONGBLOCK_BF16, FP8_B256)}

# Small parity workloads: several tiles of every kernel plus ragged tails
# (vocab, hidden, ffn and context not multiples of the tile sizes), GQA, more
# than one layer, gains and selector both active.
SMALL_BF16 = Workload(
    name="small_bf16", index=10, batch=3, block_size=8, hidden=320, num_layers=2,
    num_q_heads=10, num_kv_heads=2, head_dim=64, ffn=736, vocab=3001, num_taps=3,
    tap_width=192, ctx=(40, 300), top_k=16, rank=16, weight_dtype="bf16",
    agree=("const", 0.8), gain_jitter=0.1, selector_active=True)

SMALL_FP8 = SMALL_BF16.replace(name="small_fp8", index=11, weight_dtype="fp8", batch=5,
                               block_size=7, top_k=8, vocab=2500)

SMALL_FP32 = SMALL_BF16.replace(name="small_fp32", index=12, weight_dtype="fp32", batch=2,
                                block_size=5, cold=True, ctx=(70, 70), vocab=1000)

# Many activation rows (the compute-bound, LDS-tiled GEMM path) at small
# widths: ragged row tiles, a ragged vocabulary tile, and (fp8) two row tiles.
MEDIUM_BF16 = SMALL_BF16.replace(name="medium_bf16", index=13, batch=24, ffn=768, vocab=3001)
MEDIUM_FP8 = SMALL_BF16.replace(name="medium_fp8", index=14, weight_dtype="fp8", batch=40,
                                block_size=7, ffn=768, top_k=8, vocab=2500, ctx=(40, 200))

TEST_WORKLOADS = {w.name: w for w in (SMALL_BF16, SMALL_FP8, SMALL_FP32, MEDIUM_BF16, MEDIUM_FP8)}


def get(name: str) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name]
    if name in TEST_WORKLOADS:
        return TEST_WORKLOADS[name]
    raise KeyError(name)
