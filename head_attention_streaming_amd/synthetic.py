"""Seeded synthetic inputs shared by the GPU tests, the benchmark and the oracle checks.

This module only draws numbers and builds the caller-side RoPE angle table; it holds none of
the attention, normalisation or cache arithmetic, and it imports neither the GPU library nor
the oracle.

Recipe (the pages' workloads use trained video models whose weights and data are not
available, so every tensor here is a stand-in of the same shape and dtype):
  * a fresh ``torch.Generator`` seeded per tensor set; fp32 N(0, 1) draws in the order
    q, k, v (then gamma_q, gamma_k), each cast round-to-nearest-even to the I/O dtype;
  * RMSNorm weights: bf16(1 + 0.1 * N(0, 1)), held as fp32 (the learned weights are unknown);
  * RoPE angles: theta_{p,r} = p * base^(-2r/d) computed in fp64 from absolute stream positions
    p and stored as fp32 [L, d/2] -- the expanded per-position angle table that the page
    "flashdreams.accelerated" (section "Multi Head Attention Definition") says the attention
    module receives from its caller.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16, "e4m3": torch.float8_e4m3fn}


def normal(shape, dtype: str, gen: torch.Generator, scale: float = 1.0) -> torch.Tensor:
    """fp32 N(0, 1) * scale, cast to the dtype (CPU tensor; e4m3 = unscaled float8_e4m3fn)."""
    x = torch.randn(tuple(shape), generator=gen, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x.to(DTYPES[dtype])


def attention_inputs(B: int, Lq: int, Lk: int, Hq: int, Hkv: int, d: int, dtype: str, seed: int,
                     q_scale: float = 1.0):
    """q [B, Lq, Hq, d], k and v [B, Lk, Hkv, d], drawn in that order from one generator."""
    g = torch.Generator().manual_seed(seed)
    q = normal((B, Lq, Hq, d), dtype, g, q_scale)
    k = normal((B, Lk, Hkv, d), dtype, g)
    v = normal((B, Lk, Hkv, d), dtype, g)
    return q, k, v


def norm_weight(d: int, gen: torch.Generator) -> torch.Tensor:
    """Synthetic RMSNorm weight: bf16(1 + 0.1 N(0,1)) values held in fp32 [d]."""
    w = 1.0 + 0.1 * torch.randn((d,), generator=gen, dtype=torch.float32)
    return w.to(torch.bfloat16).to(torch.float32)


def rope_angles(positions, d: int, base: float = 10000.0) -> torch.Tensor:
    """fp32 [len(positions), d/2] table of p * base^(-2r/d), computed in fp64."""
    p = np.asarray(positions, dtype=np.float64)[:, None]
    r = np.arange(d // 2, dtype=np.float64)[None, :]
    ang = p * np.power(float(base), -2.0 * r / d)
    return torch.from_numpy(ang.astype(np.float32))


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a CPU tensor: uint16 for bf16/f16, uint8 for float8_e4m3fn."""
    if t.dtype == torch.float8_e4m3fn:
        return t.contiguous().view(torch.uint8).numpy()
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclass(frozen=True)
class Workload:
    """One benchmark configuration (shapes and dtypes of the pages' workloads)."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lk: int
    d: int
    dtype: str
    causal: bool
    scale: float
    seed: int
    prologue: str = "none"   # "none" | "qk_norm_rope" (streaming self-attention) | "q_norm" (cross)
    chunk: int = 0           # streaming: chunk length (= Lq)
    window: int = 0          # streaming: cache capacity in tokens (sink 0)
    attn_window: tuple | None = None  # local attention band (left, right) around i + Lk - Lq
    rope_scope: str = "before"        # streaming: RoPE before or after the K/V cache update
    cache_dtype: str = "bf16"         # streaming: element type of the K/V cache and attention inputs
    v_cache_dtype: str | None = None  # V kept in another type (f16: the type P*V uses), same results
    fp8_probs: bool = False           # e4m3: softmax probabilities rounded to E4M3 for an FP8 P*V

    @property
    def flops(self) -> float:
        """Attention flop count 4 * B * H * Lq * Lk * d (the metric's formula)."""
        return 4.0 * self.B * self.Hq * self.Lq * self.Lk * self.d


WORKLOADS = {
    # non-causal MHA, [1, 257, 8, 128] bf16, scale 1/sqrt(128)
    "mha_257_bf16": Workload("mha_257_bf16", 1, 8, 8, 257, 257, 128, "bf16", False, 128 ** -0.5, 1001),
    # the same queries over 20 keys: a workgroup's fixed cost (one masked key tile, no loop)
    "mha_257x20_bf16": Workload("mha_257x20_bf16", 1, 8, 8, 257, 20, 128, "bf16", False, 128 ** -0.5, 1001),
    # causal MHA, [2, 2048, 8, 64] fp16, scale 1/8
    "causal_2048_f16": Workload("causal_2048_f16", 2, 8, 8, 2048, 2048, 64, "f16", True, 0.125, 1002),
    # streaming self-attention: 40 heads, d 128, chunk 1785, rolling cache of 4 chunks (7140 keys)
    "stream_self_1785x4": Workload("stream_self_1785x4", 1, 40, 40, 1785, 7140, 128, "bf16", False,
                                   128 ** -0.5, 1300, "qk_norm_rope", 1785, 7140),
    # the same streaming step with after-cache RoPE: unrotated cache, visible keys rotated per step
    "stream_after_1785x4": Workload("stream_after_1785x4", 1, 40, 40, 1785, 7140, 128, "bf16", False,
                                    128 ** -0.5, 1300, "qk_norm_rope", 1785, 7140, rope_scope="after"),
    # the same streaming step with V cached in f16 (bit-identical outputs, no V conversion in attention)
    "stream_vf16_1785x4": Workload("stream_vf16_1785x4", 1, 40, 40, 1785, 7140, 128, "bf16", False,
                                   128 ** -0.5, 1300, "qk_norm_rope", 1785, 7140, v_cache_dtype="f16"),
    # the same streaming step with an FP8 E4M3 K/V cache (Q, K, V rounded to E4M3, bf16 out)
    "stream_fp8_1785x4": Workload("stream_fp8_1785x4", 1, 40, 40, 1785, 7140, 128, "bf16", False,
                                  128 ** -0.5, 1300, "qk_norm_rope", 1785, 7140, cache_dtype="e4m3"),
    # cross-attention over a static 512-token context, B = 2 (guidance pair), Q RMSNorm only
    "cross_1785x512": Workload("cross_1785x512", 2, 40, 40, 1785, 512, 128, "bf16", False,
                               128 ** -0.5, 1004, "q_norm"),
    # the same cross-attention with after-cache RoPE: the static context cache keeps unrotated keys,
    # each query chunk rotates all 512 of them (cache-relative rows) and its queries (rows after them)
    "cross_after_1785x512": Workload("cross_after_1785x512", 2, 40, 40, 1785, 512, 128, "bf16", False,
                                     128 ** -0.5, 1004, "q_norm", rope_scope="after"),
    # the cross-attention context cache with V kept in f16 (bit-identical outputs)
    "cross_vf16_1785x512": Workload("cross_vf16_1785x512", 2, 40, 40, 1785, 512, 128, "bf16", False,
                                    128 ** -0.5, 1004, "q_norm", v_cache_dtype="f16"),
    # long non-causal MHA, [1, 20480, 56, 128] bf16
    "mha_20480_bf16": Workload("mha_20480_bf16", 1, 56, 56, 20480, 20480, 128, "bf16", False,
                               128 ** -0.5, 1005),
    # 32 query heads over 32, 8 or 1 K/V heads: what re-reading a shared K/V head costs
    "mha_8192_h32_bf16": Workload("mha_8192_h32_bf16", 1, 32, 32, 8192, 8192, 128, "bf16", False, 128 ** -0.5, 1007),
    "gqa_8192_h32kv8_bf16": Workload("gqa_8192_h32kv8_bf16", 1, 32, 8, 8192, 8192, 128, "bf16", False,
                                     128 ** -0.5, 1007),
    "mqa_8192_h32kv1_bf16": Workload("mqa_8192_h32kv1_bf16", 1, 32, 1, 8192, 8192, 128, "bf16", False,
                                     128 ** -0.5, 1007),
    # the long problem with unscaled FP8 E4M3 q, k, v (bf16 out)
    "mha_20480_fp8": Workload("mha_20480_fp8", 1, 56, 56, 20480, 20480, 128, "e4m3", False,
                              128 ** -0.5, 1005),
    # the same two with the probabilities also rounded to E4M3 for an FP8 P*V product (opt-in)
    "mha_20480_fp8p": Workload("mha_20480_fp8p", 1, 56, 56, 20480, 20480, 128, "e4m3", False,
                               128 ** -0.5, 1005, fp8_probs=True),
    "stream_fp8p_1785x4": Workload("stream_fp8p_1785x4", 1, 40, 40, 1785, 7140, 128, "bf16", False,
                                   128 ** -0.5, 1300, "qk_norm_rope", 1785, 7140, cache_dtype="e4m3",
                                   fp8_probs=True),
    # sliding-window (local) attention, [4, 4096, 32, 64] fp16, 256 keys back + the query's own
    "window_4096_w256_f16": Workload("window_4096_w256_f16", 4, 32, 32, 4096, 4096, 64, "f16", False,
                                     0.125, 1006, attn_window=(256, 0)),
}
