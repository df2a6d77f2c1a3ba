"""Shared helpers for the GPU parity tests: move seeded inputs to the device, run the oracle on
the same bytes, and apply the acceptance bounds."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from head_attention_streaming_amd import synthetic

# Attention output vs the fp64 oracle rounded once to the I/O dtype (bf16 or f16 I/O, fp32
# accumulation): elementwise max-abs and mean-abs bounds.
ATTN_MAX_ABS = 8e-3
ATTN_MEAN_ABS = 1e-4


def widen(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 values of a CPU or GPU bf16/f16/float8_e4m3fn tensor, decoded by the oracle."""
    dt = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float8_e4m3fn: "e4m3"}[t.dtype]
    return oracle.decode(synthetic.bits(t.detach().cpu()), dt)


def dtype_name(t: torch.Tensor) -> str:
    return {torch.bfloat16: "bf16", torch.float16: "f16", torch.float8_e4m3fn: "e4m3"}[t.dtype]


def attention_errors(gpu_out: torch.Tensor, ref64: np.ndarray) -> dict:
    g = widen(gpu_out).reshape(ref64.shape)
    r = oracle.round_to(ref64, dtype_name(gpu_out))
    err = np.abs(g - r)
    raw = np.abs(g - ref64)
    return {"max_abs": float(err.max()) if err.size else 0.0,
            "mean_abs": float(err.mean()) if err.size else 0.0,
            "max_abs_vs_fp64": float(raw.max()) if raw.size else 0.0,
            "exact_frac": float((g == r).mean()) if err.size else 1.0}


def assert_attention_close(gpu_out: torch.Tensor, ref64: np.ndarray, what: str = "",
                           ulp_floor: bool = False) -> dict:
    """Max-abs and mean-abs bounds against RNE(oracle).

    ulp_floor: for adversarial inputs whose outputs reach |o| >= 2, one bf16 ulp (2^-6 there)
    exceeds the 8e-3 max-abs bound, so any fp32-accumulating kernel whose value lands on the
    other side of a rounding tie would fail; with ulp_floor the per-element bound is
    max(8e-3, ulp(ref)). The benchmark configurations never need it.
    """
    e = attention_errors(gpu_out, ref64)
    g = widen(gpu_out).reshape(ref64.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    r = oracle.round_to(ref64, dtype_name(gpu_out))
    err = np.abs(g - r)
    bound = np.full(ref64.shape, ATTN_MAX_ABS)
    if ulp_floor:
        bound = np.maximum(bound, oracle.ulp(ref64, dtype_name(gpu_out)))
    if err.size and (err > bound).any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: max abs {e['max_abs']:.3g} > bound; worst at {i}: gpu {g[i]!r} "
                             f"ref {ref64[i]!r} ({e})")
    assert e["mean_abs"] <= ATTN_MEAN_ABS, f"{what}: mean abs {e['mean_abs']:.3g} > {ATTN_MEAN_ABS} ({e})"
    return e


def assert_within_one_ulp(gpu_out: torch.Tensor, ref64: np.ndarray, what: str = "", min_exact: float = 0.99):
    """Prologue bound: every element within one ulp of the 16-bit format (at the reference's
    magnitude) of the fp64 value, plus 2^-20 of its head row's largest magnitude -- the slack an
    fp32 evaluation needs where the rotation cancels (c*a - s*b much smaller than a, b) -- and at
    least ``min_exact`` of the elements equal to the fp64 value rounded to nearest even."""
    dt = dtype_name(gpu_out)
    g = widen(gpu_out).reshape(ref64.shape)
    u = oracle.ulp(ref64, dt)
    slack = 2.0 ** -20 * np.abs(ref64).max(axis=-1, keepdims=True)
    err = np.abs(g - ref64)
    bad = err > u + slack
    if bad.any():
        i = np.unravel_index(np.argmax(err - u - slack), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond one ulp; worst at {i}: gpu {g[i]!r} "
                             f"ref {ref64[i]!r} ulp {u[i]!r}")
    exact = float((g == oracle.round_to(ref64, dt)).mean())
    assert exact >= min_exact, f"{what}: only {exact:.4f} of elements equal RNE(fp64)"
    return exact


def sample_rows(B: int, Lq: int, Hq: int, n: int, seed: int) -> np.ndarray:
    """n distinct flat row indices into [B, Lq, Hq], always including the first and last query
    rows of every (batch, head) pair."""
    rng = np.random.default_rng(seed)
    total = B * Lq * Hq
    fixed = []
    for b in range(B):
        for h in range(Hq):
            fixed += [(b * Lq + 0) * Hq + h, (b * Lq + Lq - 1) * Hq + h]
    extra = rng.choice(total, size=min(total, max(0, n - len(fixed))), replace=False)
    return np.unique(np.concatenate([np.array(fixed, dtype=np.int64), extra.astype(np.int64)]))


# FP8 probabilities in P*V: E4M3 keeps 3 fraction bits, so a normal probability carries a relative
# rounding error of at most U_E4M3 = 2^-4, with a standard deviation of at most SIGMA_E4M3 =
# 2^-4 / sqrt(3) (uniform over +- half a spacing at the smallest mantissa).
U_E4M3 = 2.0 ** -4
SIGMA_E4M3 = 2.0 ** -4 / 3.0 ** 0.5
E4M3_NORMAL_BINADES = 14.0   # p = 2^(x - m + 8) stays >= 2^-6 (normal) while x >= m - 14


def assert_fp8p_close(gpu_out: torch.Tensor, ref64: np.ndarray, spread_a: np.ndarray, spread_r: np.ndarray,
                      tail_a: np.ndarray, tail_w: np.ndarray, what: str = "") -> dict:
    """Acceptance of attention with E4M3-rounded probabilities against the exact fp64 result o.
    Keys within 14 binades of the row maximum round with relative error <= U; keys further below
    (the tail: subnormal or flushed in E4M3) with relative error <= 1. With A, R the spreads of V
    under the exact weights and A_tail, W_tail the tail's part of A and its weight (from
    oracle.attention_spread with tail_binades=14): per element
    |g - o| <= (U (A - A_tail) + A_tail) / (1 - U - W_tail) + ulp(o), and the mean of |g - o| <=
    1.1 * mean((SIGMA R + A_tail) / (1 - U - W_tail) + ulp(o)/2)."""
    assert (tail_w < 0.05).all(), f"{what}: tail weight {tail_w.max():.3g} leaves no useful bound"
    g = widen(gpu_out).reshape(ref64.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref64)
    u = oracle.ulp(ref64, "bf16")
    den = (1.0 - U_E4M3 - tail_w)[..., None]
    bound = (U_E4M3 * (spread_a - tail_a) + tail_a) / den + u
    if (err > bound).any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: element beyond the rounding bound at {i}: gpu {g[i]!r} ref {ref64[i]!r} "
                             f"bound {bound[i]!r}")
    mean_bound = 1.1 * float(np.mean((SIGMA_E4M3 * spread_r + tail_a) / den + u / 2))
    mean_err = float(err.mean())
    assert mean_err <= mean_bound, f"{what}: mean abs {mean_err:.3g} > {mean_bound:.3g}"
    return {"max_abs": float(err.max()), "mean_abs": mean_err, "mean_bound": mean_bound,
            "max_over_bound": float((err / bound).max()), "tail_rows": int((tail_w > 0).sum())}
