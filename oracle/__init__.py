"""Reference oracle for streaming multi-head attention (fp64, CPU).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the GPU library
(``head_attention_streaming_amd``) and imports nothing from it.

What it computes, each item citing the page "flashdreams.accelerated" (developer guide),
section "Multi Head Attention Definition", unless stated otherwise:

* ``rmsnorm``     -- the RMSNorm equation, gamma * z / sqrt(mean(z^2) + eps), head scope (m = d)
                     or inner scope (m = H*d).
* ``rope``        -- the pair-rotation equation with angle theta_{p,r}; split-half pairs
                     (r, r + d/2) or interleaved pairs (2r, 2r + 1).
* ``qk_norm_rope``-- normalisation first, then RoPE (the order the same section uses).
* ``attention``   -- the scaled dot-product equation A_h = softmax(Q_h K_h^T * scale) V_h.
                     Grouped heads: query head h reads key/value head h // (Hq // Hkv).
                     Causal: key j visible to query i iff j <= i + Lk - Lq. Local window
                     (left, right) around i + Lk - Lq, the ``window_size`` of the page
                     "optimizing-attention-flash" (section "Step 3: Enable advanced features").
* ``round_to``    -- round-to-nearest-even into bfloat16 / IEEE binary16, from the formats'
                     definitions, applied once to an fp64 value.
* ``decode``      -- exact widening of bfloat16, binary16 and OCP FP8 E4M3 (float8_e4m3fn, the
                     unscaled FP8 the quantized-SDPA option of the same page casts Q/K/V to).
* ``cache``       -- the rolling sink + window K/V cache of the page's "Generic Multi Head
                     Attention Interface" section, simulated chunk by chunk (see cache.py).

Heavy loops run in ``liboracle.so`` (oracle.c, plain fp64 C, no fused multiply-add).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import cache  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

SPLIT = 1
INTERLEAVED = 2


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, fp64, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        src = os.path.join(_HERE, "oracle.c")
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                               src, "-lm", "-o", tmp])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        D = ctypes.c_double
        lib.oracle_decode_bf16.argtypes = [P, P, I64]
        lib.oracle_decode_f16.argtypes = [P, P, I64]
        lib.oracle_decode_e4m3.argtypes = [P, P, I64]
        lib.oracle_rmsnorm.argtypes = [P, P, P, I64, I, D]
        lib.oracle_rope.argtypes = [P, P, P, I, I, I, I, I]
        lib.oracle_attention.argtypes = [P, P, P, P, P, I64, I, I, I, I, I, I, D, I64, I64, I]
        lib.oracle_attention.restype = I
        lib.oracle_attention_spread.argtypes = [P, P, P, P, P, I64, I, I, I, I, I, I, D, I64, I64, I, P, P, P, D, P,
                                                P]
        lib.oracle_attention_spread.restype = I
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 64))


# ------------------------------------------------------------------ 16-bit formats

def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Widen float bit patterns exactly to float64: 16-bit patterns (uint16/int16) for "bf16" and
    "f16", 8-bit patterns (uint8/int8) for "e4m3" (OCP FP8 E4M3, the float8_e4m3fn format)."""
    if dtype == "e4m3":
        b = np.ascontiguousarray(bits).view(np.uint8)
        out = np.empty(b.shape, dtype=np.float64)
        _load().oracle_decode_e4m3(_ptr(b), _ptr(out), b.size)
        return out
    b = np.ascontiguousarray(bits).view(np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    fn = {"bf16": _load().oracle_decode_bf16, "f16": _load().oracle_decode_f16}[dtype]
    fn(_ptr(b), _ptr(out), b.size)
    return out


_FORMATS = {
    # significant bits (including the implicit one), smallest normal exponent, largest finite value
    "bf16": (8, -126, (2.0 - 2.0 ** -7) * 2.0 ** 127),
    "f16": (11, -14, 65504.0),
    "e4m3": (4, -6, 448.0),   # OCP FP8 E4M3 (float8_e4m3fn): no infinity, overflow is NaN
}


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the nearest ``dtype`` value ("bf16", "f16", "e4m3"), ties to even, in one step.

    A value with binary exponent e (x = f * 2^e, 0.5 <= |f| < 1) has quantum
    2^(e - p) for a p-bit significand, floored at the subnormal quantum 2^(emin - p + 1).
    x / quantum is an exact power-of-two scaling, so np.rint (ties to even) rounds once.
    Values beyond the largest finite value round to +-inf (IEEE overflow rule for RNE).
    """
    p, emin, fmax = _FORMATS[dtype]
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q_exp = np.maximum(e - p, emin - p + 1)
    q = np.ldexp(np.ones_like(x), q_exp)
    r = np.rint(x / q) * q
    if dtype == "e4m3":
        # E4M3 has no infinity: a result beyond 448 after rounding (|x| > 464; 464 itself is a tie
        # that rounds to the even 448) is NaN, as is a NaN input
        r = np.where(np.abs(r) > fmax, np.nan, r)
        return np.where(x == 0, x, r)
    # overflow: anything at or beyond the midpoint between fmax and the next (virtual) step
    top = fmax + 0.5 * np.ldexp(1.0, int(np.frexp(fmax)[1]) - p)
    r = np.where(np.abs(x) >= top, np.copysign(np.inf, x), r)
    r = np.where(x == 0, x, r)  # keep the sign of zero
    return r


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of ``dtype`` values at the magnitude of x (the quantum used by round_to): in the
    binade [2^(e-1), 2^e) of x the p significant bits are 2^(e-p) apart; at and below the smallest
    normal 2^emin (zero included) the subnormals are 2^(emin-p+1) apart."""
    p, emin, _ = _FORMATS[dtype]
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.where(x == 0, emin, e)   # frexp(0) gives exponent 0, which is not zero's binade
    return np.ldexp(1.0, np.maximum(e - p, emin - p + 1))


# ------------------------------------------------------------------ RMSNorm / RoPE

def rmsnorm(z: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis of z with weight gamma (len = last axis)."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    g = np.ascontiguousarray(gamma, dtype=np.float64)
    m = z.shape[-1]
    assert g.shape == (m,)
    out = np.empty_like(z)
    _load().oracle_rmsnorm(_ptr(z), _ptr(g), _ptr(out), z.size // m, m, float(eps))
    return out


def rope(z: np.ndarray, angles: np.ndarray, style: int) -> np.ndarray:
    """Rotate feature pairs of z [B, L, H, d] by angles [L, d/2] (float64 of the given table)."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    B, L, H, d = z.shape
    a = np.ascontiguousarray(angles, dtype=np.float64)
    assert a.shape == (L, d // 2) and d % 2 == 0 and style in (SPLIT, INTERLEAVED)
    out = np.empty_like(z)
    _load().oracle_rope(_ptr(z), _ptr(a), _ptr(out), B, L, H, d, style)
    return out


def qk_norm_rope(z: np.ndarray, gamma: np.ndarray | None, eps: float, angles: np.ndarray | None,
                 style: int) -> np.ndarray:
    """Head-scope RMSNorm (skipped when gamma is None), then RoPE (skipped when angles is None)."""
    out = np.asarray(z, dtype=np.float64)
    if gamma is not None:
        out = rmsnorm(out, gamma, eps)
    if angles is not None and style != 0:
        out = rope(out, angles, style)
    return out


# ------------------------------------------------------------------ attention

def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool = False,
              rows: np.ndarray | None = None, nthreads: int | None = None,
              window: tuple[int, int] | None = None) -> np.ndarray:
    """softmax(Q K^T * scale) V in fp64.

    q: [B, Lq, Hq, d]; k, v: [B, Lk, Hkv, d] (float64 or anything convertible).
    rows: optional flat indices into [B, Lq, Hq]; then the result is [len(rows), d],
    otherwise [B, Lq, Hq, d].
    window: (left, right) local-attention band around each query's key position i + Lk - Lq
    (a negative bound is unbounded; the skill page's ``window_size=(left, right)``). causal=True
    is the band (-1, 0); giving both is an error.
    """
    if window is not None and causal:
        raise ValueError("give either causal or window")
    win_left, win_right = window if window is not None else ((-1, 0) if causal else (-1, -1))
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, Lq, Hq, d = q.shape
    Bk, Lk, Hkv, dk = k.shape
    assert v.shape == k.shape and Bk == B and dk == d and Hq % Hkv == 0
    if rows is None:
        nrows = B * Lq * Hq
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        assert rows_arr.ndim == 1 and (rows_arr.size == 0 or
                                       (rows_arr.min() >= 0 and rows_arr.max() < B * Lq * Hq))
        nrows = rows_arr.size
    out = np.empty((nrows, d), dtype=np.float64)
    rc = _load().oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                  None if rows_arr is None else _ptr(rows_arr), nrows,
                                  B, Hq, Hkv, Lq, Lk, d, float(scale), int(win_left), int(win_right),
                                  nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_attention failed")
    return out if rows is not None else out.reshape(B, Lq, Hq, d)


def attention_spread(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool = False,
                     rows: np.ndarray | None = None, nthreads: int | None = None,
                     window: tuple[int, int] | None = None, tail_binades: float = np.inf):
    """``attention`` plus what a tolerance for rounded softmax weights needs, from the exact
    weights w_j = softmax(s)_j of each row: A = sum_j w_j |v_j - o| and R = sqrt(sum_j w_j^2
    (v_j - o)^2) per output element (same shape as the output), the row's score range
    max_j s_j - min_j s_j in base-2 exponent units (shape: the output without its last axis), and
    for the keys whose score lies more than tail_binades (base-2 units) below the row maximum,
    their part of A (A_tail, the output's shape) and their total weight (W_tail, a row's shape).
    Returns (o, A, R, span, A_tail, W_tail)."""
    if window is not None and causal:
        raise ValueError("give either causal or window")
    win_left, win_right = window if window is not None else ((-1, 0) if causal else (-1, -1))
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, Lq, Hq, d = q.shape
    assert v.shape == k.shape and k.shape[0] == B and k.shape[3] == d and Hq % k.shape[2] == 0
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = B * Lq * Hq if rows is None else rows_arr.size
    out = np.empty((nrows, d))
    a = np.empty((nrows, d))
    r = np.empty((nrows, d))
    span = np.empty((nrows,))
    ta = np.empty((nrows, d))
    tw = np.empty((nrows,))
    rc = _load().oracle_attention_spread(_ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                         None if rows_arr is None else _ptr(rows_arr), nrows, B, Hq, k.shape[2],
                                         Lq, k.shape[1], d, float(scale), int(win_left), int(win_right),
                                         nthreads or default_threads(), _ptr(a), _ptr(r), _ptr(span),
                                         float(tail_binades), _ptr(ta), _ptr(tw))
    if rc != 0:
        raise RuntimeError("oracle_attention_spread failed")
    if rows is None:
        sh = (B, Lq, Hq)
        return (out.reshape(*sh, d), a.reshape(*sh, d), r.reshape(*sh, d), span.reshape(sh), ta.reshape(*sh, d),
                tw.reshape(sh))
    return out, a, r, span, ta, tw
