"""Python binding of libstreamattn.so: the C entry points under the same names.

Argument marshalling only -- tensors supply device pointers and shapes, the current PyTorch
HIP stream supplies the stream, and a non-zero status raises ``StreamAttnError`` with the
library's message. Every computation runs in the library's HIP kernels; there is no
fallback path, and a missing library raises at first use.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

SA_DTYPE_BF16, SA_DTYPE_F16, SA_DTYPE_FP8_E4M3, SA_DTYPE_BF16_F16V, SA_DTYPE_FP8_E4M3_P8 = 0, 1, 2, 3, 4
SA_ERR_SHAPE_CODE, SA_ERR_UNSUPPORTED_CODE = -2, -3
SA_NORM_NONE, SA_NORM_HEAD, SA_NORM_INNER = 0, 1, 2
SA_ROPE_NONE, SA_ROPE_SPLIT, SA_ROPE_INTERLEAVED, SA_ROPE_AFTER_CACHE = 0, 1, 2, 4

EXPORTS = ("qk_norm_rope", "qk_norm_rope_ex", "qk_norm_rope_v", "kv_cache_slot", "kv_cache_positions", "kv_cache_append",
           "kv_cache_append_ex", "kv_cache_rope", "attn_forward", "attn_forward_f16", "attn_forward_kvstride",
           "attn_forward_window", "attn_forward_workspace_bytes", "attn_forward_ws", "attn_forward_ws_static",
           "attn_forward_qnorm", "sa_last_error")

_lib = None


class StreamAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} returned {status}: {msg}")
        self.status = status


def library_path() -> str:
    return _build.LIB


def lib():
    """Load libstreamattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m head_attention_streaming_amd.build`")
        L = ctypes.CDLL(path)
        P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        L.qk_norm_rope.argtypes = [P, P, I64, P, P, I64, P, P, P, I, I, I, I, I, F, I, I, P]
        L.kv_cache_slot.argtypes = [I64, I, I, I, ctypes.POINTER(I64), ctypes.POINTER(I)]
        L.kv_cache_append.argtypes = [P, P, P, P, I, I, I, I, I, I, I64, P]
        L.kv_cache_append_ex.argtypes = [P, P, P, P, I, I, I, I, I, I, I64, I, I, P]
        L.qk_norm_rope_ex.argtypes = [P, P, I64, P, P, I64, P, P, P, I, I, I, I, I, F, I, I, I, P]
        L.qk_norm_rope_v.argtypes = [P, P, I64, P, P, I64, P, P, I64, P, P, P, P, I, I, I, I, I, F, I, I, I, P]
        L.kv_cache_positions.argtypes = [I64, I, I, I, ctypes.POINTER(I64), I]
        L.kv_cache_rope.argtypes = [P, P, P, I, I, I, I, I, I, I64, I, P]
        L.attn_forward.argtypes = [P, P, P, P, I, I, I, I, I, I, F, I, P]
        L.attn_forward_f16.argtypes = [P, P, P, P, I, I, I, I, I, I, F, I, P]
        L.attn_forward_kvstride.argtypes = [P, P, P, P, I, I, I, I, I, I, F, I, I64, I, P]
        L.attn_forward_window.argtypes = [P, P, P, P, I, I, I, I, I, I, F, I, I, I64, I, P]
        L.attn_forward_workspace_bytes.argtypes = [I]
        L.attn_forward_ws.argtypes = [P, P, P, P, I, I, I, I, I, I, F, I, I, I64, I, P, I64, P]
        L.attn_forward_ws_static.argtypes = [P, P, P, P, I, I, I, I, I, I, F, I, I, I64, I, P]
        L.attn_forward_qnorm.argtypes = [P, P, P, P, P, F, P, I, I, I, I, I, I, I, F, I, I, I64, I, P, I64, P]
        L.sa_last_error.restype = ctypes.c_char_p
        for name in EXPORTS[:-1]:
            getattr(L, name).restype = I
        L.attn_forward_workspace_bytes.restype = I64
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise StreamAttnError(fn, status, lib().sa_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t=None):
    dev = t.device if t is not None and t.is_cuda else None
    return torch.cuda.current_stream(dev).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SA_DTYPE_BF16
    if t.dtype == torch.float16:
        return SA_DTYPE_F16
    if t.dtype == torch.float8_e4m3fn:
        return SA_DTYPE_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _require_bf16(fn: str, *tensors) -> None:
    """The prologue kernels read bf16 rows: any other input type would be misread (or, for a
    one-byte type, read past its end)."""
    for t in tensors:
        if t is not None and t.dtype != torch.bfloat16:
            raise StreamAttnError(fn, SA_ERR_UNSUPPORTED_CODE, f"inputs must be bfloat16, got {t.dtype}")


def _attn_dtype(q, k, v, fp8_probs: bool = False) -> int:
    """Attention dtype code of (q, k, v): one common type, or bf16 q/k with an f16 v; with
    fp8_probs (E4M3 q, k, v only) the opt-in FP8-probability P*V."""
    if q.dtype == torch.bfloat16 and k.dtype == torch.bfloat16 and v.dtype == torch.float16:
        code = SA_DTYPE_BF16_F16V
    elif not (q.dtype == k.dtype == v.dtype):
        raise TypeError(f"unsupported attention dtypes {q.dtype}, {k.dtype}, {v.dtype}")
    else:
        code = _dtype_code(q)
    if fp8_probs:
        if code != SA_DTYPE_FP8_E4M3:
            raise TypeError("FP8 probabilities need float8_e4m3fn q, k and v")
        return SA_DTYPE_FP8_E4M3_P8
    return code


def attn_forward(q, k, v, out, scale: float, causal: bool = False):
    """out[B, Lq, Hq, d] = softmax(q k^T * scale) v for bf16 q/k/v/out (contiguous)."""
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    _check("attn_forward", lib().attn_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, Lq, Lk, d,
                                              float(scale), int(bool(causal)), _stream(q)))
    return out


def attn_forward_f16(q, k, v, out, scale: float, causal: bool = False):
    """The fp16 variant of attn_forward."""
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    _check("attn_forward_f16", lib().attn_forward_f16(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, Lq, Lk,
                                                      d, float(scale), int(bool(causal)), _stream(q)))
    return out


def attn_forward_fp8(q, k, v, out, scale: float, causal: bool = False, fp8_probs: bool = False):
    """FP8 attention: q, k, v float8_e4m3fn (contiguous), out bf16 [B, Lq, Hq, d]. fp8_probs=True
    also rounds the softmax probabilities to E4M3 for an FP8 P*V product (opt-in, less accurate)."""
    return attn_forward_kvstride(q, k, v, out, k.shape[1], scale, causal, fp8_probs=fp8_probs)


def attn_forward_kvstride(q, k, v, out, Lk: int, scale: float, causal: bool = False, fp8_probs: bool = False):
    """Attention over the first Lk tokens of k, v [B, S, Hkv, d] (S >= Lk), e.g. a rolling cache.
    bf16/f16 tensors, or float8_e4m3fn q, k, v with a bf16 out (fp8_probs: FP8 P*V)."""
    B, Lq, Hq, d = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    kv_bstride = S * Hkv * d
    _check("attn_forward_kvstride",
           lib().attn_forward_kvstride(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, Lq, int(Lk), d,
                                       float(scale), int(bool(causal)), kv_bstride, _attn_dtype(q, k, v, fp8_probs),
                                       _stream(q)))
    return out


def attn_workspace(d: int, device=None) -> torch.Tensor:
    """A workspace for attn_forward_ws on the current (or given) device."""
    n = lib().attn_forward_workspace_bytes(int(d))
    if n < 0:
        _check("attn_forward_workspace_bytes", int(n))
    return torch.empty((int(n),), dtype=torch.uint8, device=device or "cuda")


def attn_forward_ws(q, k, v, out, scale: float, workspace, Lk: int | None = None, window=(-1, -1),
                    fp8_probs: bool = False):
    """Attention over the first Lk tokens of k, v [B, S, Hkv, d] with a workspace (attn_workspace)
    that lets under-filled grids run balanced; same results as attn_forward_kvstride."""
    B, Lq, Hq, d = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    left, right = (int(x) for x in window)
    _check("attn_forward_ws",
           lib().attn_forward_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, Lq, S if Lk is None else int(Lk),
                                 d, float(scale), left, right, S * Hkv * d, _attn_dtype(q, k, v, fp8_probs),
                                 _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(q)))
    return out


def attn_forward_ws_static(q, k, v, out, scale: float, Lk: int | None = None, window=(-1, -1),
                           fp8_probs: bool = False):
    """attn_forward_ws with the library's own per-GPU scratch instead of a workspace: allocates
    nothing. Calls that overlap on one GPU race (they share that scratch)."""
    B, Lq, Hq, d = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    left, right = (int(x) for x in window)
    _check("attn_forward_ws_static",
           lib().attn_forward_ws_static(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, Lq,
                                        S if Lk is None else int(Lk), d, float(scale), left, right, S * Hkv * d,
                                        _attn_dtype(q, k, v, fp8_probs), _stream(q)))
    return out


def attn_forward_qnorm(q, k, v, out, scale: float, gamma_q, eps: float = 1e-6, workspace=None, Lk: int | None = None,
                       window=(-1, -1), rope_cs=None, rope_style: int = SA_ROPE_NONE):
    """Attention whose query rows are RMS-normalised (head scope, weights gamma_q fp32 [d]) and,
    with rope_cs (fp32 [Lq, d]: cos then sin per row, as qk_norm_rope_v writes) and rope_style
    SA_ROPE_SPLIT / SA_ROPE_INTERLEAVED, rotated as they are loaded; q itself is not modified.
    Same as qk_norm_rope on the queries followed by attn_forward_ws, without the normalised Q
    round trip through memory."""
    B, Lq, Hq, d = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    left, right = (int(x) for x in window)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("attn_forward_qnorm",
           lib().attn_forward_qnorm(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(gamma_q), float(eps), _ptr(rope_cs),
                                    int(rope_style) if rope_cs is not None else SA_ROPE_NONE, B, Hq, Hkv, Lq,
                                    S if Lk is None else int(Lk), d, float(scale), left, right, S * Hkv * d,
                                    _attn_dtype(q, k, v), _ptr(workspace), ws_bytes, _stream(q)))
    return out


def attn_forward_window(q, k, v, out, scale: float, window: tuple[int, int], Lk: int | None = None,
                        fp8_probs: bool = False):
    """Local attention: query i (key position p = i + Lk - Lq) sees keys [p - left, p + right].

    window = (left, right), -1 for an unbounded side; k, v [B, S, Hkv, d] with S >= Lk
    (Lk defaults to S). bf16 or fp16 for all four tensors.
    """
    B, Lq, Hq, d = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    left, right = (int(w) for w in window)
    _check("attn_forward_window",
           lib().attn_forward_window(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, Lq, S if Lk is None else int(Lk),
                                     d, float(scale), left, right, S * Hkv * d, _attn_dtype(q, k, v, fp8_probs),
                                     _stream(q)))
    return out


def qk_norm_rope(q_in, q_out, k_in=None, k_out=None, gamma_q=None, gamma_k=None, angles=None, eps: float = 1e-6,
                 norm_scope: int = SA_NORM_HEAD, rope_style: int = SA_ROPE_SPLIT, q_out_bstride=None,
                 k_out_bstride=None, Hkv: int | None = None):
    """RMSNorm (head or inner scope) then RoPE of q_in (and k_in) into q_out (and k_out); bf16 in,
    bf16 or float8_e4m3fn out (the type of q_out; k_out must have the same type).

    q_in [B, L, Hq, d]; k_out may be a view of a cache row range (pass k_out_bstride = S*Hkv*d).
    rope_style | SA_ROPE_AFTER_CACHE rotates the queries only (keys are normalised, unrotated).
    """
    B, L, Hq, d = q_in.shape
    if Hkv is None:
        Hkv = k_in.shape[2] if k_in is not None else 0
    if q_out_bstride is None:
        q_out_bstride = L * Hq * d
    if k_out_bstride is None:
        k_out_bstride = L * Hkv * d
    # the C call takes one output type for both row classes and reads 16-bit inputs: a key output
    # of another type would be written with the query output's element size
    _require_bf16("qk_norm_rope", q_in, k_in)
    if k_out is not None and k_out.dtype != q_out.dtype:
        raise StreamAttnError("qk_norm_rope", SA_ERR_SHAPE_CODE,
                              f"q_out ({q_out.dtype}) and k_out ({k_out.dtype}) must share one dtype")
    out_dtype = _dtype_code(q_out)
    _check("qk_norm_rope_ex", lib().qk_norm_rope_ex(_ptr(q_in), _ptr(q_out), q_out_bstride, _ptr(k_in), _ptr(k_out),
                                                    k_out_bstride, _ptr(gamma_q), _ptr(gamma_k), _ptr(angles), B, L,
                                                    Hq, Hkv, d, float(eps), norm_scope, rope_style, out_dtype,
                                                    _stream(q_in)))


def qk_norm_rope_v(k_in, k_out, v_in, v_out, gamma_k=None, angles=None, eps: float = 1e-6,
                   norm_scope: int = SA_NORM_HEAD, rope_style: int = SA_ROPE_SPLIT, rope_cs_out=None,
                   k_out_bstride=None, v_out_bstride=None, q_in=None, q_out=None, gamma_q=None, q_out_bstride=None):
    """The chunk prologue in one launch: keys normalised (and rotated unless rope_style has
    SA_ROPE_AFTER_CACHE) into k_out, values copied into v_out (both may be cache row-range views:
    pass the cache's batch strides), optional queries as in qk_norm_rope, and optionally the
    chunk's cos/sin table (fp32 [L, d]) for attn_forward_qnorm. bf16 in; out type of k_out."""
    B, L, Hkv, d = (k_in if k_in is not None else v_in).shape
    Hq = q_in.shape[2] if q_in is not None else 0
    if k_out_bstride is None:
        k_out_bstride = L * Hkv * d
    if v_out_bstride is None:
        v_out_bstride = L * Hkv * d
    if q_out_bstride is None:
        q_out_bstride = L * max(Hq, 1) * d
    _require_bf16("qk_norm_rope_v", q_in, k_in, v_in)
    outs = [t for t in (q_out, k_out, v_out) if t is not None]
    if any(t.dtype != outs[0].dtype for t in outs):
        raise StreamAttnError("qk_norm_rope_v", SA_ERR_SHAPE_CODE, "q_out, k_out and v_out must share one dtype")
    out_dtype = _dtype_code(k_out if k_out is not None else v_out)
    _check("qk_norm_rope_v", lib().qk_norm_rope_v(_ptr(q_in), _ptr(q_out), q_out_bstride, _ptr(k_in), _ptr(k_out),
                                                  k_out_bstride, _ptr(v_in), _ptr(v_out), v_out_bstride, _ptr(gamma_q),
                                                  _ptr(gamma_k), _ptr(angles), _ptr(rope_cs_out), B, L, Hq, Hkv, d,
                                                  float(eps), norm_scope, rope_style, out_dtype, _stream(k_in)))


def kv_cache_slot(chunk_idx: int, chunk_len: int, sink_size: int, window_size: int):
    """(slot_base, visible_len) of chunk ``chunk_idx`` in a rolling sink + window cache."""
    slot = ctypes.c_int64()
    vis = ctypes.c_int()
    _check("kv_cache_slot", lib().kv_cache_slot(int(chunk_idx), int(chunk_len), int(sink_size), int(window_size),
                                                ctypes.byref(slot), ctypes.byref(vis)))
    return slot.value, vis.value


def kv_cache_positions(chunk_idx: int, chunk_len: int, sink_size: int, window_size: int):
    """Logical (arrival-order) row of each visible physical cache row after chunk ``chunk_idx``."""
    _, vis = kv_cache_slot(chunk_idx, chunk_len, sink_size, window_size)
    out = (ctypes.c_int64 * max(vis, 1))()
    _check("kv_cache_positions", lib().kv_cache_positions(int(chunk_idx), int(chunk_len), int(sink_size),
                                                          int(window_size), out, vis))
    return [out[i] for i in range(vis)]


def kv_cache_rope(cache_k, k_rot, angles, chunk_idx: int, chunk_len: int, sink_size: int, window_size: int,
                  rope_style: int = SA_ROPE_SPLIT):
    """After-cache RoPE: rotate the visible rows of cache_k [B, S, Hkv, d] into k_rot (same shape)
    with angles [visible_len, d/2] indexed by logical row."""
    B, S, Hkv, d = cache_k.shape
    _require_bf16("kv_cache_rope", cache_k, k_rot)
    _check("kv_cache_rope", lib().kv_cache_rope(_ptr(cache_k), _ptr(k_rot), _ptr(angles), B, Hkv, d, int(chunk_len),
                                                int(sink_size), int(window_size), int(chunk_idx), int(rope_style),
                                                _stream(cache_k)))


def kv_cache_append(k_new, v_new, cache_k, cache_v, chunk_idx: int, sink_size: int, window_size: int):
    """Copy k_new / v_new [B, Lc, Hkv, d] (either may be None) into their cache slot range; a cache of
    another element type (float8_e4m3fn or f16 for bf16 input) receives the rounded values."""
    if k_new is None and v_new is None:
        raise StreamAttnError("kv_cache_append", -1, "both k_new and v_new are None")
    same = (k_new is None or v_new is None or
            (k_new.dtype == v_new.dtype and cache_k.dtype == cache_v.dtype))
    # one C call converts both tensors with one (source, cache) type pair, so keys and values of
    # different type pairs (e.g. a bf16 key cache with an f16 value cache) take one call each
    pairs = [(k_new, v_new, cache_k, cache_v)] if same else [(k_new, None, cache_k, None), (None, v_new, None, cache_v)]
    for kn, vn, ck, cv in pairs:
        ref = vn if vn is not None else kn
        dst = cv if vn is not None else ck
        if dst is None:
            raise StreamAttnError("kv_cache_append", -1, "a cache tensor is None for a given source")
        B, Lc, Hkv, d = ref.shape
        if ref.dtype == dst.dtype and ref.element_size() == 2:  # any 16-bit type: a byte copy
            _check("kv_cache_append", lib().kv_cache_append(_ptr(kn), _ptr(vn), _ptr(ck), _ptr(cv), B, Lc, Hkv, d,
                                                            sink_size, window_size, int(chunk_idx), _stream(ref)))
            continue
        _check("kv_cache_append_ex", lib().kv_cache_append_ex(_ptr(kn), _ptr(vn), _ptr(ck), _ptr(cv), B, Lc, Hkv, d,
                                                              sink_size, window_size, int(chunk_idx),
                                                              _dtype_code(ref), _dtype_code(dst), _stream(ref)))


class BlockKVCache:
    """Caller-side rolling cache: storage [B, sink + window, Hkv, d] plus the chunk bookkeeping.

    Lifecycle per chunk (page "Accelerated building blocks", section "Cache lifecycle"):
    before_update(c) -> write this chunk's keys/values -> attend -> after_update(c).
    """

    def __init__(self, B: int, Hkv: int, d: int, chunk_len: int, sink_size: int, window_size: int,
                 dtype=torch.bfloat16, device="cuda", after_cache_rope: bool = False, v_dtype=None):
        """dtype: element type of the cache (bf16, or float8_e4m3fn for the FP8 path). v_dtype=float16
        with a bf16 cache keeps V in the f16 type the P*V product uses (same results, no per-tile
        conversion in attention)."""
        self.B, self.Hkv, self.d = B, Hkv, d
        self.chunk_len, self.sink_size, self.window_size = chunk_len, sink_size, window_size
        S = sink_size + window_size
        self.k = torch.empty((B, S, Hkv, d), dtype=dtype, device=device)
        self.v = torch.empty((B, S, Hkv, d), dtype=v_dtype or dtype, device=device)
        # after-cache RoPE: the cache keeps unrotated keys; each step rotates the visible ones here
        self.k_rot = torch.empty_like(self.k) if after_cache_rope else None
        # the chunk's RoPE cos/sin table [Lc, d] for queries rotated inside the attention
        self.rope_cs = torch.empty((chunk_len, d), dtype=torch.float32, device=device)
        self.slot_base = 0
        self.visible_len = 0
        self._current = None
        self._last = None   # last chunk written in the current stream (None: a fresh stream)

    @property
    def capacity(self) -> int:
        return self.sink_size + self.window_size

    def reset(self):
        """Start a new stream: the next chunk must be chunk 0. The storage keeps its old rows, but
        none of them is visible again before a chunk of the new stream overwrites it (chunk c
        sees exactly the rows chunks 0 .. c of its own stream wrote), so nothing is cleared."""
        if self._current is not None:
            raise RuntimeError("reset inside before_update / after_update")
        self.slot_base = self.visible_len = 0
        self._last = None

    def before_update(self, chunk_idx: int):
        """Chunks of a stream are written in order: chunk 0 (which also restarts a used cache, as
        reset() does) or the chunk after the last one -- the visible rows are those chunks 0 .. c
        wrote, so a skipped chunk would expose rows of another stream."""
        if self._current is not None:
            raise RuntimeError("before_update called twice without after_update")
        expected = 0 if self._last is None else self._last + 1
        if chunk_idx != 0 and chunk_idx != expected:
            raise StreamAttnError("before_update", SA_ERR_SHAPE_CODE,
                                  f"chunk {chunk_idx} after chunk {self._last}: write chunks in order (0 restarts)")
        self.slot_base, self.visible_len = kv_cache_slot(chunk_idx, self.chunk_len, self.sink_size,
                                                         self.window_size)
        self._current = chunk_idx
        return self.slot_base, self.visible_len

    def k_slot_view(self):
        """Keys of the current chunk's slot range (a strided view into the cache)."""
        return self.k[:, self.slot_base:self.slot_base + self.chunk_len]

    def after_update(self, chunk_idx: int):
        if self._current != chunk_idx:
            raise RuntimeError("after_update does not match before_update")
        self._current = None
        self._last = chunk_idx


def _check_step(cache: BlockKVCache, chunk_idx: int, q_in, k_in, v_in, q_buf, out, angles, rope: bool,
                in_attn: bool) -> None:
    """What a streaming step is built for, checked before its first launch. Shapes: the chunk's
    q_in [B, Lc, Hq, d] and k_in, v_in [B, Lc, Hkv, d] contiguous, with the cache's B, Lc, Hkv
    and d (a chunk of another length would write past its slot range), Hq a multiple of Hkv,
    q_buf and out of q_in's shape, angles with the rows the RoPE scope reads. Types: bf16 inputs;
    a bf16 or E4M3 key cache whose value cache has the same type (or f16 values with bf16 keys);
    queries buffered in the key cache's type; a bf16 output."""
    fn = "stream_self_attention_step"
    B, Lc, Hkv, d = cache.B, cache.chunk_len, cache.Hkv, cache.d
    for name, t in (("k_in", k_in), ("v_in", v_in)):
        if tuple(t.shape) != (B, Lc, Hkv, d) or not t.is_contiguous():
            raise StreamAttnError(fn, SA_ERR_SHAPE_CODE,
                                  f"{name} must be a contiguous [{B}, {Lc}, {Hkv}, {d}] chunk, got {tuple(t.shape)}")
    if (q_in.dim() != 4 or tuple(q_in.shape[:2]) != (B, Lc) or q_in.shape[3] != d or q_in.shape[2] % Hkv
            or not q_in.is_contiguous()):
        raise StreamAttnError(fn, SA_ERR_SHAPE_CODE,
                              f"q_in must be a contiguous [{B}, {Lc}, Hq, {d}] chunk with Hq a multiple of {Hkv}, "
                              f"got {tuple(q_in.shape)}")
    for name, t in (("q_buf", None if in_attn else q_buf), ("out", out)):
        if t is not None and (tuple(t.shape) != tuple(q_in.shape) or not t.is_contiguous()):
            raise StreamAttnError(fn, SA_ERR_SHAPE_CODE, f"{name} must be contiguous with q_in's shape {tuple(q_in.shape)}")
    if rope:
        # before-cache RoPE reads the chunk's Lc rows; after-cache RoPE one row per visible key
        rows = kv_cache_slot(chunk_idx, Lc, cache.sink_size, cache.window_size)[1] if cache.k_rot is not None else Lc
        if (angles is None or angles.dim() != 2 or angles.shape[1] != d // 2 or angles.shape[0] < rows
                or angles.dtype != torch.float32 or not angles.is_contiguous()):
            raise StreamAttnError(fn, SA_ERR_SHAPE_CODE, f"angles must be contiguous fp32 [>= {rows}, {d // 2}]")
    _require_bf16(fn, q_in, k_in, v_in)
    kt, vt = cache.k.dtype, cache.v.dtype
    if kt not in (torch.bfloat16, torch.float8_e4m3fn):
        raise StreamAttnError(fn, SA_ERR_UNSUPPORTED_CODE, f"key cache dtype {kt} is not bf16 or float8_e4m3fn")
    if not (vt == kt or (kt == torch.bfloat16 and vt == torch.float16)):
        raise StreamAttnError(fn, SA_ERR_UNSUPPORTED_CODE,
                              f"value cache dtype {vt} with key cache dtype {kt} (same type, or f16 values with bf16 keys)")
    if cache.k_rot is not None and kt != torch.bfloat16:
        raise StreamAttnError(fn, SA_ERR_UNSUPPORTED_CODE, "after-cache RoPE is built for a bf16 cache only")
    if not in_attn and (q_buf is None or q_buf.dtype != kt):
        raise StreamAttnError(fn, SA_ERR_SHAPE_CODE,
                              f"q_buf must have the key cache's dtype {kt}, got {None if q_buf is None else q_buf.dtype}")
    if out.dtype != torch.bfloat16:
        raise StreamAttnError(fn, SA_ERR_UNSUPPORTED_CODE, f"out must be bfloat16, got {out.dtype}")


def stream_self_attention_step(cache: BlockKVCache, chunk_idx: int, q_in, k_in, v_in, q_buf, out, gamma_q,
                               gamma_k, angles, eps: float, scale: float,
                               rope_style: int = SA_ROPE_SPLIT, norm_scope: int = SA_NORM_HEAD, workspace=None,
                               query_in_attention: bool = False, fp8_probs: bool = False):
    """One streaming self-attention chunk as library calls between before_update / after_update.

    Default route: qk_norm_rope_v in one launch writes the normalised (and rotated, unless
    after-cache RoPE) queries into q_buf, the normalised keys into the chunk's cache slot and the
    values into the value cache; the attention then reads q_buf. It applies when the value cache
    has the key cache's type (bf16 or FP8 E4M3); a cache with f16 values takes qk_norm_rope (q_in
    -> q_buf, k_in -> cache keys) -> kv_cache_append (v_in -> cache values) instead, with the same
    results bit for bit.
    query_in_attention=True (bf16 cache with bf16 values, head-scope norm, bf16 q_in): the
    prologue writes keys, values and the chunk's cos/sin table (cache.rope_cs), and the attention
    (attn_forward_qnorm) normalises and rotates the raw queries as it loads them; q_buf is not
    used. This saves the query pass but reads the cos/sin table once per query block and head,
    which on the streaming shapes costs more than the pass it saves.
    A cache of float8_e4m3fn (BlockKVCache(dtype=torch.float8_e4m3fn), before-cache RoPE only) with
    an E4M3 q_buf is the FP8 path: the prologue rounds Q, K and V to E4M3 and attention runs on
    the FP8 MFMA with a bf16 out.
    Before-cache RoPE (cache.k_rot is None): angles [Lc, d/2] for the chunk's positions.
    After-cache RoPE (cache built with after_cache_rope=True): angles [visible_len, d/2] by
    logical row; the queries are rotated with the chunk's rows (the last Lc) and the keys are
    stored unrotated; kv_cache_rope then rotates the visible keys into cache.k_rot, which the
    attention reads.
    workspace (attn_workspace): lets the attention run balanced when its grid would leave CU
    slots idle. fp8_probs (FP8 cache only, opt-in): the attention also rounds its softmax
    probabilities to E4M3 for an FP8 P*V product. Returns the visible length used.
    """
    in_attn = (query_in_attention and norm_scope == SA_NORM_HEAD and cache.k.dtype == torch.bfloat16 and
               cache.v.dtype == torch.bfloat16)
    rope = rope_style != SA_ROPE_NONE
    _check_step(cache, chunk_idx, q_in, k_in, v_in, q_buf, out, angles, rope, in_attn)
    slot, visible = cache.before_update(chunk_idx)
    S = cache.capacity
    after = cache.k_rot is not None
    q_angles = angles[visible - cache.chunk_len:visible] if after else angles
    flag = SA_ROPE_AFTER_CACHE if after else 0
    style = (rope_style | flag) if rope else SA_ROPE_NONE
    bstride = S * cache.Hkv * cache.d
    if in_attn:
        qk_norm_rope_v(k_in, cache.k[:, slot:], v_in, cache.v[:, slot:], gamma_k, q_angles if rope else None, eps,
                       norm_scope, style, rope_cs_out=cache.rope_cs if rope else None, k_out_bstride=bstride,
                       v_out_bstride=bstride)
    elif cache.v.dtype == cache.k.dtype:
        qk_norm_rope_v(k_in, cache.k[:, slot:], v_in, cache.v[:, slot:], gamma_k, q_angles if rope else None, eps,
                       norm_scope, style, k_out_bstride=bstride, v_out_bstride=bstride, q_in=q_in, q_out=q_buf,
                       gamma_q=gamma_q)
    else:
        qk_norm_rope(q_in, q_buf, k_in, cache.k[:, slot:], gamma_q, gamma_k, q_angles if rope else None, eps,
                     norm_scope, style, k_out_bstride=bstride)
        kv_cache_append(None, v_in, None, cache.v, chunk_idx, cache.sink_size, cache.window_size)
    keys = cache.k
    if after:
        kv_cache_rope(cache.k, cache.k_rot, angles, chunk_idx, cache.chunk_len, cache.sink_size, cache.window_size,
                      rope_style)
        keys = cache.k_rot
    if in_attn:
        attn_forward_qnorm(q_in, keys, cache.v, out, scale, gamma_q, eps, workspace=workspace, Lk=visible,
                           rope_cs=cache.rope_cs if rope else None, rope_style=rope_style)
    elif workspace is not None:
        attn_forward_ws(q_buf, keys, cache.v, out, scale, workspace, Lk=visible, fp8_probs=fp8_probs)
    else:
        attn_forward_kvstride(q_buf, keys, cache.v, out, visible, scale, False, fp8_probs=fp8_probs)
    cache.after_update(chunk_idx)
    return visible


def context_kv(k_in, v_in, cache_k, cache_v, gamma_k=None, eps: float = 1e-6, norm_scope: int = SA_NORM_HEAD,
               angles=None, rope_style: int = SA_ROPE_SPLIT):
    """Static cross-attention context cache (the compute_kv step): context keys k_in [B, S, H, d]
    RMS-normalised (no weights: not normalised) into cache_k, and rotated with angles [S, d/2]
    for before-cache RoPE or left unrotated (angles None) for after-cache RoPE; values copied
    into cache_v. One prologue launch; bf16 in, the caches' type out."""
    scope = norm_scope if gamma_k is not None else SA_NORM_NONE
    style = rope_style if angles is not None else SA_ROPE_NONE
    qk_norm_rope_v(k_in, cache_k, v_in, cache_v, gamma_k, angles, eps, scope, style)


def cross_attention_step(context_k, context_v, q_in, out, gamma_q, eps: float, scale: float, q_buf=None,
                         q_angles=None, context_angles=None, k_rot=None, rope_style: int = SA_ROPE_SPLIT,
                         workspace=None):
    """One query chunk of cross-attention over a static context cache (context_kv), as library calls.

    * No RoPE (q_angles None): the query RMSNorm (head scope, gamma_q) runs inside the attention
      as it loads each query row (attn_forward_qnorm); q_buf is not used.
    * Before-cache RoPE (q_angles given, context_angles None): the cached keys were rotated by
      context_kv; qk_norm_rope normalises and rotates the queries into q_buf, then attention.
    * After-cache RoPE (q_angles and context_angles given): the cache holds unrotated keys, and
      every call rotates all S of them with the cache-relative angle rows context_angles[0:S] into
      k_rot ([B, S, H, d] bf16, not the cache). A static context cache is the rolling cache after
      its one and only chunk (chunk length = window = S, no sink), whose rows are in logical
      order, so kv_cache_rope does this. The queries are normalised and rotated with q_angles
      [Lq, d/2] into q_buf, then attention runs over k_rot.
    workspace (attn_workspace) lets the attention run balanced when its grid would leave CUs idle."""
    if q_angles is None:
        if context_angles is not None:
            raise StreamAttnError("cross_attention_step", SA_ERR_SHAPE_CODE, "context angles without query angles")
        return attn_forward_qnorm(q_in, context_k, context_v, out, scale, gamma_q, eps, workspace=workspace)
    if q_buf is None or q_buf.shape != q_in.shape or q_buf.dtype != torch.bfloat16:
        raise StreamAttnError("cross_attention_step", SA_ERR_SHAPE_CODE, "q_buf must be a bf16 tensor of q_in's shape")
    B, S, Hkv, d = context_k.shape
    keys = context_k
    if context_angles is not None:
        if k_rot is None or k_rot.shape != context_k.shape or k_rot.data_ptr() == context_k.data_ptr():
            raise StreamAttnError("cross_attention_step", SA_ERR_SHAPE_CODE, "k_rot must be a separate buffer of the cache's shape")
        if context_angles.shape[0] < S:
            raise StreamAttnError("cross_attention_step", SA_ERR_SHAPE_CODE, f"context angles need {S} rows")
        kv_cache_rope(context_k, k_rot, context_angles, 0, S, 0, S, rope_style)
        keys = k_rot
    qk_norm_rope(q_in, q_buf, None, None, gamma_q, None, q_angles, eps,
                 SA_NORM_HEAD if gamma_q is not None else SA_NORM_NONE, rope_style, Hkv=0)
    if workspace is not None:
        return attn_forward_ws(q_buf, keys, context_v, out, scale, workspace)
    return attn_forward_kvstride(q_buf, keys, context_v, out, S, scale, False)
