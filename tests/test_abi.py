"""CPU checks of the C ABI: the library loads, exports every declared symbol, validates its
arguments on the host (no GPU work happens for a rejected call), and its rolling-cache slot rule
agrees with the oracle's chunk-by-chunk simulation."""
import ctypes
import os
import re

import pytest

from head_attention_streaming_amd import binding
from oracle.cache import RollingCacheModel

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "streamattn.h")

lib = pytest.importorskip("head_attention_streaming_amd.binding").lib

# These checks hand the library fake device addresses that argument validation must reject
# before anything is launched; where a GPU is visible they are not run (they are host-side
# checks, and a validation regression must never reach a launch on real hardware).
import torch  # noqa: E402

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="host-side validation checks (no GPU)")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int64_t|int|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = lib()
    for name in _declared():
        assert hasattr(L, name), name
    # the exported symbols are C names (no C++ mangling)
    raw = ctypes.CDLL(binding.library_path())
    for name in _declared():
        assert ctypes.cast(getattr(raw, name), ctypes.c_void_p).value


def _attn(q=1, k=1, v=1, out=16, B=1, Hq=8, Hkv=8, Lq=16, Lk=16, d=128, scale=0.1, causal=0):
    # fake but aligned non-null addresses: only reached if validation passes, which these avoid
    P = lambda x: None if x is None else ctypes.c_void_p(x * 4096)
    return lib().attn_forward(P(q), P(k), P(v), P(out), B, Hq, Hkv, Lq, Lk, d, scale, causal, None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), -3), (dict(d=256), -3), (dict(Hq=6, Hkv=4), -2), (dict(causal=1, Lq=20, Lk=16), -2),
    (dict(causal=2), -5), (dict(Lq=-1), -5), (dict(Hq=0), -5), (dict(scale=0.0), -5),
    (dict(scale=float("nan")), -5), (dict(Lk=0), -2), (dict(q=None), -1), (dict(v=None), -1),
])
def test_attn_forward_rejects_bad_arguments(kw, code):
    assert _attn(**kw) == code
    assert lib().sa_last_error().decode() != ""


def test_attn_forward_misaligned_pointer():
    L = lib()
    st = L.attn_forward(ctypes.c_void_p(4096 + 2), ctypes.c_void_p(8192), ctypes.c_void_p(8192),
                        ctypes.c_void_p(8192), 1, 1, 1, 4, 4, 64, 0.1, 0, None)
    assert st == -4


def test_attn_forward_empty_is_noop():
    assert _attn(q=None, k=None, v=None, out=None, Lq=0) == 0
    assert _attn(q=None, k=None, v=None, out=None, B=0) == 0


def test_kvstride_too_small_rejected():
    L = lib()
    P = ctypes.c_void_p(4096)
    assert L.attn_forward_kvstride(P, P, P, P, 2, 4, 4, 8, 100, 64, 0.1, 0, 99 * 4 * 64, 0, None) == -2
    assert L.attn_forward_kvstride(P, P, P, P, 2, 4, 4, 8, 100, 64, 0.1, 0, 100 * 4 * 64, 7, None) == -3


def test_qk_norm_rope_rejects_bad_arguments():
    L = lib()
    P = ctypes.c_void_p(4096)
    g = ctypes.c_void_p(8192)
    # head dim not built
    assert L.qk_norm_rope(P, P, 96 * 8 * 4, None, None, 0, g, None, g, 1, 4, 8, 0, 96, 1e-6, 1, 1, None) == -3
    # inner scope with grouped key heads
    assert L.qk_norm_rope(P, P, 128 * 8 * 4, P, P, 128 * 2 * 4, g, g, g, 1, 4, 8, 2, 128, 1e-6, 2, 1, None) == -3
    # unknown norm scope; the after-cache flag without a pairing; pairing value 3
    assert L.qk_norm_rope(P, P, 128 * 8 * 4, None, None, 0, g, None, g, 1, 4, 8, 0, 128, 1e-6, 3, 1, None) == -3
    assert L.qk_norm_rope(P, P, 128 * 8 * 4, None, None, 0, g, None, g, 1, 4, 8, 0, 128, 1e-6, 1, 4, None) == -3
    assert L.qk_norm_rope(P, P, 128 * 8 * 4, None, None, 0, g, None, g, 1, 4, 8, 0, 128, 1e-6, 1, 7, None) == -3
    # RoPE enabled without angles
    assert L.qk_norm_rope(P, P, 128 * 8 * 4, None, None, 0, g, None, None, 1, 4, 8, 0, 128, 1e-6, 1, 1, None) == -1
    # head norm without weights
    assert L.qk_norm_rope(P, P, 128 * 8 * 4, None, None, 0, None, None, g, 1, 4, 8, 0, 128, 1e-6, 1, 1, None) == -1
    # k_in without k_out
    assert L.qk_norm_rope(P, P, 128 * 8 * 4, P, None, 0, g, g, g, 1, 4, 8, 8, 128, 1e-6, 1, 1, None) == -1
    # output batch stride smaller than one batch
    assert L.qk_norm_rope(P, P, 100, None, None, 0, g, None, g, 2, 4, 8, 0, 128, 1e-6, 1, 1, None) == -2


def test_kv_cache_append_rejects_bad_arguments():
    L = lib()
    P = ctypes.c_void_p(4096)
    assert L.kv_cache_append(None, None, P, P, 1, 16, 2, 64, 0, 64, 0, None) == -1
    assert L.kv_cache_append(None, P, None, None, 1, 16, 2, 64, 0, 64, 0, None) == -1
    assert L.kv_cache_append(None, P, None, P, 1, 16, 2, 64, 8, 64, 0, None) == -5   # sink not a multiple
    assert L.kv_cache_append(None, P, None, P, 1, 16, 2, 64, 0, 8, 0, None) == -5    # window < chunk
    assert L.kv_cache_append(None, P, None, P, 1, 16, 2, 96, 0, 64, 0, None) == -3
    assert L.kv_cache_append(None, P, None, P, 1, 16, 2, 64, 0, 64, -1, None) == -5


@pytest.mark.parametrize("Lc,sink,window", [(1785, 0, 7140), (10, 10, 30), (10, 20, 10), (3, 0, 3), (7, 14, 35)])
def test_kv_cache_slot_matches_oracle_simulation(Lc, sink, window):
    model = RollingCacheModel(Lc, sink, window)
    for c in range(2 * (sink + window) // Lc + 7):
        expect_slot = model.write(c)
        slot, vis = binding.kv_cache_slot(c, Lc, sink, window)
        assert slot == expect_slot, c
        assert vis == model.visible_len(), c


def test_kv_cache_slot_large_chunk_index():
    slot, vis = binding.kv_cache_slot(10 ** 15, 16, 32, 64)
    assert vis == 96 and slot == 32 + ((10 ** 15 - 2) % 4) * 16
    with pytest.raises(binding.StreamAttnError):
        binding.kv_cache_slot(-1, 16, 0, 64)


def _win(left, right, Lq=16, Lk=16, q=1):
    P = lambda x: None if x is None else ctypes.c_void_p(x * 4096)
    return lib().attn_forward_window(P(q), P(1), P(1), P(16), 1, 8, 8, Lq, Lk, 128, 0.1, left, right,
                                     Lk * 8 * 128, 0, None)


@pytest.mark.parametrize("left,right,Lq,Lk,code", [
    (-2, 0, 16, 16, -5), (4, -7, 16, 16, -5),          # bounds below -1
    (4, 0, 20, 16, -2),                                # causal band with Lq > Lk: first query sees nothing
    (-1, 3, 20, 16, -2),                               # Lq > Lk + right
])
def test_attn_forward_window_rejects_bad_arguments(left, right, Lq, Lk, code):
    assert _win(left, right, Lq, Lk) == code
    assert lib().sa_last_error().decode() != ""


def test_attn_forward_window_accepts_lq_up_to_lk_plus_right():
    # Lq = Lk + right passes shape validation; the null q pointer is what stops the call
    assert _win(-1, 4, 20, 16, q=None) == -1


@pytest.mark.parametrize("Lc,sink,window", [(1785, 0, 7140), (10, 10, 30), (10, 20, 10), (3, 0, 3), (7, 14, 35)])
def test_kv_cache_positions_match_oracle_arrival_order(Lc, sink, window):
    """Physical row -> logical row of the visible keys, against the oracle's chunk simulation:
    the logical order is the visible chunks in arrival order (sinks first)."""
    model = RollingCacheModel(Lc, sink, window)
    for c in range(2 * (sink + window) // Lc + 7):
        model.write(c)
        pos = binding.kv_cache_positions(c, Lc, sink, window)
        vis = model.visible_chunks()
        assert len(pos) == model.visible_len()
        expect = [0] * len(pos)
        for logical_chunk, chunk in enumerate(vis):
            s0 = model.slot_of(chunk)
            for i in range(Lc):
                expect[s0 + i] = logical_chunk * Lc + i
        assert pos == expect, (c, pos[:: max(1, Lc)], expect[:: max(1, Lc)])


def test_kv_cache_rope_rejects_bad_arguments():
    L = lib()
    P, Q = ctypes.c_void_p(4096), ctypes.c_void_p(8192)
    assert L.kv_cache_rope(P, Q, P, 1, 4, 128, 16, 0, 64, 0, 3, None) == -3      # pairing
    assert L.kv_cache_rope(P, Q, P, 1, 4, 128, 16, 0, 64, 0, 0, None) == -3      # no rotation
    assert L.kv_cache_rope(P, Q, P, 1, 4, 96, 16, 0, 64, 0, 1, None) == -3       # head dim
    assert L.kv_cache_rope(P, P, P, 1, 4, 128, 16, 0, 64, 0, 1, None) == -2      # in place
    assert L.kv_cache_rope(P, Q, None, 1, 4, 128, 16, 0, 64, 0, 1, None) == -1   # no angles
    assert L.kv_cache_rope(P, Q, P, 1, 4, 128, 16, 8, 64, 0, 1, None) == -5      # sink not a multiple
    assert L.kv_cache_rope(P, Q, P, 1, 0, 128, 16, 0, 64, 0, 1, None) == -5      # no heads
    out = (ctypes.c_int64 * 4)()
    assert L.kv_cache_positions(5, 16, 0, 64, out, 4) == -5                      # output too small


def test_fp8_kv_stride_must_be_16_bytes():
    L = lib()
    P = ctypes.c_void_p(4096)
    # 100*4*64 + 8 elements is 16-byte aligned for 16-bit types but not for one-byte FP8
    assert L.attn_forward_kvstride(P, P, P, P, 2, 4, 4, 8, 100, 64, 0.1, 0, 100 * 4 * 64 + 8, 2, None) == -4
    assert L.attn_forward_kvstride(P, P, P, P, 2, 4, 4, 8, 100, 64, 0.1, 0, 100 * 4 * 64, 9, None) == -3


def test_typed_prologue_and_append_reject_bad_arguments():
    L = lib()
    P, g = ctypes.c_void_p(4096), ctypes.c_void_p(8192)
    # qk_norm_rope_ex: f16 output is not built; FP8 output needs 16-element aligned batch strides
    assert L.qk_norm_rope_ex(P, P, 128 * 8 * 4, None, None, 0, g, None, g, 1, 4, 8, 0, 128, 1e-6, 1, 1, 1, None) == -3
    assert L.qk_norm_rope_ex(P, P, 128 * 8 * 4 + 8, None, None, 0, g, None, g, 2, 4, 8, 0, 128, 1e-6, 1, 1, 2,
                             None) == -2
    # kv_cache_append_ex: conversions that do not exist
    assert L.kv_cache_append_ex(None, P, None, P, 1, 16, 2, 64, 0, 64, 0, 1, 2, None) == -3   # f16 -> fp8
    assert L.kv_cache_append_ex(None, P, None, P, 1, 16, 2, 64, 0, 64, 0, 2, 0, None) == -3   # fp8 -> bf16
    assert L.kv_cache_append_ex(None, P, None, P, 1, 16, 2, 64, 0, 64, 0, 0, 7, None) == -3   # unknown type


def test_attn_forward_qnorm_rejects_bad_arguments():
    L = lib()
    P, g = ctypes.c_void_p(4096), ctypes.c_void_p(8192)

    def call(gamma=g, eps=1e-6, cs=None, style=0, Hq=8, Hkv=8, dtype=0, d=128):
        return L.attn_forward_qnorm(P, P, P, P, gamma, eps, cs, style, 1, Hq, Hkv, 16, 16, d, 0.1, -1, -1,
                                    16 * Hkv * d, dtype, None, 0, None)

    assert call(gamma=None) == -1
    assert call(gamma=ctypes.c_void_p(8192 + 4)) == -4
    assert call(eps=-1.0) == -5
    assert call(eps=float("nan")) == -5
    assert call(dtype=2) == -3          # FP8 queries: no fused norm
    assert call(dtype=9) == -3
    assert call(Hq=6, Hkv=4) == -2
    assert call(d=96) == -3
    assert call(style=1) == -1          # RoPE without its cos/sin table
    assert call(cs=g) == -1             # a table without a pairing
    assert call(cs=g, style=3) == -3
    assert call(cs=ctypes.c_void_p(8192 + 8), style=1) == -4
    assert lib().sa_last_error().decode() != ""


def test_qk_norm_rope_v_rejects_bad_arguments():
    L = lib()
    P, g, a = ctypes.c_void_p(4096), ctypes.c_void_p(8192), ctypes.c_void_p(12288)
    S = 64 * 8 * 128  # a cache of 64 rows

    def call(q=(None, None), k=(P, P), v=(P, P), gq=None, gk=g, ang=a, cs=None, Hkv=8, d=128, style=1, out=0,
             vbs=S, kbs=S, scope=1):
        return L.qk_norm_rope_v(q[0], q[1], 16 * 8 * d, k[0], k[1], kbs, v[0], v[1], vbs, gq, gk, ang, cs, 1, 16, 8,
                                Hkv, d, 1e-6, scope, style, out, None)

    assert call(k=(None, None), v=(None, None)) == -1      # no rows at all
    assert call(v=(P, None)) == -1                         # v_in without v_out
    assert call(q=(P, None)) == -1
    assert call(gq=g) == -2                                # query weights without queries
    assert call(gk=None) == -1                             # key weights missing
    assert call(cs=g, style=0, ang=None) == -2             # cos/sin table without RoPE
    assert call(cs=ctypes.c_void_p(8192 + 4)) == -4
    assert call(vbs=16 * 8 * 128 - 8) == -2                # value batch stride below one chunk
    assert call(vbs=S + 8, out=2) == -2                    # FP8 strides must be 16-element multiples
    assert call(Hkv=0) == -5
    assert call(d=96) == -3
    assert call(out=1) == -3
    assert lib().sa_last_error().decode() != ""


def test_binding_qk_norm_rope_v_requires_one_output_dtype():
    """The one-launch prologue writes every output row in one type (the C-ABI takes a single
    out_dtype), so the binding rejects query/key/value outputs of different dtypes before any
    library call."""
    import torch
    from head_attention_streaming_amd import binding
    k = torch.zeros((1, 4, 2, 64), dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    q = torch.zeros((1, 4, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(binding.StreamAttnError) as e:
        binding.qk_norm_rope_v(k, torch.empty_like(k), v, torch.empty_like(v, dtype=torch.float16))
    assert e.value.status == binding.SA_ERR_SHAPE_CODE
    with pytest.raises(binding.StreamAttnError) as e:
        binding.qk_norm_rope_v(k, torch.empty_like(k), v, torch.empty_like(v), q_in=q,
                               q_out=torch.empty_like(q, dtype=torch.float8_e4m3fn))
    assert e.value.status == binding.SA_ERR_SHAPE_CODE


def test_binding_qk_norm_rope_requires_one_output_dtype():
    """qk_norm_rope writes query and key rows with one output type (the C call takes a single
    out_dtype): a key output of another type would be written with the query output's element
    size, so the binding rejects it before any library call; non-bf16 inputs are rejected too."""
    import torch
    from head_attention_streaming_amd import binding
    q = torch.zeros((1, 4, 2, 64), dtype=torch.bfloat16)
    k = torch.zeros_like(q)
    with pytest.raises(binding.StreamAttnError) as e:
        binding.qk_norm_rope(q, torch.empty_like(q), k, torch.empty_like(k, dtype=torch.float8_e4m3fn))
    assert e.value.status == binding.SA_ERR_SHAPE_CODE
    with pytest.raises(binding.StreamAttnError) as e:
        binding.qk_norm_rope(q.half(), torch.empty_like(q), k, torch.empty_like(k))
    assert e.value.status == binding.SA_ERR_UNSUPPORTED_CODE


class _RecordingLib:
    """Stands in for the loaded library: records each entry point's arguments and returns 0."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append((name, args))
            return 0
        return fn


def test_binding_kv_cache_append_one_call_per_type_pair(monkeypatch):
    """A bf16 key cache with an f16 value cache: one C call converts both tensors with a single
    (source, cache) type pair, so the binding issues one call per tensor, each with its own pair
    (the key copy must not be converted to f16, nor a 2-byte row be copied into an FP8 cache)."""
    import torch
    from head_attention_streaming_amd import binding
    rec = _RecordingLib()
    monkeypatch.setattr(binding, "lib", lambda: rec)
    monkeypatch.setattr(binding, "_stream", lambda t=None: None)
    k = torch.zeros((1, 4, 2, 64), dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    ck = torch.zeros((1, 8, 2, 64), dtype=torch.bfloat16)
    cv = torch.zeros((1, 8, 2, 64), dtype=torch.float16)
    binding.kv_cache_append(k, v, ck, cv, 0, 0, 8)
    names = [c[0] for c in rec.calls]
    assert names == ["kv_cache_append", "kv_cache_append_ex"]
    kargs, vargs = rec.calls[0][1], rec.calls[1][1]
    assert kargs[0] == k.data_ptr() and kargs[1] is None and kargs[2] == ck.data_ptr() and kargs[3] is None
    assert vargs[0] is None and vargs[1] == v.data_ptr() and vargs[3] == cv.data_ptr()
    assert vargs[-3:-1] == (binding.SA_DTYPE_BF16, binding.SA_DTYPE_F16)
    # FP8 key cache, bf16 value cache: the key rows are rounded to E4M3, the values byte-copied
    rec.calls.clear()
    ck8 = torch.zeros((1, 8, 2, 64), dtype=torch.float8_e4m3fn)
    binding.kv_cache_append(k, v, ck8, ck, 0, 0, 8)
    assert [c[0] for c in rec.calls] == ["kv_cache_append_ex", "kv_cache_append"]
    assert rec.calls[0][1][-3:-1] == (binding.SA_DTYPE_BF16, binding.SA_DTYPE_FP8_E4M3)
    # same types: one call for both
    rec.calls.clear()
    binding.kv_cache_append(k, v, ck, torch.zeros_like(ck), 0, 0, 8)
    assert [c[0] for c in rec.calls] == ["kv_cache_append"]


@pytest.mark.parametrize("kdt,vdt,qdt,code", [
    ("float8_e4m3fn", "float16", "float8_e4m3fn", -3),   # FP8 keys with 16-bit values: not built
    ("float8_e4m3fn", "bfloat16", "float8_e4m3fn", -3),
    ("bfloat16", "bfloat16", "float8_e4m3fn", -2),      # queries buffered in another type
    ("bfloat16", "float16", "float16", -2),
    ("float16", "float16", "float16", -3),              # f16 key cache: not built
])
def test_binding_streaming_step_rejects_unbuilt_dtype_combinations(kdt, vdt, qdt, code, monkeypatch):
    """The streaming step checks the (key cache, value cache, query buffer) types before its first
    launch, so no kernel ever writes rows of one type at another type's element size."""
    import torch
    from head_attention_streaming_amd import binding
    rec = _RecordingLib()
    monkeypatch.setattr(binding, "lib", lambda: rec)
    B, Lc, H, d = 1, 4, 2, 64
    cache = binding.BlockKVCache(B, H, d, Lc, 0, 2 * Lc, dtype=getattr(torch, kdt), device="cpu",
                                 v_dtype=getattr(torch, vdt))
    x = torch.zeros((B, Lc, H, d), dtype=torch.bfloat16)
    q_buf = torch.zeros((B, Lc, H, d), dtype=getattr(torch, qdt))
    out = torch.zeros((B, Lc, H, d), dtype=torch.bfloat16)
    g = torch.ones(d)
    ang = torch.zeros((Lc, d // 2))
    with pytest.raises(binding.StreamAttnError) as e:
        binding.stream_self_attention_step(cache, 0, x, x, x, q_buf, out, g, g, ang, 1e-6, 0.125)
    assert e.value.status == code
    assert rec.calls == [] and cache._current is None  # nothing launched, no chunk opened


def _step_args(B=1, Lc=4, H=2, d=64, **over):
    import torch
    a = dict(q_in=torch.zeros((B, Lc, H, d), dtype=torch.bfloat16), k_in=torch.zeros((B, Lc, H, d), dtype=torch.bfloat16),
             v_in=torch.zeros((B, Lc, H, d), dtype=torch.bfloat16), q_buf=torch.zeros((B, Lc, H, d), dtype=torch.bfloat16),
             out=torch.zeros((B, Lc, H, d), dtype=torch.bfloat16), gamma_q=torch.ones(d), gamma_k=torch.ones(d),
             angles=torch.zeros((Lc, d // 2)))
    a.update(over)
    return a


@pytest.mark.parametrize("what", ["short_chunk", "long_chunk", "kv_heads", "head_dim", "q_heads_not_multiple",
                                  "noncontiguous_k", "out_shape", "angles_rows", "angles_dtype", "batch"])
def test_binding_streaming_step_rejects_shape_changes(what, monkeypatch):
    """A chunk whose shape differs from the cache's (length, heads, head dim, batch), or angles
    with too few rows, is rejected before any launch: a longer chunk would otherwise be written
    past its slot range into the next chunk's rows or past the cache."""
    import torch
    from head_attention_streaming_amd import binding
    rec = _RecordingLib()
    monkeypatch.setattr(binding, "lib", lambda: rec)
    B, Lc, H, d = 1, 4, 2, 64
    cache = binding.BlockKVCache(B, H, d, Lc, 0, 2 * Lc, device="cpu")
    bf = dict(dtype=torch.bfloat16)
    bad = {
        "short_chunk": dict(k_in=torch.zeros((B, Lc - 1, H, d), **bf)),
        "long_chunk": dict(q_in=torch.zeros((B, Lc + 1, H, d), **bf), k_in=torch.zeros((B, Lc + 1, H, d), **bf),
                           v_in=torch.zeros((B, Lc + 1, H, d), **bf), q_buf=torch.zeros((B, Lc + 1, H, d), **bf),
                           out=torch.zeros((B, Lc + 1, H, d), **bf), angles=torch.zeros((Lc + 1, d // 2))),
        "kv_heads": dict(v_in=torch.zeros((B, Lc, H + 1, d), **bf)),
        "head_dim": dict(q_in=torch.zeros((B, Lc, H, 128), **bf)),
        "q_heads_not_multiple": dict(q_in=torch.zeros((B, Lc, 3, d), **bf), q_buf=torch.zeros((B, Lc, 3, d), **bf),
                                     out=torch.zeros((B, Lc, 3, d), **bf)),
        "noncontiguous_k": dict(k_in=torch.zeros((B, H, Lc, d), **bf).transpose(1, 2)),
        "out_shape": dict(out=torch.zeros((B, Lc, H + 2, d), **bf)),
        "angles_rows": dict(angles=torch.zeros((Lc - 1, d // 2))),
        "angles_dtype": dict(angles=torch.zeros((Lc, d // 2), dtype=torch.float64)),
        "batch": dict(q_in=torch.zeros((2, Lc, H, d), **bf), k_in=torch.zeros((2, Lc, H, d), **bf),
                      v_in=torch.zeros((2, Lc, H, d), **bf), q_buf=torch.zeros((2, Lc, H, d), **bf),
                      out=torch.zeros((2, Lc, H, d), **bf)),
    }[what]
    a = _step_args(B, Lc, H, d, **bad)
    with pytest.raises(binding.StreamAttnError) as e:
        binding.stream_self_attention_step(cache, 0, a["q_in"], a["k_in"], a["v_in"], a["q_buf"], a["out"],
                                           a["gamma_q"], a["gamma_k"], a["angles"], 1e-6, 0.125)
    assert e.value.status == binding.SA_ERR_SHAPE_CODE
    assert rec.calls == [] and cache._current is None


def test_block_kv_cache_lifecycle_order_and_reset():
    """Chunks of a stream are written in order; chunk 0 (or reset()) restarts the stream; a
    skipped or repeated chunk is rejected (it would expose rows another stream wrote)."""
    from head_attention_streaming_amd import binding
    cache = binding.BlockKVCache(1, 2, 64, 4, 4, 8, device="cpu")
    for c in range(5):
        assert cache.before_update(c) == binding.kv_cache_slot(c, 4, 4, 8)
        cache.after_update(c)
    for bad in (4, 6, 3):
        with pytest.raises(binding.StreamAttnError):
            cache.before_update(bad)
    assert cache.before_update(0) == (0, 4)   # a restart sees only its own first chunk
    cache.after_update(0)
    assert cache.before_update(1) == (4, 8)
    with pytest.raises(RuntimeError):
        cache.reset()                          # not between before_update and after_update
    cache.after_update(1)
    cache.reset()
    with pytest.raises(binding.StreamAttnError):
        cache.before_update(2)
    assert cache.before_update(0) == (0, 4)


def test_fp8_probability_dtype_is_accepted_and_qnorm_rejects_it():
    """dtype 4 (E4M3 with FP8 probabilities) passes validation like dtype 2 (an empty problem is a
    no-op), needs 16-byte K/V batch strides in bytes, and the fused query norm rejects it."""
    lib = binding.lib()
    p = ctypes.c_void_p(4096)
    assert lib.attn_forward_kvstride(p, p, p, p, 0, 8, 8, 16, 16, 128, 0.1, 0, 16 * 8 * 128, 4, None) == 0
    assert lib.attn_forward_kvstride(p, p, p, p, 1, 8, 8, 16, 16, 128, 0.1, 0, 16 * 8 * 128 + 8, 4, None) == -4
    assert lib.attn_forward_kvstride(p, p, p, p, 1, 8, 8, 16, 16, 128, 0.1, 0, 16 * 8 * 128, 5, None) == -3
    g = ctypes.c_void_p(8192)
    assert lib.attn_forward_qnorm(p, p, p, p, g, 1e-6, None, 0, 1, 8, 8, 16, 16, 128, 0.1, -1, -1, 16 * 8 * 128, 4,
                                  None, 0, None) == -3
