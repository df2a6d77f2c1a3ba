"""GPU parity of the opt-in FP8-probability attention (SA_DTYPE_FP8_E4M3_P8): E4M3 q, k, v, the
softmax probabilities rounded to E4M3 for an FP8 P*V product with V in E4M3, bf16 out. Compared
with the exact fp64 attention of the same E4M3 inputs under the bound derived from the rounding
(tests/parity.py::assert_fp8p_close): per element u/(1-u) * sum_j w_j |v_j - o| + one ulp, and a
mean-abs bound from the rounding variance. Special cases are exact: a single visible key returns
its value, q = 0 returns the mean of V."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from head_attention_streaming_amd import binding, synthetic
from parity import E4M3_NORMAL_BINADES, assert_attention_close, assert_fp8p_close, sample_rows, widen

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # name, B, Lq, Lk, Hq, Hkv, d, window (None: full), rows sampled (None: every row)
    ("gqa_d128_ragged", 1, 130, 300, 4, 2, 128, None, None),
    ("mha_d64_b2", 2, 257, 257, 3, 3, 64, None, None),
    ("causal_rect_d128", 1, 200, 333, 2, 2, 128, (-1, 0), None),
    ("window_d64", 1, 400, 400, 2, 1, 64, (64, 0), None),
    ("split_keys_d128", 1, 256, 2000, 2, 2, 128, None, None),       # few blocks, long loop: key-split shape
    ("wide_grid_d128", 1, 4000, 700, 64, 16, 128, None, 2048),      # 256-row blocks
    ("long_c5_shape", 1, 20480, 20480, 56, 56, 128, None, 1024),    # the long problem's shape
]


def _inputs(name, B, Lq, Lk, Hq, Hkv, d):
    return synthetic.attention_inputs(B, Lq, Lk, Hq, Hkv, d, "e4m3", seed=zlib.crc32(name.encode()) % 10000)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp8_probabilities_within_rounding_bound(case):
    name, B, Lq, Lk, Hq, Hkv, d, window, nrows = case
    print(f"[case] {case}", flush=True)
    q, k, v = _inputs(name, B, Lq, Lk, Hq, Hkv, d)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    scale = d ** -0.5
    binding.attn_forward_window(qd, kd, vd, out, scale, window or (-1, -1), fp8_probs=True)
    torch.cuda.synchronize()
    Q, K, V = (widen(x).reshape(x.shape) for x in (q, k, v))
    rows = None if nrows is None else sample_rows(B, Lq, Hq, nrows, seed=7)
    o, a, r, _, ta, tw = oracle.attention_spread(Q, K, V, scale, window=window, rows=rows,
                                                 tail_binades=E4M3_NORMAL_BINADES)
    got = out if rows is None else out.reshape(-1, d)[torch.from_numpy(rows).to(DEV)]
    print(assert_fp8p_close(got, o, a, r, ta, tw, name), flush=True)


def test_fp8_probabilities_balanced_launch_and_streaming_cache():
    """The balanced launch (persistent workgroups, pieces merged from a workspace) at the
    streaming shape, and the same attention through the streaming step's FP8 cache."""
    B, Lq, Lk, H, d = 1, 1785, 7140, 40, 128
    q, k, v = _inputs("balanced", B, Lq, Lk, H, H, d)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    binding.attn_forward_ws(qd, kd, vd, out, d ** -0.5, binding.attn_workspace(d), fp8_probs=True)
    torch.cuda.synchronize()
    Q, K, V = (widen(x).reshape(x.shape) for x in (q, k, v))
    rows = sample_rows(B, Lq, H, 2048, seed=11)
    o, a, r, _, ta, tw = oracle.attention_spread(Q, K, V, d ** -0.5, rows=rows, tail_binades=E4M3_NORMAL_BINADES)
    assert_fp8p_close(out.reshape(-1, d)[torch.from_numpy(rows).to(DEV)], o, a, r, ta, tw, "balanced")


def test_fp8_probabilities_exact_special_cases():
    """One visible key: the output is that key's value (bf16 holds every E4M3 value). q = 0: every
    probability is 2^8, an E4M3 value, so the output is the mean of V within the 16-bit bounds."""
    g = torch.Generator().manual_seed(5)
    k = synthetic.normal((1, 1, 2, 128), "e4m3", g)
    v = synthetic.normal((1, 1, 2, 128), "e4m3", g)
    q = synthetic.normal((1, 70, 2, 128), "e4m3", g)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    binding.attn_forward_fp8(q.to(DEV), k.to(DEV), v.to(DEV), out, 0.1, fp8_probs=True)
    torch.cuda.synchronize()
    assert np.array_equal(widen(out).reshape(q.shape), np.broadcast_to(widen(v).reshape(v.shape), q.shape))
    q0 = torch.zeros((2, 90, 3, 64), dtype=torch.float8_e4m3fn)
    k0 = synthetic.normal((2, 500, 3, 64), "e4m3", g)
    v0 = synthetic.normal((2, 500, 3, 64), "e4m3", g)
    out0 = torch.empty(q0.shape, dtype=torch.bfloat16, device=DEV)
    binding.attn_forward_fp8(q0.to(DEV), k0.to(DEV), v0.to(DEV), out0, 0.125, fp8_probs=True)
    torch.cuda.synchronize()
    V0 = widen(v0).reshape(v0.shape)
    ref = np.broadcast_to(V0.mean(axis=1, keepdims=True), q0.shape)
    assert_attention_close(out0, np.ascontiguousarray(ref), "q = 0")


def test_fp8_probabilities_streaming_step_fp8_cache():
    """The streaming step with an FP8 E4M3 cache and fp8_probs through fill and eviction: every
    chunk within the rounding bound of the exact attention over the visible E4M3 keys."""
    from oracle.cache import RollingCacheModel
    B, Lc, H, d, sink, window = 1, 96, 4, 128, 96, 192
    eps, scale = 1e-6, d ** -0.5
    cache = binding.BlockKVCache(B, H, d, Lc, sink, window, dtype=torch.float8_e4m3fn, device=DEV)
    model = RollingCacheModel(Lc, sink, window)
    g = torch.Generator().manual_seed(6600)
    gq, gk = synthetic.norm_weight(d, g), synthetic.norm_weight(d, g)
    kst, vals = {}, {}
    for c in range(5):
        gc = torch.Generator().manual_seed(6600 + c)
        q, k, v = (synthetic.normal((B, Lc, H, d), "bf16", gc) for _ in range(3))
        ang = synthetic.rope_angles(np.arange(c * Lc, (c + 1) * Lc), d)
        q_buf = torch.empty((B, Lc, H, d), dtype=torch.float8_e4m3fn, device=DEV)
        out = torch.empty((B, Lc, H, d), dtype=torch.bfloat16, device=DEV)
        binding.stream_self_attention_step(cache, c, q.to(DEV), k.to(DEV), v.to(DEV), q_buf, out, gq.to(DEV),
                                           gk.to(DEV), ang.to(DEV), eps, scale, fp8_probs=True)
        torch.cuda.synchronize()
        model.write(c)
        # the attention's inputs are what the prologue stored (checked elsewhere): use them as given
        Q = widen(q_buf).reshape(q.shape)
        kst[c] = widen(cache.k[:, model.slot_of(c):model.slot_of(c) + Lc].contiguous()).reshape(k.shape)
        vals[c] = widen(cache.v[:, model.slot_of(c):model.slot_of(c) + Lc].contiguous()).reshape(v.shape)
        vis = model.visible_chunks()
        K = np.concatenate([kst[x] for x in vis], axis=1)
        V = np.concatenate([vals[x] for x in vis], axis=1)
        o, a, r, _, ta, tw = oracle.attention_spread(Q, K, V, scale, tail_binades=E4M3_NORMAL_BINADES)
        assert_fp8p_close(out, o, a, r, ta, tw, f"chunk {c}")
