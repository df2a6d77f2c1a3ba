"""GPU parity of the streaming path: qk_norm_rope (per-head RMSNorm + RoPE), kv_cache_append
(bit-exact), and streaming self-attention / cross-attention end to end, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from head_attention_streaming_amd import binding, synthetic
from oracle.cache import RollingCacheModel
from parity import assert_attention_close, assert_within_one_ulp, sample_rows, widen

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENTINEL = 0x7E11  # a bf16 NaN pattern no copy produces


def _oracle_prologue(x, gamma, eps, angles, style, inner=False):
    """Oracle RMSNorm (head scope, or inner scope over all heads of a token) then RoPE, fp64."""
    g = None if gamma is None else gamma.double().numpy()
    a = None if angles is None else angles.double().numpy()
    z = widen(x).reshape(x.shape)
    if inner and g is not None:
        B, L, H, d = x.shape
        z = oracle.rmsnorm(z.reshape(B, L, H * d), g, eps).reshape(B, L, H, d)
        g = None
    return oracle.qk_norm_rope(z, g, eps, a, style)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("style", [binding.SA_ROPE_SPLIT, binding.SA_ROPE_INTERLEAVED, binding.SA_ROPE_NONE])
@pytest.mark.parametrize("with_k", [True, False])
def test_qk_norm_rope_matches_oracle(d, style, with_k):
    B, L, Hq, Hkv = 2, 37, 5, 3
    print(f"[case] d={d} style={style} with_k={with_k}", flush=True)
    g = torch.Generator().manual_seed(100 + d + style)
    q = synthetic.normal((B, L, Hq, d), "bf16", g, 2.0)
    k = synthetic.normal((B, L, Hkv, d), "bf16", g, 0.5)
    gq, gk = synthetic.norm_weight(d, g), synthetic.norm_weight(d, g)
    ang = synthetic.rope_angles(np.arange(5000, 5000 + L), d) if style else None
    qd, kd = q.to(DEV), k.to(DEV)
    qo = torch.empty_like(qd)
    ko = torch.empty_like(kd) if with_k else None
    binding.qk_norm_rope(qd, qo, kd if with_k else None, ko, gq.to(DEV), gk.to(DEV) if with_k else None,
                         ang.to(DEV) if style else None, 1e-6, binding.SA_NORM_HEAD, style)
    torch.cuda.synchronize()
    assert_within_one_ulp(qo, _oracle_prologue(q, gq, 1e-6, ang, style), "q")
    if with_k:
        assert_within_one_ulp(ko, _oracle_prologue(k, gk, 1e-6, ang, style), "k")


@pytest.mark.parametrize("d,H,with_k", [(128, 5, True), (64, 5, True), (128, 7, False), (128, 80, True),
                                         (64, 150, True)])
def test_qk_norm_rope_inner_scope(d, H, with_k):
    """Inner-scope RMSNorm (m = H*d over all heads of a token) then split RoPE. H*2 rows above 128
    (d = 128) or 256 (d = 64) exercise the path that reads the rows twice."""
    B, L = 2, 9
    print(f"[case] inner d={d} H={H} with_k={with_k}", flush=True)
    g = torch.Generator().manual_seed(200 + d + H)
    q = synthetic.normal((B, L, H, d), "bf16", g, 2.0)
    k = synthetic.normal((B, L, H, d), "bf16", g, 0.5)
    gq, gk = synthetic.norm_weight(H * d, g), synthetic.norm_weight(H * d, g)
    ang = synthetic.rope_angles(np.arange(300, 300 + L), d)
    qd, kd = q.to(DEV), k.to(DEV)
    qo = torch.empty_like(qd)
    ko = torch.empty_like(kd) if with_k else None
    binding.qk_norm_rope(qd, qo, kd if with_k else None, ko, gq.to(DEV), gk.to(DEV) if with_k else None,
                         ang.to(DEV), 1e-6, binding.SA_NORM_INNER, binding.SA_ROPE_SPLIT)
    torch.cuda.synchronize()
    assert_within_one_ulp(qo, _oracle_prologue(q, gq, 1e-6, ang, oracle.SPLIT, inner=True), "q inner")
    if with_k:
        assert_within_one_ulp(ko, _oracle_prologue(k, gk, 1e-6, ang, oracle.SPLIT, inner=True), "k inner")


@pytest.mark.parametrize("style", [binding.SA_ROPE_SPLIT, binding.SA_ROPE_INTERLEAVED])
def test_qk_norm_rope_after_cache_rotates_queries_only(style):
    B, L, Hq, Hkv, d = 1, 33, 4, 2, 128
    g = torch.Generator().manual_seed(17 + style)
    q = synthetic.normal((B, L, Hq, d), "bf16", g)
    k = synthetic.normal((B, L, Hkv, d), "bf16", g)
    gq, gk = synthetic.norm_weight(d, g), synthetic.norm_weight(d, g)
    ang = synthetic.rope_angles(np.arange(40, 40 + L), d)
    qd, kd = q.to(DEV), k.to(DEV)
    qo, ko = torch.empty_like(qd), torch.empty_like(kd)
    binding.qk_norm_rope(qd, qo, kd, ko, gq.to(DEV), gk.to(DEV), ang.to(DEV), 1e-6, binding.SA_NORM_HEAD,
                         style | binding.SA_ROPE_AFTER_CACHE)
    torch.cuda.synchronize()
    assert_within_one_ulp(qo, _oracle_prologue(q, gq, 1e-6, ang, style), "q rotated")
    assert_within_one_ulp(ko, _oracle_prologue(k, gk, 1e-6, None, 0), "k normalised only")


@pytest.mark.parametrize("Lc,sink,window,chunk,d", [(40, 40, 120, 6, 128), (40, 0, 120, 1, 128), (32, 64, 64, 7, 64)])
def test_kv_cache_rope_matches_oracle(Lc, sink, window, chunk, d):
    """Every visible cache row rotated with the angles of its arrival-order row (from the oracle's
    cache simulation); rows past the visible length untouched."""
    B, H = 2, 3
    S = sink + window
    model = RollingCacheModel(Lc, sink, window)
    for c in range(chunk + 1):
        model.write(c)
    n = model.visible_len()
    g = torch.Generator().manual_seed(Lc + chunk)
    cache = synthetic.normal((B, S, H, d), "bf16", g)
    ang = synthetic.rope_angles(np.arange(n) * 3 + 11, d)
    k_rot = torch.full((B, S, H, d), 0, dtype=torch.int16).fill_(SENTINEL).view(torch.bfloat16).to(DEV)
    binding.kv_cache_rope(cache.to(DEV), k_rot, ang.to(DEV), chunk, Lc, sink, window, binding.SA_ROPE_SPLIT)
    torch.cuda.synchronize()
    got = k_rot.cpu()
    logical = np.empty(n, dtype=np.int64)
    for j, x in enumerate(model.visible_chunks()):
        s0 = model.slot_of(x)
        logical[s0:s0 + Lc] = j * Lc + np.arange(Lc)
    ref = oracle.rope(widen(cache[:, :n]).reshape(B, n, H, d), ang.double().numpy()[logical], oracle.SPLIT)
    assert_within_one_ulp(got[:, :n], ref, "k_rot")
    assert bool((got[:, n:].view(torch.int16) == SENTINEL).all()), "rows past the visible length were written"


def test_qk_norm_rope_without_norm_and_in_place():
    B, L, H, d = 1, 20, 4, 128
    g = torch.Generator().manual_seed(3)
    q = synthetic.normal((B, L, H, d), "bf16", g)
    ang = synthetic.rope_angles(np.arange(L) * 97, d)
    qd = q.to(DEV)
    binding.qk_norm_rope(qd, qd, None, None, None, None, ang.to(DEV), 0.0, binding.SA_NORM_NONE,
                         binding.SA_ROPE_SPLIT)  # in place, rotation only
    torch.cuda.synchronize()
    assert_within_one_ulp(qd, _oracle_prologue(q, None, 0.0, ang, oracle.SPLIT), "rope only")


def test_qk_norm_rope_full_streaming_chunk():
    """Prologue of the streaming workload at full size: [1, 1785, 40, 128] q and k, split RoPE at
    absolute positions of chunk 5, keys written straight into a 4-chunk cache slot range."""
    L, H, d, S = 1785, 40, 128, 7140
    c = 5
    g = torch.Generator().manual_seed(1300 + c)
    q = synthetic.normal((1, L, H, d), "bf16", g)
    k = synthetic.normal((1, L, H, d), "bf16", g)
    gq, gk = synthetic.norm_weight(d, g), synthetic.norm_weight(d, g)
    ang = synthetic.rope_angles(np.arange(c * L, (c + 1) * L), d)
    slot, _ = binding.kv_cache_slot(c, L, 0, S)
    cache = torch.full((1, S, H, d), 0, dtype=torch.int16, device=DEV)
    cache.fill_(SENTINEL)
    cache = cache.view(torch.bfloat16)
    qo = torch.empty((1, L, H, d), dtype=torch.bfloat16, device=DEV)
    binding.qk_norm_rope(q.to(DEV), qo, k.to(DEV), cache[:, slot:], gq.to(DEV), gk.to(DEV), ang.to(DEV), 1e-6,
                         binding.SA_NORM_HEAD, binding.SA_ROPE_SPLIT, k_out_bstride=S * H * d)
    torch.cuda.synchronize()
    assert_within_one_ulp(qo, _oracle_prologue(q, gq, 1e-6, ang, oracle.SPLIT), "q chunk")
    assert_within_one_ulp(cache[:, slot:slot + L], _oracle_prologue(k, gk, 1e-6, ang, oracle.SPLIT), "k chunk")
    untouched = torch.cat([cache[:, :slot], cache[:, slot + L:]], dim=1).view(torch.int16)
    assert bool((untouched == SENTINEL).all())


@pytest.mark.parametrize("B,Lc,H,d,sink,window", [(2, 16, 3, 64, 16, 48), (1, 1785, 40, 128, 0, 7140)])
def test_kv_cache_append_bit_exact_fill_and_eviction(B, Lc, H, d, sink, window):
    print(f"[case] B={B} Lc={Lc} H={H} d={d} sink={sink} window={window}", flush=True)
    S = sink + window
    model = RollingCacheModel(Lc, sink, window)
    cache_k = torch.full((B, S, H, d), SENTINEL, dtype=torch.int16, device=DEV)
    cache_v = torch.full((B, S, H, d), SENTINEL, dtype=torch.int16, device=DEV)
    expect_k = torch.full((B, S, H, d), SENTINEL, dtype=torch.int16)
    expect_v = torch.full((B, S, H, d), SENTINEL, dtype=torch.int16)
    n_chunks = 2 * S // Lc + 2
    g = torch.Generator().manual_seed(55)
    for c in range(n_chunks):
        kc = torch.randint(-32768, 32767, (B, Lc, H, d), generator=g, dtype=torch.int16)
        vc = torch.randint(-32768, 32767, (B, Lc, H, d), generator=g, dtype=torch.int16)
        s0 = model.write(c)
        expect_k[:, s0:s0 + Lc] = kc
        expect_v[:, s0:s0 + Lc] = vc
        binding.kv_cache_append(kc.to(DEV), vc.to(DEV), cache_k, cache_v, c, sink, window)
        torch.cuda.synchronize()
        assert torch.equal(cache_k.cpu(), expect_k), f"K cache differs after chunk {c}"
        assert torch.equal(cache_v.cpu(), expect_v), f"V cache differs after chunk {c}"


def _streaming_run(B, Lc, H, d, sink, window, n_chunks, rows_per_chunk, seed0, style=binding.SA_ROPE_SPLIT,
                   after_cache=False, inner=False, fp8=False, workspace=False):
    """Run the streaming loop on the GPU and compare every chunk's output with the oracle.
    workspace: pass an attention workspace, as the benchmark's steps do, so grids with a mostly
    idle last round run balanced.

    Before-cache RoPE: angles at absolute stream positions c*Lc + i rotate the chunk's queries
    and keys, and the cache stores rotated keys. After-cache RoPE: the cache stores normalised,
    unrotated keys; each step rotates the visible keys at their rows 0 .. n-1 of the visible
    sequence (arrival order) and the queries at the last Lc rows."""
    eps, scale = 1e-6, d ** -0.5
    cdt = torch.float8_e4m3fn if fp8 else torch.bfloat16
    rnd = "e4m3" if fp8 else "bf16"   # the type the cache and the attention inputs hold
    cache = binding.BlockKVCache(B, H, d, Lc, sink, window, dtype=cdt, device=DEV, after_cache_rope=after_cache)
    model = RollingCacheModel(Lc, sink, window)
    g = torch.Generator().manual_seed(seed0)
    gdim = H * d if inner else d
    gq, gk = synthetic.norm_weight(gdim, g), synthetic.norm_weight(gdim, g)
    gqd, gkd = gq.to(DEV), gk.to(DEV)
    scope = binding.SA_NORM_INNER if inner else binding.SA_NORM_HEAD
    kstar, vals = {}, {}
    results = []
    ws = binding.attn_workspace(d) if workspace else None
    for c in range(n_chunks):
        gc = torch.Generator().manual_seed(seed0 + c)
        q = synthetic.normal((B, Lc, H, d), "bf16", gc)
        k = synthetic.normal((B, Lc, H, d), "bf16", gc)
        v = synthetic.normal((B, Lc, H, d), "bf16", gc)
        model.write(c)
        n = model.visible_len()
        if after_cache:
            ang = synthetic.rope_angles(np.arange(n), d)       # rows of the visible sequence
            ang_q = ang[n - Lc:]
        else:
            ang = ang_q = synthetic.rope_angles(np.arange(c * Lc, (c + 1) * Lc), d)
        q_buf = torch.empty((B, Lc, H, d), dtype=cdt, device=DEV)
        out = torch.empty((B, Lc, H, d), dtype=torch.bfloat16, device=DEV)
        vis_len = binding.stream_self_attention_step(cache, c, q.to(DEV), k.to(DEV), v.to(DEV), q_buf, out, gqd, gkd,
                                                     ang.to(DEV), eps, scale, style, scope, workspace=ws)
        torch.cuda.synchronize()
        # oracle: prologue in fp64, rounded once to the bf16 the cache stores; logical window
        qs = oracle.round_to(_oracle_prologue(q, gq, eps, ang_q, style, inner), rnd)
        kstar[c] = oracle.round_to(_oracle_prologue(k, gk, eps, None if after_cache else ang, style, inner), rnd)
        vals[c] = oracle.round_to(widen(v).reshape(v.shape), rnd)
        vis = model.visible_chunks()
        assert vis_len == n
        K = np.concatenate([kstar[x] for x in vis], axis=1)
        if after_cache:  # rotated visible keys enter attention as bf16, like the cache's keys
            K = oracle.round_to(oracle.rope(K, ang.double().numpy(), style), "bf16")
        V = np.concatenate([vals[x] for x in vis], axis=1)
        if rows_per_chunk is None:
            ref = oracle.attention(qs, K, V, scale)
            got = out
        else:
            rows = sample_rows(B, Lc, H, rows_per_chunk, seed=c)
            ref = oracle.attention(qs, K, V, scale, rows=rows)
            got = out.reshape(-1, d)[torch.from_numpy(rows).to(DEV)]
        results.append(assert_attention_close(got, ref, f"chunk {c}"))
        # the cache holds V (rounded to the cache type) at the model's slot, bit for bit
        s0 = model.slot_of(c)
        got_v = widen(cache.v[:, s0:s0 + Lc]).reshape(v.shape)
        assert np.array_equal(got_v, vals[c])
    return results


def test_streaming_small_with_sink_full_compare():
    # sink 1 chunk + window 3 chunks: fill (chunks 0-3) and several evictions (4-8)
    _streaming_run(B=2, Lc=100, H=4, d=128, sink=100, window=300, n_chunks=9, rows_per_chunk=None, seed0=4000)


def test_streaming_interleaved_rope_d64():
    _streaming_run(B=1, Lc=64, H=3, d=64, sink=0, window=192, n_chunks=5, rows_per_chunk=None, seed0=4100,
                   style=binding.SA_ROPE_INTERLEAVED)


def test_streaming_after_cache_rope_with_sink():
    # after-cache RoPE, sink 1 chunk + window 3 chunks: fill and evictions; the sink's position
    # moves next to the window each step
    _streaming_run(B=2, Lc=100, H=4, d=128, sink=100, window=300, n_chunks=8, rows_per_chunk=None, seed0=4200,
                   after_cache=True)


def test_streaming_after_cache_interleaved_d64_no_sink():
    _streaming_run(B=1, Lc=64, H=3, d=64, sink=0, window=192, n_chunks=5, rows_per_chunk=None, seed0=4300,
                   style=binding.SA_ROPE_INTERLEAVED, after_cache=True)


def test_streaming_inner_scope_norm():
    # inner-scope Q/K RMSNorm (one RMS over all heads of a token), before-cache RoPE
    _streaming_run(B=1, Lc=96, H=6, d=128, sink=0, window=288, n_chunks=4, rows_per_chunk=None, seed0=4400,
                   inner=True)


def test_streaming_inner_scope_after_cache_d64():
    _streaming_run(B=2, Lc=50, H=4, d=64, sink=50, window=100, n_chunks=5, rows_per_chunk=None, seed0=4500,
                   inner=True, after_cache=True)


def test_streaming_after_cache_full_size_with_sink():
    """After-cache RoPE at full size: chunks of 1785 tokens x 40 heads x 128, cache of one sink
    chunk + a 3-chunk window (7140 keys), chunks 0-5 (fill, then eviction); sampled rows."""
    w = synthetic.WORKLOADS["stream_self_1785x4"]
    print(f"[case] after-cache {w}", flush=True)
    _streaming_run(B=1, Lc=w.chunk, H=w.Hq, d=w.d, sink=w.chunk, window=w.window - w.chunk, n_chunks=6,
                   rows_per_chunk=512, seed0=w.seed + 50, after_cache=True, workspace=True)


def test_streaming_fp8_cache_with_sink():
    # FP8 E4M3 cache: Q and K rounded by the prologue, V by the append; sink + 3-chunk window
    _streaming_run(B=2, Lc=100, H=4, d=128, sink=100, window=300, n_chunks=7, rows_per_chunk=None, seed0=4600,
                   fp8=True)


def test_streaming_fp8_cache_full_size():
    """FP8 streaming at full size: 1785 x 40 x 128 chunks, 4-chunk cache; sampled rows."""
    w = synthetic.WORKLOADS["stream_self_1785x4"]
    print(f"[case] fp8 {w}", flush=True)
    _streaming_run(B=1, Lc=w.chunk, H=w.Hq, d=w.d, sink=0, window=w.window, n_chunks=6, rows_per_chunk=512,
                   seed0=w.seed + 70, fp8=True, workspace=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("inner", [False, True])
def test_qk_norm_rope_fp8_output(d, inner):
    B, L, H = 2, 23, 4
    g = torch.Generator().manual_seed(300 + d + inner)
    q = synthetic.normal((B, L, H, d), "bf16", g, 2.0)
    k = synthetic.normal((B, L, H, d), "bf16", g, 0.5)
    gq = synthetic.norm_weight(H * d if inner else d, g)
    gk = synthetic.norm_weight(H * d if inner else d, g)
    ang = synthetic.rope_angles(np.arange(70, 70 + L), d)
    qo = torch.empty((B, L, H, d), dtype=torch.float8_e4m3fn, device=DEV)
    ko = torch.empty_like(qo)
    binding.qk_norm_rope(q.to(DEV), qo, k.to(DEV), ko, gq.to(DEV), gk.to(DEV), ang.to(DEV), 1e-6,
                         binding.SA_NORM_INNER if inner else binding.SA_NORM_HEAD, binding.SA_ROPE_SPLIT)
    torch.cuda.synchronize()
    assert_within_one_ulp(qo, _oracle_prologue(q, gq, 1e-6, ang, oracle.SPLIT, inner), "q e4m3")
    assert_within_one_ulp(ko, _oracle_prologue(k, gk, 1e-6, ang, oracle.SPLIT, inner), "k e4m3")


@pytest.mark.parametrize("cache_dtype", [torch.float8_e4m3fn, torch.float16])
def test_kv_cache_append_casts_bit_exact(cache_dtype):
    """bf16 chunks into an E4M3 or f16 cache: each value rounded to nearest even, bit for bit
    (the oracle rounds the same bf16 values from their exact fp64 form); other rows untouched."""
    B, Lc, H, d, sink, window = 2, 16, 3, 64, 16, 48
    S = sink + window
    name = "e4m3" if cache_dtype == torch.float8_e4m3fn else "f16"
    cache = torch.zeros((B, S, H, d), dtype=cache_dtype, device=DEV)
    model = RollingCacheModel(Lc, sink, window)
    expect = np.zeros((B, S, H, d))
    g = torch.Generator().manual_seed(17)
    for c in range(6):
        v = synthetic.normal((B, Lc, H, d), "bf16", g, 3.0)
        v[0, 0, 0, :4] = torch.tensor([300.0, -470.0, 1e-4, 65504.0 * 2]).to(torch.bfloat16)  # saturation, subnormal, overflow
        binding.kv_cache_append(None, v.to(DEV), None, cache, c, sink, window)
        s0 = model.write(c)
        expect[:, s0:s0 + Lc] = oracle.round_to(widen(v).reshape(v.shape), name)
    torch.cuda.synchronize()
    got = widen(cache).reshape(expect.shape)
    same = (got == expect) | (np.isnan(got) & np.isnan(expect)) | (np.isinf(got) & np.isinf(expect) & (np.sign(got) == np.sign(expect)))
    assert same.all(), np.argwhere(~same)[:5]


def test_streaming_f16_v_cache_equals_bf16_cache():
    """A cache that keeps V in f16 (bf16 K) gives bit-identical streaming outputs to a bf16 cache
    (the f16 cache takes the two-launch prologue, the bf16 one the one-launch prologue; both
    attend on the same normalised queries)."""
    B, Lc, H, d, sink, window = 1, 120, 4, 128, 120, 360
    outs = {}
    for v_dtype in (None, torch.float16):
        cache = binding.BlockKVCache(B, H, d, Lc, sink, window, device=DEV, v_dtype=v_dtype)
        g = torch.Generator().manual_seed(4700)
        gq, gk = synthetic.norm_weight(d, g).to(DEV), synthetic.norm_weight(d, g).to(DEV)
        res = []
        for c in range(6):
            gc = torch.Generator().manual_seed(4700 + c)
            q, k, v = (synthetic.normal((B, Lc, H, d), "bf16", gc).to(DEV) for _ in range(3))
            ang = synthetic.rope_angles(np.arange(c * Lc, (c + 1) * Lc), d).to(DEV)
            q_buf = torch.empty_like(q)
            out = torch.empty_like(q)
            binding.stream_self_attention_step(cache, c, q, k, v, q_buf, out, gq, gk, ang, 1e-6, d ** -0.5)
            res.append(out.clone())
        torch.cuda.synchronize()
        outs[v_dtype] = res
    for c, (a, b) in enumerate(zip(outs[None], outs[torch.float16])):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"chunk {c}"


def test_streaming_self_attention_full_size():
    """Streaming self-attention at full size, in the benchmark's configuration (one-launch
    prologue, attention with a workspace, so the full cache's 280-block grid runs balanced):
    chunks of 1785 tokens x 40 heads x 128, rolling cache of 4 chunks (7140 keys), chunks 0-5
    (fill, then eviction); sampled rows each chunk."""
    w = synthetic.WORKLOADS["stream_self_1785x4"]
    print(f"[case] {w}", flush=True)
    _streaming_run(B=1, Lc=w.chunk, H=w.Hq, d=w.d, sink=0, window=w.window, n_chunks=6, rows_per_chunk=512,
                   seed0=w.seed, workspace=True)


def test_cross_attention_full_size():
    """Cross-attention: B=2, 40 heads, 1785 queries with Q RMSNorm (no RoPE) over a static
    512-token K/V context; sampled rows."""
    w = synthetic.WORKLOADS["cross_1785x512"]
    print(f"[case] {w}", flush=True)
    g = torch.Generator().manual_seed(w.seed)
    q = synthetic.normal((w.B, w.Lq, w.Hq, w.d), "bf16", g)
    k = synthetic.normal((w.B, w.Lk, w.Hkv, w.d), "bf16", g)
    v = synthetic.normal((w.B, w.Lk, w.Hkv, w.d), "bf16", g)
    gq = synthetic.norm_weight(w.d, g)
    qd = q.to(DEV)
    qs = torch.empty_like(qd)
    binding.qk_norm_rope(qd, qs, None, None, gq.to(DEV), None, None, 1e-6, binding.SA_NORM_HEAD,
                         binding.SA_ROPE_NONE)
    out = torch.empty_like(qd)
    binding.attn_forward(qs, k.to(DEV), v.to(DEV), out, w.scale, False)
    torch.cuda.synchronize()
    q_ref = oracle.round_to(_oracle_prologue(q, gq, 1e-6, None, 0), "bf16")
    assert_within_one_ulp(qs, _oracle_prologue(q, gq, 1e-6, None, 0), "q norm")
    rows = sample_rows(w.B, w.Lq, w.Hq, 4096, seed=3)
    ref = oracle.attention(q_ref, widen(k).reshape(k.shape), widen(v).reshape(v.shape), w.scale, rows=rows)
    assert_attention_close(out.reshape(-1, w.d)[torch.from_numpy(rows).to(DEV)], ref, w.name)


FUSED_QNORM_CASES = [
    # name, B, Lq, Lk, Hq, Hkv, d, q/k dtype, v dtype, window, workspace
    ("qnorm_bf16_d128_ragged", 2, 300, 200, 4, 2, 128, "bf16", "bf16", (-1, -1), False),
    ("qnorm_f16_d64", 1, 257, 513, 3, 3, 64, "f16", "f16", (-1, -1), False),
    ("qnorm_window_bf16_d128", 1, 400, 400, 2, 2, 128, "bf16", "bf16", (100, 0), False),
    ("qnorm_bf16qk_f16v_d128", 1, 200, 300, 4, 4, 128, "bf16", "f16", (-1, -1), False),
    ("qnorm_wide_grid_bf16_d128", 1, 4000, 333, 64, 16, 128, "bf16", "bf16", (-1, -1), False),
    ("qnorm_balanced_stream_shape", 1, 1785, 7140, 40, 40, 128, "bf16", "bf16", (-1, -1), True),
]


@pytest.mark.parametrize("case", FUSED_QNORM_CASES, ids=[c[0] for c in FUSED_QNORM_CASES])
def test_attention_with_fused_query_norm_matches_oracle(case):
    """attn_forward_qnorm: each query row is RMS-normalised (head scope) and rounded once as it
    is loaded; compared with the oracle's normalised query, rounded once, then attention."""
    name, B, Lq, Lk, Hq, Hkv, d, qk_dt, v_dt, window, use_ws = case
    print(f"[case] {case}", flush=True)
    g = torch.Generator().manual_seed(zlib_seed(name))
    q = synthetic.normal((B, Lq, Hq, d), qk_dt, g, 2.0)
    k = synthetic.normal((B, Lk, Hkv, d), qk_dt, g)
    v = synthetic.normal((B, Lk, Hkv, d), v_dt, g)
    gq = synthetic.norm_weight(d, g)
    qd = q.to(DEV)
    q_before = qd.clone()
    out = torch.empty_like(qd)
    ws = binding.attn_workspace(d) if use_ws else None
    binding.attn_forward_qnorm(qd, k.to(DEV), v.to(DEV), out, d ** -0.5, gq.to(DEV), 1e-6, workspace=ws,
                               window=window)
    torch.cuda.synchronize()
    assert torch.equal(qd.view(torch.int16), q_before.view(torch.int16)), "q must not be modified"
    q_ref = oracle.round_to(_oracle_prologue(q, gq, 1e-6, None, 0), qk_dt)
    win = None if window == (-1, -1) else window
    rows = sample_rows(B, Lq, Hq, 3000, seed=5) if B * Lq * Hq > 20000 else None
    ref = oracle.attention(q_ref, widen(k).reshape(k.shape), widen(v).reshape(v.shape), d ** -0.5, rows=rows,
                           window=win)
    got = out if rows is None else out.reshape(-1, d)[torch.from_numpy(rows).to(DEV)]
    assert_attention_close(got, ref, name)


def test_cross_attention_fused_query_norm_full_size():
    """The cross-attention configuration (B=2, 40 heads, 1785 queries over a 512-token context)
    with the Q RMSNorm fused into the attention: sampled rows against the oracle, and every
    output within the attention bounds of the two-kernel path (prologue, then attention)."""
    w = synthetic.WORKLOADS["cross_1785x512"]
    print(f"[case] fused {w}", flush=True)
    g = torch.Generator().manual_seed(w.seed)
    q = synthetic.normal((w.B, w.Lq, w.Hq, w.d), "bf16", g)
    k = synthetic.normal((w.B, w.Lk, w.Hkv, w.d), "bf16", g)
    v = synthetic.normal((w.B, w.Lk, w.Hkv, w.d), "bf16", g)
    gq = synthetic.norm_weight(w.d, g)
    qd, kd, vd, gd = q.to(DEV), k.to(DEV), v.to(DEV), gq.to(DEV)
    fused = torch.empty_like(qd)
    binding.attn_forward_qnorm(qd, kd, vd, fused, w.scale, gd, 1e-6)
    qs = torch.empty_like(qd)
    binding.qk_norm_rope(qd, qs, None, None, gd, None, None, 1e-6, binding.SA_NORM_HEAD, binding.SA_ROPE_NONE)
    two = torch.empty_like(qd)
    binding.attn_forward(qs, kd, vd, two, w.scale, False)
    torch.cuda.synchronize()
    diff = (fused.float() - two.float()).abs()
    assert diff.max().item() <= 8e-3 and diff.mean().item() <= 1e-4, (diff.max().item(), diff.mean().item())
    q_ref = oracle.round_to(_oracle_prologue(q, gq, 1e-6, None, 0), "bf16")
    rows = sample_rows(w.B, w.Lq, w.Hq, 4096, seed=4)
    ref = oracle.attention(q_ref, widen(k).reshape(k.shape), widen(v).reshape(v.shape), w.scale, rows=rows)
    assert_attention_close(fused.reshape(-1, w.d)[torch.from_numpy(rows).to(DEV)], ref, "fused " + w.name)


def zlib_seed(name: str) -> int:
    import zlib
    return zlib.crc32(name.encode()) % 10000


@pytest.mark.parametrize("d,style,after,out8,with_q", [
    (128, binding.SA_ROPE_SPLIT, False, False, False),
    (64, binding.SA_ROPE_INTERLEAVED, False, False, True),
    (128, binding.SA_ROPE_SPLIT, True, False, False),
    (128, binding.SA_ROPE_SPLIT, False, True, False),
    (64, binding.SA_ROPE_NONE, False, False, False),
    (128, binding.SA_ROPE_SPLIT, False, True, True),   # the FP8 streaming step's prologue
])
def test_qk_norm_rope_v_matches_oracle(d, style, after, out8, with_q):
    """The one-launch chunk prologue: keys normalised (rotated unless after-cache) within one ulp
    of the oracle, values copied bit for bit (or rounded to E4M3 like the append), queries as in
    qk_norm_rope, and the chunk's cos/sin table within a few fp32 ulps of cos/sin of the angles;
    rows outside the slot untouched."""
    B, L, Hq, Hkv, S, s0 = 2, 29, 6, 3, 96, 32
    print(f"[case] d={d} style={style} after={after} out8={out8} with_q={with_q}", flush=True)
    g = torch.Generator().manual_seed(500 + d + style + 2 * after + 4 * out8)
    q = synthetic.normal((B, L, Hq, d), "bf16", g, 2.0)
    k = synthetic.normal((B, L, Hkv, d), "bf16", g, 0.5)
    v = synthetic.normal((B, L, Hkv, d), "bf16", g, 3.0)
    gq, gk = synthetic.norm_weight(d, g), synthetic.norm_weight(d, g)
    ang = synthetic.rope_angles(np.arange(900, 900 + L), d) if style else None
    cdt = torch.float8_e4m3fn if out8 else torch.bfloat16
    ck = torch.zeros((B, S, Hkv, d), dtype=cdt, device=DEV)
    cv = torch.zeros_like(ck)
    cs = torch.full((L, d), -7.0, device=DEV) if style else None
    qo = torch.empty((B, L, Hq, d), dtype=cdt, device=DEV) if with_q else None
    flag = binding.SA_ROPE_AFTER_CACHE if (after and style) else 0
    binding.qk_norm_rope_v(k.to(DEV), ck[:, s0:], v.to(DEV), cv[:, s0:], gk.to(DEV), None if ang is None else ang.to(DEV),
                           1e-6, binding.SA_NORM_HEAD, style | flag, rope_cs_out=cs, k_out_bstride=S * Hkv * d,
                           v_out_bstride=S * Hkv * d, q_in=q.to(DEV) if with_q else None, q_out=qo,
                           gamma_q=gq.to(DEV) if with_q else None)
    torch.cuda.synchronize()
    rnd = "e4m3" if out8 else "bf16"
    kref = _oracle_prologue(k, gk, 1e-6, None if (after or not style) else ang, style)
    assert_within_one_ulp(ck[:, s0:s0 + L].contiguous(), kref, "k")
    vref = oracle.round_to(widen(v).reshape(v.shape), rnd)
    got_v = widen(cv[:, s0:s0 + L].contiguous()).reshape(vref.shape)
    assert np.array_equal(got_v, vref)
    for t in (ck, cv):  # rows outside the slot stay zero
        assert not t[:, :s0].float().abs().sum().item() and not t[:, s0 + L:].float().abs().sum().item()
    if with_q:
        assert_within_one_ulp(qo, _oracle_prologue(q, gq, 1e-6, ang, style), "q")
    if style:
        a64 = ang.double().numpy()
        tab = cs.double().cpu().numpy()
        assert np.abs(tab[:, :d // 2] - np.cos(a64)).max() < 4e-7
        assert np.abs(tab[:, d // 2:] - np.sin(a64)).max() < 4e-7


def _two_launch_step(cache, c, q, k, v, q_buf, out, gq, gk, ang, scale, style):
    """The chunk step composed from the separate calls: qk_norm_rope (Q -> q_buf, K -> cache
    slot), kv_cache_append (V), kv_cache_rope (after-cache RoPE), attention on q_buf."""
    slot, visible = cache.before_update(c)
    after = cache.k_rot is not None
    q_ang = ang[visible - cache.chunk_len:visible] if after else ang
    flag = binding.SA_ROPE_AFTER_CACHE if after else 0
    binding.qk_norm_rope(q, q_buf, k, cache.k[:, slot:], gq, gk, q_ang, 1e-6, binding.SA_NORM_HEAD, style | flag,
                         k_out_bstride=cache.capacity * cache.Hkv * cache.d)
    binding.kv_cache_append(None, v, None, cache.v, c, cache.sink_size, cache.window_size)
    keys = cache.k
    if after:
        binding.kv_cache_rope(cache.k, cache.k_rot, ang, c, cache.chunk_len, cache.sink_size, cache.window_size,
                              style)
        keys = cache.k_rot
    binding.attn_forward_kvstride(q_buf, keys, cache.v, out, visible, scale, False)
    cache.after_update(c)


@pytest.mark.parametrize("style,after", [(binding.SA_ROPE_SPLIT, False), (binding.SA_ROPE_INTERLEAVED, False),
                                         (binding.SA_ROPE_SPLIT, True)])
def test_streaming_routes_agree(style, after):
    """stream_self_attention_step's routes through fill and eviction: the default one-launch
    prologue (qk_norm_rope_v: Q, K and V in one launch) equals the two-launch composition
    (qk_norm_rope -> kv_cache_append) bit for bit in the caches and the outputs; the route with
    the query norm and RoPE inside the attention (query_in_attention) leaves the same caches and
    outputs within the attention bounds of the others."""
    B, Lc, H, d, sink, window = 1, 96, 4, 128, 96, 192
    print(f"[case] style={style} after={after}", flush=True)
    caches = [binding.BlockKVCache(B, H, d, Lc, sink, window, device=DEV, after_cache_rope=after) for _ in range(3)]
    for cch in caches:
        cch.k.zero_()
        cch.v.zero_()
    g = torch.Generator().manual_seed(77)
    gq, gk = synthetic.norm_weight(d, g).to(DEV), synthetic.norm_weight(d, g).to(DEV)
    for c in range(6):
        gc = torch.Generator().manual_seed(7000 + c)
        q, k, v = (synthetic.normal((B, Lc, H, d), "bf16", gc).to(DEV) for _ in range(3))
        n = min((c + 1) * Lc, sink + window)
        ang = synthetic.rope_angles(np.arange(n) if after else np.arange(c * Lc, (c + 1) * Lc), d).to(DEV)
        outs = [torch.empty_like(q) for _ in range(3)]
        bufs = [torch.empty_like(q) for _ in range(3)]
        binding.stream_self_attention_step(caches[0], c, q, k, v, bufs[0], outs[0], gq, gk, ang, 1e-6, d ** -0.5,
                                           style, binding.SA_NORM_HEAD)
        _two_launch_step(caches[1], c, q, k, v, bufs[1], outs[1], gq, gk, ang, d ** -0.5, style)
        binding.stream_self_attention_step(caches[2], c, q, k, v, bufs[2], outs[2], gq, gk, ang, 1e-6, d ** -0.5,
                                           style, binding.SA_NORM_HEAD, query_in_attention=True)
        torch.cuda.synchronize()
        for i in (1, 2):
            assert torch.equal(caches[0].k.view(torch.int16), caches[i].k.view(torch.int16)), (c, i)
            assert torch.equal(caches[0].v.view(torch.int16), caches[i].v.view(torch.int16)), (c, i)
        assert torch.equal(bufs[0].view(torch.int16), bufs[1].view(torch.int16)), c
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), c
        diff = (outs[0].float() - outs[2].float()).abs()
        assert diff.max().item() <= 8e-3 and diff.mean().item() <= 1e-4, (c, diff.max().item(), diff.mean().item())


@pytest.mark.parametrize("v_dtype", [None, torch.float16], ids=["one_launch", "two_launch"])
def test_streaming_without_norm_or_rope(v_dtype):
    """The streaming step with neither RMSNorm nor RoPE (no weights, no angles), on both prologue
    routes: the cache holds the raw keys and values, and each chunk's output is plain attention
    of the raw queries over the visible chunks (oracle rolling-cache model), through eviction."""
    B, Lc, H, d, sink, window = 2, 48, 2, 64, 48, 96
    print(f"[case] no norm, no rope, v_dtype={v_dtype}", flush=True)
    cache = binding.BlockKVCache(B, H, d, Lc, sink, window, device=DEV, v_dtype=v_dtype)
    model = RollingCacheModel(Lc, sink, window)
    keys, vals = {}, {}
    for c in range(6):
        gc = torch.Generator().manual_seed(6100 + c)
        q, k, v = (synthetic.normal((B, Lc, H, d), "bf16", gc) for _ in range(3))
        q_buf = torch.empty((B, Lc, H, d), dtype=torch.bfloat16, device=DEV)
        out = torch.empty_like(q_buf)
        vis_len = binding.stream_self_attention_step(cache, c, q.to(DEV), k.to(DEV), v.to(DEV), q_buf, out, None, None,
                                                     None, 1e-6, d ** -0.5, binding.SA_ROPE_NONE, binding.SA_NORM_NONE)
        torch.cuda.synchronize()
        model.write(c)
        keys[c], vals[c] = widen(k).reshape(k.shape), widen(v).reshape(v.shape)
        vis = model.visible_chunks()
        assert vis_len == model.visible_len()
        ref = oracle.attention(widen(q).reshape(q.shape), np.concatenate([keys[x] for x in vis], axis=1),
                               np.concatenate([vals[x] for x in vis], axis=1), d ** -0.5)
        assert_attention_close(out, ref, f"chunk {c}")
        s0 = model.slot_of(c)
        assert np.array_equal(widen(cache.k[:, s0:s0 + Lc]).reshape(k.shape), keys[c])
        assert np.array_equal(widen(q_buf).reshape(q.shape), widen(q).reshape(q.shape))


@pytest.mark.parametrize("B,Lq,S,H,d,style,mode,rows_n", [
    (2, 300, 130, 4, 128, binding.SA_ROPE_SPLIT, "after", None),
    (1, 97, 65, 3, 64, binding.SA_ROPE_INTERLEAVED, "after", None),
    (2, 130, 200, 2, 128, binding.SA_ROPE_SPLIT, "before", None),
    (2, 200, 64, 4, 64, binding.SA_ROPE_NONE, "none", None),
    (2, 1785, 512, 40, 128, binding.SA_ROPE_SPLIT, "after", 4096),   # the cross-attention workload's shape
], ids=["after_split_d128", "after_interleaved_d64", "before_split_d128", "norm_only_d64", "after_full_size"])
def test_cross_attention_context_cache_rope_scopes(B, Lq, S, H, d, style, mode, rows_n):
    """Cross-attention over a static context cache built once by context_kv (keys RMS-normalised;
    rotated there for before-cache RoPE, left unrotated for after-cache RoPE), then one query
    chunk through cross_attention_step, called twice (the cache is reused and stays unrotated).
    After-cache RoPE rotates all S cached keys with the cache-relative rows 0 .. S-1 of the
    context angle table and the queries with their own rows (here positions S + i, right after
    the context). Oracle: RMSNorm, RoPE in fp64, each rounded once to the bf16 that is stored or
    attended; every row (sampled rows at full size)."""
    print(f"[case] B={B} Lq={Lq} S={S} H={H} d={d} style={style} mode={mode}", flush=True)
    eps, scale = 1e-6, d ** -0.5
    g = torch.Generator().manual_seed(8100 + S + d)
    q = synthetic.normal((B, Lq, H, d), "bf16", g)
    k = synthetic.normal((B, S, H, d), "bf16", g)
    v = synthetic.normal((B, S, H, d), "bf16", g)
    gq, gk = synthetic.norm_weight(d, g), synthetic.norm_weight(d, g)
    ctx_ang = synthetic.rope_angles(np.arange(S), d)
    q_ang = synthetic.rope_angles(np.arange(S, S + Lq), d)
    ck = torch.full((B, S, H, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    cv = torch.full_like(ck, float("nan"))
    binding.context_kv(k.to(DEV), v.to(DEV), ck, cv, gk.to(DEV), eps,
                       angles=ctx_ang.to(DEV) if mode == "before" else None, rope_style=style)
    ck_before = ck.clone()
    k_rot = torch.empty_like(ck) if mode == "after" else None
    q_buf = torch.empty((B, Lq, H, d), dtype=torch.bfloat16, device=DEV)
    outs = []
    for _ in range(2):
        out = torch.full((B, Lq, H, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        binding.cross_attention_step(ck, cv, q.to(DEV), out, gq.to(DEV), eps, scale, q_buf=q_buf,
                                     q_angles=q_ang.to(DEV) if mode != "none" else None,
                                     context_angles=ctx_ang.to(DEV) if mode == "after" else None, k_rot=k_rot,
                                     rope_style=style)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(ck.view(torch.int16), ck_before.view(torch.int16))   # the cache is never rotated in place
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    # the context cache: normalised keys (rotated for before-cache RoPE), values bit for bit
    kcache_ref = _oracle_prologue(k, gk, eps, ctx_ang if mode == "before" else None, style)
    assert_within_one_ulp(ck, kcache_ref, "context keys")
    assert np.array_equal(widen(cv).reshape(v.shape), widen(v).reshape(v.shape))
    K = widen(ck).reshape(k.shape)   # what the cache holds
    if mode == "after":
        rot = oracle.rope(K, ctx_ang.double().numpy(), style)
        assert_within_one_ulp(k_rot, rot, "rotated keys")
        K = oracle.round_to(rot, "bf16")
    Q = oracle.round_to(_oracle_prologue(q, gq, eps, q_ang if mode != "none" else None, style), "bf16")
    V = widen(v).reshape(v.shape)
    if rows_n is None:
        assert_attention_close(outs[0], oracle.attention(Q, K, V, scale), mode)
    else:
        rows = sample_rows(B, Lq, H, rows_n, seed=5)
        ref = oracle.attention(Q, K, V, scale, rows=rows)
        assert_attention_close(outs[0].reshape(-1, d)[torch.from_numpy(rows).to(DEV)], ref, mode)


@pytest.mark.parametrize("after", [False, True], ids=["before_cache_rope", "after_cache_rope"])
def test_cache_reset_matches_fresh_cache(after):
    """A cache used by one stream (fill and eviction), then restarted at chunk 0 by a second
    stream, gives that stream the outputs of a fresh cache bit for bit (stale rows of the first
    stream are never visible), and matches the oracle's rolling-cache model of the second stream."""
    B, Lc, H, d, sink, window = 1, 64, 4, 128, 64, 128
    eps, scale = 1e-6, d ** -0.5
    print(f"[case] reset after={after}", flush=True)
    used = binding.BlockKVCache(B, H, d, Lc, sink, window, device=DEV, after_cache_rope=after)
    fresh = binding.BlockKVCache(B, H, d, Lc, sink, window, device=DEV, after_cache_rope=after)
    g = torch.Generator().manual_seed(9100)
    gq, gk = synthetic.norm_weight(d, g).to(DEV), synthetic.norm_weight(d, g).to(DEV)

    def chunk(seed, c):
        gc = torch.Generator().manual_seed(seed + c)
        return [synthetic.normal((B, Lc, H, d), "bf16", gc) for _ in range(3)]

    def angles(c):
        n = min((c + 1) * Lc, sink + window)
        return synthetic.rope_angles(np.arange(n) if after else np.arange(c * Lc, (c + 1) * Lc), d)

    def run(cache, seed, c):
        q, k, v = chunk(seed, c)
        q_buf = torch.empty((B, Lc, H, d), dtype=torch.bfloat16, device=DEV)
        out = torch.empty_like(q_buf)
        binding.stream_self_attention_step(cache, c, q.to(DEV), k.to(DEV), v.to(DEV), q_buf, out, gq, gk,
                                           angles(c).to(DEV), eps, scale)
        return out

    for c in range(5):              # first stream: fill, then two evictions
        run(used, 500, c)
    used.reset()
    model = RollingCacheModel(Lc, sink, window)
    kstar, vals = {}, {}
    for c in range(4):              # second stream on both caches
        o_used, o_fresh = run(used, 700, c), run(fresh, 700, c)
        torch.cuda.synchronize()
        assert torch.equal(o_used.view(torch.int16), o_fresh.view(torch.int16)), c
        q, k, v = chunk(700, c)
        model.write(c)
        n = model.visible_len()
        ang = angles(c)
        ang_q = ang[n - Lc:] if after else ang
        qs = oracle.round_to(_oracle_prologue(q, gq.cpu(), eps, ang_q, binding.SA_ROPE_SPLIT), "bf16")
        kstar[c] = oracle.round_to(_oracle_prologue(k, gk.cpu(), eps, None if after else ang, binding.SA_ROPE_SPLIT),
                                   "bf16")
        vals[c] = widen(v).reshape(v.shape)
        K = np.concatenate([kstar[x] for x in model.visible_chunks()], axis=1)
        if after:
            K = oracle.round_to(oracle.rope(K, ang.double().numpy(), binding.SA_ROPE_SPLIT), "bf16")
        V = np.concatenate([vals[x] for x in model.visible_chunks()], axis=1)
        assert_attention_close(o_used, oracle.attention(qs, K, V, scale), f"restarted chunk {c}")
