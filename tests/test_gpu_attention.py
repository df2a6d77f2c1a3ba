"""GPU parity of attn_forward / attn_forward_f16 / attn_forward_kvstride against the fp64 oracle.

Sizes span several 128-query and 64-key tiles with ragged tails; the full-size workloads are
checked on sampled rows (the oracle computes each sampled row exactly over all its keys)."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from head_attention_streaming_amd import binding, synthetic
from parity import assert_attention_close, sample_rows, widen

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(q, k, v, scale, causal, dtype):
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.empty_like(qd)
    if dtype == "bf16":
        binding.attn_forward(qd, kd, vd, out, scale, causal)
    else:
        binding.attn_forward_f16(qd, kd, vd, out, scale, causal)
    torch.cuda.synchronize()
    return out


CASES = [
    # name, B, Lq, Lk, Hq, Hkv, d, dtype, causal
    ("noncausal_257_bf16_d128", 1, 257, 257, 8, 8, 128, "bf16", False),
    ("ragged_gqa_f16_d64", 2, 200, 333, 4, 2, 64, "f16", False),
    ("causal_square_f16_d64", 2, 190, 190, 3, 3, 64, "f16", True),
    ("causal_rect_bf16_d128", 1, 100, 300, 2, 2, 128, "bf16", True),
    ("causal_square_bf16_d128", 1, 300, 300, 2, 2, 128, "bf16", True),
    ("single_query_single_key", 1, 1, 1, 1, 1, 128, "bf16", False),
    ("tile_plus_one", 1, 129, 65, 2, 1, 128, "bf16", False),
    ("tile_minus_one", 1, 127, 63, 2, 2, 64, "bf16", False),
    ("mqa_bf16_d128", 1, 150, 200, 8, 1, 128, "bf16", False),
    ("f16_d128", 1, 200, 250, 2, 2, 128, "f16", False),
    ("bf16_d64_batch", 3, 130, 70, 2, 2, 64, "bf16", False),
    ("one_key_many_queries", 2, 300, 1, 2, 2, 128, "bf16", False),
    ("causal_one_row_f16", 1, 1, 97, 2, 2, 64, "f16", True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_attention_matches_oracle(case):
    name, B, Lq, Lk, Hq, Hkv, d, dtype, causal = case
    print(f"[case] {case}", flush=True)
    q, k, v = synthetic.attention_inputs(B, Lq, Lk, Hq, Hkv, d, dtype, seed=zlib.crc32(name.encode()) % 10000)
    scale = d ** -0.5
    out = _run(q, k, v, scale, causal, dtype)
    ref = oracle.attention(widen(q).reshape(q.shape), widen(k).reshape(k.shape), widen(v).reshape(v.shape),
                           scale, causal)
    assert_attention_close(out, ref, name)


def test_causal_2048_f16_full():
    """Causal MHA [2, 2048, 8, 64] fp16, scale 1/8: every output element."""
    w = synthetic.WORKLOADS["causal_2048_f16"]
    print(f"[case] {w}", flush=True)
    q, k, v = synthetic.attention_inputs(w.B, w.Lq, w.Lk, w.Hq, w.Hkv, w.d, w.dtype, w.seed)
    out = _run(q, k, v, w.scale, True, "f16")
    ref = oracle.attention(widen(q).reshape(q.shape), widen(k).reshape(k.shape), widen(v).reshape(v.shape),
                           w.scale, True)
    assert_attention_close(out, ref, w.name)


def test_noncausal_20480_bf16_sampled_rows():
    """Long non-causal MHA [1, 20480, 56, 128] bf16: 2048+ sampled rows, each over all 20480 keys."""
    w = synthetic.WORKLOADS["mha_20480_bf16"]
    print(f"[case] {w}", flush=True)
    q, k, v = synthetic.attention_inputs(w.B, w.Lq, w.Lk, w.Hq, w.Hkv, w.d, w.dtype, w.seed)
    out = _run(q, k, v, w.scale, False, "bf16")
    rows = sample_rows(w.B, w.Lq, w.Hq, 2048, seed=7)
    ref = oracle.attention(widen(q).reshape(q.shape), widen(k).reshape(k.shape), widen(v).reshape(v.shape),
                           w.scale, False, rows=rows)
    got = out.reshape(-1, w.d)[torch.from_numpy(rows).to(DEV)]
    assert_attention_close(got, ref, w.name)


def test_peaky_softmax():
    q, k, v = synthetic.attention_inputs(1, 257, 257, 4, 4, 128, "bf16", seed=31, q_scale=8.0)
    out = _run(q, k, v, 128 ** -0.5, False, "bf16")
    ref = oracle.attention(widen(q).reshape(q.shape), widen(k).reshape(k.shape), widen(v).reshape(v.shape),
                           128 ** -0.5)
    assert_attention_close(out, ref, "peaky", ulp_floor=True)


def test_scores_rising_across_tiles_forces_rescale():
    # q = 1 on every feature; key j gets + t_j on every feature with t_j rising: the row maximum
    # moves into every new key tile, so each tile rescales the partial output.
    B, Lq, Lk, H, d = 1, 130, 517, 2, 128
    g = torch.Generator().manual_seed(77)
    q = torch.ones((B, Lq, H, d)).to(torch.bfloat16)
    t = torch.linspace(0.0, 3.0, Lk).view(1, Lk, 1, 1)
    k = (0.3 * torch.randn((B, Lk, H, d), generator=g) + t).to(torch.bfloat16)
    v = torch.randn((B, Lk, H, d), generator=g).to(torch.bfloat16)
    scale = 0.05
    out = _run(q, k, v, scale, False, "bf16")
    ref = oracle.attention(widen(q).reshape(q.shape), widen(k).reshape(k.shape), widen(v).reshape(v.shape), scale)
    assert_attention_close(out, ref, "rising")


def test_maximum_in_last_tile():
    q, k, v = synthetic.attention_inputs(1, 64, 300, 2, 2, 128, "bf16", seed=5)
    k[:, 297] = q[:, 10]  # key 297 (last, ragged tile) aligns with query 10: a dominant score
    k[:, 297] = (k[:, 297].float() * 3).to(torch.bfloat16)
    out = _run(q, k, v, 128 ** -0.5, False, "bf16")
    ref = oracle.attention(widen(q).reshape(q.shape), widen(k).reshape(k.shape), widen(v).reshape(v.shape),
                           128 ** -0.5)
    assert_attention_close(out, ref, "max_last_tile")


def test_kvstride_reads_prefix_of_larger_buffer():
    B, Lq, S, Lk, H, d = 2, 140, 400, 333, 3, 128
    q, k, v = synthetic.attention_inputs(B, Lq, S, H, H, d, "bf16", seed=9)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.empty_like(qd)
    binding.attn_forward_kvstride(qd, kd, vd, out, Lk, 0.1, False)
    torch.cuda.synchronize()
    ref = oracle.attention(widen(q).reshape(q.shape), widen(k[:, :Lk]).reshape(B, Lk, H, d),
                           widen(v[:, :Lk]).reshape(B, Lk, H, d), 0.1)
    assert_attention_close(out, ref, "kvstride")


def test_deterministic_repeat():
    q, k, v = synthetic.attention_inputs(1, 333, 1000, 4, 4, 128, "bf16", seed=11)
    a = _run(q, k, v, 0.09, False, "bf16")
    b = _run(q, k, v, 0.09, False, "bf16")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_empty_query_is_noop():
    q = torch.empty((1, 0, 2, 128), dtype=torch.bfloat16, device=DEV)
    k = torch.randn((1, 5, 2, 128), device=DEV).to(torch.bfloat16)
    binding.attn_forward(q, k, k, torch.empty_like(q), 0.1, False)
    torch.cuda.synchronize()


WIDE_CASES = [
    # at least four (batch, head, 256-row block) workgroups per CU: the 8-wave launch shape,
    # except causal rows of at most 4096 keys, which run 128-row blocks of 4 waves
    ("wide_ragged_bf16_d128", 1, 4000, 333, 64, 64, 128, "bf16", False),
    ("wide_causal_f16_d64", 2, 2000, 2000, 64, 64, 64, "f16", True),
    ("wide_gqa_causal_bf16_d128", 4, 1000, 1100, 64, 8, 128, "bf16", True),
    ("wide_long_causal_8wave_bf16_d128", 1, 4500, 4600, 64, 16, 128, "bf16", True),
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=[c[0] for c in WIDE_CASES])
def test_attention_wide_grid_sampled_rows(case):
    name, B, Lq, Lk, Hq, Hkv, d, dtype, causal = case
    print(f"[case] {case}", flush=True)
    q, k, v = synthetic.attention_inputs(B, Lq, Lk, Hq, Hkv, d, dtype, seed=zlib.crc32(name.encode()) % 10000)
    out = _run(q, k, v, d ** -0.5, causal, dtype)
    rows = sample_rows(B, Lq, Hq, 3000, seed=11)
    ref = oracle.attention(widen(q).reshape(q.shape), widen(k).reshape(k.shape), widen(v).reshape(v.shape),
                           d ** -0.5, causal, rows=rows)
    assert_attention_close(out.reshape(-1, d)[torch.from_numpy(rows).to(DEV)], ref, name)


def _shape_cases():
    """Shapes that land in each launch regime for this device's CU count: 8-wave workgroups with
    the keys split in two (at most one 128-row block per CU and at least 512 keys) or in four
    (d = 64, at least 1024 keys, no band; causal blocks paired when they would take two rounds),
    4-wave workgroups (short key loops, or between one and
    four 128-row blocks per CU)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks4 = (3 * cus) // 2          # 128-row blocks: 1.5 per CU -> 4-wave workgroups
    H4 = 64
    Lq4 = -(-blocks4 // H4) * 128 - 37
    return [
        # name, B, Lq, Lk, Hq, Hkv, d, dtype, causal, window
        ("split_ragged_bf16_d128", 1, 300, 1111, 4, 2, 128, "bf16", False, None),
        ("split_causal_f16_d64", 2, 600, 600, 3, 3, 64, "f16", True, None),
        ("short_keys_bf16_d128", 1, 100, 20, 2, 2, 128, "bf16", False, None),
        ("split_odd_tiles_bf16_d128", 2, 129, 513, 3, 1, 128, "bf16", False, None),
        ("split_window_bf16_d128", 1, 700, 700, 2, 2, 128, "bf16", False, (100, 30)),
        ("wave4_bf16_d128", 1, Lq4, 900, H4, 16, 128, "bf16", False, None),
        ("wave4_causal_f16_d64", 1, Lq4, Lq4, H4, H4, 64, "f16", True, None),
        ("wave4_window_bf16_d128", 1, Lq4, Lq4 + 50, H4, 8, 128, "bf16", False, (200, 0)),
        # d = 64, rows over >= 1024 keys: four key groups over 64-row blocks (causal, or few blocks),
        # ragged key tails, groups stepping past the block's last tile; a band keeps two groups
        ("split4_causal_f16_d64", 2, 1000, 1100, 3, 3, 64, "f16", True, None),
        ("split4_ragged_gqa_bf16_d64", 1, 333, 1500, 4, 2, 64, "bf16", False, None),
        ("split4_causal_odd_bf16_d64", 1, 1090, 1090, 2, 1, 64, "bf16", True, None),
        ("split_window_f16_d64", 1, 1100, 1100, 2, 2, 64, "f16", False, (256, 0)),
        # causal 64-row blocks that would need two rounds: paired blocks (i, n - 1 - i), an odd
        # block count (the middle block alone), ragged last block, bottom-right causal offset
        ("pair4_causal_odd_bf16_d64", 1, 33 * 64 - 21, 33 * 64 + 19, cus // 17, cus // 17, 64, "bf16", True, None),
        # paired blocks with a batch of two and grouped K/V heads (4 query heads per K/V head)
        ("pair4_causal_gqa_batch_f16_d64", 2, 18 * 64 - 30, 18 * 64 - 30, cus // 32, cus // 128, 64, "f16", True, None),
    ]


@pytest.mark.parametrize("idx", range(14))
def test_launch_regimes_sampled_rows(idx):
    name, B, Lq, Lk, Hq, Hkv, d, dtype, causal, window = _shape_cases()[idx]
    print(f"[case] {name} B={B} Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} d={d} {dtype} causal={causal} window={window}",
          flush=True)
    q, k, v = synthetic.attention_inputs(B, Lq, Lk, Hq, Hkv, d, dtype, seed=zlib.crc32(name.encode()) % 10000)
    scale = d ** -0.5
    if window is None:
        out = _run(q, k, v, scale, causal, dtype)
    else:
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        out = torch.empty_like(qd)
        binding.attn_forward_window(qd, kd, vd, out, scale, window)
        torch.cuda.synchronize()
    rows = sample_rows(B, Lq, Hq, 3000, seed=idx)
    ref = oracle.attention(widen(q).reshape(q.shape), widen(k).reshape(k.shape), widen(v).reshape(v.shape),
                           scale, causal, rows=rows, window=window)
    assert_attention_close(out.reshape(-1, d)[torch.from_numpy(rows).to(DEV)], ref, name)


@pytest.mark.parametrize("causal,Lk", [(False, 1111), (True, 700), (False, 90)])
def test_f16_v_with_bf16_qk_equals_bf16_path(causal, Lk):
    """bf16 q/k with an f16 v (a cache that keeps V in f16) gives exactly the bf16-v result for
    the same values (the bf16 path rounds V to f16 itself when staging), and matches the oracle."""
    B, Lq, H, d = 2, 300 if not causal else Lk, 4, 128
    q, k, v = synthetic.attention_inputs(B, Lq, Lk, H, H, d, "bf16", seed=Lk + causal)
    v16 = v.to(torch.float16)  # RNE, exact for these values' range
    qd, kd = q.to(DEV), k.to(DEV)
    a = torch.empty_like(qd)
    b = torch.empty_like(qd)
    binding.attn_forward_kvstride(qd, kd, v16.to(DEV), a, Lk, d ** -0.5, causal)
    binding.attn_forward_kvstride(qd, kd, v.to(DEV), b, Lk, d ** -0.5, causal)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = oracle.attention(widen(q).reshape(q.shape), widen(k).reshape(k.shape), widen(v16).reshape(v.shape),
                           d ** -0.5, causal)
    assert_attention_close(a, ref, "f16 v")


BIG_CASES = [
    # name, Lk, dtype, causal: 64 K/V heads x d=128; rows up to one tile past Lk span
    # (Lk + 64) * 64 * 128 * elem bytes; 4 GiB or more takes per-tile resources
    ("big_bf16", 262200, "bf16", False),
    ("big_bf16_causal", 262200, "bf16", True),
    ("big_fp8", 524400, "e4m3", False),
    ("limit_bf16_just_under_4gib", 262079, "bf16", False),   # the largest Lk on one resource
]


@pytest.mark.parametrize("case", BIG_CASES, ids=[c[0] for c in BIG_CASES])
def test_kv_regions_at_and_past_4gib(case):
    """K/V regions whose rows reach 4 GiB (4.3 GB tensors): every head's rows are read through
    32-bit buffer offsets, from a base that moves with the tile past the limit; just under it,
    from one resource with offsets up to the last tile. Three heads are checked against the
    oracle on their own slices (all 40 query rows, every key, ragged last tile)."""
    name, Lk, dt, causal = case
    B, Lq, H, d = 1, 40, 64, 128
    elem = 1 if dt == "e4m3" else 2
    big = (Lk + 64) * H * d * elem > 0xFFFFFFFF
    assert big == name.startswith("big"), name
    print(f"[case] {name} B={B} Lq={Lq} Lk={Lk} H={H} d={d} {dt} causal={causal}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(4242)
    def draw(L):
        x = torch.randn((B, L, H, d), generator=g, device=DEV, dtype=torch.bfloat16)
        return x.to(torch.float8_e4m3fn) if dt == "e4m3" else x
    q, k, v = draw(Lq), draw(Lk), draw(Lk)
    out = torch.empty((B, Lq, H, d), dtype=torch.bfloat16, device=DEV)
    if dt == "e4m3":
        binding.attn_forward_fp8(q, k, v, out, d ** -0.5, causal=causal)
    else:
        binding.attn_forward(q, k, v, out, d ** -0.5, causal)
    torch.cuda.synchronize()
    for h in (0, 37, 63):
        qh, kh, vh = (t[:, :, h:h + 1].contiguous().cpu() for t in (q, k, v))
        ref = oracle.attention(widen(qh).reshape(qh.shape), widen(kh).reshape(kh.shape),
                               widen(vh).reshape(vh.shape), d ** -0.5, causal)
        assert_attention_close(out[:, :, h:h + 1].contiguous(), ref, f"{name} head {h}")
    del q, k, v, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("Lk", [2047, 2048, 4100])
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_probability_threshold_rows(Lk, d):
    """bf16 launches whose rows all see at least 2048 keys (no mask) round the probabilities to
    bf16 for a bf16 P*V product; shorter rows keep f16 probabilities. Every row on both sides of
    the threshold, against the oracle, within the standard bounds."""
    B, Lq, H = 1, 300, 4
    print(f"[case] Lk={Lk} d={d}", flush=True)
    q, k, v = synthetic.attention_inputs(B, Lq, Lk, H, H, d, "bf16", seed=2040 + Lk + d)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    binding.attn_forward(q.to(DEV), k.to(DEV), v.to(DEV), out, d ** -0.5)
    torch.cuda.synchronize()
    Q, K, V = (widen(x).reshape(x.shape) for x in (q, k, v))
    assert_attention_close(out, oracle.attention(Q, K, V, d ** -0.5), f"Lk={Lk} d={d}")
