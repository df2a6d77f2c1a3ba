"""GPU parity of attn_forward_window (local attention) against the fp64 oracle.

The window (left, right) is placed around each query's key position i + Lk - Lq, as in the
oracle. Cases cover edges that fall inside a key tile, on tile boundaries, bands narrower than
one tile, one-sided bands, bands wider than the sequence, grouped heads, a K/V prefix of a
larger buffer and the 256-row launch shape."""
import zlib

import pytest
import torch

import oracle
from head_attention_streaming_amd import binding, synthetic
from parity import assert_attention_close, sample_rows, widen

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(name, B, Lq, Lk, Hq, Hkv, d, dtype):
    return synthetic.attention_inputs(B, Lq, Lk, Hq, Hkv, d, dtype, seed=zlib.crc32(name.encode()) % 10000)


def _ref(q, k, v, scale, window, rows=None):
    return oracle.attention(widen(q).reshape(q.shape), widen(k).reshape(k.shape), widen(v).reshape(v.shape),
                            scale, window=window, rows=rows)


def _run(q, k, v, scale, window, Lk=None):
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.empty_like(qd)
    binding.attn_forward_window(qd, kd, vd, out, scale, window, Lk=Lk)
    torch.cuda.synchronize()
    return out


CASES = [
    # name, B, Lq, Lk, Hq, Hkv, d, dtype, (left, right)
    ("sliding_causal_256_bf16_d128", 1, 1000, 1000, 2, 2, 128, "bf16", (256, 0)),
    ("symmetric_100_37_f16_d64", 2, 700, 700, 2, 2, 64, "f16", (100, 37)),
    ("tile_aligned_64_63_bf16_d128", 1, 600, 600, 2, 2, 128, "bf16", (64, 63)),
    ("narrow_5_3_bf16_d64", 1, 333, 333, 3, 3, 64, "bf16", (5, 3)),
    ("single_key_0_0_bf16_d128", 2, 300, 300, 2, 2, 128, "bf16", (0, 0)),
    ("left_only_rect_f16_d128", 1, 200, 650, 2, 1, 128, "f16", (150, -1)),
    ("right_only_lq_gt_lk_bf16_d64", 1, 305, 300, 2, 2, 64, "bf16", (-1, 5)),
    ("left_and_right_rect_gqa_bf16_d128", 2, 150, 777, 8, 2, 128, "bf16", (300, 20)),
    ("decode_row_window_f16_d64", 1, 1, 1000, 4, 4, 64, "f16", (130, 0)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_window_matches_oracle(case):
    name, B, Lq, Lk, Hq, Hkv, d, dtype, window = case
    print(f"[case] {case}", flush=True)
    q, k, v = _inputs(name, B, Lq, Lk, Hq, Hkv, d, dtype)
    out = _run(q, k, v, d ** -0.5, window)
    assert_attention_close(out, _ref(q, k, v, d ** -0.5, window), name)


def test_window_wider_than_sequence_equals_unwindowed():
    """Bands that reach past both ends of the keys give exactly the causal / full results."""
    q, k, v = _inputs("wide_band", 1, 300, 420, 2, 2, 128, "bf16")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for window, causal in (((5000, 0), True), ((419, 0), True), ((-1, 5000), False), ((419, 299), False)):
        print(f"[case] window={window}", flush=True)
        a = torch.empty_like(qd)
        b = torch.empty_like(qd)
        binding.attn_forward_window(qd, kd, vd, a, 0.1, window)
        binding.attn_forward(qd, kd, vd, b, 0.1, causal)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), window


def test_window_over_prefix_of_larger_buffer():
    B, Lq, S, Lk, H, d = 2, 140, 500, 333, 3, 128
    q, k, v = synthetic.attention_inputs(B, Lq, S, H, H, d, "bf16", seed=19)
    out = _run(q, k, v, 0.1, (90, 0), Lk=Lk)
    ref = _ref(q, k[:, :Lk].contiguous(), v[:, :Lk].contiguous(), 0.1, (90, 0))
    assert_attention_close(out, ref, "window_prefix")


WIDE_CASES = [
    # at least four 256-row blocks per CU: bands of at most 2049 keys run 128-row blocks of 4
    # waves, wider ones 256-row blocks of 8 waves
    ("wide_sliding_1024_bf16_d128", 1, 8192, 8192, 32, 32, 128, "bf16", (1024, 0)),
    ("wide_symmetric_f16_d64", 2, 4000, 4000, 32, 8, 64, "f16", (700, 300)),
    ("wide_band_3101_8wave_bf16_d128", 1, 8192, 8192, 32, 32, 128, "bf16", (2500, 600)),
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=[c[0] for c in WIDE_CASES])
def test_window_wide_grid_sampled_rows(case):
    name, B, Lq, Lk, Hq, Hkv, d, dtype, window = case
    print(f"[case] {case}", flush=True)
    q, k, v = _inputs(name, B, Lq, Lk, Hq, Hkv, d, dtype)
    out = _run(q, k, v, d ** -0.5, window)
    rows = sample_rows(B, Lq, Hq, 3000, seed=13)
    ref = _ref(q, k, v, d ** -0.5, window, rows=rows)
    assert_attention_close(out.reshape(-1, d)[torch.from_numpy(rows).to(DEV)], ref, name)
