"""GPU parity of FP8 E4M3 attention (float8_e4m3fn q, k, v; bf16 out) against the fp64 oracle.

The oracle decodes the same E4M3 codes exactly and evaluates the SDPA definition; the FP8 kernel
multiplies the exact E4M3 values on the FP8 MFMA and widens V exactly to f16, so the bf16 bounds
of the 16-bit kernels apply unchanged."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from head_attention_streaming_amd import binding, synthetic
from parity import assert_attention_close, sample_rows, widen

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(name, B, Lq, Lk, Hq, Hkv, d):
    return synthetic.attention_inputs(B, Lq, Lk, Hq, Hkv, d, "e4m3", seed=zlib.crc32(name.encode()) % 10000)


def _run(q, k, v, scale, causal=False, window=None):
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    if window is None:
        binding.attn_forward_fp8(qd, kd, vd, out, scale, causal)
    else:
        binding.attn_forward_window(qd, kd, vd, out, scale, window)
    torch.cuda.synchronize()
    return out


def _ref(q, k, v, scale, causal=False, window=None, rows=None):
    return oracle.attention(widen(q).reshape(q.shape), widen(k).reshape(k.shape), widen(v).reshape(v.shape),
                            scale, causal, rows=rows, window=window)


CASES = [
    # name, B, Lq, Lk, Hq, Hkv, d, causal, window
    ("fp8_noncausal_257_d128", 1, 257, 257, 8, 8, 128, False, None),
    ("fp8_ragged_gqa_d64", 2, 200, 333, 4, 2, 64, False, None),
    ("fp8_causal_square_d64", 2, 190, 190, 3, 3, 64, True, None),
    ("fp8_causal_rect_d128", 1, 100, 300, 2, 2, 128, True, None),
    ("fp8_split_keys_d128", 1, 300, 1111, 4, 2, 128, False, None),
    ("fp8_split_keys_causal_d64", 2, 600, 600, 3, 3, 64, True, None),
    ("fp8_window_d128", 1, 700, 700, 2, 2, 128, False, (100, 30)),
    ("fp8_one_key", 2, 70, 1, 2, 2, 128, False, None),
    ("fp8_mqa_d128", 1, 150, 200, 8, 1, 128, False, None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp8_attention_matches_oracle(case):
    name, B, Lq, Lk, Hq, Hkv, d, causal, window = case
    print(f"[case] {case}", flush=True)
    q, k, v = _inputs(name, B, Lq, Lk, Hq, Hkv, d)
    out = _run(q, k, v, d ** -0.5, causal, window)
    assert_attention_close(out, _ref(q, k, v, d ** -0.5, causal, window), name)


def test_fp8_every_value_code_passes_exactly():
    """One key per query: the output is V itself. V holds every finite E4M3 code (subnormals,
    448, negative zero), so the exact widening of V to f16 is checked code by code; every E4M3
    value is a bf16 value, so the bf16 output must equal it bit for bit."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    d, H = 128, 2
    n = -(-codes.size * 1 // (H * d)) + 1
    vals = np.resize(codes, (1, n, H, d))
    q = torch.zeros((1, n, H, d), dtype=torch.uint8).view(torch.float8_e4m3fn)
    k = torch.zeros((1, n, H, d), dtype=torch.uint8).view(torch.float8_e4m3fn)
    v = torch.from_numpy(vals.copy()).view(torch.float8_e4m3fn)
    out = _run(q, k, v, 0.1, window=(0, 0))  # query i sees key i only
    expect = torch.from_numpy(widen(v).reshape(v.shape)).to(torch.bfloat16)
    got = out.cpu()
    assert torch.equal(got.view(torch.int16)[got != 0], expect.view(torch.int16)[got != 0])
    assert torch.equal(got == 0, expect == 0)


def test_fp8_large_scores():
    """Scores far beyond the 16-bit input range (E4M3 values up to 448 on every feature)."""
    g = torch.Generator().manual_seed(3)
    q = (torch.randn((1, 130, 2, 128), generator=g) * 100).clamp(-448, 448).to(torch.float8_e4m3fn)
    k = (torch.randn((1, 300, 2, 128), generator=g) * 100).clamp(-448, 448).to(torch.float8_e4m3fn)
    v = torch.randn((1, 300, 2, 128), generator=g).to(torch.float8_e4m3fn)
    out = _run(q, k, v, 1e-4)
    assert_attention_close(out, _ref(q, k, v, 1e-4), "fp8 large scores", ulp_floor=True)


def test_fp8_wide_grid_sampled_rows():
    """256-row workgroups: [2, 4000, 64, 8, 128] E4M3, causal."""
    B, L, Hq, Hkv, d = 2, 4000, 64, 8, 128
    q, k, v = _inputs("fp8_wide", B, L, L, Hq, Hkv, d)
    out = _run(q, k, v, d ** -0.5, True)
    rows = sample_rows(B, L, Hq, 3000, seed=5)
    ref = _ref(q, k, v, d ** -0.5, True, rows=rows)
    assert_attention_close(out.reshape(-1, d)[torch.from_numpy(rows).to(DEV)], ref, "fp8 wide causal")


def test_fp8_long_20480_sampled_rows():
    """Long non-causal FP8 attention [1, 20480, 56, 128]: sampled rows over all keys."""
    w = synthetic.WORKLOADS["mha_20480_bf16"]
    q, k, v = synthetic.attention_inputs(w.B, w.Lq, w.Lk, w.Hq, w.Hkv, w.d, "e4m3", w.seed)
    out = _run(q, k, v, w.scale)
    rows = sample_rows(w.B, w.Lq, w.Hq, 2048, seed=7)
    ref = _ref(q, k, v, w.scale, rows=rows)
    assert_attention_close(out.reshape(-1, w.d)[torch.from_numpy(rows).to(DEV)], ref, "fp8 20480")
