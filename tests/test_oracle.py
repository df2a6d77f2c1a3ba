"""Pins for the fp64 oracle: closed forms, invariants, brute force and library cross-checks.

Every check here ties the oracle to something other than itself -- a value worked out by hand
from the definitions on the page "flashdreams.accelerated" (section "Multi Head Attention
Definition"), an algebraic invariant of those definitions, or an independent library routine
(PyTorch float64 SDPA / rms_norm, numpy's binary16 conversion). No check re-types the oracle's
own formula.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from head_attention_streaming_amd import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def _sdpa64(q, k, v, scale, causal=False, mask=None):
    """PyTorch CPU float64 SDPA on [B, L, H, d] arrays (library cross-check)."""
    tq = torch.from_numpy(np.ascontiguousarray(q)).permute(0, 2, 1, 3)
    tk = torch.from_numpy(np.ascontiguousarray(k)).permute(0, 2, 1, 3)
    tv = torch.from_numpy(np.ascontiguousarray(v)).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, is_causal=causal,
                                                         scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


# ------------------------------------------------------------------ 16-bit formats

def test_decode_matches_library_for_every_pattern():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f16 = oracle.decode(pats, "f16")
    ref16 = pats.view(np.float16).astype(np.float64)
    same = (f16 == ref16) | (np.isnan(f16) & np.isnan(ref16))
    assert same.all()
    bf = oracle.decode(pats, "bf16")
    refbf = torch.from_numpy(pats.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    same = (bf == refbf) | (np.isnan(bf) & np.isnan(refbf))
    assert same.all()


def test_decode_known_values():
    pats = np.array([0x3F80, 0xC000, 0x7F80, 0x0001, 0x3C00], dtype=np.uint16)
    assert list(oracle.decode(pats[:4], "bf16")) == [1.0, -2.0, math.inf, 2.0 ** -133]
    f = oracle.decode(np.array([0x3C00, 0x7BFF, 0x0001, 0x3555, 0xC400], dtype=np.uint16), "f16")
    assert list(f) == [1.0, 65504.0, 2.0 ** -24, 0.333251953125, -4.0]


def test_decode_e4m3_every_pattern_and_known_values():
    """OCP FP8 E4M3 (float8_e4m3fn): all 256 codes against torch's float8_e4m3fn, and values
    worked out from the format (bias 7, 3 fraction bits, subnormals, only S.1111.111 is NaN)."""
    pats = np.arange(256, dtype=np.uint8)
    got = oracle.decode(pats, "e4m3")
    ref = torch.from_numpy(pats.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert ((got == ref) | (np.isnan(got) & np.isnan(ref))).all()
    known = {0x38: 1.0, 0x40: 2.0, 0xB8: -1.0, 0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6,
             0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x3C: 1.5, 0x33: 0.6875, 0x00: 0.0, 0x78: 256.0}
    for code, value in known.items():
        assert oracle.decode(np.array([code], dtype=np.uint8), "e4m3")[0] == value, hex(code)
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.isfinite(got[[c for c in range(256) if c not in (0x7F, 0xFF)]]).all()  # no infinities


def test_round_to_bf16_hand_cases():
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -30, -(1 + 2 ** -8 + 2 ** -30),
                  2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 0.0, -0.0, 3.0e38, 3.5e38])
    r = oracle.round_to(x, "bf16")
    # tie to even (down), tie to even (up), just above a tie (direct rounding, no fp32 detour),
    # smallest subnormal, half of it (tie to even 0), 1.5x half (rounds up), zeros, large, overflow
    expect = [1.0, 1 + 2 ** -6, 1 + 2 ** -7, -(1 + 2 ** -7), 2.0 ** -133, 0.0, 2.0 ** -133, 0.0, -0.0,
              float(torch.tensor(3.0e38).to(torch.bfloat16).double()), math.inf]
    assert list(r) == expect
    assert math.copysign(1.0, r[8]) == -1.0


def test_round_to_matches_libraries():
    # fp32-representable inputs: torch's float32 -> bfloat16 conversion is round-to-nearest-even
    x32 = (RNG.standard_normal(200000) * np.exp(RNG.uniform(-30, 30, 200000))).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_to(x32.astype(np.float64), "bf16"), ref)
    # numpy converts float64 -> float16 directly with round-to-nearest-even
    x64 = RNG.standard_normal(200000) * np.exp(RNG.uniform(-12, 9, 200000))
    ref16 = x64.astype(np.float16).astype(np.float64)
    assert np.array_equal(oracle.round_to(x64, "f16"), ref16)


# ------------------------------------------------------------------ attention

@pytest.mark.parametrize("case", _load("attention_two_keys.json")["cases"], ids=lambda c: c["name"])
def test_attention_hand_worked_two_key_cases(case):
    q, k, v = (np.array(case[n], dtype=np.float64) for n in ("q", "k", "v"))
    out = oracle.attention(q, k, v, case["scale"], case["causal"])
    np.testing.assert_allclose(out, np.array(case["expected"]), rtol=0, atol=1e-12)


def test_attention_single_key_returns_v():
    q, k, v = _rand(2, 5, 3, 16), _rand(2, 1, 3, 16), _rand(2, 1, 3, 16)
    out = oracle.attention(q, k, v, 0.25)
    np.testing.assert_allclose(out, np.broadcast_to(v, out.shape), rtol=0, atol=1e-14)


def test_attention_zero_query_returns_mean_of_v():
    q, k, v = np.zeros((1, 4, 2, 8)), _rand(1, 37, 2, 8), _rand(1, 37, 2, 8)
    out = oracle.attention(q, k, v, 0.3)
    mean = v.mean(axis=1, keepdims=True)
    np.testing.assert_allclose(out, np.broadcast_to(mean, out.shape), rtol=0, atol=1e-14)


def test_attention_causal_first_row_returns_v0():
    q, k, v = _rand(2, 9, 3, 8), _rand(2, 9, 3, 8), _rand(2, 9, 3, 8)
    out = oracle.attention(q, k, v, 0.5, causal=True)
    np.testing.assert_allclose(out[:, 0], v[:, 0], rtol=0, atol=1e-14)


def test_attention_brute_force_two_heads_sigmoid():
    # B=1, H=2, L=2, d=2 from random values: o = sigmoid(s0 - s1) v0 + sigmoid(s1 - s0) v1
    q, k, v = _rand(1, 2, 2, 2), _rand(1, 2, 2, 2), _rand(1, 2, 2, 2)
    out = oracle.attention(q, k, v, 0.7)
    for i in range(2):
        for h in range(2):
            s0 = 0.7 * (q[0, i, h, 0] * k[0, 0, h, 0] + q[0, i, h, 1] * k[0, 0, h, 1])
            s1 = 0.7 * (q[0, i, h, 0] * k[0, 1, h, 0] + q[0, i, h, 1] * k[0, 1, h, 1])
            w0 = 1.0 / (1.0 + math.exp(s1 - s0))
            w1 = 1.0 / (1.0 + math.exp(s0 - s1))
            np.testing.assert_allclose(out[0, i, h], w0 * v[0, 0, h] + w1 * v[0, 1, h], rtol=0, atol=1e-14)


@pytest.mark.parametrize("shape", [(1, 7, 2, 13, 16), (2, 33, 3, 65, 64), (1, 64, 4, 64, 128)])
def test_attention_matches_torch_sdpa_float64(shape):
    B, Lq, H, Lk, d = shape
    q, k, v = _rand(B, Lq, H, d), _rand(B, Lk, H, d), _rand(B, Lk, H, d)
    out = oracle.attention(q, k, v, d ** -0.5)
    np.testing.assert_allclose(out, _sdpa64(q, k, v, d ** -0.5), rtol=1e-12, atol=1e-13)


def test_attention_causal_bottom_right_matches_masked_sdpa():
    B, Lq, Lk, H, d = 1, 5, 12, 2, 8
    q, k, v = _rand(B, Lq, H, d), _rand(B, Lk, H, d), _rand(B, Lk, H, d)
    out = oracle.attention(q, k, v, 0.35, causal=True)
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    mask = torch.from_numpy(j <= i + (Lk - Lq))
    np.testing.assert_allclose(out, _sdpa64(q, k, v, 0.35, mask=mask), rtol=1e-12, atol=1e-13)
    # square causal equals torch's is_causal
    q2, k2, v2 = _rand(2, 17, 2, 8), _rand(2, 17, 2, 8), _rand(2, 17, 2, 8)
    np.testing.assert_allclose(oracle.attention(q2, k2, v2, 0.35, causal=True),
                               _sdpa64(q2, k2, v2, 0.35, causal=True), rtol=1e-12, atol=1e-13)


def test_attention_key_permutation_invariance():
    q, k, v = _rand(1, 6, 2, 16), _rand(1, 40, 2, 16), _rand(1, 40, 2, 16)
    perm = RNG.permutation(40)
    a = oracle.attention(q, k, v, 0.25)
    b = oracle.attention(q, k[:, perm], v[:, perm], 0.25)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_attention_score_shift_invariance_large_offset():
    # k_j + u with q.u = const per query: every score of a row moves by the same amount (~ +1000)
    d = 16
    q, k, v = _rand(1, 3, 1, d), _rand(1, 25, 1, d), _rand(1, 25, 1, d)
    u = q[0, 0, 0] / np.dot(q[0, 0, 0], q[0, 0, 0]) * 4000.0   # q0.u = 4000, scale 0.25 -> +1000
    a = oracle.attention(q[:, :1], k, v, 0.25)
    b = oracle.attention(q[:, :1], k + u, v, 0.25)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-10)
    assert np.isfinite(b).all()


def test_attention_constant_and_linear_in_v():
    q, k = _rand(1, 5, 2, 8), _rand(1, 19, 2, 8)
    c = _rand(8)
    vc = np.broadcast_to(c, (1, 19, 2, 8)).copy()
    np.testing.assert_allclose(oracle.attention(q, k, vc, 0.4), np.broadcast_to(c, (1, 5, 2, 8)),
                               rtol=0, atol=1e-13)
    v1, v2 = _rand(1, 19, 2, 8), _rand(1, 19, 2, 8)
    lhs = oracle.attention(q, k, 2.0 * v1 - 3.0 * v2, 0.4)
    rhs = 2.0 * oracle.attention(q, k, v1, 0.4) - 3.0 * oracle.attention(q, k, v2, 0.4)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_attention_one_hot_limit():
    q, k, v = _rand(1, 1, 1, 8), _rand(1, 30, 1, 8), _rand(1, 30, 1, 8)
    k[0, 17, 0] = q[0, 0, 0] * 100.0   # score gap of hundreds: weight of every other key < e^-300
    out = oracle.attention(q, k, v, 1.0)
    np.testing.assert_allclose(out[0, 0, 0], v[0, 17, 0], rtol=0, atol=1e-12)


def test_attention_gqa_equals_repeated_kv_heads():
    q, k, v = _rand(2, 9, 6, 16), _rand(2, 21, 2, 16), _rand(2, 21, 2, 16)
    a = oracle.attention(q, k, v, 0.25)
    b = oracle.attention(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), 0.25)
    np.testing.assert_allclose(a, b, rtol=0, atol=0)


def test_attention_scale_folds_into_query():
    q, k, v = _rand(1, 6, 2, 32), _rand(1, 50, 2, 32), _rand(1, 50, 2, 32)
    np.testing.assert_allclose(oracle.attention(q, k, v, 0.17), oracle.attention(0.17 * q, k, v, 1.0),
                               rtol=1e-12, atol=1e-13)


def test_attention_row_subset_equals_full():
    q, k, v = _rand(2, 11, 3, 8), _rand(2, 13, 3, 8), _rand(2, 13, 3, 8)
    full = oracle.attention(q, k, v, 0.3, causal=True)
    rows = np.array([0, 5, 17, 65, 32, 2 * 11 * 3 - 1])
    sub = oracle.attention(q, k, v, 0.3, causal=True, rows=rows)
    np.testing.assert_array_equal(sub, full.reshape(-1, 8)[rows])


# ------------------------------------------------------------------ RMSNorm

@pytest.mark.parametrize("case", _load("norm_rope_closed_form.json")["rmsnorm"], ids=lambda c: c["note"][:20])
def test_rmsnorm_hand_worked(case):
    out = oracle.rmsnorm(np.array([case["z"]]), np.array(case["gamma"]), case["eps"])
    np.testing.assert_allclose(out[0], case["expected"], rtol=0, atol=1e-15)


def test_rmsnorm_unit_rms_and_scale_invariance_and_gamma_linearity():
    z = _rand(50, 128)
    one = oracle.rmsnorm(z, np.ones(128), 0.0)
    np.testing.assert_allclose(np.sqrt((one ** 2).mean(axis=1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(oracle.rmsnorm(7.5 * z, np.ones(128), 0.0), one, rtol=1e-14, atol=1e-15)
    g1, g2 = _rand(128), _rand(128)
    np.testing.assert_allclose(oracle.rmsnorm(z, 2 * g1 + g2, 1e-6),
                               2 * oracle.rmsnorm(z, g1, 1e-6) + oracle.rmsnorm(z, g2, 1e-6),
                               rtol=1e-12, atol=1e-13)


def test_rmsnorm_matches_torch_float64():
    z, g = _rand(3, 7, 5, 64), _rand(64)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(z), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rmsnorm(z, g, 1e-6), ref, rtol=1e-13, atol=1e-14)
    # inner scope (m = H*d) is the same routine over a flattened token
    zi = z.reshape(3, 7, 5 * 64)
    gi = _rand(5 * 64)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(zi), (320,), torch.from_numpy(gi), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rmsnorm(zi, gi, 1e-6), ref, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------------ RoPE

@pytest.mark.parametrize("case", _load("norm_rope_closed_form.json")["rope"], ids=lambda c: c["note"][:20])
def test_rope_hand_worked(case):
    style = {"split": oracle.SPLIT, "interleaved": oracle.INTERLEAVED}[case["style"]]
    z = np.array(case["z"]).reshape(1, 1, 1, 4)
    out = oracle.rope(z, np.array([case["angles"]]), style)
    np.testing.assert_allclose(out.reshape(-1), case["expected"], rtol=0, atol=1e-15)


def _angles(positions, d):
    return synthetic.rope_angles(positions, d).numpy().astype(np.float64)


def test_rope_angle_table_values():
    a = _angles([0, 1, 3000], 128)
    assert np.all(a[0] == 0)
    assert a[1, 0] == 1.0 and a[2, 0] == 3000.0
    # omega_32 = 10000^(-64/128) = 1/100
    np.testing.assert_allclose(a[1, 32], 0.01, rtol=1e-7)
    np.testing.assert_allclose(a[2, 32], 30.0, rtol=1e-7)


@pytest.mark.parametrize("style", [oracle.SPLIT, oracle.INTERLEAVED])
def test_rope_preserves_pair_norms(style):
    d = 64
    z = _rand(2, 9, 3, d)
    out = oracle.rope(z, _angles(np.arange(100, 109), d), style)
    if style == oracle.SPLIT:
        pa, pb = np.arange(d // 2), np.arange(d // 2) + d // 2
    else:
        pa, pb = np.arange(0, d, 2), np.arange(1, d, 2)
    np.testing.assert_allclose(out[..., pa] ** 2 + out[..., pb] ** 2, z[..., pa] ** 2 + z[..., pb] ** 2,
                               rtol=1e-13, atol=1e-13)


def test_rope_relative_position_identity():
    # <R_p q, R_p' k> = <R_(p-p') q, k> with angles p * omega_r (computed here in fp64)
    d = 32
    omega = 10000.0 ** (-2.0 * np.arange(d // 2) / d)
    q, k = _rand(1, 1, 1, d), _rand(1, 1, 1, d)
    for p, pp in [(7, 3), (120, 119), (5, 40)]:
        lhs = np.sum(oracle.rope(q, (p * omega)[None], oracle.SPLIT) * oracle.rope(k, (pp * omega)[None], oracle.SPLIT))
        rhs = np.sum(oracle.rope(q, ((p - pp) * omega)[None], oracle.SPLIT) * k)
        np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_rope_split_equals_interleaved_under_feature_permutation():
    d = 16
    z = _rand(1, 4, 2, d)
    ang = _angles(np.arange(4), d)
    perm = np.empty(d, dtype=int)          # interleaved position 2r <- split r, 2r+1 <- split r+d/2
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    split = oracle.rope(z, ang, oracle.SPLIT)
    inter = oracle.rope(z[..., perm], ang, oracle.INTERLEAVED)
    np.testing.assert_allclose(inter, split[..., perm], rtol=0, atol=1e-15)


def test_rope_complex_multiplication_form():
    d = 8
    z = _rand(1, 3, 1, d)
    ang = _angles([2, 50, 999], d)
    out = oracle.rope(z, ang, oracle.INTERLEAVED)
    zc = z[..., 0::2] + 1j * z[..., 1::2]
    rc = zc * np.exp(1j * ang)[None, :, None, :]
    np.testing.assert_allclose(out[..., 0::2], rc.real, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(out[..., 1::2], rc.imag, rtol=1e-13, atol=1e-13)


def test_qk_norm_rope_order_is_norm_then_rope():
    d = 16
    z, g = _rand(1, 3, 2, d), _rand(d)
    ang = _angles([5, 6, 7], d)
    out = oracle.qk_norm_rope(z, g, 1e-6, ang, oracle.SPLIT)
    np.testing.assert_allclose(out, oracle.rope(oracle.rmsnorm(z, g, 1e-6), ang, oracle.SPLIT), rtol=0, atol=0)
    # with gamma = 1 the rotation preserves the unit RMS of each head
    out1 = oracle.qk_norm_rope(z, np.ones(d), 0.0, ang, oracle.SPLIT)
    np.testing.assert_allclose(np.sqrt((out1 ** 2).mean(axis=-1)), 1.0, rtol=1e-13)


# ------------------------------------------------------------------ local window (left, right)

def _band_mask(Lq, Lk, left, right):
    pos = np.arange(Lq)[:, None] + (Lk - Lq)
    j = np.arange(Lk)[None, :]
    m = np.ones((Lq, Lk), dtype=bool)
    if left >= 0:
        m &= j >= pos - left
    if right >= 0:
        m &= j <= pos + right
    return torch.from_numpy(m)


@pytest.mark.parametrize("Lq,Lk,left,right", [(9, 9, 2, 1), (5, 12, 3, 0), (7, 20, -1, 2), (11, 11, 4, -1)])
def test_window_matches_banded_sdpa(Lq, Lk, left, right):
    q, k, v = _rand(2, Lq, 2, 8), _rand(2, Lk, 2, 8), _rand(2, Lk, 2, 8)
    out = oracle.attention(q, k, v, 0.4, window=(left, right))
    np.testing.assert_allclose(out, _sdpa64(q, k, v, 0.4, mask=_band_mask(Lq, Lk, left, right)),
                               rtol=1e-12, atol=1e-13)


def test_window_special_cases():
    q, k, v = _rand(1, 6, 2, 8), _rand(1, 10, 2, 8), _rand(1, 10, 2, 8)
    full = oracle.attention(q, k, v, 0.3)
    np.testing.assert_array_equal(oracle.attention(q, k, v, 0.3, window=(-1, -1)), full)
    np.testing.assert_array_equal(oracle.attention(q, k, v, 0.3, window=(10, 10)), full)
    np.testing.assert_array_equal(oracle.attention(q, k, v, 0.3, window=(-1, 0)),
                                  oracle.attention(q, k, v, 0.3, causal=True))
    # (0, 0): query i sees only key i + Lk - Lq
    diag = oracle.attention(q, k, v, 0.3, window=(0, 0))
    np.testing.assert_allclose(diag, v[:, 4:10], rtol=0, atol=1e-14)
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, 0.3, causal=True, window=(1, 0))


def test_window_two_keys_sigmoid():
    # window (1, 0) on a square problem: row i >= 1 sees keys i-1 and i
    q, k, v = _rand(1, 5, 1, 4), _rand(1, 5, 1, 4), _rand(1, 5, 1, 4)
    out = oracle.attention(q, k, v, 0.8, window=(1, 0))
    for i in range(1, 5):
        s_prev = 0.8 * float(np.dot(q[0, i, 0], k[0, i - 1, 0]))
        s_cur = 0.8 * float(np.dot(q[0, i, 0], k[0, i, 0]))
        w_cur = 1.0 / (1.0 + math.exp(s_prev - s_cur))
        np.testing.assert_allclose(out[0, i, 0], w_cur * v[0, i, 0] + (1.0 - w_cur) * v[0, i - 1, 0],
                                   rtol=0, atol=1e-13)
    np.testing.assert_allclose(out[0, 0, 0], v[0, 0, 0], rtol=0, atol=1e-14)


# ------------------------------------------------------------------ after-cache RoPE positions

def _angles64(positions, d):
    p = np.asarray(positions, dtype=np.float64)[:, None]
    return p * np.power(10000.0, -2.0 * np.arange(d // 2)[None, :] / d)


def _after_vs_before(Lc, sink, window, n_chunks, d=8, H=2, seed=0):
    from oracle.cache import RollingCacheModel
    rng = np.random.default_rng(seed)
    model = RollingCacheModel(Lc, sink, window)
    keys, vals = {}, {}
    for c in range(n_chunks):
        keys[c] = rng.standard_normal((1, Lc, H, d))
        vals[c] = rng.standard_normal((1, Lc, H, d))
        model.write(c)
    c = n_chunks - 1
    q = rng.standard_normal((1, Lc, H, d))
    vis = model.visible_chunks()
    K = np.concatenate([keys[x] for x in vis], axis=1)
    V = np.concatenate([vals[x] for x in vis], axis=1)
    # before-cache: keys keep the absolute stream positions they were written at
    abs_pos = np.concatenate([np.arange(x * Lc, (x + 1) * Lc) for x in vis])
    before = oracle.attention(oracle.rope(q, _angles64(np.arange(c * Lc, (c + 1) * Lc), d), oracle.SPLIT),
                              oracle.rope(K, _angles64(abs_pos, d), oracle.SPLIT), V, 0.3)
    # after-cache: every visible key at its row of the visible sequence, queries at the last Lc rows
    n = model.visible_len()
    after = oracle.attention(oracle.rope(q, _angles64(np.arange(n - Lc, n), d), oracle.SPLIT),
                             oracle.rope(K, _angles64(np.arange(n), d), oracle.SPLIT), V, 0.3)
    return before, after


def test_after_cache_positions_equal_absolute_without_sinks():
    """RoPE scores depend only on position differences. Without sinks the visible window is a
    contiguous run of the stream, so cache-relative positions (after-cache RoPE) give the same
    attention as absolute positions (before-cache RoPE)."""
    before, after = _after_vs_before(Lc=4, sink=0, window=12, n_chunks=6)
    np.testing.assert_allclose(after, before, rtol=0, atol=1e-12)


def test_after_cache_positions_close_the_gap_after_a_sink():
    """With a sink chunk and evictions the sink sits right before the window in cache-relative
    positions, far from it in absolute ones: the two readings must differ."""
    before, after = _after_vs_before(Lc=4, sink=4, window=8, n_chunks=6)
    assert np.abs(after - before).max() > 1e-3


def test_round_to_e4m3_matches_the_format_and_torch():
    """RNE into OCP E4M3 (float8_e4m3fn): hand cases from the format (3 fraction bits, subnormal
    quantum 2^-9, largest 448, no infinity) and torch's float8_e4m3fn cast on many values."""
    hand = {1.0625: 1.0, 1.1875: 1.25, 1.0625 + 2 ** -20: 1.125, 2.0 ** -10: 0.0, 3 * 2.0 ** -11: 2.0 ** -9,
            448.0: 448.0, 464.0: 448.0, 300.0: 288.0, -0.3: -0.3125, 2.0 ** -9: 2.0 ** -9, 0.0: 0.0}
    for x, want in hand.items():
        assert oracle.round_to(np.array([x]), "e4m3")[0] == want, x
    assert np.isnan(oracle.round_to(np.array([464.5, -500.0, 1e9]), "e4m3")).all()
    rng = np.random.default_rng(5)
    vals = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 200.0)])
    codes = oracle.decode(np.arange(256, dtype=np.uint8), "e4m3")
    codes = codes[np.isfinite(codes)]
    mids = (np.sort(codes)[1:] + np.sort(codes)[:-1]) / 2      # exact ties between neighbours
    # float32 inputs (torch casts through float32, so a float64 input one step off a tie would be
    # rounded twice there); the neighbours of each tie are float32 neighbours
    m32 = mids.astype(np.float32)
    vals = np.concatenate([vals.astype(np.float32), codes.astype(np.float32), m32,
                           np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(-np.inf))])
    vals = vals[np.abs(vals) <= 464.0]
    ours = oracle.round_to(vals.astype(np.float64), "e4m3")
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------------ ulp (the tolerance quantum)

@pytest.mark.parametrize("dtype,x,spacing", [
    # bf16: 8 significant bits. Binade [1, 2) has spacing 2^-7, [2, 4) 2^-6, [0.5, 1) 2^-8;
    # below the smallest normal 2^-126 the spacing stays 2^-133 (subnormals)
    ("bf16", 1.0, 2.0 ** -7), ("bf16", 1.999, 2.0 ** -7), ("bf16", 2.0, 2.0 ** -6), ("bf16", 0.75, 2.0 ** -8),
    ("bf16", -3.0, 2.0 ** -6), ("bf16", 2.0 ** -126, 2.0 ** -133), ("bf16", 2.0 ** -130, 2.0 ** -133),
    ("bf16", 0.0, 2.0 ** -133), ("bf16", 5.0, 2.0 ** -5),
    # f16: 11 significant bits, smallest normal 2^-14, largest finite 65504 = (2 - 2^-10) 2^15
    ("f16", 1.0, 2.0 ** -10), ("f16", 65504.0, 32.0), ("f16", 2.0 ** -14, 2.0 ** -24),
    ("f16", 2.0 ** -20, 2.0 ** -24), ("f16", 0.0, 2.0 ** -24), ("f16", 1000.0, 0.5),
    # E4M3: 4 significant bits, smallest normal 2^-6, largest finite 448 = 1.75 * 2^8
    ("e4m3", 1.0, 2.0 ** -3), ("e4m3", 448.0, 32.0), ("e4m3", 2.0 ** -6, 2.0 ** -9),
    ("e4m3", 2.0 ** -8, 2.0 ** -9), ("e4m3", 0.0, 2.0 ** -9), ("e4m3", 20.0, 2.0),
])
def test_ulp_hand_derived_spacings(dtype, x, spacing):
    """Spacings worked out by hand from each format's significand width and smallest normal
    exponent (the formats' definitions), not from the oracle's expression."""
    assert oracle.ulp(np.array([x]), dtype)[0] == spacing


@pytest.mark.parametrize("dtype,tdt,idt,lo,hi", [
    ("bf16", torch.bfloat16, torch.int16, -133, 127),
    ("f16", torch.float16, torch.int16, -24, 15),
    ("e4m3", torch.float8_e4m3fn, torch.uint8, -9, 8),
])
def test_ulp_equals_gap_to_next_bit_pattern(dtype, tdt, idt, lo, hi):
    """For 10^5 magnitudes spread over the format's whole range (subnormals included), ulp(x)
    equals the gap between the largest representable value <= x and the value of the next bit
    pattern, both decoded by torch: positive encodings are ordered like their values, so the next
    pattern is the next representable number."""
    rng = np.random.default_rng(7)
    x = np.exp2(rng.uniform(lo, hi + 0.999, size=100_000))
    x = x[x < {"bf16": 3.3e38, "f16": 65504.0, "e4m3": 448.0}[dtype]]
    bits = torch.from_numpy(x).to(tdt).view(idt).to(torch.int64)

    def val(b):
        return b.to(idt).view(tdt).to(torch.float64).numpy()

    xt = torch.from_numpy(x)
    # step the encoding to the largest value <= x (the conversion may have rounded up, or, for
    # bf16 via fp32, twice down)
    for _ in range(3):
        bits = torch.where(torch.from_numpy(val(bits)) > xt, bits - 1, bits)
        bits = torch.where(torch.from_numpy(val(bits + 1)) <= xt, bits + 1, bits)
    below, above = val(bits), val(bits + 1)
    assert (below <= x).all() and (above > x).all()
    np.testing.assert_array_equal(oracle.ulp(x, dtype), above - below)
    np.testing.assert_array_equal(oracle.ulp(-x, dtype), above - below)


# ------------------------------------------------------------------ spread of V under the weights

def test_attention_spread_single_key_is_zero():
    """One visible key: weight 1, o = v, so both spreads and the score range are exactly 0."""
    q, k, v = _rand(1, 3, 2, 8), _rand(1, 1, 2, 8), _rand(1, 1, 2, 8)
    o, a, r, span, ta, tw = oracle.attention_spread(q, k, v, 0.3)
    assert np.array_equal(o, np.broadcast_to(v, o.shape))
    assert not a.any() and not r.any() and not span.any() and not ta.any() and not tw.any()


def test_attention_spread_uniform_weights_closed_form():
    """q = 0: every weight is 1/N, so o = mean(V), A = mean |v - mean| and R = sqrt(sum (v - mean)^2) / N,
    computed here from V alone; the score range is 0."""
    B, Lq, Lk, H, d = 2, 3, 37, 2, 16
    q, k, v = np.zeros((B, Lq, H, d)), _rand(B, Lk, H, d), _rand(B, Lk, H, d)
    o, a, r, span, _, _ = oracle.attention_spread(q, k, v, 0.7)
    mean = v.mean(axis=1, keepdims=True)                       # [B, 1, H, d]
    np.testing.assert_allclose(o, np.broadcast_to(mean, o.shape), rtol=0, atol=1e-14)
    np.testing.assert_allclose(a, np.broadcast_to(np.abs(v - mean).mean(axis=1, keepdims=True), a.shape),
                               rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r, np.broadcast_to(np.sqrt(((v - mean) ** 2).sum(axis=1, keepdims=True)) / Lk,
                                                  r.shape), rtol=1e-12, atol=1e-15)
    assert not span.any()


def test_attention_spread_two_keys_hand_worked():
    """Two keys with score gap ln 3 (weights 3/4, 1/4): v0 - o = w1 (v0 - v1), v1 - o = w0 (v1 - v0),
    so A = 2 w0 w1 |v0 - v1| = (3/8)|v0 - v1|, R = sqrt(2) w0 w1 |v0 - v1| = (3 sqrt(2)/16)|v0 - v1|,
    and the score range is log2(3)."""
    q = np.array([[[[math.log(3.0), 0.0]]]])
    k = np.array([[[[1.0, 0.0]], [[0.0, 1.0]]]])
    v = np.array([[[[4.0, 8.0]], [[0.0, -4.0]]]])
    o, a, r, span, ta, tw = oracle.attention_spread(q, k, v, 1.0, tail_binades=1.5)
    dv = np.array([4.0, 12.0])
    # key 1 lies log2(3) ~ 1.58 binades below key 0: with a 1.5-binade threshold it is the tail,
    # carrying weight 1/4 and w1 |v1 - o| = w1 w0 |v0 - v1| of A
    np.testing.assert_allclose(tw[0, 0, 0], 0.25, rtol=1e-14)
    np.testing.assert_allclose(ta[0, 0, 0], 3.0 / 16.0 * dv, rtol=1e-13)
    _, _, _, _, ta2, tw2 = oracle.attention_spread(q, k, v, 1.0, tail_binades=1.6)
    assert not ta2.any() and not tw2.any()
    np.testing.assert_allclose(o[0, 0, 0], [3.0, 5.0], rtol=1e-14)
    np.testing.assert_allclose(a[0, 0, 0], 3.0 / 8.0 * dv, rtol=1e-13)
    np.testing.assert_allclose(r[0, 0, 0], 3.0 * math.sqrt(2.0) / 16.0 * dv, rtol=1e-13)
    np.testing.assert_allclose(span[0, 0, 0], math.log2(3.0), rtol=1e-13)


def test_attention_spread_rows_and_windows_match_full():
    """Row subsets and windowed rows give the same o as ``attention`` and the same spreads as the
    full computation."""
    q, k, v = _rand(2, 9, 4, 8), _rand(2, 13, 2, 8), _rand(2, 13, 2, 8)
    o, a, r, span, ta, tw = oracle.attention_spread(q, k, v, 0.5, window=(3, 1), tail_binades=0.5)
    np.testing.assert_array_equal(o, oracle.attention(q, k, v, 0.5, window=(3, 1)))
    assert (ta <= a + 1e-15).all() and (tw <= 1.0).all() and tw.any()
    rows = np.array([5, 0, 71, 33])
    o2, a2, r2, s2, ta2, tw2 = oracle.attention_spread(q, k, v, 0.5, window=(3, 1), rows=rows, tail_binades=0.5)
    np.testing.assert_array_equal(ta2, ta.reshape(-1, 8)[rows])
    np.testing.assert_array_equal(tw2, tw.reshape(-1)[rows])
    np.testing.assert_array_equal(o2, o.reshape(-1, 8)[rows])
    np.testing.assert_array_equal(a2, a.reshape(-1, 8)[rows])
    np.testing.assert_array_equal(r2, r.reshape(-1, 8)[rows])
    np.testing.assert_array_equal(s2, span.reshape(-1)[rows])
