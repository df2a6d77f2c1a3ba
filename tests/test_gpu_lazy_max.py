"""GPU parity of the exponent offset's sum check (the 16-bit d = 128 kernels other than the plain
bf16-probability launch, and the 8-wave one-key-group d = 64 ones): no per-tile maximum is taken,
and a tile whose probability sum exceeds 2^15 in some lane, or overflows f16, is recomputed after
raising the offset to the tile maximum.
Each case plants keys late in the key loop that some query rows align with, so those rows' scores
jump 15-50 binades past every earlier tile's (two jumps per row, in different tiles): the
recompute path runs mid-loop, in balanced pieces and split loops as well. The planted rows and a
random sample of the others are checked against the fp64 oracle with the one-ulp floor: a planted
key is a multiple of one query, so it also gives some other rows a dominant score, and all such
rows have outputs close to one value row, up to |v| ~ 4, where one bf16 ulp exceeds 8e-3."""
import numpy as np
import pytest
import torch

import oracle
from head_attention_streaming_amd import binding, synthetic
from parity import assert_attention_close, sample_rows, widen

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # name, B, Lq, Lk, Hq, Hkv, d, dtype, window, workspace, (first, second) planted key
    # positions as fractions of the key range, score multipliers of the two planted keys
    ("balanced_bf16_probs_stream_shape", 1, 1785, 7140, 40, 40, 128, "bf16", (-1, -1), True, (0.42, 0.91), (1.5, 3.0)),
    ("plain_8wave_f16_overflow", 1, 4096, 4096, 16, 16, 128, "f16", (-1, -1), False, (0.55, 0.97), (2.0, 4.0)),
    ("plain_4wave_bf16_cross_shape", 2, 1785, 512, 40, 40, 128, "bf16", (-1, -1), True, (0.5, 0.9), (1.5, 3.0)),
    ("window_1024_bf16", 1, 4096, 4096, 8, 8, 128, "bf16", (1024, 0), False, (-0.6, -0.1), (1.5, 3.0)),
    ("split_small_grid_bf16_probs", 1, 64, 4096, 16, 16, 128, "bf16", (-1, -1), True, (0.5, 0.95), (1.5, 3.0)),
    ("plain_8wave_d64_f16", 1, 8192, 8192, 16, 16, 64, "f16", (-1, -1), False, (0.3, 0.8), (2.0, 4.0)),
]


def _plant(q, k, frac, mult, window, seed):
    """For 4 query rows per head, overwrite two keys of the same K head with multiples of the
    row's query: key positions at the given fractions of Lk (for a window: offsets below the row's
    own position, as fractions of the left window). Returns the flat [B, Lq, Hq] indices of the
    planted rows."""
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    group = Hq // Hkv
    rng = np.random.default_rng(seed)
    rows, used = [], set()
    for b in range(B):
        for h in range(0, Hq, group):  # one query head per K/V head, so planted keys never collide
            hk = h // group
            for qi in rng.choice(np.arange(Lq // 2, Lq), size=4, replace=False):
                pos = int(qi) + Lk - Lq
                if window[0] >= 0:
                    keys = [pos + int(f * window[0]) for f in frac]
                else:
                    keys = [int(f * Lk) for f in frac]
                keys = [min(max(kk, 0), Lk - 1) for kk in keys]
                if any((b, hk, kk) in used for kk in keys) or keys[0] == keys[1]:
                    continue
                for kk, m in zip(keys, mult):
                    k[b, kk, hk] = (q[b, qi, h].float() * m).to(k.dtype)
                    used.add((b, hk, kk))
                rows.append((b * Lq + int(qi)) * Hq + h)
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_sum_check_recompute_mid_loop(idx):
    name, B, Lq, Lk, Hq, Hkv, d, dtype, window, use_ws, frac, mult = CASES[idx]
    print(f"[case] {name} B={B} Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} d={d} {dtype} window={window}", flush=True)
    q, k, v = synthetic.attention_inputs(B, Lq, Lk, Hq, Hkv, d, dtype, seed=6100 + idx)
    planted = _plant(q, k, frac, mult, window, seed=idx)
    assert len(planted) >= 4, name
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.empty_like(qd)
    scale = d ** -0.5
    if use_ws:
        binding.attn_forward_ws(qd, kd, vd, out, scale, binding.attn_workspace(d), window=window)
    else:
        binding.attn_forward_window(qd, kd, vd, out, scale, window)
    torch.cuda.synchronize()
    Q, K, V = (widen(x).reshape(x.shape) for x in (q, k, v))
    win = None if window == (-1, -1) else window
    ref_p = oracle.attention(Q, K, V, scale, rows=planted, window=win)
    flat = out.reshape(-1, d)
    assert_attention_close(flat[torch.from_numpy(planted).to(DEV)], ref_p, name + " planted rows", ulp_floor=True)
    others = np.setdiff1d(sample_rows(B, Lq, Hq, 2048, seed=idx), planted)
    ref_o = oracle.attention(Q, K, V, scale, rows=others, window=win)
    assert_attention_close(flat[torch.from_numpy(others).to(DEV)], ref_o, name, ulp_floor=True)
