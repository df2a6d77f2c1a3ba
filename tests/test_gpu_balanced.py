"""GPU parity of balanced launches (attn_forward_ws): grids whose last round of 4-wave
workgroups would leave CU slots idle run as 2 x CUs persistent workgroups, each with the same
number of whole query blocks plus an equal piece of the key tiles of the remaining blocks; the
pieces are merged from the workspace. Compared with the fp64 oracle on every row of the split
blocks and a sample of the rest; shapes are chosen from the device's CU count."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from head_attention_streaming_amd import binding, synthetic
from parity import assert_attention_close, sample_rows, widen

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _cases():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = 2 * cus + 2 * cus // 9 + 1           # just over one round of 4-wave workgroups
    Lq40 = -(-units // 40) * 128 - 85              # 40 heads, ragged last query block
    Lq64 = -(-units // 64) * 128 - 28
    return [
        # name, B, Lq, Lk, Hq, Hkv, d, dtype; key loops of at least 32 tiles (32 keys at d=128,
        # 64 at d=64) with a ragged last tile
        ("bal_bf16_d128_ragged", 1, Lq40, 1061, 40, 40, 128, "bf16"),
        ("bal_f16_d64_gqa", 1, Lq64, 2100, 64, 16, 64, "f16"),
        ("bal_bf16_batch2", 2, -(-units // 80) * 128 - 3, 1040, 40, 8, 128, "bf16"),
        ("bal_fp8_d128", 1, Lq40, 1500, 40, 40, 128, "e4m3"),
        # 8 surplus units of 34 tiles over 2 x CUs workgroups: most pieces are empty
        ("bal_sparse_surplus", 1, (2 * cus // 8 + 1) * 128 - 7, 1061, 8, 8, 128, "bf16"),
        ("bal_stream_shape", 1, 1785, 7140, 40, 40, 128, "bf16"),
    ]


def _split_rows(B, Lq, Hq):
    """Every row of the query blocks that a balanced launch splits between workgroups: the units
    past the last whole round of 2 x CUs, in (batch, head, 128-row query block) order."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nq = -(-Lq // 128)
    units = B * Hq * nq
    rows = []
    for u in range(units - units % (2 * cus), units):
        qb, bh = u % nq, u // nq
        h, b = bh % Hq, bh // Hq
        rows += [(b * Lq + t) * Hq + h for t in range(qb * 128, min(Lq, qb * 128 + 128))]
    return np.array(rows, dtype=np.int64)


@pytest.mark.parametrize("idx", range(6))
def test_balanced_matches_oracle(idx):
    name, B, Lq, Lk, Hq, Hkv, d, dtype = _cases()[idx]
    print(f"[case] {name} B={B} Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} d={d} {dtype}", flush=True)
    q, k, v = synthetic.attention_inputs(B, Lq, Lk, Hq, Hkv, d, dtype, seed=zlib.crc32(name.encode()) % 10000)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.empty(q.shape, dtype=torch.float16 if dtype == "f16" else torch.bfloat16, device=DEV)
    ws = binding.attn_workspace(d)
    binding.attn_forward_ws(qd, kd, vd, out, d ** -0.5, ws)
    torch.cuda.synchronize()
    Q, K, V = (widen(x).reshape(x.shape) for x in (q, k, v))
    split = _split_rows(B, Lq, Hq)
    assert len(split) > 0, name
    rows = np.union1d(split, sample_rows(B, Lq, Hq, 4096, seed=idx))
    ref = oracle.attention(Q, K, V, d ** -0.5, rows=rows)
    assert_attention_close(out.reshape(-1, d)[torch.from_numpy(rows).to(DEV)], ref, name)


def test_balanced_repeat_is_deterministic_and_small_workspace_falls_back():
    name, B, Lq, Lk, Hq, Hkv, d, dtype = _cases()[0]
    q, k, v = synthetic.attention_inputs(B, Lq, Lk, Hq, Hkv, d, dtype, seed=3)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ws = binding.attn_workspace(d)
    a, b, c, e = (torch.empty_like(qd) for _ in range(4))
    binding.attn_forward_ws(qd, kd, vd, a, 0.1, ws)
    binding.attn_forward_ws(qd, kd, vd, b, 0.1, ws)
    binding.attn_forward_ws(qd, kd, vd, c, 0.1, ws[:1024])      # too small: the plain launch
    binding.attn_forward_kvstride(qd, kd, vd, e, Lk, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(c.view(torch.int16), e.view(torch.int16))
    # the balanced launch ran: whole query blocks take the plain 4-wave launch's arithmetic and
    # match it bit for bit; split blocks sum their key tiles in another order and differ somewhere
    split = torch.zeros(B * Lq * Hq, dtype=torch.bool, device=DEV)
    split[torch.from_numpy(_split_rows(B, Lq, Hq)).to(DEV)] = True
    ab, cb = a.reshape(-1, d).view(torch.int16), c.reshape(-1, d).view(torch.int16)
    assert torch.equal(ab[~split], cb[~split])
    assert not torch.equal(ab[split], cb[split])
    rows = np.union1d(_split_rows(B, Lq, Hq), sample_rows(B, Lq, Hq, 4096, seed=7))
    ref = oracle.attention(widen(q).reshape(q.shape), widen(k).reshape(k.shape), widen(v).reshape(v.shape), 0.1,
                           rows=rows)
    ri = torch.from_numpy(rows).to(DEV)
    assert_attention_close(a.reshape(-1, d)[ri], ref, "balanced")
    assert_attention_close(c.reshape(-1, d)[ri], ref, "fallback")
