"""GPU parity of balanced launches (attn_forward_ws): grids of 256-row query blocks that would
leave the CUs under 90 % busy over their rounds run as one persistent 8-wave workgroup per CU,
each with the same number of whole blocks plus an equal piece of the key tiles (64 keys) of the
remaining blocks; the pieces are merged from the workspace. Compared with the fp64 oracle on
every row of the split blocks and a sample of the rest; shapes are chosen from the device's CU
count."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from head_attention_streaming_amd import binding, synthetic
from parity import assert_attention_close, sample_rows, widen

pytestmark = pytest.mark.gpu
DEV = "cuda"
BM = 256  # query rows per block of a balanced launch


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _cases():
    cus = _cus()
    units = cus + cus // 9 + 1                    # just over one round of blocks
    Lq40 = -(-units // 40) * BM - 85              # 40 heads, ragged last query block
    Lq64 = -(-units // 64) * BM - 28
    return [
        # name, B, Lq, Lk, Hq, Hkv, d, dtype; key loops of at least 16 tiles with a ragged last one
        ("bal_bf16_d128_ragged", 1, Lq40, 2100, 40, 40, 128, "bf16"),
        ("bal_f16_d64_gqa", 1, Lq64, 2100, 64, 16, 64, "f16"),
        ("bal_bf16_batch2", 2, -(-units // 80) * BM - 3, 2080, 40, 8, 128, "bf16"),
        ("bal_fp8_d128", 1, Lq40, 2500, 40, 40, 128, "e4m3"),
        # 4 surplus blocks of 33 tiles over CUs workgroups: most pieces are empty
        ("bal_sparse_surplus", 1, (cus // 4 + 1) * BM - 7, 2100, 4, 4, 128, "bf16"),
        ("bal_stream_shape", 1, 1785, 7140, 40, 40, 128, "bf16"),
        # the shortest balanced key loops: 16 tiles (ragged), 24 tiles at d = 64
        ("bal_bf16_16_tiles", 1, Lq40, 1000, 40, 40, 128, "bf16"),
        ("bal_f16_d64_24_tiles", 1, Lq64, 1500, 64, 16, 64, "f16"),
    ]


def _split_rows(B, Lq, Hq):
    """Every row of the query blocks that a balanced launch splits between workgroups: the blocks
    past the last whole round of one per CU, in (batch, head, 256-row block) order."""
    nq = -(-Lq // BM)
    units = B * Hq * nq
    rows = []
    for u in range(units - units % _cus(), units):
        qb, bh = u % nq, u // nq
        h, b = bh % Hq, bh // Hq
        rows += [(b * Lq + t) * Hq + h for t in range(qb * BM, min(Lq, qb * BM + BM))]
    return np.array(rows, dtype=np.int64)


@pytest.mark.parametrize("idx", range(8))
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


def test_balanced_whole_blocks_bit_exact_repeatable_and_small_workspace_falls_back():
    # 27 blocks x 40 heads = 1080 on 256 CUs: the plain launch is the same 8-wave shape (at least
    # four blocks per CU), 5 rounds 84 % busy, so the balanced one takes 4 whole blocks per
    # workgroup and splits the other 56
    cus = _cus()
    Hq, Lk, d = 40, 2100, 128
    Lq = -(-(4 * cus + cus // 8) // Hq) * BM - 3
    print(f"[case] bit-exact B=1 Lq={Lq} Lk={Lk} Hq={Hq} d={d}", flush=True)
    q, k, v = synthetic.attention_inputs(1, Lq, Lk, Hq, Hq, d, "bf16", seed=3)
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
    # the balanced launch ran: whole query blocks take the plain launch's arithmetic and match it
    # bit for bit; split blocks sum their key tiles in another order and differ somewhere
    split_rows = _split_rows(1, Lq, Hq)
    assert len(split_rows) > 0
    split = torch.zeros(Lq * Hq, dtype=torch.bool, device=DEV)
    split[torch.from_numpy(split_rows).to(DEV)] = True
    ab, cb = a.reshape(-1, d).view(torch.int16), c.reshape(-1, d).view(torch.int16)
    assert torch.equal(ab[~split], cb[~split])
    assert not torch.equal(ab[split], cb[split])
    rows = np.union1d(split_rows, sample_rows(1, Lq, Hq, 4096, seed=7))
    ref = oracle.attention(widen(q).reshape(q.shape), widen(k).reshape(k.shape), widen(v).reshape(v.shape), 0.1,
                           rows=rows)
    ri = torch.from_numpy(rows).to(DEV)
    assert_attention_close(a.reshape(-1, d)[ri], ref, "balanced")
    assert_attention_close(c.reshape(-1, d)[ri], ref, "fallback")


def _split_cases():
    cus = _cus()
    q_rows = cus // 4 // 8 * 128  # 8 heads: exactly a quarter as many 128-row blocks as CUs
    return [
        # name, B, Lq, Lk, Hq, Hkv, d, dtype: d = 128 grids of at most cus / 4 128-row blocks
        # over key loops of at least 32 tiles (64 keys), whose key tiles are split over the CUs
        ("split_bf16_d128_64q", 1, 64, 4096, 16, 16, 128, "bf16"),
        ("split_f16_gqa_ragged", 1, 100, 3000, 8, 2, 128, "f16"),
        ("split_bf16_one_query_batch2", 2, 1, 2100, 16, 4, 128, "bf16"),
        ("split_fp8_d128", 1, 64, 2500, 8, 8, 128, "e4m3"),
        ("split_bf16_quarter_grid_32_tiles", 1, q_rows, 2048, 8, 8, 128, "bf16"),
    ]


@pytest.mark.parametrize("idx", range(5))
def test_split_key_small_grid_matches_oracle(idx):
    # every row against the oracle; the split changes the order in which a row's key tiles are
    # summed, so the result differs from the plain launch's somewhere, while a workspace too
    # small for the split takes the plain launch bit for bit
    name, B, Lq, Lk, Hq, Hkv, d, dtype = _split_cases()[idx]
    print(f"[case] {name} B={B} Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} d={d} {dtype}", flush=True)
    q, k, v = synthetic.attention_inputs(B, Lq, Lk, Hq, Hkv, d, dtype, seed=zlib.crc32(name.encode()) % 10000)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    odt = torch.float16 if dtype == "f16" else torch.bfloat16
    out, small, plain = (torch.empty(q.shape, dtype=odt, device=DEV) for _ in range(3))
    ws = binding.attn_workspace(d)
    binding.attn_forward_ws(qd, kd, vd, out, d ** -0.5, ws)
    binding.attn_forward_ws(qd, kd, vd, small, d ** -0.5, ws[:1024])
    if dtype == "e4m3":
        binding.attn_forward_fp8(qd, kd, vd, plain, d ** -0.5, False)
    else:
        binding.attn_forward_kvstride(qd, kd, vd, plain, Lk, d ** -0.5, False)
    torch.cuda.synchronize()
    assert torch.equal(small.view(torch.int16), plain.view(torch.int16)), name
    assert not torch.equal(out.view(torch.int16), plain.view(torch.int16)), name
    Q, K, V = (widen(x).reshape(x.shape) for x in (q, k, v))
    ref = oracle.attention(Q, K, V, d ** -0.5)
    assert_attention_close(out.reshape(-1, d), ref.reshape(-1, d), name)
