"""The allocation-free entry point (attn_forward_ws_static): the balanced launch with its partial
results in the library's per-GPU scratch array instead of a caller workspace. Called through the
C ABI on two calls in a row -- the second on a smaller input, so partials left in the scratch by
the first must not leak into it -- and compared with attn_forward_ws on the same inputs (the same
kernels, so bit for bit) and with the fp64 oracle on every row of the split query blocks."""
import numpy as np
import pytest
import torch

import oracle
from head_attention_streaming_amd import binding, synthetic
from parity import assert_attention_close, widen

pytestmark = pytest.mark.gpu
DEV = "cuda"
BM = 256  # query rows per block of a balanced launch


def _cases():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = cus + cus // 9 + 1   # just over one round of 256-row blocks: a balanced grid
    return [
        # name, B, Lq, Lk, Hq, Hkv, d, dtype (key loops of at least 16 tiles of 64 keys)
        ("static_bf16_d128", 1, -(-units // 40) * BM - 85, 2100, 40, 40, 128, "bf16"),
        ("static_f16_d64_gqa_smaller", 1, -(-units // 64) * BM - 200, 1990, 64, 16, 64, "f16"),
    ], cus


def _split_rows(B, Lq, Hq, cus):
    nq = -(-Lq // BM)
    units = B * Hq * nq
    rows = []
    for u in range(units - units % cus, units):
        qb, bh = u % nq, u // nq
        h, b = bh % Hq, bh // Hq
        rows += [(b * Lq + t) * Hq + h for t in range(qb * BM, min(Lq, qb * BM + BM))]
    return np.array(rows, dtype=np.int64)


def test_static_scratch_matches_workspace_launch_on_two_calls():
    cases, cus = _cases()
    sizes = []
    for i, (name, B, Lq, Lk, Hq, Hkv, d, dtype) in enumerate(cases):
        print(f"[case] {name} B={B} Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} d={d} {dtype}", flush=True)
        q, k, v = synthetic.attention_inputs(B, Lq, Lk, Hq, Hkv, d, dtype, seed=4200 + i)
        sizes.append(q.numel() + k.numel())
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        odt = torch.float16 if dtype == "f16" else torch.bfloat16
        out_static = torch.full(q.shape, float("nan"), dtype=odt, device=DEV)
        out_ws = torch.full(q.shape, float("nan"), dtype=odt, device=DEV)
        binding.attn_forward_ws_static(qd, kd, vd, out_static, d ** -0.5)
        binding.attn_forward_ws(qd, kd, vd, out_ws, d ** -0.5, binding.attn_workspace(d))
        torch.cuda.synchronize()
        assert torch.equal(out_static.view(torch.int16), out_ws.view(torch.int16)), name
        Q, K, V = (widen(x).reshape(x.shape) for x in (q, k, v))
        rows = _split_rows(B, Lq, Hq, cus)
        assert len(rows) > 0, name
        ref = oracle.attention(Q, K, V, d ** -0.5, rows=rows)
        assert_attention_close(out_static.reshape(-1, d)[torch.from_numpy(rows).to(DEV)], ref, name)
    assert sizes[1] < sizes[0]


def test_static_scratch_rejects_bad_arguments_before_launch():
    q = torch.zeros((1, 16, 8, 96), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(binding.StreamAttnError) as e:
        binding.attn_forward_ws_static(q, q, q, torch.empty_like(q), 0.1)
    assert e.value.status == binding.SA_ERR_UNSUPPORTED_CODE


def test_static_scratch_split_key_small_grid_on_two_calls():
    # the split key loops of small d = 128 grids (few query rows over 32+ key tiles) through the
    # allocation-free entry point: bit for bit as with a caller workspace, every row against the
    # oracle, the second call on a smaller input
    cases = [("static_split_64q_4096k", 1, 64, 4096, 16, 16, 128, "bf16"),
             ("static_split_one_query_smaller", 2, 1, 2100, 16, 4, 128, "bf16")]
    sizes = []
    for i, (name, B, Lq, Lk, Hq, Hkv, d, dtype) in enumerate(cases):
        print(f"[case] {name} B={B} Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} d={d} {dtype}", flush=True)
        q, k, v = synthetic.attention_inputs(B, Lq, Lk, Hq, Hkv, d, dtype, seed=4300 + i)
        sizes.append(q.numel() + k.numel())
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        out_static = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        out_ws = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        binding.attn_forward_ws_static(qd, kd, vd, out_static, d ** -0.5)
        binding.attn_forward_ws(qd, kd, vd, out_ws, d ** -0.5, binding.attn_workspace(d))
        torch.cuda.synchronize()
        assert torch.equal(out_static.view(torch.int16), out_ws.view(torch.int16)), name
        Q, K, V = (widen(x).reshape(x.shape) for x in (q, k, v))
        assert_attention_close(out_static.reshape(-1, d), oracle.attention(Q, K, V, d ** -0.5).reshape(-1, d), name)
    assert sizes[1] < sizes[0]
