"""LDS race check: the attention kernels built with SA_LDS_CHECK=1 (libstreamattn_ldscheck.so:
one LDS slot for K and one for V, each written only after a barrier that follows every read of
its previous tile) must give the fast double-buffered build's outputs bit for bit, on every
launch shape (8-wave, 4-wave, key-split, balanced, 4 GiB-free small shapes), every input type
(bf16 with f16 or bf16 probabilities, f16, FP8 with f16 or FP8 probabilities, bf16 with f16 V),
and the masked paths (causal, windows, key tails, the fused query norm). A barrier missing from
the fast pipeline would let a wave read a tile that another wave is overwriting; the check build
cannot, so the outputs would differ."""
import pytest
import torch

from head_attention_streaming_amd import binding, build, synthetic

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def check_lib():
    """The check library's handle, configured by the binding (the fast one is restored after)."""
    fast, path = binding.lib(), build.LIB
    try:
        binding._lib = None
        build.LIB = build.LIB_LDS_CHECK
        handle = binding.lib()
    finally:
        binding._lib, build.LIB = fast, path
    return fast, handle


def _both(check_lib, fn):
    fast, chk = check_lib
    outs = []
    for h in (fast, chk):
        binding._lib = h
        try:
            outs.append(fn())
        finally:
            binding._lib = fast
    torch.cuda.synchronize()
    return outs


CASES = [
    # name, B, Lq, Lk, Hq, Hkv, d, dtype, window, workspace, qnorm
    ("4wave_bf16_tail", 2, 300, 333, 4, 2, 128, "bf16", (-1, -1), False, False),
    ("8wave_grid_f16_d64", 1, 4096, 700, 72, 8, 64, "f16", (-1, -1), False, False),
    ("keysplit_bf16", 1, 256, 1500, 4, 4, 128, "bf16", (-1, -1), False, False),
    ("bf16_probs_long", 1, 300, 4100, 4, 4, 128, "bf16", (-1, -1), False, False),
    ("balanced_stream", 1, 1785, 7140, 40, 40, 128, "bf16", (-1, -1), True, False),
    ("causal_f16_d64", 2, 700, 700, 8, 8, 64, "f16", (-1, 0), False, False),
    ("four_groups_causal_f16_d64", 2, 1000, 1100, 3, 3, 64, "f16", (-1, 0), False, False),
    ("paired_blocks_causal_bf16_d64", 1, 2091, 2131, 15, 15, 64, "bf16", (-1, 0), False, False),
    ("window_bf16", 1, 900, 1000, 4, 2, 128, "bf16", (200, 30), False, False),
    ("fp8", 1, 333, 1200, 4, 2, 128, "e4m3", (-1, -1), False, False),
    ("fp8_probs", 1, 333, 1200, 4, 2, 128, "e4m3p", (-1, 0), False, False),
    ("bf16_f16v_qnorm", 1, 500, 600, 4, 4, 128, "bf16vf16", (-1, -1), False, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_lds_check_build_matches_fast_build(case, check_lib):
    name, B, Lq, Lk, Hq, Hkv, d, dtype, window, use_ws, qnorm = case
    print(f"[case] {case}", flush=True)
    base = {"e4m3p": "e4m3", "bf16vf16": "bf16"}.get(dtype, dtype)
    q, k, v = synthetic.attention_inputs(B, Lq, Lk, Hq, Hkv, d, base, seed=700 + Lq)
    if dtype == "bf16vf16":
        v = v.to(torch.float16)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    odt = torch.float16 if dtype == "f16" else torch.bfloat16
    ws = binding.attn_workspace(d) if use_ws else None
    gq = synthetic.norm_weight(d, torch.Generator().manual_seed(5)).to(DEV)

    def run():
        out = torch.full(q.shape, float("nan"), dtype=odt, device=DEV)
        if qnorm:
            binding.attn_forward_qnorm(qd, kd, vd, out, d ** -0.5, gq, 1e-6, workspace=ws, window=window)
        elif use_ws:
            binding.attn_forward_ws(qd, kd, vd, out, d ** -0.5, ws, window=window)
        else:
            binding.attn_forward_window(qd, kd, vd, out, d ** -0.5, window, fp8_probs=dtype == "e4m3p")
        return out

    fast, chk = _both(check_lib, run)
    assert not torch.isnan(fast.float()).any()
    assert torch.equal(fast.view(torch.int16), chk.view(torch.int16)), name
