"""GPU parity of the streaming step on seeded random configurations: chunk length, sink and
window sizes (whole chunks), heads, head size, RoPE pairing and scope, norm scope, cache type and
the attention workspace drawn from a fixed seed. Each run streams until the cache has evicted
twice and compares every chunk's output (all rows) with the oracle's rolling-cache model, and
the cached values bit for bit."""
import numpy as np
import pytest

from head_attention_streaming_amd import binding
from test_gpu_streaming import _streaming_run

pytestmark = pytest.mark.gpu


def _configs():
    rng = np.random.RandomState(1785)
    out = []
    for i in range(10):
        Lc = int(rng.choice([1, 7, 32, 63, 64, 65, 100, 130]))
        sink = Lc * int(rng.choice([0, 0, 1, 2]))
        window = Lc * int(rng.choice([1, 2, 3, 5]))
        H = int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128]))
        style = int(rng.choice([binding.SA_ROPE_SPLIT, binding.SA_ROPE_INTERLEAVED]))
        kind = str(rng.choice(["before", "before", "after", "inner", "fp8"]))
        B = int(rng.choice([1, 2]))
        ws = bool(rng.randint(2))
        n_chunks = (sink + window) // Lc + 2
        out.append((f"cfg{i}", B, Lc, H, d, sink, window, n_chunks, style, kind, ws))
    return out


CONFIGS = _configs()


@pytest.mark.parametrize("cfg", CONFIGS, ids=[c[0] for c in CONFIGS])
def test_random_streaming_matches_oracle(cfg):
    name, B, Lc, H, d, sink, window, n_chunks, style, kind, ws = cfg
    print(f"[case] {cfg}", flush=True)
    _streaming_run(B=B, Lc=Lc, H=H, d=d, sink=sink, window=window, n_chunks=n_chunks, rows_per_chunk=None,
                   seed0=5000 + 10 * int(name[3:]), style=style, after_cache=kind == "after",
                   inner=kind == "inner", fp8=kind == "fp8", workspace=ws)
