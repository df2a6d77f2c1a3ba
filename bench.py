#!/usr/bin/env python3
"""Throughput benchmark of the streaming-attention hot path on one MI355X.

Default workload: long non-causal MHA forward [1, 20480, 56, 128] bf16 (scale 1/sqrt(128)), one
attn_forward call per step. Other workloads (``--workload``) time the other configurations,
including a full streaming self-attention step (prologue + cache append + attention).

Prints ONE JSON line: metric/value (attention TFLOP/s = 4*B*H*Lq*Lk*d / step time), the
dominant kernel's roofline (HIP-event timing of that kernel alone), and the fp64 CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (4·B·H·Lq·Lk·d) and % of bf16 MFMA peak, 1×MI355X"
PEAK_MFMA_16BIT = 2516.6   # TFLOP/s, dense bf16/fp16 MFMA, 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_MFMA_FP8 = 5033.2     # TFLOP/s, dense FP8 MFMA (twice the 16-bit rate)
# FP8 attention: Q K^T (half the flops) on FP8 MFMA, P V (the other half) on f16 MFMA
PEAK_MFMA_FP8_F16 = 1.0 / (0.5 / PEAK_MFMA_FP8 + 0.5 / PEAK_MFMA_16BIT)
PEAK_HBM = 8000.0          # GB/s
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed steps before the timed ones (default: at least 5 and at least 100 ms of GPU work, "
                        "so the GPU reaches its steady clock; the count run is reported)")
    p.add_argument("--workload", default="mha_20480_bf16")
    p.add_argument("--no-workspace", action="store_true",
                   help="streaming / cross workloads: plain attention launch instead of the balanced one")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time for the CPU baseline")
    return p.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "head_attention_streaming_amd", "csrc", "attn_fwd.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per launch measured with rocprofv3 PMC counters (committed summary), or None
    when no summary exists or the kernel source changed since it was taken."""
    path = os.path.join(PROFILE_DIR, f"attn_fwd_{workload}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def make_workload(name: str, dev: str, use_ws: bool = True):
    """Build device buffers and return (step_fn, kernel_fn, info)."""
    import numpy as np
    import torch

    from head_attention_streaming_amd import binding, synthetic

    if name == "copy_calibration":
        # plain 16-byte vector copy of a known size (the cache-append kernel): 512 MiB read and
        # 512 MiB written per launch; used to calibrate the HBM byte counters
        n_tok, H, d = 16384, 128, 128   # 16384 * 128 * 128 * 2 B = 512 MiB
        src = torch.empty((1, n_tok, H, d), dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)

        def copy():
            binding.kv_cache_append(None, src, None, dst, 0, 0, n_tok)
        info = {"workload": name, "bytes_read": src.numel() * 2, "bytes_written": src.numel() * 2}
        return None, copy, copy, info, None

    w = synthetic.WORKLOADS[name]
    info = {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Lq": w.Lq, "Lk": w.Lk, "d": w.d,
            "causal": w.causal, "scale": w.scale, "io_dtype": w.dtype, "prologue": w.prologue}
    if w.prologue == "none":
        q, k, v = synthetic.attention_inputs(w.B, w.Lq, w.Lk, w.Hq, w.Hkv, w.d, w.dtype, w.seed)
        q, k, v = q.to(dev), k.to(dev), v.to(dev)
        if w.dtype == "e4m3":
            out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
            info["compute"] = ("Q K^T and P V (E4M3 probabilities, E4M3 V) on FP8 E4M3 MFMA, fp32 accumulation, "
                               "bf16 out" if w.fp8_probs else
                               "Q K^T on FP8 E4M3 MFMA, P V on f16 MFMA, fp32 accumulation, bf16 out")

            def step():
                binding.attn_forward_fp8(q, k, v, out, w.scale, w.causal, fp8_probs=w.fp8_probs)
            return w, step, step, info, (q, k, v)
        out = torch.empty_like(q)
        if w.attn_window is not None:
            info["window"] = list(w.attn_window)

            def step():
                binding.attn_forward_window(q, k, v, out, w.scale, w.attn_window)
            return w, step, step, info, (q, k, v)
        fwd = binding.attn_forward if w.dtype == "bf16" else binding.attn_forward_f16

        def step():
            fwd(q, k, v, out, w.scale, w.causal)
        return w, step, step, info, (q, k, v)

    if w.prologue == "q_norm":
        g = torch.Generator().manual_seed(w.seed)
        q = synthetic.normal((w.B, w.Lq, w.Hq, w.d), "bf16", g).to(dev)
        k = synthetic.normal((w.B, w.Lk, w.Hkv, w.d), "bf16", g).to(dev)
        v = synthetic.normal((w.B, w.Lk, w.Hkv, w.d), "bf16", g).to(dev)
        if w.v_cache_dtype:
            v = v.to(synthetic.DTYPES[w.v_cache_dtype])  # the context cache keeps V in that type
            info["v_cache_dtype"] = w.v_cache_dtype
        gq = synthetic.norm_weight(w.d, g).to(dev)
        out = torch.empty_like(q)
        ws = binding.attn_workspace(w.d, dev) if use_ws else None
        info["balanced"] = use_ws
        if w.rope_scope == "after":
            # after-cache RoPE over a static context: the cache (built once, outside the step)
            # holds normalised, unrotated keys; each step rotates all of them into k_rot with the
            # cache-relative angle rows and normalises and rotates the queries (rows after them)
            gk = synthetic.norm_weight(w.d, g).to(dev)
            ck, cv, k_rot = torch.empty_like(k), torch.empty_like(v), torch.empty_like(k)
            binding.context_kv(k, v, ck, cv, gk, 1e-6)
            ctx_ang = synthetic.rope_angles(np.arange(w.Lk), w.d).to(dev)
            q_ang = synthetic.rope_angles(np.arange(w.Lk, w.Lk + w.Lq), w.d).to(dev)
            q_buf = torch.empty_like(q)

            def step():
                binding.cross_attention_step(ck, cv, q, out, gq, 1e-6, w.scale, q_buf=q_buf, q_angles=q_ang,
                                             context_angles=ctx_ang, k_rot=k_rot, workspace=ws)

            def kern():
                binding.attn_forward_ws(q_buf, k_rot, cv, out, w.scale, ws) if ws is not None else \
                    binding.attn_forward_kvstride(q_buf, k_rot, cv, out, w.Lk, w.scale, False)

            def rot_keys():
                binding.kv_cache_rope(ck, k_rot, ctx_ang, 0, w.Lk, 0, w.Lk, binding.SA_ROPE_SPLIT)

            def q_prologue():
                binding.qk_norm_rope(q, q_buf, None, None, gq, None, q_ang, 1e-6, binding.SA_NORM_HEAD,
                                     binding.SA_ROPE_SPLIT, Hkv=0)
            kbytes = 2 * w.B * w.Lk * w.Hkv * w.d
            qbytes = 2 * w.B * w.Lq * w.Hq * w.d
            info["hbm_steps"] = {"kv_cache_rope": (rot_keys, 2 * kbytes + w.Lk * (w.d // 2) * 4),
                                 "qk_norm_rope_q": (q_prologue, 2 * qbytes + w.Lq * (w.d // 2) * 4 + w.d * 4)}
            info["step"] = ("kv_cache_rope(all context keys -> k_rot) + qk_norm_rope(Q) + attention "
                            "(cross_attention_step, after-cache RoPE)")
            return w, step, kern, info, (q, k, v)

        def kern():  # the Q RMSNorm is fused into the attention kernel's query load
            binding.attn_forward_qnorm(q, k, v, out, w.scale, gq, 1e-6, workspace=ws)

        step = kern
        info["step"] = "attention with the Q RMSNorm fused into its query load (attn_forward_qnorm)"
        return w, step, kern, info, (q, k, v)

    # streaming self-attention: steady state (cache full, every step evicts the oldest chunk)
    Lc, S = w.chunk, w.window
    after = w.rope_scope == "after"
    cdt = synthetic.DTYPES[w.cache_dtype]
    vdt = synthetic.DTYPES[w.v_cache_dtype] if w.v_cache_dtype else None
    cache = binding.BlockKVCache(w.B, w.Hkv, w.d, Lc, 0, S, dtype=cdt, device=dev, after_cache_rope=after,
                                 v_dtype=vdt)
    if vdt is not None:
        info["v_cache_dtype"] = w.v_cache_dtype
    g = torch.Generator().manual_seed(w.seed)
    gq, gk = synthetic.norm_weight(w.d, g).to(dev), synthetic.norm_weight(w.d, g).to(dev)
    # Rotating input sets (10 x 55 MB) and query buffers (4 x 18 MB): together with the two cache
    # tensors (2 x 73 MB) each HBM-bound step cycles over ~770 MB of distinct bytes, three times
    # the 256 MB Infinity Cache, so no input or output of a timed call is still cache-resident.
    nsets, nbufs = 10, 4
    sets = []
    for i in range(nsets):
        gi = torch.Generator().manual_seed(w.seed + i)
        sets.append([synthetic.normal((w.B, Lc, w.Hq, w.d), "bf16", gi).to(dev) for _ in range(3)])
    q_bufs = [torch.empty((w.B, Lc, w.Hq, w.d), dtype=cdt, device=dev) for _ in range(nbufs)]
    q_buf = q_bufs[0]
    out = torch.empty((w.B, Lc, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
    state = {"c": 0}
    if after:  # rows 0 .. visible-1 of the visible sequence (visible = S once the cache is full)
        vis_angles = synthetic.rope_angles(np.arange(S), w.d).to(dev)
        angles = [vis_angles[:min(S, (c + 1) * Lc)] for c in range(8)]
    else:      # absolute stream positions of chunk c
        angles = [synthetic.rope_angles(np.arange(c * Lc, (c + 1) * Lc), w.d).to(dev) for c in range(8)]

    ws = binding.attn_workspace(w.d, dev) if use_ws else None
    info["balanced"] = use_ws

    def step():
        c = state["c"]
        q, k, v = sets[c % nsets]
        binding.stream_self_attention_step(cache, c, q, k, v, q_buf, out, gq, gk, angles[min(c, 7)], 1e-6, w.scale,
                                           workspace=ws, fp8_probs=w.fp8_probs)
        state["c"] = c + 1

    for _ in range(S // Lc):  # fill the cache before timing
        step()

    # the step's route (stream_self_attention_step's default): Q, K and V through one prologue
    # launch when the value cache has the key cache's type, else prologue + append; then attention
    one_launch = vdt is None
    info["route"] = ("qk_norm_rope_v (Q -> q_buf, K and V -> cache) + attention" if one_launch else
                     "qk_norm_rope (Q -> q_buf, K -> cache) + kv_cache_append (V) + attention")

    def kern():
        keys = cache.k_rot if after else cache.k
        if ws is not None:
            binding.attn_forward_ws(q_buf, keys, cache.v, out, w.scale, ws, Lk=S, fp8_probs=w.fp8_probs)
        else:
            binding.attn_forward_kvstride(q_buf, keys, cache.v, out, S, w.scale, False, fp8_probs=w.fp8_probs)

    # the HBM-bound steps alone, on rotating input sets, query buffers and cache slots (each input
    # set is read once per 10 calls; outputs go to one of 4 query buffers and one of the cache's
    # S / Lc chunk slots)
    rot = {"i": 0}
    nslots = S // Lc

    def next_set():
        i = rot["i"]
        rot["i"] = i + 1
        return sets[i % nsets], q_bufs[i % nbufs], (i % nslots) * Lc

    q_ang = angles[7][S - Lc:] if after else angles[0]
    flag = binding.SA_ROPE_AFTER_CACHE if after else 0
    gq_in = synthetic.norm_weight(w.Hq * w.d, g).to(dev)
    gk_in = synthetic.norm_weight(w.Hkv * w.d, g).to(dev)

    def prologue(scope=binding.SA_NORM_HEAD):
        (q, k, _), qb, slot = next_set()
        inner = scope == binding.SA_NORM_INNER
        binding.qk_norm_rope(q, qb, k, cache.k[:, slot:], gq_in if inner else gq, gk_in if inner else gk, q_ang,
                             1e-6, scope, binding.SA_ROPE_SPLIT | flag, k_out_bstride=S * w.Hkv * w.d)

    def append():  # sources rotate over all 30 chunk-sized input tensors (550 MB), not just the Vs
        i = rot["i"]
        rot["i"] = i + 1
        binding.kv_cache_append(None, sets[(i // 3) % nsets][i % 3], None, cache.v, i % nslots, 0, S)

    def prologue_v():  # the one-launch prologue: queries, keys and values
        (q, k, v), qb, slot = next_set()
        binding.qk_norm_rope_v(k, cache.k[:, slot:], v, cache.v[:, slot:], gk, q_ang, 1e-6, binding.SA_NORM_HEAD,
                               binding.SA_ROPE_SPLIT | flag, k_out_bstride=S * w.Hkv * w.d,
                               v_out_bstride=S * w.Hkv * w.d, q_in=q, q_out=qb, gamma_q=gq)

    elem = 2 * w.B * Lc * w.Hq * w.d  # bytes of one [B, Lc, H, d] bf16 tensor
    out_elem = elem // 2 if w.cache_dtype == "e4m3" else elem   # the same tensor in the cache type
    info["cache_dtype"] = w.cache_dtype
    info["hbm_steps"] = {
        # q, k read (bf16) + written (cache type), angles, gammas
        "qk_norm_rope": (prologue, 2 * elem + 2 * out_elem + Lc * (w.d // 2) * 4 + 2 * w.d * 4),
        "qk_norm_rope_inner": (lambda: prologue(binding.SA_NORM_INNER),
                               2 * elem + 2 * out_elem + Lc * (w.d // 2) * 4 + 2 * w.Hq * w.d * 4),
        "kv_cache_append": (append, elem + out_elem),                            # v read + written
    }
    if one_launch:  # q, k, v read (bf16) + written (cache type), angles, gammas
        info["hbm_steps"]["qk_norm_rope_v"] = (prologue_v, 3 * elem + 3 * out_elem + Lc * (w.d // 2) * 4 + 2 * w.d * 4)
        # the copy ceiling at this size: the plain 16-byte copy kernel moving the one-launch
        # prologue's bytes (three chunks in, three out), over 5 rotating buffer pairs (550 MB)
        cp_src = [torch.empty((w.B, 3 * Lc, w.Hq, w.d), dtype=torch.bfloat16, device=dev).fill_(1.0) for _ in range(5)]
        cp_dst = [torch.empty_like(x) for x in cp_src]

        def copy_same_bytes():
            i = rot["i"]
            rot["i"] = i + 1
            binding.kv_cache_append(None, cp_src[i % 5], None, cp_dst[i % 5], 0, 0, 3 * Lc)
        if w.cache_dtype == "bf16":
            info["hbm_steps"]["copy_same_bytes"] = (copy_same_bytes, 6 * elem)
    if after:
        def cache_rope():
            binding.kv_cache_rope(cache.k, cache.k_rot, angles[7], state["c"] - 1, Lc, 0, S, binding.SA_ROPE_SPLIT)
        kbytes = 2 * w.B * S * w.Hkv * w.d
        info["hbm_steps"]["kv_cache_rope"] = (cache_rope, 2 * kbytes + S * (w.d // 2) * 4)  # cache K read, k_rot written, angles
        info["step"] = (("qk_norm_rope_v(Q rotated, K normalised->cache, V->cache)" if one_launch else
                         "qk_norm_rope(Q rotated, K normalised->cache) + kv_cache_append(V)") +
                        " + kv_cache_rope(visible K -> k_rot) + attention, cache full")
    else:
        info["step"] = (("qk_norm_rope_v(Q, K->cache, V->cache)" if one_launch else
                         "qk_norm_rope(Q,K->cache) + kv_cache_append(V)") + " + attention, cache full")
    info["cache_tokens"] = S
    return w, step, kern, info, None


def visible_keys(w, i):
    """Keys each query row i (array of query indices) attends to under the workload's mask."""
    import numpy as np
    p = i + (w.Lk - w.Lq)
    lo, hi = np.zeros_like(p), np.full_like(p, w.Lk - 1)
    if w.causal:
        hi = np.minimum(hi, p)
    if w.attn_window is not None:
        left, right = w.attn_window
        if left >= 0:
            lo = np.maximum(lo, p - left)
        if right >= 0:
            hi = np.minimum(hi, p + right)
    return hi - lo + 1


def workload_flops(w) -> float:
    """Flops per step: the metric's formula 4*B*H*Lq*Lk*d; a local-attention band counts only
    the keys inside it (4*B*H*d*sum of visible keys), which is the work the band leaves."""
    if w.attn_window is None:
        return w.flops
    import numpy as np
    return 4.0 * w.B * w.Hq * w.d * float(visible_keys(w, np.arange(w.Lq)).sum())


def warm_up(fn, warmup):
    """Runs `warmup` untimed steps; with None, at least 5 steps and at least 100 ms of GPU work
    (short steps need many to bring the GPU to its steady clock). Returns the count run."""
    import torch
    if warmup is not None:
        for _ in range(warmup):
            fn()
        return warmup
    n, t0 = 0, time.perf_counter()
    while n < 5 or time.perf_counter() - t0 < 0.1:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()  # the host must not run far ahead of the GPU
    return n


def time_loop(fn, steps, warmup):
    import torch
    warm_up(fn, warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall * 1e3 / steps


def shader_clock_mhz(fn, seconds: float = 1.0):
    """Shader clock under the step's own load: runs `fn` back to back for about `seconds` while
    one `amd-smi metric -c` call reads the current clock of every XCD; returns (mean, min, max)
    in MHz, or None when the tool is missing or reports nothing. Called after the timed region,
    so it never perturbs the timing."""
    import re
    import shutil
    import subprocess
    import threading

    import torch
    tool = shutil.which("amd-smi")
    if tool is None:
        return None
    box = {}

    def sample():
        time.sleep(seconds / 2)
        try:
            r = subprocess.run([tool, "metric", "-c"], capture_output=True, text=True, timeout=20)
            box["text"] = r.stdout
        except (OSError, subprocess.SubprocessError):
            box["text"] = ""

    th = threading.Thread(target=sample, daemon=True)
    t0 = time.perf_counter()
    th.start()
    n = 0
    while th.is_alive() or time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()  # keep the host within a few steps of the GPU
    torch.cuda.synchronize()
    clk = [int(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)\s*MHz", box.get("text", ""))]
    if not clk:
        return None
    return round(sum(clk) / len(clk), 1), min(clk), max(clk)


def cpu_baseline(w, tensors, target_s: float):
    """The fp64 oracle on a bounded row sample of the same inputs; returns a dict."""
    import numpy as np
    import oracle
    from head_attention_streaming_amd import synthetic

    if tensors is None:  # streaming: time the attention rows of one full-cache step
        import torch
        g = torch.Generator().manual_seed(w.seed)
        q, k, v = synthetic.attention_inputs(w.B, w.Lq, w.Lk, w.Hq, w.Hkv, w.d, w.dtype, w.seed)
    else:
        q, k, v = (t.cpu() for t in tensors)
    dt = w.dtype
    qn = oracle.decode(synthetic.bits(q), dt).reshape(q.shape)
    kn = oracle.decode(synthetic.bits(k), dt).reshape(k.shape)
    vn = oracle.decode(synthetic.bits(v), dt).reshape(v.shape)
    total = w.B * w.Lq * w.Hq
    threads = oracle.default_threads()
    rng = np.random.default_rng(0)

    def run(n):
        rows = np.sort(rng.choice(total, size=min(n, total), replace=False))
        t0 = time.perf_counter()
        oracle.attention(qn, kn, vn, w.scale, w.causal, rows=rows, nthreads=threads, window=w.attn_window)
        return rows, time.perf_counter() - t0

    n = max(threads * 4, 64)
    rows, t = run(n)
    while t < 0.5 and len(rows) < total:
        n *= 4
        rows, t = run(n)
    n_full = min(total, int(len(rows) * target_s / max(t, 1e-6)))
    if n_full > len(rows):
        rows, t = run(n_full)
    # flops of the sampled rows: 4*d per visible key of each row
    fl = 4.0 * w.d * float(visible_keys(w, (rows // w.Hq) % w.Lq).sum())
    full = workload_flops(w)
    return {"value": fl / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} of {total} query rows (random, seed 0), each over all its keys; "
                      f"{t:.1f} s wall, fp64, {threads} threads",
            "seconds": round(t, 2),
            # the whole problem at the sample's rate (every row costs 4*d flops per visible key)
            "full_problem_seconds_extrapolated": round(t * full / fl, 1)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    dev = "cuda:0"
    torch.cuda.set_device(0)
    w, step, kern, info, tensors = make_workload(args.workload, dev, use_ws=not args.no_workspace)

    torch.cuda.synchronize()
    if w is None:  # calibration copy: report GB/s only
        ms, _ = time_loop(step, args.steps, args.warmup)
        gbs = (info["bytes_read"] + info["bytes_written"]) / (ms * 1e-3) / 1e9
        print(json.dumps({"workload": info["workload"], "ms": round(ms, 4), "GB/s": round(gbs, 1), **info}))
        return
    args.warmup = warm_up(step, args.warmup)  # the steps' own warm-up; the count goes into the JSON line
    ms_step, wall_ms = time_loop(step, args.steps, 0)
    ms_kern, _ = time_loop(kern, args.steps, 2) if kern is not step else (ms_step, wall_ms)

    # The sampler reads the instantaneous clock: between the host submissions of launches much
    # shorter than a millisecond the GPU idles and amd-smi reports idle clocks, so only long
    # launches are sampled.
    clock = shader_clock_mhz(kern) if ms_kern >= 1.0 else None
    hbm = {}
    for name, (fn, nbytes) in info.pop("hbm_steps", {}).items():
        ms_h, _ = time_loop(fn, args.steps, args.warmup)
        hbm[name] = {"us": round(ms_h * 1e3, 2), "bytes": nbytes, "GB/s": round(nbytes / (ms_h * 1e-3) / 1e9, 1),
                     "frac_of_8TB/s": round(nbytes / (ms_h * 1e-3) / 1e9 / PEAK_HBM, 3)}
    if hbm:
        info["hbm_kernels"] = hbm

    flops = workload_flops(w)
    fp8 = w.dtype == "e4m3" or w.cache_dtype == "e4m3"
    peak = PEAK_MFMA_FP8 if w.fp8_probs else PEAK_MFMA_FP8_F16 if fp8 else PEAK_MFMA_16BIT
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (ms_kern * 1e-3) / 1e12
    traffic = traffic_from_profile(w.name)
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3" if fp8 else w.dtype,
        "data": "synthetic",
        "config": dict(info, flops_per_step=flops, pct_of_bf16_peak=round(100 * value / PEAK_MFMA_16BIT, 2),
                       wall_ms_per_step=round(wall_ms, 4),
                       shader_clock_mhz=None if clock is None else
                       {"mean": clock[0], "min": clock[1], "max": clock[2],
                        "how": "amd-smi metric -c, every XCD, read while the kernel ran back to back "
                               "right after the timed steps"},
                       **({} if ms_kern >= 1.0 else
                          {"shader_clock_note": "not sampled: launches under 1 ms leave the GPU idle "
                                                "between host submissions, where amd-smi reads idle clocks"})),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1), "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": f"attn_fwd_kernel<{w.d},{('e4m3p8' if w.fp8_probs else 'e4m3') if fp8 else w.dtype}>",
                     "kernel_ms": round(ms_kern, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, tensors, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
