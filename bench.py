"""Benchmark of the routed-attention hot path on one MI355X.

Headline (``value``): mixed-bit KV decode bandwidth on the 1.3B-shaped decode workload --
24 layers x 32 sequences x 16 heads x head_dim 128, cached context 8192, widths
{2: .3, 4: .4, 8: .2, 16: .1}, modes {skip: .2, local: .4, full: .4}, w = 512.  One step =
for every layer: quantize-write the new token of every sequence (Eq. 4) and run routed decode
attention (Eq. 2) over the cache.  After each step the layers are truncated back to 8192
cached tokens, so every step sees the same context.

Second object (``prefill``): routed prefill on the 160M-shaped workload -- 12 layers x 4
sequences x T = 2048 x 12 heads x head_dim 64, w = 256; one step = the 12 layer calls
(quantize-write of the prompt, then causal routed attention), tokens/s = 4 * 2048 / step time.

Third object (``gqa``): the same two measurements on grouped-query variants of the two
workloads (decode: 16 query heads over 4 KV heads; prefill: 12 over 3), without a CPU baseline.

Fourth object (``baselines``): the pages' comparison points run through the same kernels on the
same shapes -- dense (every token bf16, every head full), KV quantization only at one width for
every token (b = 4, b = 2; every head full), routing only (bf16 cache, routed modes) and TriRoute
-- for decode (4 layers of the 1.3B-shaped decode) and prefill (the 160M-shaped prefill), each
with its time per layer and its speedup over dense.

Fifth object (``controller``): the routing controller (Eq. 5, Eq. 11, hard argmax) that writes
the mode and width arrays, timed on one layer's tokens for the 160M and 1.3B prefill shapes and a
1.3B decode step, with random weights.

Sixth object (``moe``): the expert FFN of Eq. 3 (8 SwiGLU experts plus the null expert, top-2),
timed on one layer's tokens for the 160M and 1.3B shapes and a 1.3B decode step, random weights.

Seventh object (``small``): the workloads whose whole step fits in the 256 MB last-level cache --
the tiny prefill (T = 256, 4 heads), the 160M decode (8 sequences, 2048 cached, 12 heads) and
the 1.3B long-context decode (1 sequence, 65536 cached) -- timed iteration by iteration with the
last-level cache evicted before each (a 512 MB buffer rewritten), the median reported.

The line also carries the seed of the inputs, the sha256 of the library's sources and the git
revision (null where the tree has no .git).

Accounting (algorithmic, from the realized seeded draws):
  decode bytes  = per attended (key, KV head): 2*D*b/8 codes + 16 B (s, z of K and V) for b < 16,
                  4*D for b = 16, counted once over the union of the windows of the query heads
                  that read the KV head; plus per non-skip (seq, query head) 2*D (q); per (seq,
                  query head) 2*D (out); plus the new token's write: 4*D read + its stored bytes
                  per KV head.
  prefill flops = 4*D per attended (query, key, head) pair.

Timing: warmup steps, then K steps between HIP events on the launch stream (torch's current
stream), synchronized on both sides.  A second pass of the same steps with the library's
per-kernel event timing enabled gives each kernel's average launch duration (roofline).
The CPU oracle (``cpu_baseline``) is timed on a bounded sample of the same inputs, on this host,
in spawned worker processes (one BLAS thread each, up to 16): decode = all 32 sequences of layer
0, each the step repeated --cpu-reps times (Eq. 4 on the new token, then Eq. 2 for its heads) on
a cache quantized beforehand (untimed); prefill = the whole step, one job per (layer, sequence).
Its value = the sample's algorithmic bytes (tokens) / (timed work / workers).
"""

from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import CONFIGS, layer_inputs  # noqa: E402

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s

# HBM traffic of the dominant kernels from rocprofv3 PMC passes (FETCH_SIZE, then WRITE_SIZE,
# KiB per dispatch, averaged over the timed launches), each divided by what the same counter
# read per byte of a plain 1 GiB device-to-device copy in the same run (``--calib-copy-mib``).
# Keyed by (kernel, workload): a figure describes one kernel on one workload only.  ``sources``
# lists the files the kernel is built from and their sha256 when the counters were taken: once
# any of them changes the figures no longer describe the kernel and the bench reports traffic
# as null.
TRAFFIC = {
    ("k_decode", "1.3b-decode-L24-B32-C8192-H16-D128"): {
        "fetch_kib": 175694.5, "write_kib": 2623.0, "fetch_per_byte": 0.500101, "write_per_byte": 1.0,
        "profile": "profiles/k_decode_1.3b-decode-L24-B32-C8192-H16-D128.md",
        "sources": {
            "mixed_precision_kv_tr_amd/csrc/decode.cpp.hip": "a45df512c8053dd187f88531bde9651dc0672ced2f92470d335e88e354bc64ae",
            "mixed_precision_kv_tr_amd/csrc/common.h": "ff7f42e41c0f7a910aa65712bb1a08697c255e0874e1a77bccd1b967ce083556",
            "mixed_precision_kv_tr_amd/csrc/layout.h": "68327b740f988dfc84020652ed95c482ff0a871587eefe9dfba27d8ca782d454",
            "include/triroute.h": "a878c5fe6a6d6f81c3e4f878b7ce714770ac11b44a59e099e3ba3d3b5428bee2",
        },
    },
    ("k_decode", "1.3b-gqa-decode-L24-B32-C8192-H16-KV4-D128"): {
        "fetch_kib": 89435.0, "write_kib": 4640.3, "fetch_per_byte": 0.500103, "write_per_byte": 1.0,
        "profile": "profiles/k_decode_1.3b-gqa-decode-L24-B32-C8192-H16-KV4-D128.md",
        "sources": {
            "mixed_precision_kv_tr_amd/csrc/decode.cpp.hip": "a45df512c8053dd187f88531bde9651dc0672ced2f92470d335e88e354bc64ae",
            "mixed_precision_kv_tr_amd/csrc/common.h": "ff7f42e41c0f7a910aa65712bb1a08697c255e0874e1a77bccd1b967ce083556",
            "mixed_precision_kv_tr_amd/csrc/layout.h": "68327b740f988dfc84020652ed95c482ff0a871587eefe9dfba27d8ca782d454",
            "include/triroute.h": "a878c5fe6a6d6f81c3e4f878b7ce714770ac11b44a59e099e3ba3d3b5428bee2",
        },
    },
    ("k_prefill_attn", "160m-prefill-L12-B4-T2048-H12-D64"): {
        "fetch_kib": 19258.2, "write_kib": 19043.9, "fetch_per_byte": 0.500103, "write_per_byte": 1.0,
        "profile": "profiles/k_prefill_attn_160m-prefill-L12-B4-T2048-H12-D64.md",
        "sources": {
            "mixed_precision_kv_tr_amd/csrc/prefill.cpp.hip": "af4ba0a1ed87eba042bc59e7c0e7eb069b4e8043c4b5a0d229a4430e331ee717",
            "mixed_precision_kv_tr_amd/csrc/common.h": "ff7f42e41c0f7a910aa65712bb1a08697c255e0874e1a77bccd1b967ce083556",
            "mixed_precision_kv_tr_amd/csrc/layout.h": "68327b740f988dfc84020652ed95c482ff0a871587eefe9dfba27d8ca782d454",
            "mixed_precision_kv_tr_amd/csrc/kv_write.h": "e9bf3bbc3fdaf24942e01dc74f503c5dda652b9b89b312eb428744f02eef8ca8",
            "include/triroute.h": "a878c5fe6a6d6f81c3e4f878b7ce714770ac11b44a59e099e3ba3d3b5428bee2",
        },
    },
    ("k_prefill_attn", "160m-gqa-prefill-L12-B4-T2048-H12-KV3-D64"): {
        "fetch_kib": 19111.8, "write_kib": 19052.2, "fetch_per_byte": 0.500103, "write_per_byte": 1.0,
        "profile": "profiles/k_prefill_attn_160m-gqa-prefill-L12-B4-T2048-H12-KV3-D64.md",
        "sources": {
            "mixed_precision_kv_tr_amd/csrc/prefill.cpp.hip": "af4ba0a1ed87eba042bc59e7c0e7eb069b4e8043c4b5a0d229a4430e331ee717",
            "mixed_precision_kv_tr_amd/csrc/common.h": "ff7f42e41c0f7a910aa65712bb1a08697c255e0874e1a77bccd1b967ce083556",
            "mixed_precision_kv_tr_amd/csrc/layout.h": "68327b740f988dfc84020652ed95c482ff0a871587eefe9dfba27d8ca782d454",
            "mixed_precision_kv_tr_amd/csrc/kv_write.h": "e9bf3bbc3fdaf24942e01dc74f503c5dda652b9b89b312eb428744f02eef8ca8",
            "include/triroute.h": "a878c5fe6a6d6f81c3e4f878b7ce714770ac11b44a59e099e3ba3d3b5428bee2",
        },
    },
}

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 MFMA, TFLOP/s
METRIC = "mixed-bit KV decode GB/s (% HBM peak); routed prefill tokens/s (% MFMA peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def row_bytes(b: np.ndarray, D: int) -> np.ndarray:
    """Stored bytes of one (token, head): K and V codes plus fp32 (s, z) pairs, or bf16."""
    return np.where(b == 16, 4 * D, 2 * D * b // 8 + 16)


def decode_layer_bytes(bits: np.ndarray, mode: np.ndarray, C: int, w: int, D: int, kv_heads: int = 0):
    """Algorithmic bytes of one decode layer: (split-kernel bytes, whole-layer bytes).

    bits [B, C+1] (position C is the new token), mode [B, H] over H query heads; kv_heads KV
    heads (0 = H), query head h reading KV head h // (H / kv_heads).  A KV head's rows are
    counted once over the union of the windows of the query heads that read it."""
    B, H = mode.shape
    Hkv = kv_heads or H
    G = H // Hkv
    rb = row_bytes(bits.astype(np.int64), D)               # [B, C+1]
    csum = np.concatenate([np.zeros((B, 1), np.int64), np.cumsum(rb, axis=1)], axis=1)
    attn = 0
    for s in range(B):
        for hk in range(Hkv):
            ms = [int(m) for m in mode[s, hk * G:(hk + 1) * G]]
            active = [m for m in ms if m in (1, 2)]
            if not active:
                continue
            lo = 0 if 2 in active else max(0, C - w)
            attn += int(csum[s, C + 1] - csum[s, lo]) + 2 * D * len(active)    # keys + q
    out = B * H * 2 * D
    write = int((4 * D + rb[:, C]).sum()) * Hkv
    return attn, attn + out + write


def prefill_layer_flops(mode: np.ndarray, w: int, D: int) -> int:
    """4*D per attended pair; mode [B, T, H]."""
    B, T, H = mode.shape
    t = np.arange(T)
    keys = np.where(mode == 2, (t + 1)[None, :, None], np.where(mode == 1, (np.minimum(t, w) + 1)[None, :, None], 0))
    return int(keys.sum()) * 4 * D


def pool_pages_needed(bits_layers, P: dict, slack: int = 4) -> int:
    total = 0
    for bits in bits_layers:                               # [B, T] per layer
        for b, p in P.items():
            cnt = (bits == b).sum(axis=1)
            total += int(np.ceil(cnt / p).sum())
        total += slack * bits.shape[0]
    return total


def _sha256(path: str) -> str:
    import hashlib
    with open(os.path.join(ROOT, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(kernel: str, workload: str):
    """Calibrated HBM bytes per launch of ``kernel`` on ``workload`` if its sources are unchanged,
    else None."""
    t = TRAFFIC.get((kernel, workload))
    if not t or any(_sha256(f) != h for f, h in t["sources"].items()):
        return None
    return int(t["fetch_kib"] * 1024 / t["fetch_per_byte"] + t["write_kib"] * 1024 / t["write_per_byte"])


SOURCE_GLOBS = ("mixed_precision_kv_tr_amd/csrc", "include", "workloads")


def source_digest() -> str:
    """sha256 (first 16 hex digits) over the kernel sources, the header, the workload generator
    and this file: identifies the code a line was measured with (the GPU machine has no git)."""
    import hashlib
    h = hashlib.sha256()
    files = [os.path.join(d, f) for d in SOURCE_GLOBS for f in sorted(os.listdir(os.path.join(ROOT, d)))
             if os.path.isfile(os.path.join(ROOT, d, f)) and not f.endswith(".pyc")]
    for rel in sorted(files) + ["bench.py"]:
        h.update(rel.encode())
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def git_sha():
    """HEAD's commit if this tree is a git checkout, else None."""
    import subprocess
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        return r.stdout.strip() or None if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        return None


def built_from():
    """The commit the library was built from, as recorded by the build (None if not recorded)."""
    try:
        with open(os.path.join(ROOT, "mixed_precision_kv_tr_amd", "_build", "REVISION")) as f:
            return f.read().strip() or None
    except OSError:
        return None


def copy_calibration(mib: int, reps: int = 5):
    """Plain device-to-device copies of a known size, for scaling the PMC byte counters.

    uint8 -> int8, so torch runs its elementwise copy kernel (n bytes read, n written) rather
    than a DMA blit that the counters would not see."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(n, dtype=torch.int8, device="cuda")
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[calib] {reps} copies of {n} bytes")
    del src, dst


def time_graph(step, calls: int, replays: int = 10) -> float:
    """ms per call of `step` captured `calls` times in one HIP graph (torch.cuda.graph) and
    replayed `replays` times between HIP events: the device time of back-to-back calls without
    the host's per-call launch cost, as a serving loop that replays a captured step sees it.
    `step` takes the capture stream's handle."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step(s.cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = torch.cuda.current_stream().cuda_stream
        for _ in range(calls):
            step(st)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (replays * calls)


def time_steps(step, K: int) -> float:
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(K):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / K


LLC_FLUSH_BYTES = 512 << 20      # > the 256 MB last-level cache (Infinity Cache)


def time_iters(step, iters: int, flush_buf=None) -> list:
    """Per-iteration HIP-event times (ms) on the current stream.  With flush_buf, the buffer is
    rewritten between iterations, outside the events, so that every iteration starts with a
    cold last-level cache."""
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    evs = []
    for i in range(iters):
        if flush_buf is not None:
            flush_buf.fill_(i & 0x7f)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


# --------------------------------------------------------------------------------------------
# CPU oracle baseline (runs in spawned worker processes on this host, one BLAS thread each)

def _oracle_decode_worker(args):
    """One sequence of a decode step: its cached positions 0..C-1 are quantized and dequantized
    first (untimed: the cache exists before the step); then, timed, `reps` times: Eq. 4 on the
    new token C, and Eq. 2 for its one query per head over positions 0..C."""
    import oracle
    q, k, v, bits, mode, C, w, reps = args
    Hkv = k.shape[1]
    k_hat = np.empty(k.shape, dtype=np.float64)
    v_hat = np.empty(v.shape, dtype=np.float64)
    b_old = np.broadcast_to(bits[:C, None].astype(np.int64), (C, Hkv))
    for src, dst in ((k, k_hat), (v, v_hat)):
        c_, s_, z_ = oracle.quantize(src[:C], b_old)
        dst[:C] = oracle.dequantize(c_, s_, z_, b_old)
    b_new = np.full((1, Hkv), int(bits[C]), dtype=np.int64)
    qf = oracle.bf16_bits_to_f32(q).astype(np.float64)[None]
    t0 = time.perf_counter()
    for _ in range(reps):
        for src, dst in ((k, k_hat), (v, v_hat)):
            c_, s_, z_ = oracle.quantize(src[C:C + 1], b_new)
            dst[C:C + 1] = oracle.dequantize(c_, s_, z_, b_new)
        oracle.routed_attention(qf, k_hat, v_hat, mode[None], np.array([C]), w)
    return time.perf_counter() - t0


def _oracle_prefill_worker(args):
    """One (layer, sequence) of a prefill step, timed whole: Eq. 4 on every token, then Eq. 2 for
    every query."""
    import oracle
    q, k, v, bits, mode, w = args
    t0 = time.perf_counter()
    oracle.attend_cached(q, k, v, bits, mode, np.arange(k.shape[0]), w)
    return time.perf_counter() - t0


def run_pool(fn, jobs, workers):
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers, initializer=_pool_init) as pool:
        t0 = time.perf_counter()
        cpu_times = pool.map(fn, jobs, chunksize=1)
        wall = time.perf_counter() - t0
    return wall, cpu_times


def _pool_init():
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    sys.path.insert(0, ROOT)


def cpu_workers() -> int:
    """Cores this process may run on, capped at the 16 a one-GPU machine gives a job."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# --------------------------------------------------------------------------------------------

def bench_decode(tr, args, cfg=CONFIGS[3], baseline=True, flush=False):
    """Decode steps of a workload: per layer, the new token's quantize-write and routed decode.
    flush: time iterations one by one with the last-level cache evicted before each (workloads
    whose whole step fits in it); the step time is then the median."""
    B, H, D, C, w, Lyr = cfg.batch, cfg.heads, cfg.head_dim, cfg.tokens, cfg.window, cfg.layers
    Hkv = cfg.num_kv_heads
    dev = torch.device("cuda")
    log(f"[decode] generating {Lyr} layers of {cfg.name}")
    per_layer, samples = [], []
    pcb = args.page_code_bytes or 4096
    ptok = {b: pcb * 8 // (D * b) for b in (2, 4, 8, 16)}
    cache = None
    acc_attn, acc_total = [], []
    for layer in range(Lyr):
        case = layer_inputs(cfg, layer, seed=args.seed, device=dev)
        bits_np = case["bits"].cpu().numpy()
        mode_np = case["mode"].cpu().numpy()
        if cache is None:
            # pool sized from layer 0's realized width mix, with 25% headroom for the others
            pool_pages = int(pool_pages_needed([bits_np], ptok) * Lyr * 1.25) + 64
            cache = tr.tr_kv_cache_alloc(Lyr, B, Hkv, D, C + 1, page_code_bytes=args.page_code_bytes,
                                         pool_pages=pool_pages, num_query_heads=H, prefill_tokens=-1)
        tr.tr_kv_quantize_write(cache, layer, case["k"][:, :C].contiguous(), case["v"][:, :C].contiguous(),
                                case["bits"][:, :C].contiguous())
        a, t = decode_layer_bytes(bits_np, mode_np, C, w, D, Hkv)
        acc_attn.append(a)
        acc_total.append(t)
        per_layer.append({x: case[x][:, C:C + 1].contiguous() for x in ("k", "v", "bits")} |
                         {"q": case["q"].contiguous(), "mode": case["mode"].contiguous()})
        if layer == 0 and baseline and not args.no_cpu_baseline:
            for s in range(B):
                samples.append((u16(case["q"][s]), u16(case["k"][s]), u16(case["v"][s]), bits_np[s],
                                mode_np[s], C, w, args.cpu_reps))
        del case
    torch.cuda.synchronize()
    st = tr.tr_kv_cache_status(cache)
    if st != 0:
        raise RuntimeError(f"cache fill failed with status {st}")
    outs = [torch.empty((B, H, D), dtype=torch.bfloat16, device=dev) for _ in range(Lyr)]

    def step():
        for layer in range(Lyr):
            p = per_layer[layer]
            tr.tr_kv_quantize_write(cache, layer, p["k"], p["v"], p["bits"])
            tr.tr_routed_attn_decode(cache, layer, p["q"], p["mode"], w, outs[layer])
        for layer in range(Lyr):
            tr.tr_kv_cache_truncate(cache, layer, C)

    flush_buf = torch.empty(LLC_FLUSH_BYTES, dtype=torch.uint8, device=dev) if flush else None
    for _ in range(args.warmup):
        step()
    log(f"[decode] timing {args.steps} steps" + (" (last-level cache flushed before each)" if flush else ""))
    if flush:
        ms = float(np.median(time_iters(step, args.steps, flush_buf)))
    else:
        ms = time_steps(step, args.steps)
    st = tr.tr_kv_cache_status(cache)
    if st != 0:
        raise RuntimeError(f"decode steps failed with status {st}")
    step_bytes = float(sum(acc_total))
    gbs = step_bytes / (ms * 1e-3) / 1e9

    # per-kernel durations: same steps with event timing inside the library
    tr.tr_profile_read(cache)
    tr.tr_profile_enable(cache, True)
    if flush:
        time_iters(step, args.steps, flush_buf)
    else:
        for _ in range(args.steps):
            step()
    prof = tr.tr_profile_read(cache)
    tr.tr_profile_enable(cache, False)
    n_split, ms_split = prof["decode_split"]
    avg_split_ms = ms_split / max(1, n_split)
    bytes_per_launch = float(np.mean(acc_attn))
    achieved = bytes_per_launch / (avg_split_ms * 1e-3) / 1e9
    kname = "k_decode"
    roof = {"bound": "hbm", "kernel": kname, "traffic_unit": "bytes per launch", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(kname, cfg.name),
            "avg_launch_us": round(avg_split_ms * 1e3, 2), "bytes_per_launch": int(bytes_per_launch),
            "kernels_us_per_step": {k: round(v[1] * 1e3 / args.steps, 1) for k, v in prof.items() if v[0]}}

    cpu = None
    if samples:
        workers = min(cpu_workers(), len(samples))
        log(f"[decode] oracle on {len(samples)} sequences, {workers} worker processes")
        wall, times = run_pool(_oracle_decode_worker, samples, workers)
        s_bytes = 0
        for (q, k, v, bits, mode, C_, w_, reps) in samples:
            s_bytes += decode_layer_bytes(bits[None], mode[None], C_, w_, D, Hkv)[1] * reps
        busy = float(sum(times))
        cpu = {"value": round(s_bytes / (busy / workers) / 1e9, 6), "unit": "GB/s", "cores": workers,
               "kind": "oracle", "cpu_model": cpu_model(),
               "sample": f"layer 0, all {B} sequences of {cfg.name}: per sequence, the step repeated "
                         f"{args.cpu_reps} times (Eq. 4 on the new token, Eq. 2 for its {H} query heads over "
                         f"{C + 1} positions) on a cache quantized beforehand (untimed); {busy:.2f} s of "
                         f"timed work on {workers} worker processes (one BLAS thread each), value = the "
                         f"sample's algorithmic bytes / (timed work / workers)"}
    cache.close()
    return {"ms": ms, "gbs": gbs, "bytes": step_bytes, "roofline": roof, "cpu": cpu, "cfg": cfg}


def bench_prefill(tr, args, cfg=CONFIGS[2], baseline=True, flush=False):
    """Prefill steps of a workload: every layer's quantize-write of the prompt and routed
    attention of its queries.  flush: as for bench_decode."""
    B, H, D, T, w, Lyr = cfg.batch, cfg.heads, cfg.head_dim, cfg.tokens, cfg.window, cfg.layers
    dev = torch.device("cuda")
    log(f"[prefill] generating {Lyr} layers of {cfg.name}")
    cases = [layer_inputs(cfg, layer, seed=args.seed, device=dev) for layer in range(Lyr)]
    flops = [prefill_layer_flops(c["mode"].cpu().numpy(), w, D) for c in cases]
    cache = tr.tr_kv_cache_alloc(Lyr, B, cfg.num_kv_heads, D, T, page_code_bytes=args.page_code_bytes,
                                 num_query_heads=H)
    outs = [torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev) for _ in range(Lyr)]

    def step():
        for layer in range(Lyr):
            c = cases[layer]
            tr.tr_kv_cache_truncate(cache, layer, 0)
            tr.tr_routed_attn_prefill(cache, layer, c["q"], c["k"], c["v"], c["bits"], c["mode"], T, w, outs[layer])

    flush_buf = torch.empty(LLC_FLUSH_BYTES, dtype=torch.uint8, device=dev) if flush else None
    for _ in range(args.warmup):
        step()
    log(f"[prefill] timing {args.steps} steps" + (" (last-level cache flushed before each)" if flush else ""))
    if flush:
        ms = float(np.median(time_iters(step, args.steps, flush_buf)))
    else:
        ms = time_steps(step, args.steps)
    st = tr.tr_kv_cache_status(cache)
    if st != 0:
        raise RuntimeError(f"prefill steps failed with status {st}")
    tok_s = B * T / (ms * 1e-3)
    tflops = sum(flops) / (ms * 1e-3) / 1e12

    tr.tr_profile_read(cache)
    tr.tr_profile_enable(cache, True)
    if flush:
        time_iters(step, args.steps, flush_buf)
    else:
        for _ in range(args.steps):
            step()
    prof = tr.tr_profile_read(cache)
    tr.tr_profile_enable(cache, False)
    n_attn, ms_attn = prof["prefill_attn"]
    avg_ms = ms_attn / max(1, n_attn)
    fl_per_launch = float(np.mean(flops))
    achieved = fl_per_launch / (avg_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "kernel": "k_prefill_attn", "achieved": round(achieved, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("k_prefill_attn", cfg.name), "traffic_unit": "bytes per launch",
            "avg_launch_us": round(avg_ms * 1e3, 2), "flops_per_launch": int(fl_per_launch),
            "kernels_us_per_step": {k: round(v[1] * 1e3 / args.steps, 1) for k, v in prof.items() if v[0]}}
    cpu = None
    if baseline and not args.no_cpu_baseline:
        jobs = []
        for layer, c in enumerate(cases):
            for s in range(B):
                jobs.append((u16(c["q"][s]), u16(c["k"][s]), u16(c["v"][s]), c["bits"][s].cpu().numpy(),
                             c["mode"][s].cpu().numpy(), w))
        workers = min(cpu_workers(), len(jobs))
        log(f"[prefill] oracle on {len(jobs)} (layer, sequence) jobs, {workers} worker processes")
        wall, times = run_pool(_oracle_prefill_worker, jobs, workers)
        busy = float(sum(times))
        cpu = {"value": round(B * T / (busy / workers), 3), "unit": "tokens/s", "cores": workers, "kind": "oracle",
               "cpu_model": cpu_model(),
               "sample": f"the whole step of {cfg.name}: {Lyr} layers x {B} sequences, each job one (layer, "
                         f"sequence): Eq. 4 on its {T} tokens, then Eq. 2 for every query and head; {busy:.2f} s "
                         f"of work on {workers} worker processes (one BLAS thread each), value = "
                         f"{B * T} tokens / (work / workers)"}
    cache.close()
    return {"ms": ms, "tok_s": tok_s, "tflops": tflops, "roofline": roof, "cpu": cpu, "cfg": cfg}


def bench_small(tr, args):
    """The workloads whose step fits in the last-level cache, each timed with the cache evicted
    before every iteration (median of the iterations): the tiny prefill (T = 256, 1 layer), the
    160M-shaped decode step (B = 8, C = 2048) and the long-context decode (B = 1, C = 65536)."""
    out = {}
    r = bench_prefill(tr, args, CONFIGS[0], baseline=False, flush=True)
    out["tiny_prefill"] = {"workload": r["cfg"].name, "value": round(r["tok_s"], 1), "unit": "tokens/s",
                           "us_per_step": round(r["ms"] * 1e3, 2), "tflops": round(r["tflops"], 3),
                           "mfma_frac": round(r["tflops"] / MFMA_BF16_PEAK_TFLOPS, 5), "roofline": r["roofline"]}
    for key, cid in (("decode_160m", 1), ("longctx_decode", 4)):
        r = bench_decode(tr, args, CONFIGS[cid], baseline=False, flush=True)
        out[key] = {"workload": r["cfg"].name, "value": round(r["gbs"], 1), "unit": "GB/s",
                    "us_per_step": round(r["ms"] * 1e3, 2), "hbm_frac": round(r["gbs"] / HBM_PEAK_GBS, 4),
                    "bytes_per_step": int(r["bytes"]), "roofline": r["roofline"]}
    return out


# The pages' baselines as configurations of the same kernels: dense (every token stored as
# bf16, every head attending fully), KV-quantization only (one width for every token, every
# head full; per-token groups like the rest of the cache, not KIVI's per-channel keys), routing
# only (bf16 cache, routed modes) and TriRoute (both).  Same
# shapes, windows and seeded q/k/v as the workload; only the width and mode draws change.
BASELINE_VARIANTS = (
    ("dense_bf16", {16: 1.0}, {"full": 1.0}),
    ("kv_quant_uniform_b4", {4: 1.0}, {"full": 1.0}),
    ("kv_quant_uniform_b2", {2: 1.0}, {"full": 1.0}),
    ("routing_only_bf16", {16: 1.0}, None),
    ("triroute", None, None),
)


def bench_baselines(tr, args):
    """Decode (4 layers of the 1.3B-shaped decode) and prefill (the 160M-shaped prefill) per variant."""
    from dataclasses import replace
    res = {}
    for kind, base, layers in (("decode", CONFIGS[3], args.baseline_layers), ("prefill", CONFIGS[2], None)):
        out = {}
        for name, bw, mw in BASELINE_VARIANTS:
            cfg = replace(base, layers=layers or base.layers, bit_weights=bw or base.bit_weights,
                          mode_weights=mw or base.mode_weights)
            if kind == "decode":
                r = bench_decode(tr, args, cfg, baseline=False)
                out[name] = {"ms_per_layer": round(r["ms"] / cfg.layers, 5), "bytes_per_layer": int(r["bytes"] / cfg.layers),
                             "gbs": round(r["gbs"], 1), "kernel_us": r["roofline"]["avg_launch_us"]}
            else:
                r = bench_prefill(tr, args, cfg, baseline=False)
                out[name] = {"ms_per_layer": round(r["ms"] / cfg.layers, 5), "tok_s": round(r["tok_s"], 1),
                             "tflops": round(r["tflops"], 2), "kernel_us": r["roofline"]["avg_launch_us"]}
        d = out["dense_bf16"]["ms_per_layer"]
        for v in out.values():
            v["speedup_vs_dense"] = round(d / v["ms_per_layer"], 3)
        res[kind] = {"shape": (f"{base.name} shape, {layers or base.layers} layers"), "variants": out}
    return res


def bench_controller(tr, args):
    """Routing controller (Eq. 5 + Eq. 11 + hard argmax) on one layer's tokens: a 160M-shaped
    prefill layer (4 x 2048 tokens, d = 768, 12 heads), a 1.3B-shaped one (d = 2048, 16 heads) and
    a 1.3B decode step (32 tokens).  Random weights (no trained controller exists); 8 side features.
    Bytes: x (2 d per token) + decisions (heads + 1 per token) + the weights once; FLOP: the trunk
    and heads, 2 * (d + 8) * 128 + 2 * 128 * 128 + 2 * 128 * (3 heads + 4) per token.
    us_per_call: 50 calls captured in a HIP graph and replayed (device time, no per-call host
    launch cost); eager_us_per_call: the same calls launched one by one from Python, which for
    the small decode call measures the host's launch rate rather than the kernels."""
    from workloads import controller_case
    out = {}
    for name, M, d, H in (("prefill_160m", 8192, 768, 12), ("prefill_1.3b", 8192, 2048, 16), ("decode_1.3b", 32, 2048, 16)):
        c = controller_case(M, d, H, d_side=8, seed=args.seed, device="cuda")
        mode = torch.empty((M, H), dtype=torch.uint8, device="cuda")
        bits = torch.empty((M,), dtype=torch.uint8, device="cuda")
        cw = tr.ControllerWeights(c["w"])
        stream = torch.cuda.current_stream().cuda_stream
        call = lambda: tr.tr_controller_route(cw, c["x"], c["side"], M, mode, bits, stream)
        for _ in range(5):
            call()
        ms_eager = time_steps(call, 200)
        ms = time_graph(lambda st: tr.tr_controller_route(cw, c["x"], c["side"], M, mode, bits, st), 50)
        wbytes = sum(v.numel() * v.element_size() for v in c["w"].values())
        nbytes = M * (2 * d + 4 * 8 + H + 1) + wbytes
        flops = M * (2 * (d + 8) * 128 + 2 * 128 * 128 + 2 * 128 * (3 * H + 4))
        out[name] = {"tokens": M, "d": d, "heads": H, "us_per_call": round(ms * 1e3, 2),
                     "eager_us_per_call": round(ms_eager * 1e3, 2),
                     "tokens_per_s": round(M / (ms * 1e-3), 1), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
        del c
    return out


def bench_moe(tr, args):
    """Expert FFN (Eq. 3): E = 8 SwiGLU experts plus the null expert, top-2, on one layer's tokens:
    the 160M prefill layer (8192 tokens, d = 768, expert width 1024 = half the model's 2048 FFN),
    the 1.3B one (d = 2048, expert width 2688 ~ half of 5461, rounded to 128) and a 1.3B decode step
    (32 tokens).  Random weights; gate logits N(0, 1).  FLOP: 6 d d_e per (token, non-null expert)."""
    from workloads import moe_case
    out = {}
    for name, M, d, de in (("prefill_160m", 8192, 768, 1024), ("prefill_1.3b", 8192, 2048, 2688),
                           ("decode_1.3b", 32, 2048, 2688)):
        c = moe_case(M, d, de, 8, seed=args.seed, device="cuda")
        moe = tr.tr_moe_alloc(d, de, 8, 2, M)
        tr.tr_moe_set_weights(moe, c["w_gate"], c["w_up"], c["w_down"])
        y = torch.empty((M, d), dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        call = lambda: tr.tr_moe_ffn(moe, c["x"], c["z"], M, y, stream)
        for _ in range(3):
            call()
        ms = time_steps(call, 50)
        chosen = torch.topk(c["z"], 2, dim=1).indices
        active = int((chosen != 0).sum())
        flops = 6.0 * d * de * active
        out[name] = {"tokens": M, "d": d, "d_expert": de, "experts": 8, "top_k": 2, "us_per_call": round(ms * 1e3, 2),
                     "tokens_per_s": round(M / (ms * 1e-3), 1), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                     "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "active_choices": active}
        moe.close()
        del c
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=1234)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=2,
                    help="decode oracle: timed repetitions of each sampled sequence's step")
    ap.add_argument("--only", choices=["decode", "prefill", "small", "gqa_decode", "gqa_prefill", "baselines",
                                       "controller", "moe"], default=None)
    ap.add_argument("--no-small", action="store_true", help="skip the workloads that fit in the last-level cache")
    ap.add_argument("--no-gqa", action="store_true", help="skip the grouped-query workloads")
    ap.add_argument("--no-baselines", action="store_true", help="skip the dense / uniform-width / routing-only runs")
    ap.add_argument("--no-controller", action="store_true", help="skip the routing-controller timing")
    ap.add_argument("--no-moe", action="store_true", help="skip the expert-FFN timing")
    ap.add_argument("--baseline-layers", type=int, default=4, help="decode layers per baseline variant")
    ap.add_argument("--page-code-bytes", type=int, default=0,
                    help="cache page size: K (and V) code bytes per head per page; 0 = the library default")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run plain copies of this many MiB (PMC counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (decode and prefill shard by "
              "(sequence, head) with no exchange; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import mixed_precision_kv_tr_amd as tr

    if args.calib_copy_mib:
        copy_calibration(args.calib_copy_mib)

    dec = bench_decode(tr, args) if args.only in (None, "decode") else None
    pre = bench_prefill(tr, args) if args.only in (None, "prefill") else None
    small = bench_small(tr, args) if (args.only is None and not args.no_small) or args.only == "small" else None
    gqa = args.only is None and not args.no_gqa
    gdec = bench_decode(tr, args, CONFIGS[5], baseline=False) if gqa or args.only == "gqa_decode" else None
    gpre = bench_prefill(tr, args, CONFIGS[6], baseline=False) if gqa or args.only == "gqa_prefill" else None
    base = (bench_baselines(tr, args) if (args.only is None and not args.no_baselines) or args.only == "baselines"
            else None)
    ctl = (bench_controller(tr, args) if (args.only is None and not args.no_controller) or args.only == "controller"
           else None)
    moe = bench_moe(tr, args) if (args.only is None and not args.no_moe) or args.only == "moe" else None

    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "data": "synthetic",
            "seed": args.seed, "source_sha256": source_digest(), "git_sha": git_sha(), "library_built_from": built_from()}
    if dec:
        cfg = dec["cfg"]
        line.update({"value": round(dec["gbs"], 1), "unit": "GB/s", "ms_per_step": round(dec["ms"], 4),
                     "dtype": "fp32", "hbm_frac": round(dec["gbs"] / HBM_PEAK_GBS, 4),
                     "config": {"workload": cfg.name, "layers": cfg.layers, "batch": cfg.batch,
                                "context": cfg.tokens, "heads": cfg.heads, "head_dim": cfg.head_dim,
                                "window": cfg.window, "bytes_per_step": int(dec["bytes"])},
                     "roofline": dec["roofline"], "cpu_baseline": dec["cpu"]})
    if pre:
        cfg = pre["cfg"]
        pobj = {"workload": cfg.name, "value": round(pre["tok_s"], 1), "unit": "tokens/s",
                "ms_per_step": round(pre["ms"], 4), "dtype": "bf16 QK / fp16 PV MFMA, fp32 softmax",
                "tflops": round(pre["tflops"], 2), "mfma_frac": round(pre["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
                "roofline": pre["roofline"], "cpu_baseline": pre["cpu"]}
        if dec:
            line["prefill"] = pobj
        else:
            line.update({"value": pobj["value"], "unit": "tokens/s", "ms_per_step": pobj["ms_per_step"],
                         "dtype": "bf16", "config": {"workload": cfg.name}, "roofline": pobj["roofline"],
                         "cpu_baseline": pobj["cpu_baseline"]})
    if small:
        if "value" in line:
            line["small"] = small
        else:
            o = small["decode_160m"]
            line.update({"value": o["value"], "unit": o["unit"], "ms_per_step": round(o["us_per_step"] / 1e3, 5),
                         "dtype": "fp32", "config": {"workload": o["workload"]}, "roofline": o["roofline"],
                         "cpu_baseline": None, "small": small})
    # grouped-query workloads: same objects, no CPU baseline
    extra = {}
    if gdec:
        extra["decode"] = {"workload": gdec["cfg"].name, "value": round(gdec["gbs"], 1), "unit": "GB/s",
                           "ms_per_step": round(gdec["ms"], 4), "hbm_frac": round(gdec["gbs"] / HBM_PEAK_GBS, 4),
                           "bytes_per_step": int(gdec["bytes"]), "roofline": gdec["roofline"]}
    if gpre:
        extra["prefill"] = {"workload": gpre["cfg"].name, "value": round(gpre["tok_s"], 1), "unit": "tokens/s",
                            "ms_per_step": round(gpre["ms"], 4), "tflops": round(gpre["tflops"], 2),
                            "roofline": gpre["roofline"]}
    if moe:
        if "value" in line:
            line["moe"] = moe
        else:
            line.update({"value": moe["prefill_1.3b"]["tflops"], "unit": "TFLOP/s",
                         "config": {"workload": "expert FFN, 8192 tokens, d = 2048, 8 experts, top-2"}, "moe": moe})
    if ctl:
        if "value" in line:
            line["controller"] = ctl
        else:
            line.update({"value": ctl["prefill_1.3b"]["tokens_per_s"], "unit": "tokens/s",
                         "config": {"workload": "routing controller, 8192 tokens, d = 2048, 16 heads"},
                         "controller": ctl})
    if base:
        if "value" in line:
            line["baselines"] = base
        else:
            line.update({"value": base["decode"]["variants"]["triroute"]["speedup_vs_dense"], "unit": "x vs dense",
                         "config": {"workload": base["decode"]["shape"]}, "baselines": base})
    if extra:
        if "value" in line:
            line["gqa"] = extra
        else:
            o = extra.get("decode") or extra.get("prefill")
            line.update({"value": o["value"], "unit": o["unit"], "ms_per_step": o["ms_per_step"],
                         "dtype": "fp32" if "decode" in extra else "bf16", "config": {"workload": o["workload"]},
                         "roofline": o["roofline"], "cpu_baseline": None})
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
