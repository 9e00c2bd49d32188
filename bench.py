"""Benchmark of the low-bit MLA decode hot path on one MI355X.

One step = the whole path on one batch: the fused quantize-append of one new
token per sequence (the writer, including the recent-window migration) and
one split-KV decode + log-sum-exp combine over every sequence's full
context.  Inputs are synthetic (seeded generator, shapes and value
distributions of the pages' MLA models) and resident in HBM before timing.

Prints one JSON line: KV tokens/s (sum of context lengths decoded per
second), the decode kernel's roofline fraction (algorithmic bytes or flops
per launch / its own duration from HIP events on its stream) and the CPU
oracle's throughput on a bounded sample.

    python bench.py [--workload dsv3_c4r4_128k] [--steps 50] [--warmup 10]

With --bf16-sweep it instead times the decode call (plan + decode + combine)
of the same kernels on a C4R4 cache and on an all-bf16 cache (recent window
>= N, so every token is read from bf16) at the workload's head count, for
contexts 1K..1M at batch 8 and 32, the comparison the pages make between the
low-bit and the bf16 cache; one JSON line with every point.  With --mtp it
times the decode of 1, 2 and 4 query tokens per sequence (speculative steps,
causal visibility) on the workload's cache: the queries share one read of it.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
DEFAULT_WORKLOAD = "dsv3_c4r4_128k"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--instances", type=int, default=3,
                    help="cache copies rotated across steps so the 256 MB Infinity Cache cannot serve them")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--bf16-sweep", action="store_true",
                    help="C4R4 vs all-bf16 decode latency at contexts 1K..1M, batch 8 and 32")
    ap.add_argument("--mtp", action="store_true",
                    help="decode of 1, 2 and 4 query tokens per sequence on the workload's cache")
    ap.add_argument("--sweep-contexts", default="1024,4096,16384,65536,131072,1048576")
    ap.add_argument("--sweep-batches", default="8,32")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def kv_bytes_per_token(bits_c: int) -> int:
    return 512 * bits_c // 8 + 32 + 36


def algorithmic(seq_lens, heads, bits_c, n_bf=132):
    """Algorithmic bytes and flops of one decode over these lengths.

    bytes/seq = packed bytes of non-bf16 tokens + 1152 B per bf16 token + 4 B per page-table entry
                + H * (576*2 q + 512*2 out + 4 lse);  flops/seq = 2 * H * (576 + 512) * N."""
    n = np.asarray(seq_lens, dtype=np.int64)
    nb = np.minimum(n, n_bf)
    by = kv_bytes_per_token(bits_c) * (n - nb) + 1152 * nb + 4 * ((n + 63) // 64) + heads * (1152 + 1024 + 4)
    fl = 2 * heads * (576 + 512) * n
    return int(by.sum()), int(fl.sum())


class Hip:
    """hipEvent timing through the HIP runtime (events recorded on the kernels' own stream)."""

    def __init__(self):
        import glob
        cands = ["libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"] + glob.glob("/opt/rocm*/lib/libamdhip64.so*")
        for c in cands:
            try:
                self.L = ctypes.CDLL(c)
                break
            except OSError:
                continue
        P = ctypes.c_void_p
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(P)]
        self.L.hipEventRecord.argtypes = [P, P]
        self.L.hipEventSynchronize.argtypes = [P]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
        self.L.hipEventDestroy.argtypes = [P]

    def event(self):
        e = ctypes.c_void_p()
        assert self.L.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, ev, stream):
        assert self.L.hipEventRecord(ev, stream) == 0

    def elapsed_ms(self, a, b):
        f = ctypes.c_float()
        assert self.L.hipEventSynchronize(b) == 0
        assert self.L.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return float(f.value)


def cpu_baseline(w, budget_s):
    """The oracle as it stands (quantize -> select -> exact fp64 attention), all heads, on the first
    sequences of the workload, scaled to KV tokens/s."""
    import mla_inputs as mi
    import oracle
    q = mi.queries(w.seed, w.batch, w.heads)
    tokens, t_used, seqs, heads_done = 0, 0.0, 0, w.heads
    order = np.argsort(-w.seq_lens)  # longest first
    for b in order:
        n = int(w.seq_lens[b])
        rows = mi.rows(w.seed, int(b), n, threads=16)
        t0 = time.perf_counter()
        oracle.decode_sequence(rows, q[b], w.scale, w.bits_c)
        t_used += time.perf_counter() - t0
        tokens += n
        seqs += 1
        if t_used >= budget_s:
            break
    return {"value": tokens / t_used, "unit": "KV tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{seqs} sequence(s) x {heads_done} heads, {tokens} context tokens, quantize+select+"
                      f"fp64 attention, {t_used:.1f} s wall"}


def cpu_model():
    """The host CPU's model name (first "model name" line of /proc/cpuinfo), or the platform's."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def _code_only(text):
    """C/C++ source without its comments and blank lines (string literals kept as they are)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"':  # string literal: copied through its closing quote
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            while i < n and text[i] != "\n":
                i += 1
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return "\n".join(l.rstrip() for l in "".join(out).splitlines() if l.strip())


def source_digest():
    """Digest of the decode kernels' code (comments and blank lines excluded): the committed counter
    summaries name the digest of the code they were taken on."""
    h = hashlib.sha256()
    for f in ("decode.hip", "decode64.hip", "decode16.hip", "decode_common.h", "mla_internal.h"):
        h.update(_code_only(open(os.path.join(ROOT, "bit_mla_kv_amd", "csrc", f)).read()).encode())
    return h.hexdigest()[:16]


def committed_traffic(workload):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, if it was taken on the
    current decode source (else None)."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"decode source digest: `([0-9a-f]+)`", txt)
    m_val = re.search(r"HBM bytes per decode launch \(calibrated\): ([0-9.eE+]+)", txt)
    if not (m_src and m_val) or m_src.group(1) != source_digest():
        return None
    return float(m_val.group(1))


def committed_mfma_busy(workload):
    """Fraction of the matrix cores' cycles busy during the decode kernel (SQ_VALU_MFMA_BUSY_CYCLES
    over 1024 SIMDs x 2.4 GHz x the kernel's duration), from the committed rocprofv3 SQ counter
    summary, if it was taken on the current decode source (else None)."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_sq_counters.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"decode source digest: `([0-9a-f]+)`", txt)
    m_row = re.search(r"^\| `decode(?:64|16)_kernel<\d>` \|.*\| ([0-9.]+) \|$", txt, re.M)
    if not (m_src and m_row) or m_src.group(1) != source_digest():
        return None
    return float(m_row.group(1))


def bf16_sweep(args):
    """Decode latency of a C4R4 cache vs an all-bf16 cache (n_recent >= N) on the same kernels.
    Every sequence holds the same synthetic rows (the timing does not depend on the values); both
    caches are filled through the HIP writer from one device copy of the rows."""
    import torch
    import mla_inputs as mi
    import bit_mla_kv_amd as m
    from bit_mla_kv_amd import cache_builder as cb

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = mi.workload(args.workload)
    H = w.heads
    contexts = [int(x) for x in args.sweep_contexts.split(",")]
    batches = [int(x) for x in args.sweep_batches.split(",")]
    n_max = max(contexts)
    rows = cb.to_device_bf16(mi.rows(w.seed, 0, n_max, mi.outlier_channels(w.seed), threads=16), dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    hip = Hip()
    steps, warm = max(3, min(args.steps, 20)), max(1, min(args.warmup, 5))

    def fill(layout, B, N):
        """Prefill every slot through the writer in chunks of up to 1M tokens a call; returns the
        cache and the writer's GPU time (HIP events around its calls only)."""
        cache = cb.allocate_for(layout, [N] * B, mi.page_permutation(w.seed, B * ((N + 63) // 64) + 8), device=dev)
        lens = torch.full((B,), N, dtype=torch.int32, device=dev)
        calls = []
        for b in range(B):
            for c0 in range(0, N, 1 << 20):
                c1 = min(N, c0 + (1 << 20))
                calls.append((torch.full((c1 - c0,), b, dtype=torch.int32, device=dev),
                              torch.arange(c0, c1, dtype=torch.int32, device=dev), c0, c1))
        torch.cuda.synchronize()
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, sh)
        for sl, pos, c0, c1 in calls:
            m.quantize_append(cache, rows[c0:c1], sl, pos, lens, stream=sh)
        hip.record(e1, sh)
        return cache, hip.elapsed_ms(e0, e1)

    def time_decode(cache, B, N):
        q = cb.to_device_bf16(mi.queries(w.seed, B, H).reshape(B * H, -1), dev).view(B, H, 576)
        out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        ws = m.alloc_workspace(cache.layout, B, H, N, dev)
        slots = torch.arange(B, dtype=torch.int32, device=dev)
        lens = torch.full((B,), N, dtype=torch.int32, device=dev)
        for _ in range(warm):
            m.decode(cache, q, slots, lens, N, w.scale, out, lse, ws, stream=sh)
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, sh)
        for _ in range(steps):
            m.decode(cache, q, slots, lens, N, w.scale, out, lse, ws, stream=sh)
        hip.record(e1, sh)
        torch.cuda.synchronize()
        return hip.elapsed_ms(e0, e1) / steps

    points = []
    for B in batches:
        for N in contexts:
            res = {"batch": B, "context": N}
            for mode, layout in (("c4r4", m.make_layout(w.bits_c)), ("bf16", m.make_layout(w.bits_c, 4, max(N, 128)))):
                cache, t_fill = fill(layout, B, N)
                torch.cuda.synchronize()
                if mode == "c4r4":  # prefill of B x N tokens (quantize, pack, sink / ring copies)
                    res["prefill_tokens_per_s"] = round(B * N / (t_fill * 1e-3), 1)
                res[f"{mode}_ms"] = round(time_decode(cache, B, N), 5)
                del cache
                torch.cuda.empty_cache()
            res["c4r4_vs_bf16_pct"] = round(100.0 * (res["c4r4_ms"] / res["bf16_ms"] - 1.0), 2)
            print(json.dumps(res), file=sys.stderr, flush=True)
            points.append(res)
    print(json.dumps({"metric": "decode latency, C4R4 cache vs all-bf16 cache on the same kernels",
                      "unit": "ms per decode call (plan + decode + combine)", "n_gpus": 1, "heads": H,
                      "bits": f"C{w.bits_c}R4", "steps": steps, "warmup": warm, "data": "synthetic",
                      "points": points}))


def mtp(args):
    """Decode of q_len = 1, 2, 4 query tokens per sequence on one cache of the workload's shape."""
    import torch
    import mla_inputs as mi
    import bit_mla_kv_amd as m
    from bit_mla_kv_amd import cache_builder as cb

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = mi.workload(args.workload)
    B, H = w.batch, w.heads
    lens = w.seq_lens.astype(np.int64)
    layout = m.make_layout(w.bits_c)
    cache = cb.allocate_for(layout, lens, mi.page_permutation(w.seed, int(((lens + 63) // 64).sum()) + 8), device=dev)
    outl = mi.outlier_channels(w.seed)
    for b in range(B):
        cb.prefill(cache, b, mi.rows(w.seed, b, int(lens[b]), outl, threads=16))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    hip = Hip()
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    max_len = int(lens.max())
    steps, warm = max(3, min(args.steps, 30)), max(1, min(args.warmup, 5))
    points = []
    for q_len in (1, 2, 4):
        q = cb.to_device_bf16(mi.queries(w.seed, B * q_len, H).reshape(B * q_len * H, -1), dev).view(B, q_len, H, 576)
        out = torch.empty((B, q_len, H, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, q_len, H), dtype=torch.float32, device=dev)
        ws = m.alloc_workspace(layout, B, q_len * H, max_len, dev)
        for _ in range(warm):
            m.decode_multi(cache, q, slots, sl, max_len, w.scale, out, lse, ws, stream=sh)
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, sh)
        for _ in range(steps):
            m.decode_multi(cache, q, slots, sl, max_len, w.scale, out, lse, ws, stream=sh)
        hip.record(e1, sh)
        ms = hip.elapsed_ms(e0, e1) / steps
        points.append({"q_len": q_len, "ms": round(ms, 5), "ms_per_query": round(ms / q_len, 5),
                       "kv_tokens_per_s": round(float(lens.sum()) / (ms * 1e-3), 1)})
    print(json.dumps({"metric": "multi-token query decode (plan + decode + combine) on one cache",
                      "unit": "ms per decode call", "n_gpus": 1, "workload": w.name, "batch": B, "heads": H,
                      "context": int(max_len), "steps": steps, "warmup": warm, "data": "synthetic",
                      "points": points}))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the low-bit MLA decode path is built and timed on a single "
              "MI355X (run without --gpus or with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.bf16_sweep:
        bf16_sweep(args)
        return
    if args.mtp:
        mtp(args)
        return

    import torch
    import mla_inputs as mi
    import bit_mla_kv_amd as m
    from bit_mla_kv_amd import cache_builder as cb

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = mi.workload(args.workload)
    B, H, bits = w.batch, w.heads, w.bits_c
    total_steps = args.warmup + args.steps
    R = max(1, args.instances)
    # every instance receives one new token per sequence each R steps
    grow = (total_steps + R - 1) // R
    final_lens = w.seq_lens.astype(np.int64)
    start_lens = np.maximum(final_lens - grow, 1) if w.steps_append == 0 else final_lens
    max_len = int((start_lens + grow).max())
    layout = m.make_layout(bits)

    t_setup = time.perf_counter()
    perm = mi.page_permutation(w.seed, int(((start_lens + grow + 63) // 64).sum()) + 8)
    base = cb.allocate_for(layout, start_lens, perm, spare_tokens=grow, device=dev)
    outl = mi.outlier_channels(w.seed)
    new_rows = np.empty((grow, B, 576), np.uint16)
    for b in range(B):
        n0 = int(start_lens[b])
        rows = mi.rows(w.seed, b, n0 + grow, outl, threads=16)
        cb.prefill(base, b, rows[:n0])
        new_rows[:, b] = rows[n0:n0 + grow]
        del rows
    torch.cuda.synchronize()
    caches = [base]
    for _ in range(R - 1):
        c = m.PagedCache(layout, base.pages.clone(), base.sink.clone(), base.recent.clone(), base.block_table.clone())
        caches.append(c)
    lens = [start_lens.astype(np.int64).copy() for _ in range(R)]
    q = cb.to_device_bf16(mi.queries(w.seed, B, H).reshape(B * H, -1), dev).view(B, H, 576)
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = m.alloc_workspace(layout, B, H, max_len, dev)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    new_dev = cb.to_device_bf16(new_rows.reshape(grow * B, 576), dev).view(grow, B, 576)
    # per-step positions / lengths, prepared before timing: step i appends at lens_i and decodes lens_i + 1
    plan = []
    for i in range(total_steps):
        r = i % R
        pos = lens[r].copy()
        lens[r] += 1
        plan.append((r, i // R, torch.tensor(pos, dtype=torch.int32, device=dev),
                     torch.tensor(pos + 1, dtype=torch.int32, device=dev), pos + 1))
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    hip = Hip()
    ev_k = [(hip.event(), hip.event()) for _ in range(args.steps)]

    def step(i, timed_idx=None):
        r, k, pos, after, _ = plan[i]
        m.quantize_append(caches[r], new_dev[k], slots, pos, after, stream=sh)
        if timed_idx is not None:
            m.profile_decode_events(*ev_k[timed_idx])
        m.decode(caches[r], q, slots, after, max_len, w.scale, out, lse, ws, stream=sh)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    tokens = sum(int(plan[args.warmup + j][4].sum()) for j in range(args.steps))
    t0 = time.perf_counter()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, sh)
    for j in range(args.steps):
        step(args.warmup + j, j)
    hip.record(e1, sh)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = hip.elapsed_ms(e0, e1)
    k_ms = [hip.elapsed_ms(a, b) for a, b in ev_k]
    k_avg_ms = float(np.mean(k_ms))
    ms_per_step = total_ms / args.steps
    value = tokens / (total_ms * 1e-3)

    # decode-kernel roofline on the average timed launch
    alg = [algorithmic(plan[args.warmup + j][4], H, bits) for j in range(args.steps)]
    by_per_launch = float(np.mean([a[0] for a in alg]))
    fl_per_launch = float(np.mean([a[1] for a in alg]))
    gbs = by_per_launch / (k_avg_ms * 1e-3) / 1e9
    tfs = fl_per_launch / (k_avg_ms * 1e-3) / 1e12
    t_hbm = by_per_launch / (HBM_PEAK_GBS * 1e9)
    t_mfma = fl_per_launch / (MFMA_F16_PEAK_TFLOPS * 1e12)
    traffic = committed_traffic(args.workload)
    if t_mfma > t_hbm:
        roof = {"bound": "mfma", "achieved": round(tfs, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tfs / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)

    res = {
        "metric": "C4R4 MLA decode: KV tokens/s and achieved HBM GB/s (% of peak), 128K ctx",
        "value": round(value, 1), "unit": "KV tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded generator: c ~ N(0,1) with 8 outlier channels x20, k_r = RoPE(N(0,1)), "
                "q ~ N(0,1), bf16)",
        "config": {"workload": w.name, "batch": B, "heads": H, "d_c": 512, "d_r": 64,
                   "bits": f"C{bits}R4", "context": int(max_len) if w.steps_append == 0 else "log-uniform 1K-128K",
                   "page_tokens": 64, "sink": 4, "recent": 128, "kv_tokens_per_step": int(tokens / args.steps),
                   "cache_instances": R, "parallelism": "single GPU"},
        "hbm_gbps_algorithmic": round(gbs, 1), "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "decode_kernel_ms": round(k_avg_ms, 5), "decode_kernel_ms_p10_p90": [round(float(np.percentile(k_ms, 10)), 5),
                                                                           round(float(np.percentile(k_ms, 90)), 5)],
        "roofline": roof,
        "mfma_busy_counter": committed_mfma_busy(args.workload),
        "cpu_baseline": cpu,
        "setup_s": round(t_setup, 1), "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
