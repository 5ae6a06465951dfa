"""Benchmark of the MI355X HSA forward (one GPU).

Workloads (synthetic, seeded; shapes of the paper's setting):
  prefill_128K : B=2, L=131072 query rows over their own 131072-token history,
                 32 q heads / 4 kv heads, d=128, top-K 16, bf16.   (headline `value`)
  decode_16M   : 16 single-token queries over one 16,777,216-token history,
                 8 q heads / 1 kv head, d=128, top-K 32, bf16.     (reported beside it)

A step is one hsa_forward call (landmark scan, top-K, per-chunk attention, blend)
over the whole batch, inputs resident in HBM.  Each step is preceded, outside its
HIP-event window, by a 1 GiB read that evicts L2 and the 256 MB Infinity Cache,
so every step starts cold.  ms_per_step is the mean event-timed step (the
call's kernel launches made directly; median, p10 and p90 beside it); the wall
time of the whole timed region (flushes included) is wall_ms_per_step, the same
step without the flush warm_ms_per_step, and the step replayed from a captured
HIP graph (checked bit for bit against the direct call) graph_ms_per_step.

roofline: a second pass of `steps` cold forwards has the library record HIP events
around each kernel stage on the launch stream (hsa_forward_profiled); the stage
with the largest mean duration is the dominant kernel, priced against MI355X
peaks by its algorithmic work per launch:
  decode  scan   -> HBM bytes of the eligible landmarks and q_ret;
          attend -> HBM bytes of the distinct selected chunks' K/V, q_attn, out;
  prefill attend -> bf16 MFMA FLOPs, 4*G*64*d per selection;
          scan   -> bf16 MFMA FLOPs, 2*d per candidate.
  traffic: HBM bytes per launch from two rocprofv3 counter passes (FETCH_SIZE,
  WRITE_SIZE) scaled by a 1 GiB calibration copy, read from the summary under
  profiles/ (null when none exists or the kernel sources changed since).
step_roofline: the whole step against t_roof = max(compulsory bytes / 8 TB/s,
MFMA FLOPs / 2.5 PFLOP/s); frac = t_roof / ms_per_step.
cpu_baseline: the fp64 oracle on a bounded, stratified sample of query rows of the
same workload, timed on this host's cores (test infrastructure, not the product).

Further workloads (--workloads, all in the default run): prefill_32K (the 32K
training window: B=1, 8 q heads / 1 kv head, d=128, top-K 8), chunked_1M
(8,192 new rows appended to a 1,048,576-token history, 32 q / 4 kv heads,
top-K 32; HBM-bound: roofline in bytes), global_32K (top-K covering all 512
chunks of the 32K window: global HSA), backward_32K (hsa_backward on the 32K
window for the forward's selection; roofline on the per-item MFMA kernel,
10*G*64*d FLOP per selection), crossover (HSA forward vs dense causal SDPA
from 4K to 256K tokens by default, --crossover-max up to 1M; also against
dense attention at the bf16 MFMA peak).  Every cpu_baseline names the host's
CPU model and the threads the oracle used.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA
N_SIMDS = 256 * 4                # 256 CUs x 4 SIMDs
N_XCDS = 8                       # GRBM_GUI_ACTIVE comes summed over the 8 XCDs
VALU_FP32_PEAK_TFLOPS = 78.6     # 256 CU x 64 lanes x 2 FLOP (FMA) x 2.4 GHz, non-packed

WORKLOADS = {"prefill_128K": 2, "decode_16M": 3, "prefill_32K": 1, "global_32K": 1, "backward_32K": 1,
             "chunked_1M": 4}
# global_32K: the 32K training-window prefill with a top-K covering all 512
# chunks (global HSA of the warm-up stage); the dense fused kernel runs it
OVERRIDES = {"global_32K": dict(top_k=512, name="global_hsa_32K_gqa8")}

# the kernel behind each (workload, stage) of the plan the library picks for it
KERNELS = {
    ("decode_16M", "scan"): "scan_wide_kernel<true, 128>",
    ("decode_16M", "attend"): "attend_decode_kernel<128, 8>",
    ("decode_16M", "landmarks"): "chunk_landmark_kernel<true, 128>",
    ("global_32K", "attend"): "attend_global_kernel<128, 8, 2>",
    ("chunked_1M", "scan"): "scan_block_kernel<128, 64>",
    ("chunked_1M", "bucket"): "chunk_count/scan/scatter kernels",
    ("chunked_1M", "attend"): "chunk_attend_kernel<128, 8>",
    ("chunked_1M", "combine"): "chunk_combine_kernel<128, 8>",
    ("backward_32K", "bucket"): "chunk_count/scan/scatter + bin_sort kernels",
    ("backward_32K", "attend"): "bwd_item_kernel<128, 8>",
    ("backward_32K", "combine"): "bwd_dq/bwd_chunk/bwd_landmark kernels",
    ("prefill_32K", "scan"): "scan_block_kernel<128, 64>",
    ("prefill_32K", "bucket"): "chunk_count/scan/scatter kernels",
    ("prefill_32K", "attend"): "chunk_attend_kernel<128, 8>",
    ("prefill_32K", "combine"): "chunk_combine_kernel<128, 8>",
    ("prefill_128K", "scan"): "scan_block_kernel<128, 32>",
    ("prefill_128K", "bucket"): "chunk_count/scan/scatter kernels",
    ("prefill_128K", "attend"): "chunk_attend_kernel<128, 8>",
    ("prefill_128K", "combine"): "chunk_combine_kernel<128, 8>",
}
COPY_BYTES = 1 << 30          # calibration copy: 2^28 fp32 read and written
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model() -> str:
    """The host CPU's model name (first processor entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def to_dev(a, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(a).to("cuda:0")


class Timer:
    """Cold-cache timing of one call (all its kernels) with HIP events.

    Each step enqueues a 1 GiB read of an unrelated buffer (evicting L2 and the
    256 MB Infinity Cache with clean lines; a write would leave dirty lines whose
    write-back competes with the timed step), then event e0, the call (its
    kernel launches, or a captured graph's replay), event e1.  The read keeps
    the GPU busy while the host enqueues e0 and the call, so the events bracket
    GPU work only.  Events live on torch's current stream, which is the stream
    the library launches on.  On ROCm a graph replay starts its first kernel
    several microseconds later than the same launches made directly, which
    shows on steps of tens of microseconds."""

    def __init__(self):
        import torch
        self.torch = torch
        self.flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        self.sink = torch.empty((), dtype=torch.float32, device="cuda:0")
        self.pool = []

    def cold(self):
        self.torch.sum(self.flush, dim=0, out=self.sink)

    def events(self, n):
        torch = self.torch
        while len(self.pool) < n:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            e1.record()
            self.pool.append((e0, e1))
        torch.cuda.synchronize()
        return self.pool[:n]

    def capture(self, fn):
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def time(self, graph, steps, flush=True):
        """Graph replays: (mean, median, wall) ms."""
        m = self.time_eager(graph.replay, steps, flush)
        return m["mean"], m["median"], m["wall"]

    def time_eager(self, fn, steps, flush=True):
        """`steps` calls of fn() (each enqueues one step), each bracketed by
        events, after the cache-evicting read when flush.  Returns mean,
        median, p10, p90 of the event times and the host wall time per step,
        all in ms."""
        torch = self.torch
        evs = self.events(steps)
        self.cold()                        # the flush's first launch after a capture is slow on the host
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e0, e1 in evs:
            if flush:
                self.cold()
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        ms = [e0.elapsed_time(e1) for e0, e1 in evs]
        return dict(mean=float(np.mean(ms)), median=float(np.median(ms)), p10=float(np.percentile(ms, 10)),
                    p90=float(np.percentile(ms, 90)), wall=wall * 1e3)


    def stages(self, call, steps):
        """Mean duration (ms) of each kernel stage over `steps` cold eager calls;
        call(evs) runs one forward with the library recording evs[stage] =
        (start, end) on the launch stream."""
        import ultra_long_context_amd as hsa
        torch = self.torch
        evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for n in hsa.STAGES} for _ in range(steps)]
        for d in evs:                      # create the events before the marker
            for e0, e1 in d.values():
                e0.record()
                e1.record()
        marker = torch.cuda.Event(enable_timing=True)
        marker.record()
        for d in evs:
            self.cold()
            call(d)
        torch.cuda.synchronize()
        out = {}
        for n in hsa.STAGES:
            # a stage the plan does not run keeps its events from before the marker
            if all(marker.elapsed_time(d[n][0]) > 0 for d in evs):
                out[n] = float(np.mean([d[n][0].elapsed_time(d[n][1]) for d in evs]))
        return out


def distinct_chunks(idx_t, cfg) -> int:
    """U: distinct (batch, kv head, chunk) triples selected (each chunk's K/V read once)."""
    import torch
    idx = idx_t.to(torch.int64)
    B, Lq, Hkv, K = idx.shape
    nc = cfg.n_chunks
    bg = (torch.arange(B, device=idx.device).view(B, 1, 1, 1) * Hkv
          + torch.arange(Hkv, device=idx.device).view(1, 1, Hkv, 1))
    key = torch.where(idx >= 0, bg * nc + idx, torch.full_like(idx, -1))
    return int(torch.unique(key[key >= 0]).numel())


def algorithmic(cfg, U, elem=2):
    """Compulsory bytes / FLOPs of one forward (landmarks read once, selected chunks once)."""
    B, Lq, Hq, Hkv, d, K = cfg.batch, cfg.q_len, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.top_k
    pos = cfg.q_pos0 + np.arange(Lq, dtype=np.int64)
    n = np.minimum(pos // 64, cfg.n_chunks)
    cand = int(n.sum()) * B * Hkv
    sel = int(np.minimum(n, K).sum()) * B * Hkv
    nmax = int(n.max())
    lm_bytes = B * Hkv * nmax * d * elem
    q_ret = B * Lq * Hkv * d * elem
    qa = B * Lq * Hq * d * elem
    return dict(candidates=cand, selections=sel, landmark_bytes=lm_bytes, q_ret_bytes=q_ret,
                q_attn_bytes=qa, out_bytes=qa, kv_bytes=U * 2 * 64 * d * elem,
                bytes=lm_bytes + q_ret + 2 * qa + U * 2 * 64 * d * elem,
                scan_flops=2 * d * cand, attend_flops=4 * cfg.group * 64 * d * sel,
                bwd_flops=10 * cfg.group * 64 * d * sel, partial_bytes=sel * cfg.group * d * 2)


# source file of each kernel family; a kernel's traffic figure goes stale when
# its file or a shared header changes
KERNEL_FILES = {
    "scan_wide_kernel": "retrieve.hip", "scan_block_kernel": "retrieve.hip", "scan_topk_kernel": "retrieve.hip",
    "attend_decode_kernel": "attend_decode.hip", "merge_lists_kernel": "attend_decode.hip",
    "chunk_attend_kernel": "attend_chunk.hip", "chunk_combine_kernel": "attend_chunk.hip",
    "attend_global_kernel": "attend_global.hip", "chunk_landmark_kernel": "landmarks.hip",
    "bwd_item_kernel": "backward.hip", "bwd_dq_kernel": "backward.hip",
}
SHARED_HEADERS = ("hsa_device.h", "hsa_internal.h")


def source_digest(kernel: str = "") -> str:
    """sha256 over the kernel's source file and the shared device headers (all
    kernel sources for an unknown kernel)."""
    import hashlib
    h = hashlib.sha256()
    src = os.path.join(ROOT, "ultra_long_context_amd", "csrc")
    fam = KERNEL_FILES.get(kernel.split("<")[0])
    files = sorted(os.listdir(src)) if fam is None else [fam, *SHARED_HEADERS]
    for f in files:
        if f.endswith((".hip", ".h")):
            with open(os.path.join(src, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def traffic_file(workload, kernel):
    return os.path.join(PROFILES, "%s_%s_hbm_traffic.txt" % (kernel.split("<")[0], workload))


def mfma_file(workload, kernel):
    return os.path.join(PROFILES, "%s_%s_mfma.txt" % (kernel.split("<")[0], workload))


def summary_fields(path, kernel):
    """key: value lines of a committed counter summary, or None if there is none
    or the kernel sources changed since it was taken."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k_, v_ = line.split(":", 1)
                kv[k_.strip()] = v_.strip()
    if kv.get("source_digest") != source_digest(kernel):
        return None
    return kv


def measured_mfma_busy(workload, kernel):
    """Fraction of SIMD cycles the MFMA unit was busy during the kernel, from the
    committed counter summary (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x
    SIMDs), or None."""
    kv = summary_fields(mfma_file(workload, kernel), kernel)
    return None if kv is None else float(kv["mfma_busy_percent"]) / 100.0


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed counter summary, or None if there
    is none or the kernel sources changed since it was taken."""
    path = traffic_file(workload, kernel)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k_, v_ = line.split(":", 1)
                kv[k_.strip()] = v_.strip()
    if kv.get("source_digest") != source_digest(kernel):
        return None
    return float(kv["traffic_bytes_per_launch"])


def roofline(workload, stage, ms, alg):
    """Roofline entry for one kernel stage: algorithmic bytes or FLOPs per launch
    over its measured duration."""
    kernel = KERNELS.get((workload, stage), stage)
    prefill = workload.startswith("prefill") or workload.startswith("global")
    if stage == "attend" and workload.startswith("backward"):
        units = ("mfma", alg["bwd_flops"], "10*G*64*d FLOP per selection x %d selections "
                 "(S, dP, dq, dV, dk products)" % alg["selections"])
    elif stage == "combine" and workload.startswith("backward"):
        units = ("hbm", alg["bwd_combine_bytes"], "per-pair dq partials (G*d*4 B) + per-item dV, dk "
                 "partials (2*64*d*4 B) read, fp32 gradients written")
    elif stage == "combine" and not workload.startswith("backward"):
        units = ("hbm", alg["partial_bytes"] + alg["out_bytes"],
                 "G*d*2 B fp16 partial per selection x %d + out" % alg["selections"])
    elif stage == "attend" and workload.startswith("global"):
        units = ("mfma", alg["attend_flops"] + alg["scan_flops"],
                 "4*G*64*d FLOP per (row, eligible chunk) x %d + 2*d per retrieval score x %d"
                 % (alg["selections"], alg["candidates"]))
    elif stage == "attend" and prefill:
        units = ("mfma", alg["attend_flops"], "4*G*64*d FLOP per selection x %d selections"
                 % alg["selections"])
    elif stage == "scan" and prefill:
        units = ("mfma", alg["scan_flops"], "2*d FLOP per candidate x %d candidates" % alg["candidates"])
    elif stage == "attend":
        units = ("hbm", alg["kv_bytes"] + alg["q_attn_bytes"] + alg["out_bytes"],
                 "2*64*d*2 B per distinct selected chunk x U + q_attn + out")
    else:
        units = ("hbm", alg["landmark_bytes"] + alg["q_ret_bytes"],
                 "d*2 B per eligible landmark + q_ret")
    bound, amount, how = units
    if bound == "mfma":
        achieved, peak, unit = amount / (ms / 1e3) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = amount / (ms / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s"
    res = dict(bound=bound, achieved=achieved, peak=peak, unit=unit, frac=achieved / peak,
               traffic=measured_traffic(workload, kernel), kernel=kernel, stage=stage,
               kernel_ms=ms, algorithmic_per_launch=amount, algorithmic_units=how)
    mb = measured_mfma_busy(workload, kernel)
    if bound == "mfma" or mb is not None:
        res["mfma_busy_counter"] = mb
    return res


def step_roofline(nbytes, flops, ms):
    """Whole-step roofline: t_roof = max(bytes / HBM peak, FLOPs / bf16 MFMA peak)
    over the measured step time."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9) * 1e3
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e3
    t_roof = max(t_hbm, t_mfma)
    return dict(bound="hbm" if t_hbm >= t_mfma else "mfma", t_roof_ms=t_roof, t_hbm_ms=t_hbm,
                t_mfma_ms=t_mfma, frac=t_roof / ms)


def bench_backward(name, cfg, steps, warmup, timer, cpu_baseline):
    """One step = hsa_backward over the whole batch for the forward's selection."""
    import torch
    import ultra_long_context_amd as hsa
    import workloads as W

    t = time.perf_counter()
    inp = W.generate(cfg)
    dout_np = W.cotangent(cfg)
    log("[bench] %s: inputs generated in %.1fs" % (name, time.perf_counter() - t))
    q_ret, lm, q_attn, k, v = [to_dev(a, cfg.dtype) for a in (inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v)]
    dout = to_dev(dout_np, cfg.dtype)
    _, idx, sc = hsa.forward(q_ret, lm, q_attn, k, v, q_pos0=cfg.q_pos0, top_k=cfg.top_k, return_topk=True)
    f = dict(dtype=torch.float32, device="cuda:0")
    grads = tuple(torch.empty(t_.shape, **f) for t_ in (q_ret, lm, q_attn, k, v))

    def step():
        hsa.backward(q_ret, lm, q_attn, k, v, idx, sc, dout, out=grads)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    eager = [g.clone() for g in grads]
    g_step = timer.capture(step)
    g_step.replay()
    torch.cuda.synchronize()
    if not all(torch.equal(a, b) for a, b in zip(grads, eager)):
        raise RuntimeError("graph replay differs from the eager backward")
    log("[bench] %s: warmup done, graph replay matches eager bit for bit" % name)
    tm = timer.time_eager(step, steps)
    ms_mean, ms_med, wall_ms = tm["mean"], tm["median"], tm["wall"]
    graph_ms, _, _ = timer.time(g_step, steps)
    log("[bench] %s: %.4f ms/step (median %.4f, p10 %.4f, p90 %.4f, wall incl. flush %.3f; graph replay %.4f)" % (
        name, ms_mean, ms_med, tm["p10"], tm["p90"], wall_ms, graph_ms))
    warm_mean = timer.time_eager(step, steps, flush=False)["mean"]
    stage_ms = timer.stages(lambda evs: hsa.backward(q_ret, lm, q_attn, k, v, idx, sc, dout, out=grads,
                                                     stage_events=evs), steps)
    log("[bench] %s: kernel stages (ms) %s" % (name, json.dumps(stage_ms)))
    U = distinct_chunks(idx, cfg)
    alg = algorithmic(cfg, U)
    n_pairs = int((idx >= 0).sum().item())
    items = n_pairs // 64 + U          # upper bound on work items: one partial block per used bin
    d, G = cfg.head_dim, cfg.group
    alg["bwd_combine_bytes"] = (n_pairs * G * d * 4 + items * 2 * 64 * d * 4
                                + 4 * (q_ret.numel() + lm.numel() + q_attn.numel() + k.numel() + v.numel()))
    # compulsory bytes: bf16 inputs (selected chunks' K/V once), the selection,
    # fp32 gradients written once
    grads_bytes = 4 * sum(g.numel() for g in grads)
    alg["bwd_bytes"] = (alg["q_ret_bytes"] + alg["landmark_bytes"] + 2 * alg["q_attn_bytes"] + alg["kv_bytes"]
                        + idx.numel() * 8 + grads_bytes)
    qtok = cfg.batch * cfg.q_len
    res = dict(workload=name, config=cfg, value=qtok / (ms_mean / 1e3), ms_per_step=ms_mean,
               ms_median=ms_med, ms_p10=tm["p10"], ms_p90=tm["p90"], wall_ms_per_step=wall_ms,
               warm_ms_per_step=warm_mean, graph_ms_per_step=graph_ms, stage_ms=stage_ms, alg=alg, U=U)
    dom = max(stage_ms, key=stage_ms.get)
    res["roofline"] = roofline(name, dom, stage_ms[dom], alg)
    res["hbm_frac_whole_step"] = (alg["bwd_bytes"] / 8e12) / (ms_mean / 1e3)
    res["step_roofline"] = step_roofline(alg["bwd_bytes"], alg["bwd_flops"], ms_mean)
    if cpu_baseline:
        res["cpu_baseline"] = oracle_backward_baseline(cfg, inp, dout_np, idx.cpu().numpy(), sc.cpu().numpy())
        res["cpu_baseline"]["gpu_over_cpu"] = res["value"] / res["cpu_baseline"]["value"]
    del q_ret, lm, q_attn, k, v, dout, grads, eager, inp
    torch.cuda.empty_cache()
    return res


def oracle_backward_baseline(cfg, inp, dout, idx, sc, budget_s=15.0):
    """fp64 oracle backward on every s-th query row (with the whole K/V history)."""
    import oracle
    total = cfg.batch * cfg.q_len

    def run(rows):
        r = np.asarray(rows)
        t = time.perf_counter()
        oracle.backward(inp.q_ret[:, r], inp.landmarks, inp.q_attn[:, r], inp.k, inp.v, dout[:, r],
                        idx[:, r], sc[:, r], qk_norm=cfg.qk_norm)
        return time.perf_counter() - t

    probe = np.linspace(0, cfg.q_len - 1, num=min(cfg.q_len, 64), dtype=np.int64)
    per_row = run(probe) / len(probe)
    n = int(max(64, min(cfg.q_len, budget_s / max(per_row, 1e-9))))
    stride = max(1, cfg.q_len // n)
    rows = np.arange(0, cfg.q_len, stride, dtype=np.int64)
    dt = run(rows)
    threads = min(oracle.max_threads(), cfg.batch * cfg.n_kv_heads)   # parallel over (batch, kv head)
    log("[bench] oracle backward: %d rows in %.1fs on %d threads" % (len(rows), dt, threads))
    return dict(value=cfg.batch * len(rows) / dt, unit="query-tokens/s", cores=threads, kind="oracle",
                cpu_model=cpu_model(),
                sample="%d of %d query rows (every %d-th row of each sequence, all heads), %.1f s" % (
                    cfg.batch * len(rows), total, stride, dt))


CROSSOVER_LENGTHS = (4096, 8192, 16384, 32768, 65536, 131072, 262144, 524288, 1048576)
CROSSOVER_DEFAULT_MAX = 262144   # dense SDPA past 256K takes seconds per call


def bench_crossover(steps, warmup, timer, lengths=CROSSOVER_LENGTHS):
    """HSA forward against dense causal attention (torch SDPA, flash or
    memory-efficient backend only) on the 32K training window's head layout
    (B=1, 8 q heads / 1 kv head, d=128, top-K 8) at growing L = Lq = Lkv.
    Inputs: seeded N(0,1) bf16 drawn on the GPU; landmarks = chunk means
    (hsa_chunk_landmarks).  Each side is timed cold as direct calls."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    import ultra_long_context_amd as hsa

    rows = []
    for L in lengths:
        gen = torch.Generator(device="cuda:0")
        gen.manual_seed(L)
        rnd = lambda *shape: torch.randn(*shape, generator=gen, device="cuda:0", dtype=torch.float32).to(torch.bfloat16)
        q_ret, q_attn = rnd(1, L, 1, 128), rnd(1, L, 8, 128)
        k, v = rnd(1, 1, L, 128), rnd(1, 1, L, 128)
        lm = hsa.chunk_landmarks(k)
        out = torch.empty_like(q_attn)

        def hsa_step():
            hsa.forward(q_ret, lm, q_attn, k, v, q_pos0=0, top_k=8, out=out)

        for _ in range(warmup):
            hsa_step()
        hsa_ms = timer.time_eager(hsa_step, steps)["mean"]
        # dense comparator: [B, H, L, d] with the kv head repeated for the 8 q heads
        qd = q_attn.permute(0, 2, 1, 3).contiguous()
        kd = k.expand(1, 8, L, 128).contiguous()
        vd = v.expand(1, 8, L, 128).contiguous()
        del q_ret, q_attn, k, v, lm, out
        dense_ms, backend = None, None
        for be in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
            try:
                with sdpa_kernel([be]):
                    def dense_step():
                        F.scaled_dot_product_attention(qd, kd, vd, is_causal=True)
                    for _ in range(warmup):
                        dense_step()
                    torch.cuda.synchronize()
                    dense_ms = timer.time_eager(dense_step, steps)["mean"]
                backend = be.name.lower()
                break
            except RuntimeError as e:
                log("[bench] crossover L=%d: SDPA %s unavailable (%s)" % (L, be.name, str(e).splitlines()[0]))
        del qd, kd, vd
        torch.cuda.empty_cache()
        # dense causal attention at the bf16 MFMA peak: 2*L^2*d FLOP per q head
        bound_ms = 2.0 * L * L * 128 * 8 / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e3
        rows.append(dict(L=L, hsa_ms=hsa_ms, dense_ms=dense_ms, dense_backend=backend,
                         hsa_over_dense=None if dense_ms is None else hsa_ms / dense_ms,
                         dense_mfma_bound_ms=bound_ms))
        log("[bench] crossover L=%d: hsa %.4f ms, dense %s ms (%s)" % (
            L, hsa_ms, "n/a" if dense_ms is None else "%.4f" % dense_ms, backend))
    faster = [r["L"] for r in rows if r["dense_ms"] is not None and r["hsa_ms"] < r["dense_ms"]]
    faster_bound = [r["L"] for r in rows if r["hsa_ms"] < r["dense_mfma_bound_ms"]]
    return dict(workload="crossover_gqa8_d128_k8", rows=rows,
                crossover_L=min(faster) if faster else None,
                crossover_L_vs_mfma_bound=min(faster_bound) if faster_bound else None,
                note="smallest L at which the HSA forward is faster than dense causal SDPA "
                     "(measured) and than dense causal attention at the bf16 MFMA peak")


def bench_workload(name, steps, warmup, timer, cpu_baseline):
    import torch
    import ultra_long_context_amd as hsa
    import workloads as W

    from dataclasses import replace as dc_replace
    cfg = dc_replace(W.CONFIGS[WORKLOADS[name]], **OVERRIDES.get(name, {}))
    if name.startswith("backward"):
        return bench_backward(name, cfg, steps, warmup, timer, cpu_baseline)
    t = time.perf_counter()
    inp = W.generate(cfg)
    log("[bench] %s: inputs generated in %.1fs" % (name, time.perf_counter() - t))
    dev = [to_dev(a, cfg.dtype) for a in (inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v)]
    q_ret, lm, q_attn, k, v = dev
    out = torch.empty_like(q_attn)

    def step():
        hsa.forward(q_ret, lm, q_attn, k, v, q_pos0=cfg.q_pos0, top_k=cfg.top_k, out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    eager = out.clone()
    g_step = timer.capture(step)
    g_step.replay()
    torch.cuda.synchronize()
    if not torch.equal(out, eager):
        raise RuntimeError("graph replay differs from the eager forward")
    log("[bench] %s: warmup done, graph replay matches eager" % name)
    tm = timer.time_eager(step, steps)
    ms_mean, ms_med, wall_ms = tm["mean"], tm["median"], tm["wall"]
    graph_ms, _, _ = timer.time(g_step, steps)
    log("[bench] %s: %.4f ms/step (median %.4f, p10 %.4f, p90 %.4f, wall incl. flush %.3f; graph replay %.4f)" % (
        name, ms_mean, ms_med, tm["p10"], tm["p90"], wall_ms, graph_ms))
    warm_mean = timer.time_eager(step, steps, flush=False)["mean"]

    # per-kernel timing: the same forward, cold, with HIP events recorded by the
    # library around each kernel stage on the launch stream
    stage_ms = timer.stages(lambda evs: hsa.forward(q_ret, lm, q_attn, k, v, q_pos0=cfg.q_pos0,
                                                    top_k=cfg.top_k, out=out, stage_events=evs),
                            steps)
    log("[bench] %s: kernel stages (ms) %s" % (name, json.dumps(stage_ms)))
    if cfg.top_k > hsa.MAX_TOP_K:          # global HSA: every eligible chunk is selected
        sel_out = (None,)
        U = cfg.batch * cfg.n_kv_heads * min(cfg.n_chunks, (cfg.q_pos0 + cfg.q_len - 1) // 64)
    else:
        sel_out = hsa.forward(q_ret, lm, q_attn, k, v, q_pos0=cfg.q_pos0, top_k=cfg.top_k,
                              return_topk=True)
        U = distinct_chunks(sel_out[1], cfg)
    alg = algorithmic(cfg, U)
    del sel_out

    qtok = cfg.batch * cfg.q_len
    res = dict(workload=name, config=cfg, value=qtok / (ms_mean / 1e3), ms_per_step=ms_mean,
               ms_median=ms_med, ms_p10=tm["p10"], ms_p90=tm["p90"], wall_ms_per_step=wall_ms,
               warm_ms_per_step=warm_mean, graph_ms_per_step=graph_ms, stage_ms=stage_ms, alg=alg, U=U)
    dom = max(stage_ms, key=stage_ms.get)
    res["roofline"] = roofline(name, dom, stage_ms[dom], alg)
    res["hbm_frac_whole_step"] = (alg["bytes"] / 8e12) / (ms_mean / 1e3)
    res["step_roofline"] = step_roofline(alg["bytes"], alg["scan_flops"] + alg["attend_flops"], ms_mean)
    if name == "decode_16M":
        # KV-cache maintenance beside the step: every chunk-mean landmark of the
        # history rebuilt from K (hsa_chunk_landmarks), an HBM stream
        lm_buf = torch.empty_like(lm)
        lm_ms = timer.time_eager(lambda: hsa.chunk_landmarks(k, out=lm_buf), steps)["mean"]
        nbytes = k.numel() * k.element_size() + lm_buf.numel() * lm_buf.element_size()
        gbs = nbytes / (lm_ms / 1e3) / 1e9
        res["landmark_rebuild"] = dict(kernel=KERNELS[(name, "landmarks")], chunks=cfg.batch * cfg.n_kv_heads * cfg.n_chunks,
                                       ms=lm_ms, bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS,
                                       unit="GB/s", frac=gbs / HBM_PEAK_GBS,
                                       traffic=measured_traffic(name, KERNELS[(name, "landmarks")]),
                                       algorithmic_per_launch=nbytes,
                                       algorithmic_units="64*d*2 B of keys read + d*2 B written per chunk")
        log("[bench] %s: landmark rebuild %.4f ms, %.0f GB/s" % (name, lm_ms, gbs))
        del lm_buf
    if cpu_baseline:
        res["cpu_baseline"] = oracle_baseline(cfg, inp)
        res["cpu_baseline"]["gpu_over_cpu"] = res["value"] / res["cpu_baseline"]["value"]
    del dev, q_ret, lm, q_attn, k, v, out, inp
    torch.cuda.empty_cache()
    return res


def oracle_baseline(cfg, inp, budget_s=20.0):
    """fp64 oracle on a stratified sample of query rows (every s-th row of each sequence)."""
    import oracle
    threads = oracle.max_threads()
    total = cfg.batch * cfg.q_len
    # calibrate on a few rows, then pick a stride so the sample takes ~budget_s
    probe = np.linspace(0, total - 1, num=min(total, 8 * threads), dtype=np.int64)
    t = time.perf_counter()
    oracle.forward(inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v, q_pos0=cfg.q_pos0,
                   top_k=cfg.top_k, rows=probe)
    per_row = (time.perf_counter() - t) / len(probe)
    n = int(max(threads, min(total, budget_s / max(per_row, 1e-9))))
    stride = max(1, total // n)
    rows = np.arange(0, total, stride, dtype=np.int64)
    t = time.perf_counter()
    oracle.forward(inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v, q_pos0=cfg.q_pos0,
                   top_k=cfg.top_k, rows=rows)
    dt = time.perf_counter() - t
    log("[bench] oracle: %d rows in %.1fs on %d threads" % (len(rows), dt, threads))
    res = dict(value=len(rows) / dt, unit="query-tokens/s", cores=threads, kind="oracle",
               cpu_model=cpu_model(),
               sample="%d of %d query rows (every %d-th row, all heads), %.1f s" % (
                   len(rows), total, stride, dt))
    if total <= 64 and threads > 1:       # decode: the same rows on one thread as well
        oracle.set_threads(1)
        try:
            t = time.perf_counter()
            oracle.forward(inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v, q_pos0=cfg.q_pos0,
                           top_k=cfg.top_k, rows=rows)
            dt1 = time.perf_counter() - t
        finally:
            oracle.set_threads(threads)
        log("[bench] oracle: %d rows in %.1fs on 1 thread" % (len(rows), dt1))
        res["value_1_thread"] = len(rows) / dt1
    return res


def pmc_mean_kib(csv_path, counter, match):
    """Mean per-dispatch value of `counter` over dispatches whose kernel name
    contains `match`, from a rocprofv3 --pmc counter_collection.csv.  The
    dispatches must share one grid size: a run over several workloads that use
    the same kernel (different grids) would be averaged across them, so it is
    refused (profile such workloads in runs of their own)."""
    import csv
    vals, grids = {}, set()
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") == counter and match in row.get("Kernel_Name", ""):
                d = row.get("Dispatch_Id") or row.get("Correlation_Id")
                vals[d] = vals.get(d, 0.0) + float(row["Counter_Value"])
                grids.add(row.get("Grid_Size"))
    if not vals:
        raise SystemExit("no %s dispatch of a kernel matching %r in %s" % (counter, match, csv_path))
    if len(grids) > 1:
        raise SystemExit("dispatches of %r in %s have several grid sizes %s: one workload per counter run"
                         % (match, csv_path, sorted(grids)))
    return float(np.mean(list(vals.values()))), len(vals)


def pmc_summary(fetch_csv, write_csv, workload, kernel, command):
    """Text summary of two counter passes: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) of `kernel`, each scaled by what the counter reads for the
    calibration copy (torch.neg over 2^28 fp32: 1 GiB read, 1 GiB written)."""
    match = kernel.split("<")[0]
    f_k, nf = pmc_mean_kib(fetch_csv, "FETCH_SIZE", match)
    w_k, nw = pmc_mean_kib(write_csv, "WRITE_SIZE", match)
    f_c, _ = pmc_mean_kib(fetch_csv, "FETCH_SIZE", "neg_kernel")
    w_c, _ = pmc_mean_kib(write_csv, "WRITE_SIZE", "neg_kernel")
    ff, fw = COPY_BYTES / (f_c * 1024.0), COPY_BYTES / (w_c * 1024.0)
    lines = [
        "# HBM traffic of %s, workload %s (rocprofv3 counter passes)" % (kernel, workload),
        "# command: %s" % command,
        "kernel: %s" % kernel,
        "workload: %s" % workload,
        "source_digest: %s" % source_digest(kernel),
        "fetch_dispatches: %d" % nf,
        "write_dispatches: %d" % nw,
        "FETCH_SIZE_KiB_per_dispatch: %.1f" % f_k,
        "WRITE_SIZE_KiB_per_dispatch: %.1f" % w_k,
        "copy_FETCH_SIZE_KiB: %.1f" % f_c,
        "copy_WRITE_SIZE_KiB: %.1f" % w_c,
        "copy_bytes_each_way: %d" % COPY_BYTES,
        "fetch_scale: %.4f" % ff,
        "write_scale: %.4f" % fw,
        "fetch_bytes_per_launch: %.0f" % (f_k * 1024.0 * ff),
        "write_bytes_per_launch: %.0f" % (w_k * 1024.0 * fw),
        "traffic_bytes_per_launch: %.0f" % (f_k * 1024.0 * ff + w_k * 1024.0 * fw),
    ]
    return "\n".join(lines) + "\n"


def pmc_dispatch_values(csv_path, counter, match):
    """Per-dispatch values of `counter` for kernels whose name contains `match`,
    with each dispatch's duration in microseconds (one grid size required, as
    in pmc_mean_kib)."""
    import csv
    vals, dur, grids = {}, {}, set()
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") == counter and match in row.get("Kernel_Name", ""):
                d = row.get("Dispatch_Id") or row.get("Correlation_Id")
                vals[d] = vals.get(d, 0.0) + float(row["Counter_Value"])
                dur[d] = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
                grids.add(row.get("Grid_Size"))
    if len(grids) > 1:
        raise SystemExit("dispatches of %r in %s have several grid sizes %s: one workload per counter run"
                         % (match, csv_path, sorted(grids)))
    return vals, dur


def mfma_summary(csv_path, workload, kernel, command):
    """Text summary of one counter pass (SQ_VALU_MFMA_BUSY_CYCLES,
    GRBM_GUI_ACTIVE, SQ_INSTS_VALU_MFMA_MOPS_BF16) for `kernel`: the MFMA busy
    fraction over all SIMDs and the bf16 MFMA work the hardware counted.
    GRBM_GUI_ACTIVE is reported summed over the XCDs, so the busy cycles of
    the SIMDs are set against GRBM_GUI_ACTIVE / N_XCDS cycles each (the same
    figure as rocprofv3's derived MfmaUtil, recorded beside it when present)."""
    match = kernel.split("<")[0]
    busy, dur = pmc_dispatch_values(csv_path, "SQ_VALU_MFMA_BUSY_CYCLES", match)
    gui, _ = pmc_dispatch_values(csv_path, "GRBM_GUI_ACTIVE", match)
    mops, _ = pmc_dispatch_values(csv_path, "SQ_INSTS_VALU_MFMA_MOPS_BF16", match)
    ds = sorted(set(busy) & set(gui) & set(mops))
    if not ds:
        raise SystemExit("no dispatch of a kernel matching %r with all three counters in %s" % (match, csv_path))
    b = float(np.mean([busy[d] for d in ds]))
    g = float(np.mean([gui[d] for d in ds]))
    flop = float(np.mean([mops[d] for d in ds])) * 512.0
    us = float(np.mean([dur[d] for d in ds]))
    util, _ = pmc_dispatch_values(csv_path, "MfmaUtil", match)   # rocprofv3's derived metric, if collected
    lines = [
        "# MFMA activity of %s, workload %s (rocprofv3 counter pass)" % (kernel, workload),
        "# command: %s" % command,
        "kernel: %s" % kernel,
        "workload: %s" % workload,
        "source_digest: %s" % source_digest(kernel),
        "dispatches: %d" % len(ds),
        "SQ_VALU_MFMA_BUSY_CYCLES_per_dispatch: %.0f" % b,
        "GRBM_GUI_ACTIVE_per_dispatch: %.0f" % g,
        "simds: %d" % N_SIMDS,
        "xcds: %d" % N_XCDS,
        "mfma_busy_percent: %.2f" % (100.0 * b / (g / N_XCDS * N_SIMDS)),
        "mfma_bf16_flop_per_dispatch: %.0f" % flop,
        "dispatch_us: %.1f" % us,
        "mfma_bf16_tflops_counted: %.1f" % (flop / (us * 1e-6) / 1e12),
    ]
    if util:
        lines.append("rocprof_MfmaUtil_percent: %.2f" % float(np.mean(list(util.values()))))
    return "\n".join(lines) + "\n"


def trace_summary(csv_path, workloads, command, gap_s=0.15):
    """Per-workload kernel statistics from a rocprofv3 --kernel-trace CSV of a
    bench.py run: dispatches are grouped into workloads at host gaps longer
    than gap_s (input generation separates the workloads, which run in the
    order `workloads`)."""
    import csv
    import re
    rows = []
    with open(csv_path, newline="") as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"],
                         int(r.get("Grid_Size_X", 0) or 0) // max(1, int(r.get("Workgroup_Size_X", 1) or 1))
                         * int(r.get("Grid_Size_Y", 1) or 1)))
    rows.sort()
    groups, cur, last_end = [], [], None
    for st, en, name, wgs in rows:
        if last_end is not None and st - last_end > gap_s * 1e9:
            groups.append(cur)
            cur = []
        cur.append((st, en, name, wgs))
        last_end = en if last_end is None else max(last_end, en)
    if cur:
        groups.append(cur)
    # the first groups may hold setup work (allocation, calibration): label the
    # last len(workloads) groups with the workload names
    labels = ["setup %d" % i for i in range(max(0, len(groups) - len(workloads)))] + list(workloads)[-len(groups):]

    def short(name):
        if "reduce" in name and "sum" in name.lower():
            return "torch sum (1 GiB cache-flush read)"
        m = re.search(r"(\w+_kernel)(<[^>]*>)?", name)
        return (m.group(1) + (m.group(2) or "")) if m else name[:48]

    lines = ["# rocprofv3 kernel statistics per workload of bench.py (times in microseconds;",
             "# cold timed calls, graph replays, eager warmup, stage-timed and selection calls)",
             "# command: %s" % command,
             "# dispatches grouped into workloads at host gaps > %.2f s (input generation)" % gap_s]
    for label, grp in zip(labels, groups):
        stats = {}
        for st, en, name, wgs in grp:
            k = (short(name), wgs)
            stats.setdefault(k, []).append((en - st) / 1e3)
        total = sum(sum(v) for v in stats.values())
        lines.append("")
        lines.append("## %s" % label)
        lines.append("%-48s %8s %6s %11s %11s %11s %6s" % ("kernel", "wgs", "calls", "avg_us", "min_us", "max_us", "pct"))
        for (name, wgs), v in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
            lines.append("%-48s %8d %6d %11.1f %11.1f %11.1f %6.1f" % (
                name[:48], wgs, len(v), float(np.mean(v)), min(v), max(v), 100.0 * sum(v) / total))
    return "\n".join(lines) + "\n"


def copy_calibration():
    """The plain copy kernel the counter passes are scaled by."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workloads",
                    default="prefill_128K,decode_16M,prefill_32K,chunked_1M,global_32K,backward_32K,crossover")
    ap.add_argument("--crossover-max", type=int, default=CROSSOVER_DEFAULT_MAX,
                    help="longest sequence of the crossover sweep (up to 1048576)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run the 1 GiB calibration copy first (for counter passes)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM traffic summary of --kernel-of from two counter passes")
    ap.add_argument("--mfma-summary", metavar="CSV",
                    help="print the MFMA activity summary of --kernel-of from one counter pass")
    ap.add_argument("--kernel-of", default="prefill_128K:attend",
                    help="workload:stage whose kernel --pmc-summary / --mfma-summary reports")
    ap.add_argument("--command", default="", help="command recorded in the --pmc-summary header")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="print per-workload kernel statistics of a rocprofv3 --kernel-trace CSV of a run "
                         "over --workloads")
    ap.add_argument("--trace-gap", type=float, default=0.15,
                    help="host gap (s) that separates workloads in --trace-summary (the crossover draws its "
                         "inputs on the GPU: a run of it alone is one group at a gap of a few seconds)")
    args = ap.parse_args()
    if args.trace_summary:
        order = ["crossover", "decode_16M", "prefill_32K", "chunked_1M", "global_32K", "backward_32K",
                 "prefill_128K"]
        wl = [w for w in order if w in args.workloads.split(",")]
        sys.stdout.write(trace_summary(args.trace_summary, wl, args.command, gap_s=args.trace_gap))
        return
    if args.mfma_summary:
        wl, stage = args.kernel_of.split(":")
        sys.stdout.write(mfma_summary(args.mfma_summary, wl, KERNELS[(wl, stage)], args.command))
        return
    if args.pmc_summary:
        wl, stage = args.kernel_of.split(":")
        sys.stdout.write(pmc_summary(args.pmc_summary[0], args.pmc_summary[1], wl,
                                     KERNELS[(wl, stage)], args.command))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the HSA forward here has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)

    import torch
    import ultra_long_context_amd as hsa
    hsa.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
    timer = Timer()
    names = [w for w in args.workloads.split(",") if w]
    results = {}
    crossover = None
    if "crossover" in names:
        names.remove("crossover")
        crossover = bench_crossover(args.steps, args.warmup, timer,
                                    lengths=tuple(L for L in CROSSOVER_LENGTHS if L <= args.crossover_max))
        if not names:
            print(json.dumps(crossover), flush=True)
            return
    for name in ["decode_16M", "prefill_32K", "chunked_1M", "global_32K", "backward_32K", "prefill_128K"]:
        if name in names:
            results[name] = bench_workload(name, args.steps, args.warmup, timer,
                                           not args.no_cpu_baseline)
    main_name = "prefill_128K" if "prefill_128K" in results else names[0]
    m = results[main_name]
    cfg = m["config"]

    def cfg_dict(c):
        return {"workload": c.name, "batch": c.batch, "q_len": c.q_len, "kv_len": c.kv_len,
                "q_pos0": c.q_pos0, "n_q_heads": c.n_q_heads, "n_kv_heads": c.n_kv_heads,
                "head_dim": c.head_dim, "top_k": c.top_k, "qk_norm": c.qk_norm}

    line = {
        "metric": "HSA fwd query-tokens/s at 128K prefill & 16M decode; % of HBM roofline",
        "value": m["value"], "unit": "query-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": m["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": cfg_dict(cfg),
        "roofline": m["roofline"],
        "ms_median": m["ms_median"], "ms_p10": m["ms_p10"], "ms_p90": m["ms_p90"],
        "wall_ms_per_step": m["wall_ms_per_step"], "warm_ms_per_step": m["warm_ms_per_step"],
        "graph_ms_per_step": m["graph_ms_per_step"],
        "hbm_frac_whole_step": m["hbm_frac_whole_step"],
        "step_roofline": m["step_roofline"],
        "stage_ms": m["stage_ms"],
    }
    if "cpu_baseline" in m:
        line["cpu_baseline"] = m["cpu_baseline"]
    for name, r in results.items():
        if name == main_name:
            continue
        sub = {k: r[k] for k in ("value", "ms_per_step", "ms_median", "ms_p10", "ms_p90", "wall_ms_per_step",
                                 "warm_ms_per_step", "graph_ms_per_step", "roofline", "hbm_frac_whole_step", "step_roofline",
                                 "landmark_rebuild") if k in r}
        sub["unit"] = "query-tokens/s"
        sub["config"] = cfg_dict(r["config"])
        sub["stage_ms"] = r["stage_ms"]
        if "cpu_baseline" in r:
            sub["cpu_baseline"] = r["cpu_baseline"]
        line[name] = sub
    if crossover is not None:
        line["crossover"] = crossover
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
