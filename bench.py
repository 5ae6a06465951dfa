"""Benchmark of the MI355X HSA forward (one GPU).

Workloads (synthetic, seeded; shapes of the paper's setting):
  prefill_128K : B=2, L=131072 query rows over their own 131072-token history,
                 32 q heads / 4 kv heads, d=128, top-K 16, bf16.   (headline `value`)
  decode_16M   : 16 single-token queries over one 16,777,216-token history,
                 8 q heads / 1 kv head, d=128, top-K 32, bf16.     (reported beside it)

A step is one hsa_forward call (landmark scan, top-K, per-chunk attention, blend)
over the whole batch, inputs resident in HBM.  Each step is preceded, outside its
HIP-event window, by a 1 GiB read that evicts L2 and the 256 MB Infinity Cache,
so every step starts cold.  ms_per_step is the mean event-timed step; the wall
time of the whole timed region (flushes included) is reported as wall_ms_per_step.

roofline: the dominant kernel of each workload is timed on its own with HIP events
on the launch stream (same cold-cache procedure) and priced against MI355X peaks:
  decode  -> landmark scan kernel(s), HBM bytes of the landmarks and queries;
  prefill -> attend/blend kernel, its contraction FLOPs.
cpu_baseline: the fp64 oracle on a bounded, stratified sample of query rows of the
same workload, timed on this host's cores (test infrastructure, not the product).
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
VALU_FP32_PEAK_TFLOPS = 78.6     # 256 CU x 64 lanes x 2 FLOP (FMA) x 2.4 GHz, non-packed

WORKLOADS = {"prefill_128K": 2, "decode_16M": 3}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(a).to("cuda:0")


class Timer:
    """Cold-cache timing of a captured HIP graph with HIP events.

    Each step enqueues a 1 GiB read of an unrelated buffer (evicting L2 and the
    256 MB Infinity Cache with clean lines; a write would leave dirty lines whose
    write-back competes with the timed step), then event e0, the graph replay,
    event e1.  The read keeps the GPU busy while the host enqueues e0 and the
    replay, so the events bracket GPU work only.  Events live on torch's current
    stream, which is the stream the library launches on."""

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
        torch = self.torch
        evs = self.events(steps)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e0, e1 in evs:
            if flush:
                self.cold()
            e0.record()
            graph.replay()
            e1.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        ms = [e0.elapsed_time(e1) for e0, e1 in evs]
        return float(np.mean(ms)), float(np.median(ms)), wall * 1e3


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
                scan_flops=2 * d * cand, attend_flops=4 * cfg.group * 64 * d * sel)


def bench_workload(name, steps, warmup, timer, cpu_baseline):
    import torch
    import ultra_long_context_amd as hsa
    import workloads as W

    cfg = W.CONFIGS[WORKLOADS[name]]
    t = time.perf_counter()
    inp = W.generate(cfg)
    log("[bench] %s: inputs generated in %.1fs" % (name, time.perf_counter() - t))
    dev = [to_dev(a, cfg.dtype) for a in (inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v)]
    q_ret, lm, q_attn, k, v = dev
    out = torch.empty_like(q_attn)
    idx = torch.empty((cfg.batch, cfg.q_len, cfg.n_kv_heads, cfg.top_k), dtype=torch.int32,
                      device="cuda:0")
    score = torch.empty(idx.shape, dtype=torch.float32, device="cuda:0")

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
    ms_mean, ms_med, wall_ms = timer.time(g_step, steps)
    log("[bench] %s: %.4f ms/step (median %.4f, wall incl. flush %.3f)" % (name, ms_mean, ms_med, wall_ms))
    warm_mean, _, _ = timer.time(g_step, steps, flush=False)

    # dominant-kernel timing through the two halves of the C ABI
    sel_out = hsa.forward(q_ret, lm, q_attn, k, v, q_pos0=cfg.q_pos0, top_k=cfg.top_k,
                          return_topk=True)
    idx.copy_(sel_out[1])
    score.copy_(sel_out[2])
    U = distinct_chunks(idx, cfg)
    alg = algorithmic(cfg, U)
    sel_i = torch.empty_like(idx)
    sel_s = torch.empty_like(score)
    ws = hsa.new_workspace(hsa.workspace_size(hsa.make_shape(
        batch=cfg.batch, q_len=cfg.q_len, kv_len=cfg.kv_len, q_pos0=cfg.q_pos0,
        n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim, top_k=cfg.top_k,
        dtype=hsa.DTYPE_BF16)), "cuda:0")

    def retrieve():
        hsa.retrieve_topk(q_ret, lm, q_pos0=cfg.q_pos0, top_k=cfg.top_k, kv_len=cfg.kv_len,
                          out=(sel_i, sel_s), workspace=ws)

    def attend():
        hsa.chunk_attend_blend(q_attn, k, v, idx, score, out=out, workspace=ws)

    r_ms, _, _ = timer.time(timer.capture(retrieve), steps)
    a_ms, _, _ = timer.time(timer.capture(attend), steps)
    log("[bench] %s: retrieve %.4f ms, attend %.4f ms, U=%d" % (name, r_ms, a_ms, U))

    qtok = cfg.batch * cfg.q_len
    res = dict(workload=name, config=cfg, value=qtok / (ms_mean / 1e3), ms_per_step=ms_mean,
               ms_median=ms_med, wall_ms_per_step=wall_ms, warm_ms_per_step=warm_mean,
               retrieve_ms=r_ms, attend_ms=a_ms, alg=alg, U=U)
    if name == "decode_16M":
        # landmark stream: every landmark and query read once per launch
        nbytes = alg["landmark_bytes"] + alg["q_ret_bytes"]
        gbs = nbytes / (r_ms / 1e3) / 1e9
        res["roofline"] = dict(bound="hbm", kernel="scan_wide_kernel (landmark scan, top-K, merge)",
                               achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s", frac=gbs / HBM_PEAK_GBS,
                               traffic=None, alg_bytes_per_launch=nbytes)
        res["hbm_frac_whole_step"] = (alg["bytes"] / 8e12) / (ms_mean / 1e3)
    else:
        fl = alg["attend_flops"]
        tf = fl / (a_ms / 1e3) / 1e12
        res["roofline"] = dict(bound="alu", kernel="attend_blend (fp32 VALU contraction)",
                               achieved=tf, peak=VALU_FP32_PEAK_TFLOPS, unit="TFLOP/s",
                               frac=tf / VALU_FP32_PEAK_TFLOPS, traffic=None,
                               alg_flops_per_launch=fl,
                               mfma_bf16_frac=tf / MFMA_BF16_PEAK_TFLOPS)
        res["hbm_frac_whole_step"] = (alg["bytes"] / 8e12) / (ms_mean / 1e3)
    if cpu_baseline:
        res["cpu_baseline"] = oracle_baseline(cfg, inp)
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
    return dict(value=len(rows) / dt, unit="query-tokens/s", cores=threads, kind="oracle",
                sample="%d of %d query rows (every %d-th row, all heads), %.1f s" % (
                    len(rows), total, stride, dt))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workloads", default="prefill_128K,decode_16M")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
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
    timer = Timer()
    names = [w for w in args.workloads.split(",") if w]
    results = {}
    for name in ["decode_16M", "prefill_128K"]:
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
        "wall_ms_per_step": m["wall_ms_per_step"], "warm_ms_per_step": m["warm_ms_per_step"],
        "hbm_frac_whole_step": m["hbm_frac_whole_step"],
        "stage_ms": {"retrieve": m["retrieve_ms"], "attend": m["attend_ms"]},
    }
    if "cpu_baseline" in m:
        line["cpu_baseline"] = m["cpu_baseline"]
    for name, r in results.items():
        if name == main_name:
            continue
        sub = {k: r[k] for k in ("value", "ms_per_step", "ms_median", "wall_ms_per_step",
                                 "warm_ms_per_step", "roofline", "hbm_frac_whole_step")}
        sub["unit"] = "query-tokens/s"
        sub["config"] = cfg_dict(r["config"])
        sub["stage_ms"] = {"retrieve": r["retrieve_ms"], "attend": r["attend_ms"]}
        if "cpu_baseline" in r:
            sub["cpu_baseline"] = r["cpu_baseline"]
        line[name] = sub
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
