"""Benchmark of the CSA2 FP4 sparse-attention decode step on one MI355X.

Default workload: Full-mode decode, batch 1, 64 query heads over a 64K-token
context (16384 FP4 entries of 512 latent + 64 RoPE channels), indexer 8 heads
x 128, Top-512.  One step = csa2_index_full -> csa2_topk ->
csa2_sparse_attn_fp4, all on the GPU through the C ABI, with every input
resident in HBM.  Inputs rotate over enough distinct sets (>= 1 GiB per
rotation) that no step finds its data in the 256 MB Infinity Cache.

Prints ONE JSON line (rank 0).  `roofline` describes the dominant kernel:
algorithmic bytes per launch over its average duration (HIP events on the
stream the kernels run on), against the 8 TB/s HBM peak.  `traffic` comes from
the committed rocprofv3 FETCH_SIZE / WRITE_SIZE measurement of that kernel
(profiles/), and is null when the kernel source changed since it was taken.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ROTATION_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="full-64k",
                    help="full-64k (default, the reported line); others for supplementary runs: "
                         "tiny-full, reindex-1m, reuse-128k, prefill-full-1m")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 256 MiB device copy (FETCH/WRITE calibration under rocprofv3)")
    return ap.parse_args()


def kernel_source_hash(name):
    p = os.path.join(ROOT, "sparse_attention_decode_csa2_amd", "csrc", name)
    h = hashlib.sha256()
    for f in (p, os.path.join(os.path.dirname(p), "csa2_device.h")):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel_file, workload):
    """Per-launch HBM bytes measured with rocprofv3 counters, if still valid."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(kernel_file):
        return None
    return rec.get("bytes_per_launch")


class FullStep:
    """Full-mode decode over R rotating input sets (B sequences each)."""

    def __init__(self, wl, R, dev):
        import torch
        from sparse_attention_decode_csa2_amd import csa2
        from sparse_attention_decode_csa2_amd import workloads as W
        self.wl, self.R, self.csa2 = wl, R, csa2
        B, N = wl.B, wl.N
        self.sets = []
        for r in range(R):
            ws = wl.scaled(seed=wl.seed * 1000 + r)
            keys = torch.stack([W.index_keys(ws, b, dev) for b in range(B)])
            codes = torch.empty(B, N, wl.d_c // 2, dtype=torch.uint8, device=dev)
            scales = torch.empty(B, N, wl.d_c // 16, dtype=torch.uint8, device=dev)
            rope = torch.empty(B, N, wl.d_r, dtype=torch.bfloat16, device=dev)
            for b in range(B):
                lat = W.latent_rows(ws, b, N, dev)
                rp = W.rope_rows(ws, b, N, dev) if wl.d_r else None
                csa2.csa2_quantize_fp4(lat, codes[b], scales[b], 0, rp, rope[b] if wl.d_r else None)
            self.sets.append(dict(ws=ws, keys=keys, codes=codes, scales=scales, rope=rope,
                                  qi=W.index_query(ws, dev), q=W.attn_query(ws, dev)))
        self.scores = torch.empty(B, N, dtype=torch.float32, device=dev)
        self.idx = torch.empty(B, wl.K, dtype=torch.int32, device=dev)
        self.top = torch.empty(B, wl.K, dtype=torch.float32, device=dev)
        self.out = torch.empty(B, wl.H, wl.d_c, dtype=torch.float32, device=dev)
        self.lse = torch.empty(B, wl.H, dtype=torch.float32, device=dev)
        tk = csa2.csa2_topk_workspace_bytes(B, N, wl.K)
        at = csa2.csa2_sparse_attn_workspace_bytes(B, wl.H, wl.d_c, wl.K)
        self.ws_topk = torch.empty(max(tk, 16), dtype=torch.uint8, device=dev) if tk else None
        self.ws_attn = torch.empty(max(at, 16), dtype=torch.uint8, device=dev) if at else None

    def bytes_per_set(self):
        s = self.sets[0]
        return sum(t.numel() * t.element_size() for t in (s["keys"], s["codes"], s["scales"], s["rope"]))

    # the three stages; `ev` optionally records events around each
    def index(self, r):
        s = self.sets[r]
        self.csa2.csa2_index_full(s["qi"], s["keys"], scores=self.scores)

    def topk(self, r):
        self.csa2.csa2_topk(self.scores, self.wl.K, out_idx=self.idx, out_score=self.top,
                            workspace=self.ws_topk)

    def attn(self, r):
        s = self.sets[r]
        self.csa2.csa2_sparse_attn_fp4(s["q"], s["codes"], s["scales"], s["rope"], self.idx,
                                       self.wl.sm_scale, out=self.out, lse=self.lse,
                                       workspace=self.ws_attn)

    def step(self, r):
        self.index(r)
        self.topk(r)
        self.attn(r)

    def alg_bytes(self):
        """Algorithmic bytes: inputs read once, outputs written once."""
        wl = self.wl
        B, N, K = wl.B, wl.N, wl.K
        entry = wl.d_c // 2 + wl.d_c // 16 + 2 * wl.d_r
        index = B * (N * wl.D_I * 2 + wl.H_I * wl.D_I * 2 + N * 4)
        topk = B * (N * 4 + K * 8)
        attn = B * (K * 4 + K * entry + wl.H * wl.D * 2 + wl.H * wl.d_c * 4 + wl.H * 4)
        step = B * (N * wl.D_I * 2 + wl.H_I * wl.D_I * 2 + K * entry + wl.H * wl.D * 2
                    + wl.H * wl.d_c * 4 + wl.H * 4 + K * 4)
        return {"index": index, "topk": topk, "attn": attn, "step": step}


def cpu_baseline(wl, budget_s):
    """The oracle, as it stands, on a bounded sample: one oracle-quantised
    cache (prepared outside the timed region) and as many Full-mode decode
    queries as fit in the budget."""
    import numpy as np
    import oracle
    from sparse_attention_decode_csa2_amd import workloads as W
    from threadpoolctl import threadpool_info
    ws = wl.scaled(B=1, seed=wl.seed * 1000)
    lat = W.bf16_bits(W.latent_rows(ws, 0, wl.N))
    codes, scales = oracle.quantize_fp4(lat)
    rope = W.bf16_bits(W.rope_rows(ws, 0, wl.N))[None] if wl.d_r else np.zeros((1, wl.N, 0), np.uint16)
    keys = W.bf16_bits(W.index_keys(ws, 0))[None]
    qs = [(W.bf16_bits(W.index_query(wl.scaled(B=1, seed=1000 + i))),
           W.bf16_bits(W.attn_query(wl.scaled(B=1, seed=1000 + i)))) for i in range(16)]
    n = 0
    t0 = time.perf_counter()
    while True:
        qi, q = qs[n % len(qs)]
        oracle.decode_full(qi, None, keys, None, q, codes[None], scales[None], rope, wl.K, wl.sm_scale)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s and n >= 3:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": n / el, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} Full-mode decode queries (batch 1, {wl.N} entries, Top-{wl.K}) over one "
                      f"oracle-quantised cache, {el:.1f} s; NumPy float64, BLAS threads={threads}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): this build has no "
              f"multi-GPU path; see DESIGN.md for how the step would shard.", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_attention_decode_csa2_amd import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = W.BY_NAME[args.workload]
    dev = "cuda"
    if wl.mode != "full":
        raise SystemExit(f"--workload {args.workload}: only Full-mode workloads are wired into bench.py")
    # size the rotation so one pass over the sets touches >= 1 GiB
    probe = FullStep(wl, 1, dev)
    R = max(2, math.ceil(ROTATION_BYTES / probe.bytes_per_set()))
    del probe
    step = FullStep(wl, R, dev)
    torch.cuda.synchronize()
    print(f"[bench] {wl.name}: {R} input sets x {step.bytes_per_set() / 2**20:.1f} MiB", file=sys.stderr,
          flush=True)

    # The host cannot enqueue a ~10 us step through Python faster than the GPU
    # runs it, so steps are captured into HIP graphs and replayed: one graph of
    # W warm-up steps, one of the K timed steps (inputs rotating over the R
    # sets), and per stage one graph of K launches of that stage alone.
    stream = torch.cuda.Stream()

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                fn(i % R)
        torch.cuda.synchronize()
        return g

    for i in range(min(args.warmup, R)):   # eager pass: sets up every buffer once
        step.step(i)
    torch.cuda.synchronize()
    g_warm = capture(step.step, max(args.warmup, 1))
    g_timed = capture(step.step, args.steps)
    stages = ["index", "topk", "attn"]
    g_stage = {s: capture(getattr(step, s), args.steps) for s in stages}

    def timed(g):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            torch.cuda.synchronize()
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    g_warm.replay()
    torch.cuda.synchronize()
    ms_per_step = timed(g_timed) / args.steps
    # kernel attribution: HIP events around K back-to-back launches of one stage
    # on the stream they are launched on
    for s in stages:
        g_stage[s].replay()          # untimed pass over the same launches
    stage_us = {s: 1000.0 * timed(g_stage[s]) / args.steps for s in stages}
    alg = step.alg_bytes()
    dom = max(stages, key=lambda s: stage_us[s])
    kernel_file = {"index": "index.hip", "topk": "topk.hip", "attn": "attn.hip"}[dom]
    achieved = alg[dom] / (stage_us[dom] * 1e-6) / 1e9
    traffic = committed_traffic(kernel_file, wl.name)

    if args.calib_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    qps = wl.B / (ms_per_step * 1e-3)
    line = {
        "metric": "decode queries/s + achieved HBM GB/s (% of peak), CSA2 FP4 sparse attn",
        "value": qps,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4(e2m1)+e4m3 cache, bf16/fp16 mfma, fp32 softmax",
        "data": "synthetic (seeded; integer indexer, RMS-normalised N(0,1) latents)",
        "config": {"workload": wl.name, "mode": wl.mode, "batch": wl.B, "entries": wl.N,
                   "context_tokens": wl.N * 4, "latent": wl.d_c, "rope": wl.d_r, "heads": wl.H,
                   "indexer": f"{wl.H_I}x{wl.D_I}", "top_k": wl.K, "rotation_sets": R},
        "step_hbm_gbs": alg["step"] / (ms_per_step * 1e-3) / 1e9,
        "step_alg_bytes": alg["step"],
        "stage_us": {s: round(v, 3) for s, v in stage_us.items()},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "alg_bytes_per_launch": alg[dom]},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
