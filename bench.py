"""Benchmark of the CSA2 FP4 sparse-attention decode step on one MI355X.

Default workload: prefill-full-1m, the largest configuration that fits one
GPU: an 8192-row post-RoPE bf16 chunk is quantised to FP4 and appended to
sequence 0, then a batch of 8 Full-mode decode queries (64 heads, indexer
8 heads x 128) scores 262144 entries per sequence (1M tokens at 4:1), takes
the Top-512 and runs the sparse attention over them.  One step =
csa2_index_topk_full_append (the chunk write, the indexer scores and their
Top-512 in one call; the chunk is written by the Top-K's last launch on the
CUs its selection leaves idle) -> csa2_sparse_attn_fp4, all on the GPU
through the C ABI, with every input resident in HBM.  The other
workloads (--workload) give the supplementary lines.

Inputs rotate over R distinct sets, R sized from the bytes one step actually
reads so that a rotation touches >= 1 GiB (4x the 256 MB Infinity Cache); the
timed steps start after the sets the warm-up used, and the line records how
many distinct sets and bytes the timed steps touched.

Prints ONE JSON line (rank 0).  `roofline` describes the dominant stage:
algorithmic bytes per call over its average duration (HIP events on the
stream the kernels run on), against the 8 TB/s HBM peak.  The dominant stage
of the Full workloads, `select` (csa2_index_topk_full, with the chunk write
at prefill-full-1m), is two launches at 1M entries: the fused indexer +
chunk Top-K kernel, then the final Top-K level; its duration covers both.  `traffic` comes from
the committed rocprofv3 FETCH_SIZE / WRITE_SIZE measurement of that kernel
(profiles/), and is null when the kernel source changed since it was taken.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
`torch_topk_us` times torch.topk on the same score rows (K launches in one
graph), the reference the pages quote for their Top-K kernel's speed-up;
the sampler line adds `csa2_topk_us`, its Top-K alone on the same rows.
`single_step_us_cold` is one step run on its own after a 512 MiB write has
evicted the caches (median of five): the latency of an isolated decode step,
beside `value`, the steady-state rate of back-to-back steps.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ROTATION_BYTES = 1 << 30
MAX_SETS = 512
DEFAULT_WORKLOAD = "prefill-full-1m"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="prefill-full-1m (default, the reported line: the largest configuration); others for "
                         "supplementary runs: tiny-full, full-64k, reindex-1m, reuse-128k, pool-build-1m, "
                         "reuse-swa-128k, sample-129k, prefill-reuse-1m")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one elementwise copy of 256 MiB (float32 negation: 256 MiB read, "
                         "256 MiB written) as the FETCH/WRITE calibration under rocprofv3")
    return ap.parse_args()


def committed_traffic(kernel_file, workload):
    """Per-launch HBM bytes of the dominant kernel measured with rocprofv3
    counters (profiles/traffic_<workload>.txt), or None when absent or taken
    on a different version of the kernel's source."""
    from sparse_attention_decode_csa2_amd.rocprof_summary import kernel_source_hash, read_traffic
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(p):
        return None
    rec = read_traffic(p)
    if rec.get("source_file") != kernel_file or rec.get("source_hash") != kernel_source_hash(kernel_file):
        return None
    return float(rec["bytes_per_launch"])


def _window_bytes(wl):
    """Algorithmic bytes of one FP8 window row (codes + row scale + RoPE part)."""
    return wl.d_c + 4 + 2 * wl.d_r


def _entry_bytes(wl):
    """Algorithmic bytes of one cache entry (codes + scales + RoPE part)."""
    return wl.d_c // 2 + wl.d_c // 16 + 2 * wl.d_r


class Step:
    """One decode step of a workload over R rotating input sets.

    Full (tiny-full, full-64k): select (indexer scores + Top-K) -> attn, each set its own caches.
    Reindex (reindex-1m): pool -> topk -> attn over one cache; sets = pools + queries.
    Reuse (reuse-128k): attn over one cache; sets = index lists + queries.
    Prefill + Full (prefill-full-1m): select (append 8192 rows + indexer scores + Top-K) -> attn.
    Pool construction (pool-build-1m): index (Full scores) -> build (the Reindex pool).
    Reuse + window (reuse-swa-128k): attn_swa (the selected entries and the FP8 window in one softmax).
    Sampler (sample-129k): sample (csa2_sample: Top-K over the vocabulary logits + the draw); sets = logits + uniforms.
    Prefill, Reuse layer (prefill-reuse-1m): attn over one cache for the 8192 queries of a chunk,
    each with its own causal list; sets = queries + lists.
    """

    def __init__(self, wl, dev, rotation_bytes=ROTATION_BYTES):
        import torch
        from sparse_attention_decode_csa2_amd import csa2
        from sparse_attention_decode_csa2_amd import workloads as W
        self.wl, self.csa2, self.W, self.dev = wl, csa2, W, dev
        B, N = wl.B, wl.N
        self.mode = wl.mode
        self.fused_select = False
        if self.mode in ("sample", "sample_full"):
            self._init_sample(wl, dev)
            return
        self.touched = self.step_read_bytes()
        self.R = min(MAX_SETS, max(2, math.ceil(rotation_bytes / self.touched)))
        if self.mode == "full":
            self.sets = [self._full_set(wl.scaled(seed=wl.seed * 1000 + r)) for r in range(self.R)]
        else:
            if self.mode != "pool_build":
                self.cache = self._cache(wl)
            if self.mode in ("reindex", "prefill_full", "pool_build"):
                self.keys = torch.stack([W.index_keys(wl, b, dev) for b in range(B)])
            self.sets = []
            for r in range(self.R):
                ws = wl.scaled(seed=wl.seed * 1000 + r)
                if self.mode == "prefill_reuse":
                    T = wl.prefill_rows
                    self.sets.append({"q": W.attn_query(ws.scaled(B=T), dev).view(1, T, wl.H, wl.D),
                                      "idx": W.chunk_index(ws).to(dev)})
                    continue
                st = {"q": W.attn_query(ws, dev)}
                # index lists and pools are drawn on the host (no device
                # random-permutation kernels in the profiled process)
                if self.mode == "reindex":
                    st["pool"], st["nb"] = (t.to(dev) for t in W.pool_blocks(ws, "cpu"))
                if self.mode in ("reindex", "prefill_full", "pool_build"):
                    st["qi"] = W.index_query(ws, dev)
                if self.mode in ("reuse", "reuse_swa"):
                    st["idx"] = W.reuse_index(ws, "cpu").to(dev)
                self.sets.append(st)
            if self.mode == "prefill_full":
                self.chunk = W.prefill_chunk(wl, dev)
                self.chunk_rope = W.prefill_rope(wl, dev)
        M = {"full": N, "prefill_full": N, "reindex": wl.P_max * wl.block, "reuse": 0, "pool_build": N,
             "reuse_swa": 0, "prefill_reuse": 0}[self.mode]
        self.M = M
        self.scores = torch.empty(B, max(M, 1), dtype=torch.float32, device=dev)
        self.positions = torch.empty(B, max(M, 1), dtype=torch.int32, device=dev)
        self.idx = torch.empty(B, wl.K, dtype=torch.int32, device=dev)
        self.top = torch.empty(B, wl.K, dtype=torch.float32, device=dev)
        self.out = torch.empty(B, wl.H, wl.d_c, dtype=torch.float32, device=dev)
        self.lse = torch.empty(B, wl.H, dtype=torch.float32, device=dev)
        tk = csa2.csa2_topk_workspace_bytes(B, M, wl.K) if M else 0
        # the fused chunk kernel runs when the rows hold a workgroup per CU
        self.fused_select = self.mode in ("full", "prefill_full") and wl.D_I <= 128 and B * -(-N // 8192) >= 256
        if self.mode in ("full", "prefill_full"):
            tk = csa2.csa2_index_topk_full_workspace_bytes(B, wl.D_I, N, wl.K)
        nq = wl.prefill_rows if self.mode == "prefill_reuse" else B
        at = csa2.csa2_sparse_attn_workspace_bytes(nq, wl.H, wl.d_c, wl.K)
        self.ws_topk = torch.empty(max(tk, 16), dtype=torch.uint8, device=dev) if tk else None
        self.ws_attn = torch.empty(max(at, 16), dtype=torch.uint8, device=dev) if at else None
        self.stages = {"full": ["select", "attn"], "reindex": ["pool", "topk", "attn"],
                       "reuse": ["attn"], "prefill_full": ["select", "attn"],
                       "pool_build": ["index", "build"], "reuse_swa": ["attn_swa"],
                       "prefill_reuse": ["attn"]}[self.mode]
        if self.mode == "prefill_reuse":
            self.out = torch.empty(1, wl.prefill_rows, wl.H, wl.d_c, dtype=torch.float32, device=dev)
            self.lse = torch.empty(1, wl.prefill_rows, wl.H, dtype=torch.float32, device=dev)
        if self.mode == "reuse_swa":
            sw = csa2.csa2_sparse_swa_attn_workspace_bytes(B, wl.H, wl.d_c, wl.K)
            self.ws_swa = torch.empty(max(sw, 16), dtype=torch.uint8, device=dev)
            Wn = wl.window
            self.win = csa2.alloc_window(B, Wn, wl.d_c, wl.d_r, dev)
            for b in range(B):
                lat = W.latent_rows(wl, b, Wn, dev, name="window")
                csa2.csa2_quantize_fp8(lat, self.win[0][b], self.win[1][b], 0,
                                       W.rope_rows(wl.scaled(seed=wl.seed + 7919), b, Wn, dev), self.win[2][b])
            self.out2 = torch.empty_like(self.out)
            self.lse2 = torch.empty_like(self.lse)
        if self.mode == "pool_build":
            self.pool_out = torch.empty(B, wl.P_max, dtype=torch.int32, device=dev)
            self.nb_out = torch.empty(B, dtype=torch.int32, device=dev)
            pb = csa2.csa2_build_pool_workspace_bytes(B, N, wl.block, wl.P_max)
            self.ws_build = torch.empty(max(pb, 16), dtype=torch.uint8, device=dev)
        if self.mode in ("reuse", "reuse_swa", "prefill_reuse"):
            self.idx = None

    def _init_sample(self, wl, dev):
        import torch
        csa2, W = self.csa2, self.W
        B, V, K = wl.B, wl.N, wl.K
        self.touched = self.step_read_bytes()
        self.R = min(MAX_SETS, max(2, math.ceil(ROTATION_BYTES / self.touched)))
        self.sets = []
        for r in range(self.R):
            ws = wl.scaled(seed=wl.seed * 1000 + r)
            self.sets.append({"logits": W.vocab_logits(ws, dev), "u": W.sampler_uniforms(ws, dev)})
        self.M = V
        self.scores = self.sets[0]["logits"]
        self.idx = torch.empty(B, K, dtype=torch.int32, device=dev)
        self.top = torch.empty(B, K, dtype=torch.float32, device=dev)
        self.token = torch.empty(B, dtype=torch.int32, device=dev)
        self.prob = torch.empty(B, dtype=torch.float32, device=dev)
        self.n_kept = torch.empty(B, dtype=torch.int32, device=dev)
        if self.mode == "sample_full":
            self.stages = ["draw_full"]
            self.ws_full = torch.empty(csa2.csa2_sample_full_workspace_bytes(B, V), dtype=torch.uint8, device=dev)
            return
        tk = csa2.csa2_topk_workspace_bytes(B, V, K)
        # the threshold filter's workspace: a 128-byte record and 16384 keys per row
        self.filtered_topk = V > 16384 and tk == B * (128 + 16384 * 8)
        self.ws_topk = torch.empty(max(tk, 16), dtype=torch.uint8, device=dev) if tk else None
        self.ws_sample = torch.empty(max(csa2.csa2_sample_workspace_bytes(B, V, K), 16), dtype=torch.uint8,
                                     device=dev)
        # one call, csa2_sample (Top-K + draw; with the threshold filter its
        # last kernel draws from the rows it writes)
        self.stages = ["sample"]

    def step_read_bytes(self):
        """Bytes one step reads from HBM (the inputs of all its stages, read
        once): the figure the rotation is sized from."""
        wl = self.wl
        B, N, K = wl.B, wl.N, wl.K
        if self.mode in ("sample", "sample_full"):
            return B * N * 4
        ent = _entry_bytes(wl)
        q = wl.H * wl.D * 2
        qi = wl.H_I * wl.D_I * 2
        return {"full": B * (N * wl.D_I * 2 + qi + K * ent + q),
                "prefill_reuse": wl.prefill_rows * (K * ent + q + K * 4),
                "reindex": B * (wl.n_blocks * wl.block * wl.D_I * 2 + qi + K * ent + q),
                "reuse": B * (K * ent + q + K * 4),
                "reuse_swa": B * (K * ent + wl.window * _window_bytes(wl) + q + K * 4),
                "prefill_full": B * (N * wl.D_I * 2 + qi + K * ent + q) + wl.prefill_rows * wl.D * 2,
                "pool_build": B * (N * wl.D_I * 2 + qi)}[self.mode]

    def draw_full(self, r):
        self.csa2.csa2_sample_full(self.sets[r]["logits"], self.wl.temperature, self.sets[r]["u"], token=self.token,
                                   prob=self.prob, workspace=self.ws_full)

    def sample(self, r):
        wl = self.wl
        self.csa2.csa2_sample(self.sets[r]["logits"], wl.K, wl.temperature, wl.top_p, self.sets[r]["u"],
                              token=self.token, prob=self.prob, n_kept=self.n_kept, workspace=self.ws_sample)

    def draw(self, r):
        wl = self.wl
        self.csa2.csa2_sample_draw(self.idx, self.top, wl.temperature, wl.top_p, self.sets[r]["u"],
                                   token=self.token, prob=self.prob, n_kept=self.n_kept)

    def torch_sampler(self, r):
        """The same draw in eager torch ops (speed reference; top_p = 1 only)."""
        import torch
        wl = self.wl
        if self.mode == "sample_full":
            c = torch.cumsum(torch.softmax(self.sets[r]["logits"] / wl.temperature, dim=1), dim=1)
            return torch.searchsorted(c, self.sets[r]["u"][:, None] * c[:, -1:], right=True)
        vals, ids = torch.topk(self.sets[r]["logits"], wl.K, dim=1)
        c = torch.cumsum(torch.softmax(vals / wl.temperature, dim=1), dim=1)
        pos = torch.searchsorted(c, self.sets[r]["u"][:, None] * c[:, -1:], right=True)
        return ids.gather(1, pos.clamp(max=wl.K - 1))

    def _cache(self, ws):
        import torch
        W, csa2, dev = self.W, self.csa2, self.dev
        B, N = ws.B, ws.N
        codes, scales, rope = csa2.alloc_cache(B, N, ws.d_c, ws.d_r, dev)
        for b in range(B):
            lat = W.latent_rows(ws, b, N, dev)
            rp = W.rope_rows(ws, b, N, dev) if ws.d_r else None
            csa2.csa2_quantize_fp4(lat, codes[b], scales[b], 0, rp, rope[b] if ws.d_r else None)
            del lat, rp
        return {"codes": codes, "scales": scales, "rope": rope}

    def _full_set(self, ws):
        import torch
        W, dev = self.W, self.dev
        st = self._cache(ws)
        st["keys"] = torch.stack([W.index_keys(ws, b, dev) for b in range(ws.B)])
        st["qi"] = W.index_query(ws, dev)
        st["q"] = W.attn_query(ws, dev)
        return st

    def _kv(self, r):
        return self.sets[r] if self.mode == "full" else self.cache

    def _keys(self, r):
        return self.sets[r]["keys"] if self.mode == "full" else self.keys

    # ---- stages
    def index(self, r):
        self.csa2.csa2_index_full(self.sets[r]["qi"], self._keys(r), scores=self.scores)

    def select(self, r):
        if self.mode == "prefill_full":
            # the chunk write rides in the scoring call (the Top-K's last
            # level runs it on the CUs its selection leaves idle)
            c, wl = self.cache, self.wl
            self.csa2.csa2_index_topk_full_append(self.sets[r]["qi"], self._keys(r), wl.K, self.chunk,
                                                  c["codes"][0], c["scales"][0], wl.prefill_row0,
                                                  self.chunk_rope, c["rope"][0], out_idx=self.idx,
                                                  out_score=self.top, workspace=self.ws_topk)
            return
        self.csa2.csa2_index_topk_full(self.sets[r]["qi"], self._keys(r), self.wl.K, out_idx=self.idx,
                                       out_score=self.top, workspace=self.ws_topk)

    def pool(self, r):
        st = self.sets[r]
        self.csa2.csa2_index_pool(st["qi"], self.keys, st["pool"], st["nb"], block=self.wl.block,
                                  scores=self.scores, positions=self.positions)

    def build(self, r):
        self.csa2.csa2_build_pool(self.scores, self.wl.P_max, block=self.wl.block, pool_blocks=self.pool_out,
                                  n_blocks=self.nb_out, workspace=self.ws_build)

    def topk(self, r):
        if self.mode == "sample":
            self.csa2.csa2_topk(self.sets[r]["logits"], self.wl.K, out_idx=self.idx, out_score=self.top,
                                workspace=self.ws_topk)
            return
        ids = self.positions if self.mode == "reindex" else None
        self.csa2.csa2_topk(self.scores, self.wl.K, ids=ids, out_idx=self.idx, out_score=self.top,
                            workspace=self.ws_topk)

    def attn_swa(self, r):
        kv, st = self.cache, self.sets[r]
        c, sg, rp = self.win
        self.csa2.csa2_sparse_swa_attn_fp4(st["q"], kv["codes"], kv["scales"], kv["rope"], st["idx"], c, sg, rp,
                                           self.wl.sm_scale, out=self.out, lse=self.lse, workspace=self.ws_swa)

    def swa(self, r):
        c, sg, rp = self.win
        self.csa2.csa2_swa_attn_fp8(self.sets[r]["q"], c, sg, rp, self.wl.sm_scale, merge_out=self.out,
                                    merge_lse=self.lse, out=self.out2, lse=self.lse2)

    def attn(self, r):
        kv, st = self._kv(r), self.sets[r]
        if self.mode == "prefill_reuse":
            self.csa2.csa2_prefill_sparse_attn_fp4(st["q"], kv["codes"], kv["scales"], kv["rope"], st["idx"],
                                                   self.wl.sm_scale, out=self.out, lse=self.lse,
                                                   workspace=self.ws_attn)
            return
        idx = st["idx"] if self.mode in ("reuse", "reuse_swa") else self.idx
        self.csa2.csa2_sparse_attn_fp4(st["q"], kv["codes"], kv["scales"], kv["rope"], idx,
                                       self.wl.sm_scale, out=self.out, lse=self.lse,
                                       workspace=self.ws_attn)

    def step(self, r):
        for s in self.stages:
            getattr(self, s)(r)

    def alg_bytes(self):
        """Algorithmic bytes per launch of each stage and per step: inputs read
        once, outputs written once."""
        wl = self.wl
        B, N, K, H = wl.B, wl.N, wl.K, wl.H
        if self.mode == "sample":
            # logits read once; uniform in, token + prob + n_kept out; candidates (ids + logits) between stages
            return {"sample": B * (N * 4 + 4 + 12), "topk": B * (N * 4 + K * 8), "draw": B * (K * 8 + 4 + 12),
                    "step": B * (N * 4 + 4 + 12)}
        if self.mode == "sample_full":
            # logits read once, uniform in, token + prob out (the drawn tile's second read is not counted)
            return {"draw_full": B * (N * 4 + 4 + 8), "step": B * (N * 4 + 4 + 8)}
        ent = _entry_bytes(wl)
        qi = wl.H_I * wl.D_I * 2
        if self.mode == "prefill_reuse":
            B = wl.prefill_rows            # the chunk's queries
        attn = B * (K * 4 + K * ent + H * wl.D * 2 + H * wl.d_c * 4 + H * 4)
        d = {"attn": attn}
        step = attn
        if self.mode == "reuse_swa":
            win = B * wl.window * _window_bytes(wl)
            d["attn_swa"] = attn + win
            d["step"] = attn + win
            return d
        if self.mode == "pool_build":
            d["index"] = B * (N * wl.D_I * 2 + qi + N * 4)
            d["build"] = B * (N * 4 + wl.P_max * 4 + 4)
            d["step"] = B * (N * wl.D_I * 2 + qi + wl.P_max * 4 + 4)
            return d
        if self.mode in ("full", "prefill_full"):
            # keys and queries read, the K (id, score) pairs written: the
            # scores themselves are not algorithmic bytes
            d["select"] = B * (N * wl.D_I * 2 + qi + K * 8)
            step += B * (N * wl.D_I * 2 + qi)
        if self.mode == "reindex":
            Mp = wl.P_max * wl.block
            d["pool"] = B * (wl.n_blocks * wl.block * wl.D_I * 2 + qi + wl.P_max * 4 + Mp * 8)
            d["topk"] = B * (Mp * 8 + K * 8)
            step += B * (wl.n_blocks * wl.block * wl.D_I * 2 + qi + wl.n_blocks * 4)
        if self.mode == "prefill_full":
            # the chunk write (bf16 rows read, FP4 records written) is part of the select call
            R = wl.prefill_rows
            chunk = R * (wl.d_c * 2 + wl.d_r * 2) + R * (wl.d_c // 2 + wl.d_c // 16 + wl.d_r * 2)
            d["select"] += chunk
            step += chunk
        d["step"] = step
        return d


def cpu_baseline(wl, budget_s):
    """The oracle, as it stands, on a bounded sample of the workload.

    Inputs for one sequence are prepared outside the timed region; then the
    oracle runs the workload's step for as many queries (sampler rows, chunk
    queries) as fit in the budget, one at a time, timed by wall clock.  The
    rate is the measured count over the measured time; in prefill-full the
    chunk write is timed once and the step rate is B / (write + B x the mean
    query time)."""
    import numpy as np
    import oracle
    from sparse_attention_decode_csa2_amd import workloads as W
    from threadpoolctl import threadpool_info
    bits = W.bf16_bits
    mode = wl.mode
    one = wl.scaled(B=1, seed=wl.seed * 1000)
    prep = []

    def cache(n):
        if mode == "full":
            codes, scales = oracle.quantize_fp4(bits(W.latent_rows(one, 0, n)))
            prep.append(f"one oracle-quantised cache of {n} entries")
        else:
            c, sc = W.random_codes(one, 0, n)
            codes, scales = c.numpy(), sc.numpy()
            prep.append(f"one cache of {n} entries (seeded random FP4 codes and E4M3 scales)")
        rope = bits(W.rope_rows(one, 0, n))[None] if wl.d_r else np.zeros((1, n, 0), np.uint16)
        return codes[None], scales[None], rope

    def queries(i):
        w1 = wl.scaled(B=1, seed=1000 + i)
        return bits(W.index_query(w1)) if wl.H_I else None, bits(W.attn_query(w1)) if wl.H else None

    n_q = 16
    qs = [queries(i) for i in range(n_q)] if mode not in ("sample", "sample_full") else []
    fixed_s = 0.0
    if mode in ("full", "prefill_full", "reindex", "pool_build"):
        keys = bits(W.index_keys(one, 0))[None]
    if mode in ("full", "prefill_full", "reindex", "reuse", "reuse_swa", "prefill_reuse"):
        codes, scales, rope = cache(wl.N)
    if mode == "prefill_full":
        chunk = bits(W.prefill_chunk(one))
        t0 = time.perf_counter()
        oracle.quantize_fp4(chunk)
        fixed_s = time.perf_counter() - t0
        prep.append(f"the {wl.prefill_rows}-row chunk write timed once ({fixed_s:.2f} s)")
    if mode == "reindex":
        pools = [W.pool_blocks(wl.scaled(B=1, seed=1000 + i)) for i in range(n_q)]
        pools = [(p.numpy(), nb.numpy()) for p, nb in pools]
    if mode in ("reuse", "reuse_swa"):
        lists = W.reuse_index(wl.scaled(B=n_q, seed=wl.seed * 1000)).numpy()
    if mode == "prefill_reuse":
        # the last chunk of the context sees all but its last few entries: lists
        # uniform over the visible range stand in for the chunk's own lists
        vis = int(W.chunk_visible(wl, 0))
        lists = W.reuse_index(wl.scaled(B=n_q, N=vis, seed=wl.seed * 1000)).numpy()
    if mode == "reuse_swa":
        wcodes, wsig = oracle.quantize_fp8(bits(W.latent_rows(one, 0, wl.window, name="window")))
        wrope = bits(W.rope_rows(one.scaled(seed=one.seed + 7919), 0, wl.window))[None]
        wcodes, wsig = wcodes[None], wsig[None]
    if mode in ("sample", "sample_full"):
        rows = [W.vocab_logits(wl.scaled(B=1, seed=1000 + i)).numpy() for i in range(n_q)]
        us = [W.sampler_uniforms(wl.scaled(B=1, seed=1000 + i)).numpy() for i in range(n_q)]

    def run(i):
        j = i % n_q
        if mode == "sample":
            oracle.sample(rows[j], wl.K, wl.temperature, wl.top_p, us[j])
            return
        if mode == "sample_full":
            oracle.sample_full(rows[j], wl.temperature, us[j])
            return
        qi, q = qs[j]
        if mode in ("full", "prefill_full"):
            oracle.decode_full(qi, None, keys, None, q, codes, scales, rope, wl.K, wl.sm_scale)
        elif mode == "reindex":
            oracle.decode_reindex(qi, None, keys, None, pools[j][0], pools[j][1], wl.block, q, codes, scales,
                                  rope, wl.K, wl.sm_scale)
        elif mode == "pool_build":
            oracle.build_pool(oracle.index_full(qi, None, keys, None), None, wl.block, wl.P_max)
        elif mode == "reuse":
            oracle.decode_reuse(lists[j:j + 1], q, codes, scales, rope, wl.sm_scale)
        elif mode == "reuse_swa":
            o, l = oracle.decode_reuse(lists[j:j + 1], q, codes, scales, rope, wl.sm_scale)
            ow, lw = oracle.swa_attn(q, wcodes, wsig, wrope, None, wl.sm_scale)
            oracle.merge_branches(o, l, ow, lw)
        elif mode == "prefill_reuse":
            oracle.prefill_sparse_attn(q[:, None], codes, scales, rope, lists[j:j + 1][:, None], wl.sm_scale)
        else:
            raise ValueError(mode)

    n = 0
    t0 = time.perf_counter()
    while True:
        run(n)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s and n >= 3:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    what = {"full": "Full-mode decode queries", "prefill_full": "Full-mode decode queries",
            "reindex": "Reindex-mode decode queries", "reuse": "Reuse-mode decode queries",
            "reuse_swa": "Reuse-mode decode queries with the window branch merged",
            "pool_build": "pool constructions (Full scores + pool)", "sample": "sampler rows",
            "sample_full": "untruncated sampler rows",
            "prefill_reuse": "prefill chunk queries"}[mode]
    if mode == "prefill_full":
        value = wl.B / (fixed_s + wl.B * el / n)
    else:
        value = n / el
    unit = "rows/s" if mode in ("sample", "sample_full") else "queries/s"
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{n} {what} (batch 1, {wl.N} {'vocabulary logits' if mode in ('sample', 'sample_full') else 'entries'}"
                      f"{'' if mode in ('sample', 'sample_full') else f', pool of {wl.P_max} blocks' if mode == 'pool_build' else f', Top-{wl.K}'}) in {el:.1f} s"
                      f"{'; ' + '; '.join(prep) if prep else ''}; NumPy float64, BLAS threads={threads}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the step has no "
              f"multi-GPU path (each GPU would run it on its own shard of the batch).", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_attention_decode_csa2_amd import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = W.BY_NAME[args.workload]
    dev = "cuda"
    step = Step(wl, dev)
    R = step.R
    torch.cuda.synchronize()
    print(f"[bench] {wl.name}: mode {wl.mode}, {R} rotating input sets", file=sys.stderr, flush=True)

    # The host cannot enqueue a ~10 us step through Python faster than the GPU
    # runs it, so steps are captured into HIP graphs and replayed: one graph of
    # W warm-up steps, one of the K timed steps (inputs rotating over the R
    # sets), and per stage one graph of K launches of that stage alone.
    stream = torch.cuda.Stream()

    def capture(fn, n, start):
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                fn((start + i) % R)
        torch.cuda.synchronize()
        return g

    for i in range(min(args.warmup, R)):   # eager pass: sets up every buffer once
        step.step(i)
    torch.cuda.synchronize()
    # the warm-up takes sets 0 .. W-1, the timed steps the next K sets (mod R),
    # the per-stage graphs the K after those
    W0 = max(args.warmup, 1)
    g_warm = capture(step.step, W0, 0)
    g_timed = capture(step.step, args.steps, W0)
    stages = step.stages
    g_stage = {s: capture(getattr(step, s), args.steps, W0 + args.steps) for s in stages}

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
    # the same selection by torch.topk (speed reference only: its order among
    # equal scores is unspecified), K launches on the stage's own score rows
    torch_topk_us = torch_sampler_us = None
    if wl.mode in ("sample", "sample_full") and wl.top_p >= 1.0:
        g_ts = capture(step.torch_sampler, args.steps, W0 + args.steps)
        g_ts.replay()
        torch_sampler_us = 1000.0 * timed(g_ts) / args.steps
        del g_ts
    csa2_topk_us = None
    if "topk" in stages or "select" in stages or wl.mode == "sample":
        if "select" in stages:      # score rows for the reference, outside the timed region
            step.index(0)
            torch.cuda.synchronize()
        g_tt = capture(lambda r: torch.topk(step.scores, wl.K, dim=1), args.steps, 0)
        g_tt.replay()
        torch_topk_us = 1000.0 * timed(g_tt) / args.steps
        del g_tt
    if wl.mode == "sample":
        # the sampler's Top-K alone (csa2_topk over the same rows), beside torch.topk
        g_ck = capture(step.topk, args.steps, W0 + args.steps)
        g_ck.replay()
        csa2_topk_us = 1000.0 * timed(g_ck) / args.steps
        del g_ck
    # one step on its own with cold caches (what an isolated decode step
    # waits for, beside the steady-state rate above): a 512 MiB write evicts
    # the L2s and the Infinity Cache before each run; median of five
    g_one = capture(step.step, 1, 0)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(5):
        flush.fill_(1)
        cold.append(1000.0 * timed(g_one))
    del flush
    single_step_us = sorted(cold)[len(cold) // 2]
    alg = step.alg_bytes()
    dom = max(stages, key=lambda s: stage_us[s])
    kernel_file = {"index": "index.hip", "pool": "index.hip", "topk": "topk.hip+topk_filter.hip", "attn": "attn.hip",
                   "sample": "topk.hip+topk_filter.hip+sample.hip",
                   "select": "index_topk.hip+topk.hip" if step.fused_select else "index_topk.hip+index.hip+topk.hip",
                   "attn_swa": "attn.hip",
                   "build": "pool.hip", "swa": "attn.hip", "draw": "sample.hip",
                   "draw_full": "sample.hip"}[dom]
    achieved = alg[dom] / (stage_us[dom] * 1e-6) / 1e9
    traffic = committed_traffic(kernel_file, wl.name)

    if args.calib_copy:
        a = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b

    n_queries = wl.prefill_rows if wl.mode == "prefill_reuse" else wl.B
    qps = n_queries / (ms_per_step * 1e-3)
    launches = {"select": ("index_topk_kernel + topk_final_append_kernel (final level + chunk write)"
                           if wl.mode == "prefill_full" else "index_topk_kernel + topk_kernel (final level)")
                if step.fused_select else "index_kernel + topk_kernel",
                "topk": "topk_estimate_kernel + topk_filter_kernel + topk_select_kernel"
                if getattr(step, "filtered_topk", False) else "topk_kernel (chunk levels)",
                "draw_full": "sample_full_stats_kernel + sample_full_kernel",
                "sample": "topk_estimate_kernel + topk_filter_kernel + topk_select_draw_kernel"
                if getattr(step, "filtered_topk", False) else "topk_kernel (chunk levels) + sample_draw_kernel"}
    roofline = {"bound": "hbm", "kernel": dom, "launches": launches.get(dom, dom), "achieved": achieved,
                "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                "alg_bytes_per_launch": alg[dom]}
    if wl.mode == "prefill_reuse":
        # the chunk's queries share one cache (134 MB, held in the Infinity
        # Cache), so the matrix cores, not HBM, bound the step: scores and
        # value products, 2 flops per multiply-add, fp16 operands
        flops = n_queries * wl.H * wl.K * (wl.D + wl.d_c) * 2
        tf = flops / (stage_us["attn"] * 1e-6) / 1e12
        roofline = {"bound": "mfma", "kernel": "attn", "achieved": tf, "peak": 2500.0, "unit": "TFLOP/s",
                    "frac": tf / 2500.0, "traffic": traffic, "alg_flops_per_launch": flops,
                    "alg_bytes_per_launch": alg["attn"], "alg_gbs": achieved}
    line = {
        "metric": ("decode sampler rows/s + achieved HBM GB/s (% of peak), Top-K + top-p draw"
                   if wl.mode == "sample" else
                   "decode sampler rows/s + achieved HBM GB/s (% of peak), untruncated draw over the vocabulary"
                   if wl.mode == "sample_full" else
                   "prefill chunk queries/s + achieved TFLOP/s (% of MFMA peak), CSA2 FP4 sparse attn"
                   if wl.mode == "prefill_reuse" else
                   "decode queries/s + achieved HBM GB/s (% of peak), CSA2 FP4 sparse attn"),
        "value": qps,
        "unit": "rows/s" if wl.mode in ("sample", "sample_full") else "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("f32 logits, f32 weights" if wl.mode in ("sample", "sample_full") else
                  "fp4(e2m1)+e4m3 cache, bf16/fp16 mfma, fp32 softmax"),
        "data": ("synthetic (seeded; N(0,1) x 4 logits, uniform draws)" if wl.mode in ("sample", "sample_full") else
                 "synthetic (seeded; integer indexer, RMS-normalised N(0,1) latents)"),
        "config": ({"workload": wl.name, "mode": wl.mode, "batch": wl.B, "vocab": wl.N, "top_k": wl.K,
                    "temperature": wl.temperature, "top_p": wl.top_p, "rotation_sets": R}
                   if wl.mode in ("sample", "sample_full") else
                   {"workload": wl.name, "mode": wl.mode, "batch": wl.B, "entries": wl.N,
                    "context_tokens": wl.N * 4, "latent": wl.d_c, "rope": wl.d_r, "heads": wl.H,
                    "indexer": f"{wl.H_I}x{wl.D_I}", "top_k": wl.K, "rotation_sets": R,
                    **({"chunk_queries": wl.prefill_rows} if wl.mode == "prefill_reuse" else {})}),
        "step_hbm_gbs": alg["step"] / (ms_per_step * 1e-3) / 1e9,
        "single_step_us_cold": round(single_step_us, 2),
        "step_alg_bytes": alg["step"],
        "step_read_bytes": step.touched,
        "timed_distinct_sets": min(args.steps, R),
        "stage_us": {s: round(v, 3) for s, v in stage_us.items()},
        "stage_gbs": {s: round(alg[s] / (stage_us[s] * 1e-6) / 1e9, 1) for s in stages},
        "torch_topk_us": None if torch_topk_us is None else round(torch_topk_us, 3),
        **({"csa2_topk_us": round(csa2_topk_us, 3)} if csa2_topk_us is not None else {}),
        "torch_sampler_us": None if torch_sampler_us is None else round(torch_sampler_us, 3),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
