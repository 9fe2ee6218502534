"""Helpers shared by the GPU parity tests: build device inputs from the seeded
generators, run the HIP path through the C-ABI binding, and hand host copies of
the very same inputs to the oracle."""

import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
from sparse_attention_decode_csa2_amd import csa2  # noqa: E402
from sparse_attention_decode_csa2_amd import workloads as W  # noqa: E402

DEV = "cuda"


def note(msg):
    """Name the case on stdout before a GPU step (flushed, so a crash still shows it)."""
    print(f"[case] {msg}", flush=True)


def np_bits(t):
    return W.bf16_bits(t)


class Cache:
    """FP4 main-KV cache of one workload, built on the GPU by csa2_quantize_fp4
    from seeded bf16 latent rows; latents of any sequence can be regenerated
    (same generator, same device) for the oracle."""

    def __init__(self, wl, B=None, device=DEV, layout="record"):
        self.wl = wl
        self.B = wl.B if B is None else B
        N, d_c, d_r = wl.N, wl.d_c, wl.d_r
        self.codes, self.scales, self.rope = csa2.alloc_cache(self.B, N, d_c, d_r, device, layout)
        for b in range(self.B):
            lat = W.latent_rows(wl, b, N, device)
            rp = W.rope_rows(wl, b, N, device) if d_r > 0 else None
            csa2.csa2_quantize_fp4(lat, self.codes[b], self.scales[b], 0, rp, self.rope[b] if d_r > 0 else None)
            del lat, rp
        self.device = device

    def latents_host(self, b, rows=None):
        lat = W.latent_rows(self.wl, b, self.wl.N, self.device)
        if rows is not None:
            lat = lat[torch.as_tensor(rows, device=self.device, dtype=torch.long)]
        return np_bits(lat)

    def rope_host(self, b, rows=None):
        if self.wl.d_r == 0:
            n = self.wl.N if rows is None else len(rows)
            return np.zeros((n, 0), dtype=np.uint16)
        rp = W.rope_rows(self.wl, b, self.wl.N, self.device)
        if rows is not None:
            rp = rp[torch.as_tensor(rows, device=self.device, dtype=torch.long)]
        return np_bits(rp)


def oracle_attention_rows(cache, b, q_bits_b, idx_b, sm_scale):
    """Oracle attention for sequence b using only the selected rows: the oracle
    quantises those rows itself from the seeded bf16 latents."""
    idx_b = np.asarray(idx_b, dtype=np.int64)
    N = cache.wl.N
    ok = (idx_b >= 0) & (idx_b < N)
    rows = np.unique(idx_b[ok])
    if rows.size == 0:
        rows = np.array([0])
    lat = cache.latents_host(b, rows)
    codes, scales = oracle.quantize_fp4(lat)
    rope = cache.rope_host(b, rows)
    remap = np.full(idx_b.shape, -1, dtype=np.int64)
    pos = {int(r): i for i, r in enumerate(rows)}
    for j, v in enumerate(idx_b):
        if ok[j]:
            remap[j] = pos[int(v)]
    out, lse = oracle.sparse_attn(q_bits_b[None], codes[None], scales[None], rope[None], remap[None],
                                  sm_scale)
    return out[0], lse[0]


def attn_close(out, lse, ref_out, ref_lse, tol=2e-3):
    """Normwise per (b, h) row: max|o - o_ref| <= tol * max|o_ref|.  lse (an
    fp32 output) within 1e-3 plus four fp32 ulps of its magnitude."""
    out = np.asarray(out, dtype=np.float64)
    ref_out = np.asarray(ref_out, dtype=np.float64)
    err = np.abs(out - ref_out).max(axis=-1)
    scale = np.abs(ref_out).max(axis=-1)
    rel = np.where(scale > 0, err / np.maximum(scale, 1e-300), err)
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= tol, f"normwise relative error {worst:.3e} > {tol}"
    if ref_lse is not None:
        a = np.asarray(lse, dtype=np.float64)
        r = np.asarray(ref_lse, dtype=np.float64)
        both_inf = np.isneginf(a) & np.isneginf(r)
        with np.errstate(invalid="ignore"):
            d = np.where(both_inf, 0.0, np.abs(a - r))
        bound = 1e-3 + 4 * 2.0 ** -23 * np.where(np.isfinite(r), np.abs(r), 0.0)
        assert np.all(d <= bound), f"lse error {float(np.max(d - bound)):.3e} above bound"
    return worst
