"""Seeded input generators (no GPU): determinism, shapes, value ranges, and the
dynamic-range invariant the FP4 format relies on."""

import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import oracle  # noqa: E402
from sparse_attention_decode_csa2_amd import workloads as W  # noqa: E402


def test_generators_are_deterministic_and_shaped():
    wl = W.WORKLOADS[1].scaled(N=2048, B=2)
    a = W.latent_rows(wl, 0, 64)
    b = W.latent_rows(wl, 0, 64)
    assert a.dtype == torch.bfloat16 and a.shape == (64, 512) and torch.equal(a, b)
    assert not torch.equal(a, W.latent_rows(wl, 1, 64))
    rms = a.float().pow(2).mean(1).sqrt()
    assert torch.allclose(rms, torch.ones_like(rms), atol=1e-2)
    k = W.index_keys(wl, 0)
    assert k.shape == (2048, 128) and k.float().min() >= -8 and k.float().max() <= 8
    assert torch.equal(k.float(), k.float().round())
    q = W.index_query(wl)
    assert q.shape == (2, 8, 128)
    blk, nb = W.pool_blocks(wl.scaled(n_blocks=64, P_max=128))
    assert blk.shape == (2, 128) and torch.all(nb == 64)
    for b in range(2):
        v = blk[b, :64]
        assert torch.all(v[1:] > v[:-1]) and v.min() >= 0 and v.max() < 2048 // 8
        assert torch.all(blk[b, 64:] == -1)
    idx = W.reuse_index(wl)
    assert idx.shape == (2, 512) and torch.all(idx[:, 1:] > idx[:, :-1])
    x = W.prefill_chunk(W.WORKLOADS[4].scaled(prefill_rows=256))
    frac = (x.float().abs() > 6).float().mean().item()
    assert 0.002 < frac < 0.03


def test_rmsnorm_rows_stay_in_normal_scale_range():
    """Unit-RMS latent rows never need a zero, subnormal or saturated E4M3
    scale (the dynamic-range property the FP4 format relies on, stated for
    RMSNorm'd inputs in [P1] section 效率组件四件, item 4)."""
    for wl in W.WORKLOADS[:4]:
        x = W.latent_rows(wl, 0, 2048)
        _, s = oracle.quantize_fp4(W.bf16_bits(x))
        assert np.all(s >= 0x08) and np.all(s < 0x7E), wl.name
    x = W.prefill_chunk(W.WORKLOADS[4].scaled(prefill_rows=2048))
    _, s = oracle.quantize_fp4(W.bf16_bits(x))
    assert np.all(s >= 0x08) and np.all(s < 0x7E)


def test_chunk_lists_are_causal_unique_sorted_and_uniform():
    """Prefill chunk lists: K distinct entries each query may see, sorted;
    every query sees its visible entries in full when it sees fewer than K;
    the lists are deterministic and cover the visible range evenly."""
    wl = W.BY_NAME["prefill-reuse-1m"].scaled(B=2, N=3000, prefill_rows=400, K=256)
    idx = W.chunk_index(wl)
    assert idx.shape == (2, 400, 256) and torch.equal(idx, W.chunk_index(wl))
    vis = W.chunk_visible(wl, torch.arange(400))
    assert int(vis[-1]) == wl.N and torch.all(torch.diff(vis) >= 0)
    for s in range(2):
        for t in range(400):
            row = idx[s, t]
            v = row[row >= 0]
            assert v.numel() == min(256, int(vis[t]))
            assert torch.all(v < vis[t]) and torch.all(torch.diff(v) > 0)
    # uniform over the visible range: each quarter of it holds about a quarter of the picks
    picks = idx[0].float() / vis[:, None].float()
    frac = torch.histc(picks[idx[0] >= 0], bins=4, min=0, max=1) / (idx[0] >= 0).sum()
    assert torch.all((frac - 0.25).abs() < 0.02), frac
    small = W.chunk_index(wl.scaled(N=40, prefill_rows=100, K=16))
    assert small[0, 0].tolist() == list(range(15)) + [-1]      # sees 15 entries: all of them, then -1


def test_sampler_inputs():
    wl = W.BY_NAME["sample-129k"].scaled(B=3, N=5000)
    x = W.vocab_logits(wl)
    u = W.sampler_uniforms(wl)
    assert x.dtype == torch.float32 and x.shape == (3, 5000) and torch.equal(x, W.vocab_logits(wl))
    assert abs(float(x.std()) - 4.0) < 0.2
    assert u.shape == (3,) and torch.all((u >= 0) & (u < 1))
