"""Prefill sparse attention (csa2_prefill_sparse_attn_fp4) on the GPU against
the oracle: T queries per sequence, each with its own causal list into its own
sequence's cache; normwise 2e-3 per (query, head) row and lse to 1e-3, the
bar of the decode attention."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, W, attn_close, csa2, note, np_bits, oracle

pytestmark = pytest.mark.gpu


def _raw_caches(wl, S, N):
    codes, scales, rope = csa2.alloc_cache(S, N, wl.d_c, wl.d_r, DEV)
    for s in range(S):
        c, sc = W.random_codes(wl, s, N, DEV)
        codes[s].copy_(c)
        scales[s].copy_(sc)
        if wl.d_r:
            rope[s].copy_(W.rope_rows(wl, s, N, DEV))
    return codes, scales, rope


def _causal_idx(wl, S, T, N, K):
    ws = wl.scaled(B=S, N=N, K=K, prefill_rows=T)
    return W.chunk_index(ws).numpy()


def _run(wl, S, T, N, K, rows=None):
    codes, scales, rope = _raw_caches(wl, S, N)
    q = W.attn_query(wl.scaled(B=S * T), DEV).view(S, T, wl.H, wl.D)
    idx = _causal_idx(wl, S, T, N, K)
    out, lse = csa2.csa2_prefill_sparse_attn_fp4(q, codes, scales, rope, torch.from_numpy(idx).to(DEV),
                                                 wl.sm_scale)
    torch.cuda.synchronize()
    return q, (codes, scales, rope), idx, out, lse


def _oracle_rows(wl, q, cache, idx, rows):
    """The oracle on the listed (s, t) rows only (one query each)."""
    codes, scales = cache[0].cpu().numpy(), cache[1].cpu().numpy()
    rope = np_bits(cache[2].contiguous())
    qb = np_bits(q)
    ro, rl = [], []
    for s, t in rows:
        o, l = oracle.prefill_sparse_attn(qb[s:s + 1, t:t + 1], codes[s:s + 1], scales[s:s + 1],
                                          rope[s:s + 1], idx[s:s + 1, t:t + 1], wl.sm_scale)
        ro.append(o[0, 0])
        rl.append(l[0, 0])
    return np.stack(ro), np.stack(rl)


CASES = [  # (workload, S, T, N, K): 16-head kernel below 128 queries, 32-head kernel at 128 and above
    (1, 1, 1, 1024, 512), (1, 1, 37, 2048, 512), (1, 2, 64, 4096, 512), (1, 3, 100, 2048, 100),
    (1, 2, 5, 600, 512), (0, 2, 9, 1024, 64),
]


@pytest.mark.parametrize("wi,S,T,N,K", CASES)
def test_prefill_vs_oracle(wi, S, T, N, K):
    wl = W.WORKLOADS[wi]
    note(f"prefill attn: {wl.name} S={S} T={T} N={N} K={K} H={wl.H}")
    q, cache, idx, out, lse = _run(wl, S, T, N, K)
    codes, scales, rope = cache
    ro, rl = oracle.prefill_sparse_attn(np_bits(q), codes.cpu().numpy(), scales.cpu().numpy(),
                                        np_bits(rope.contiguous()), idx, wl.sm_scale)
    attn_close(out.cpu().numpy().reshape(S * T, wl.H, -1), lse.cpu().numpy().reshape(S * T, wl.H),
               ro.reshape(S * T, wl.H, -1), rl.reshape(S * T, wl.H), 2e-3)


@pytest.mark.parametrize("S,T", [(2, 8), (2, 64)])
def test_prefill_equals_decode_over_replicated_caches(S, T):
    """Query (s, t) of a chunk = decode query s * T + t over a copy of
    sequence s's cache: bit for bit (same plan, same kernel, only the
    sequence base differs)."""
    wl = W.WORKLOADS[1]
    N, K = 1024, 512
    note(f"prefill vs decode over replicated caches S={S} T={T}")
    q, (codes, scales, rope), idx, out, lse = _run(wl, S, T, N, K)
    rep = lambda a: a.repeat_interleave(T, dim=0)   # noqa: E731
    dout, dlse = csa2.csa2_sparse_attn_fp4(q.reshape(S * T, wl.H, wl.D), rep(codes), rep(scales), rep(rope),
                                           torch.from_numpy(idx.reshape(S * T, K)).to(DEV), wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(out.reshape(S * T, wl.H, -1), dout)
    assert torch.equal(lse.reshape(S * T, wl.H), dlse)


def test_prefill_masked_and_empty_lists():
    wl = W.WORKLOADS[1]
    S, T, N, K = 2, 6, 1024, 512
    note("prefill attn: masked, out-of-range and empty lists")
    codes, scales, rope = _raw_caches(wl, S, N)
    q = W.attn_query(wl.scaled(B=S * T), DEV).view(S, T, wl.H, wl.D)
    rng = np.random.default_rng(3)
    idx = np.stack([np.stack([np.sort(rng.permutation(N)[:K]) for _ in range(T)]) for _ in range(S)])
    idx[0, 1, ::3] = -1
    idx[1, 2, ::4] = N + 5
    idx[1, 3, :] = -1
    out, lse = csa2.csa2_prefill_sparse_attn_fp4(q, codes, scales, rope, torch.from_numpy(idx.astype(np.int32)).to(DEV),
                                                 wl.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_sparse_attn(np_bits(q), codes.cpu().numpy(), scales.cpu().numpy(),
                                        np_bits(rope.contiguous()), idx, wl.sm_scale)
    attn_close(out.cpu().numpy().reshape(S * T, wl.H, -1), lse.cpu().numpy().reshape(S * T, wl.H),
               ro.reshape(S * T, wl.H, -1), rl.reshape(S * T, wl.H), 2e-3)


def test_prefill_full_workload_sampled_rows():
    """The benchmarked chunk (8192 queries over a 262144-entry cache, Top-512
    lists), quantised through csa2_quantize_fp4; 12 sampled queries against
    the oracle."""
    wl = W.BY_NAME["prefill-reuse-1m"]
    T = wl.prefill_rows
    note(f"prefill attn: {wl.name} T={T} N={wl.N}")
    codes, scales, rope = csa2.alloc_cache(1, wl.N, wl.d_c, wl.d_r, DEV)
    lat = W.latent_rows(wl, 0, wl.N, DEV)
    csa2.csa2_quantize_fp4(lat, codes[0], scales[0], 0, W.rope_rows(wl, 0, wl.N, DEV), rope[0])
    del lat
    q = W.attn_query(wl.scaled(B=T), DEV).view(1, T, wl.H, wl.D)
    idx = W.chunk_index(wl)
    out, lse = csa2.csa2_prefill_sparse_attn_fp4(q, codes, scales, rope, idx.to(DEV), wl.sm_scale)
    torch.cuda.synchronize()
    rows = [(0, t) for t in (0, 1, 63, 64, 1000, 4095, 4096, 5000, 8000, 8190, 8191, 2222)]
    ro, rl = _oracle_rows(wl, q, (codes, scales, rope), idx.numpy(), rows)
    ts = [t for _, t in rows]
    attn_close(out[0, ts].cpu().numpy(), lse[0, ts].cpu().numpy(), ro, rl, 2e-3)


@pytest.mark.parametrize("T", [64, 150])
def test_prefill_in_a_hip_graph_matches_eager(T):
    """csa2_prefill_sparse_attn_fp4 captured into a HIP graph and replayed
    three times, with eager work in between, reproduces the eager result bit
    for bit (128 queries: one unit per workgroup; 300: the persistent
    kernel)."""
    wl = W.WORKLOADS[1]
    S, N, K = 2, 2048, 512
    note(f"prefill attn: HIP graph capture + 3 replays vs eager S={S} T={T}")
    codes, scales, rope = _raw_caches(wl, S, N)
    q = W.attn_query(wl.scaled(B=S * T), DEV).view(S, T, wl.H, wl.D)
    idx = torch.from_numpy(_causal_idx(wl, S, T, N, K)).to(DEV)
    out = torch.empty(S, T, wl.H, wl.d_c, dtype=torch.float32, device=DEV)
    lse = torch.empty(S, T, wl.H, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(csa2.csa2_sparse_attn_workspace_bytes(S * T, wl.H, wl.d_c, K), 16), dtype=torch.uint8,
                     device=DEV)

    def step():
        csa2.csa2_prefill_sparse_attn_fp4(q, codes, scales, rope, idx, wl.sm_scale, out=out, lse=lse, workspace=ws)
    step()
    torch.cuda.synchronize()
    ref = [out.clone(), lse.clone()]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(3):
        out.fill_(0)
        lse.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), rep
        # eager work between replays: two decode queries, one per sequence of the cache
        csa2.csa2_sparse_attn_fp4(q[0, :S], codes, scales, rope, idx[0, :S], wl.sm_scale)
        torch.cuda.synchronize()



@pytest.mark.parametrize("H,dc,dr,S,T", [(40, 512, 64, 1, 300), (64, 512, 0, 2, 150), (17, 512, 64, 3, 100),
                                         (8, 128, 64, 2, 70)])
def test_prefill_head_counts_and_dims(H, dc, dr, S, T):
    """Partial 32-head groups and the variant without a RoPE part on the
    32-head kernel (S * T * ceil(H / 32) >= 256), and small head counts and
    the 128-channel latent on the 16-head kernel."""
    wl = W.WORKLOADS[1].scaled(H=H, d_c=dc, d_r=dr)
    N, K = 2048, 512
    note(f"prefill attn: H={H} d_c={dc} d_r={dr} S={S} T={T}")
    q, cache, idx, out, lse = _run(wl, S, T, N, K)
    codes, scales, rope = cache
    ro, rl = oracle.prefill_sparse_attn(np_bits(q), codes.cpu().numpy(), scales.cpu().numpy(),
                                        np_bits(rope.contiguous()), idx, wl.sm_scale)
    attn_close(out.cpu().numpy().reshape(S * T, H, -1), lse.cpu().numpy().reshape(S * T, H),
               ro.reshape(S * T, H, -1), rl.reshape(S * T, H), 2e-3)
