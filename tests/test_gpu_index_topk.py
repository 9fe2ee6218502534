"""a1 + a3 in one call (csa2_index_topk_full) on the GPU against the oracle's
index_full followed by its topk: bit-exact ids and scores.  The shapes with
at least 256 chunks of 8192 entries run the fused chunk kernel; the others
the separate indexer and Top-K kernels, whose result must be the same."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, W, csa2, note, np_bits, oracle

pytestmark = pytest.mark.gpu


def _keys(wl, B):
    return torch.stack([W.index_keys(wl, b, DEV) for b in range(B)])


def _oracle_row(q, k, K, w, nv, b):
    wb = None if w is None else w[b:b + 1].cpu().numpy().astype(np.float64)
    nb = None if nv is None else nv[b:b + 1].cpu().numpy()
    rs = oracle.index_full(np_bits(q[b:b + 1]), wb, np_bits(k[b:b + 1]), nb)
    return oracle.topk(rs, None, nb, K)


def _check(q, k, K, w=None, nv=None, rows=None, against_separate=False):
    gi, gs = csa2.csa2_index_topk_full(q, k, K, w=w, n_valid=nv)
    torch.cuda.synchronize()
    gi, gs = gi.cpu().numpy(), gs.cpu().numpy().astype(np.float64)
    B = q.shape[0]
    for b in range(B) if rows is None else rows:
        ri, rt = _oracle_row(q, k, K, w, nv, b)
        assert np.array_equal(gi[b], ri[0]), (b, np.nonzero(gi[b] != ri[0])[0][:8])
        assert np.array_equal(gs[b], rt[0], equal_nan=True), b
    if against_separate:
        sc = csa2.csa2_index_full(q, k, w=w, n_valid=nv)
        si, ss = csa2.csa2_topk(sc, K, n_valid=nv)
        torch.cuda.synchronize()
        assert np.array_equal(si.cpu().numpy(), gi)
        assert np.array_equal(ss.cpu().numpy().astype(np.float64), gs, equal_nan=True)


def test_prefill_full_1m_every_row():
    """The 1M-entry Full workload (8 sequences x 262144 entries, Top-512):
    32 chunks per row, 256 workgroups; every row against the oracle and the
    whole result against the separate kernels."""
    wl = W.BY_NAME["prefill-full-1m"]
    note(f"index_topk: {wl.name} B={wl.B} N={wl.N} K={wl.K} (fused, every row)")
    assert csa2.csa2_index_topk_full_workspace_bytes(wl.B, wl.D_I, wl.N, wl.K) == wl.B * 32 * wl.K * 8
    _check(W.index_query(wl, DEV), _keys(wl, wl.B), wl.K, against_separate=True)


def test_ragged_tail_and_n_valid():
    """N_cap not a multiple of the chunk (17 chunks per row, the last of 37
    entries), n_valid at, below and past chunk edges, zero, negative and past
    N_cap (clamped)."""
    N = 16 * 8192 + 37
    wl = W.BY_NAME["prefill-full-1m"].scaled(B=16, N=N)
    nv = torch.tensor([N, N - 1, 131072, 131071, 8192, 8191, 8193, 1, 0, -5, 2 ** 31 - 1, 70000, 16384, 100,
                       24576, 600], dtype=torch.int32, device=DEV)
    note(f"index_topk: B=16 N={N} ragged n_valid (fused)")
    q, k = W.index_query(wl, DEV), _keys(wl, 16)
    _check(q, k, 512, nv=nv, against_separate=True)
    # integer head weights keep the scores exact
    w = torch.randint(0, 4, (16, wl.H_I), device=DEV).float()
    _check(q, k, 512, w=w, nv=nv)


@pytest.mark.parametrize("H_I,D_I,K", [(8, 128, 1), (8, 128, 100), (8, 128, 2048), (1, 32, 512), (5, 64, 512),
                                       (16, 128, 512), (16, 256, 512)])
def test_head_shapes_and_k(H_I, D_I, K):
    """One chunk per row over 256 rows (fused, D_I <= 128; D_I 256 goes
    through the separate kernels)."""
    wl = W.BY_NAME["prefill-full-1m"].scaled(B=256, N=8192, H_I=H_I, D_I=D_I)
    note(f"index_topk: B=256 N=8192 H_I={H_I} D_I={D_I} K={K}")
    _check(W.index_query(wl, DEV), _keys(wl, 256), K, rows=range(0, 256, 15))


def test_tie_floods_across_chunks():
    """0/1 keys and queries: integer scores in [0, 128] over 262144 entries, so
    the K-th largest score is shared by thousands of entries in every chunk
    and the lower ids must win across chunks and levels."""
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    B, N, H_I, D_I = 8, 262144, 4, 32
    k = torch.randint(0, 2, (B, N, D_I), generator=g, device=DEV).to(torch.bfloat16)
    q = torch.randint(0, 2, (B, H_I, D_I), generator=g, device=DEV).to(torch.bfloat16)
    note(f"index_topk: tie floods B={B} N={N} D_I={D_I} (fused)")
    for K in (512, 2048):
        _check(q, k, K, against_separate=True)


def test_separate_kernels_below_a_workgroup_per_cu():
    """The Full 64k workload (one row of 16384 entries): separate kernels."""
    wl = W.BY_NAME["full-64k"]
    note(f"index_topk: {wl.name} (separate kernels)")
    assert csa2.csa2_index_topk_full_workspace_bytes(1, wl.D_I, wl.N, wl.K) == wl.N * 4
    _check(W.index_query(wl, DEV), _keys(wl, 1), wl.K)


def test_fused_call_in_a_hip_graph_matches_eager():
    """Captured into a HIP graph and replayed three times, with eager work in
    between, the fused call reproduces the eager result bit for bit."""
    wl = W.BY_NAME["prefill-full-1m"]
    note("index_topk: HIP graph capture + 3 replays vs eager")
    q, k = W.index_query(wl, DEV), _keys(wl, wl.B)
    idx = torch.empty(wl.B, wl.K, dtype=torch.int32, device=DEV)
    top = torch.empty(wl.B, wl.K, dtype=torch.float32, device=DEV)
    ws = torch.empty(csa2.csa2_index_topk_full_workspace_bytes(wl.B, wl.D_I, wl.N, wl.K), dtype=torch.uint8,
                     device=DEV)

    def step():
        csa2.csa2_index_topk_full(q, k, wl.K, out_idx=idx, out_score=top, workspace=ws)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (idx, top)]
    s = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        step()
    for rep in range(3):
        idx.fill_(0)
        top.fill_(0)
        ws.fill_(0)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]) and torch.equal(top, ref[1]), rep
        csa2.csa2_index_topk_full(q[:1], k[:1], 64)      # eager work between replays
        torch.cuda.synchronize()


def _rand_cache(wl, cap, seed):
    """Two identical FP4 caches of one sequence, filled with random bytes (so
    that rows an append must not touch are checked too)."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    ca = csa2.alloc_cache(1, cap, wl.d_c, wl.d_r, DEV)
    cb = csa2.alloc_cache(1, cap, wl.d_c, wl.d_r, DEV)
    for ta, tb in zip(ca, cb):
        if ta.numel() == 0:
            continue
        if ta.dtype == torch.uint8:
            ta.copy_(torch.randint(0, 256, ta.shape, generator=g, device=DEV, dtype=torch.uint8))
        else:
            ta.copy_(torch.randn(ta.shape, generator=g, device=DEV).to(ta.dtype))
        tb.copy_(ta)
    return ca, cb


def _append_vs_separate(wl, q, k, K, rows, cap, row0, seed=0):
    x = W.latent_rows(wl, 0, rows, DEV)
    rs = W.rope_rows(wl, 0, rows, DEV) if wl.d_r else None
    ca, cb = _rand_cache(wl, cap, seed)
    fi, fs = csa2.csa2_index_topk_full_append(q, k, K, x, ca[0][0], ca[1][0], row0, rs, ca[2][0] if wl.d_r else None)
    si, ss = csa2.csa2_index_topk_full(q, k, K)
    csa2.csa2_quantize_fp4(x, cb[0][0], cb[1][0], row0, rs, cb[2][0] if wl.d_r else None)
    torch.cuda.synchronize()
    assert torch.equal(fi, si)
    assert torch.equal(fs.view(torch.int32), ss.view(torch.int32))
    for ta, tb in zip(ca, cb):
        if ta.numel():
            assert torch.equal(ta.contiguous().view(torch.uint8), tb.contiguous().view(torch.uint8))
    return fi


def test_scoring_and_append_in_one_call():
    """csa2_index_topk_full_append = csa2_index_topk_full + csa2_quantize_fp4,
    bit for bit, on the benchmarked step (8 x 262144 entries, the 8192-row
    chunk appended by the Top-K's last level) and with ragged and tiny
    appends, no RoPE part, the separate-kernel path (one row of 16384
    entries), an empty scoring (B = 0) and an empty append."""
    wl = W.BY_NAME["prefill-full-1m"]
    note(f"index_topk + append: {wl.name} B={wl.B} N={wl.N} chunk {wl.prefill_rows} rows")
    q, k = W.index_query(wl, DEV), _keys(wl, wl.B)
    fi = _append_vs_separate(wl, q, k, wl.K, wl.prefill_rows, wl.N, wl.prefill_row0, seed=1)
    ri, _ = _oracle_row(q, k, wl.K, None, None, 3)
    assert np.array_equal(fi[3].cpu().numpy(), ri[0])
    _append_vs_separate(wl, q, k, wl.K, 1000, 4096, 5, seed=2)
    _append_vs_separate(wl, q, k, wl.K, 1, 16, 15, seed=3)
    _append_vs_separate(wl.scaled(d_r=0), q, k, wl.K, 777, 1000, 200, seed=4)
    _append_vs_separate(wl, q, k, wl.K, 0, 16, 16, seed=5)
    w64 = W.BY_NAME["full-64k"]
    note("index_topk + append: separate-kernel path, B = 0")
    _append_vs_separate(w64, W.index_query(w64, DEV), _keys(w64, 1), w64.K, 3000, 8192, 100, seed=6)
    _append_vs_separate(wl, q[:0], k[:0], wl.K, 500, 600, 50, seed=7)
    # 256 rows of one chunk each: the last level has 256 selection
    # workgroups and the append its minimum of eight
    wb = wl.scaled(B=256, N=8192)
    note("index_topk + append: B = 256 rows of 8192 entries")
    _append_vs_separate(wb, W.index_query(wb, DEV), _keys(wb, 256), wb.K, 3000, 4096, 1000, seed=8)


def test_scoring_and_append_in_a_hip_graph():
    """The one-call step captured into a HIP graph and replayed three times
    (outputs and the appended rows cleared in between, eager work between the
    replays) reproduces the eager result bit for bit."""
    wl = W.BY_NAME["prefill-full-1m"]
    note("index_topk + append: HIP graph capture + 3 replays vs eager")
    q, k = W.index_query(wl, DEV), _keys(wl, wl.B)
    x = W.latent_rows(wl, 0, wl.prefill_rows, DEV)
    rs = W.rope_rows(wl, 0, wl.prefill_rows, DEV)
    codes, scales, rope = csa2.alloc_cache(1, wl.prefill_rows, wl.d_c, wl.d_r, DEV)
    idx = torch.empty(wl.B, wl.K, dtype=torch.int32, device=DEV)
    top = torch.empty(wl.B, wl.K, dtype=torch.float32, device=DEV)
    ws = torch.empty(csa2.csa2_index_topk_full_workspace_bytes(wl.B, wl.D_I, wl.N, wl.K), dtype=torch.uint8,
                     device=DEV)

    def step():
        csa2.csa2_index_topk_full_append(q, k, wl.K, x, codes[0], scales[0], 0, rs, rope[0], out_idx=idx,
                                         out_score=top, workspace=ws)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (idx, top, codes, scales, rope)]
    s = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        step()
    for rep in range(3):
        for t in (idx, top, codes, scales, rope):
            t.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for t, r in zip((idx, top, codes, scales, rope), ref):
            assert torch.equal(t, r), rep
        csa2.csa2_index_topk_full(q[:1], k[:1], 64)      # eager work between replays
        torch.cuda.synchronize()
