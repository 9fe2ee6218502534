"""The three CSA2 decode modes end to end on the workloads' full sizes, chained
through the C-ABI exactly as the bench runs them; the oracle recomputes
every sequence from the seeded inputs (bit-exact Top-K ids and scores,
attention within 2e-3)."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, Cache, W, attn_close, csa2, note, np_bits, oracle, oracle_attention_rows

pytestmark = pytest.mark.gpu


def _keys(wl, B):
    return torch.stack([W.index_keys(wl, b, DEV) for b in range(B)])


def _check_full(wl, cache, k, qi, q, check_b, n_valid=None, fused=False):
    if fused:
        idx, top = csa2.csa2_index_topk_full(qi, k, wl.K, n_valid=n_valid)
    else:
        sc = csa2.csa2_index_full(qi, k, n_valid=n_valid)
        idx, top = csa2.csa2_topk(sc, wl.K, n_valid=n_valid)
    out, lse = csa2.csa2_sparse_attn_fp4(q, cache.codes, cache.scales, cache.rope, idx, wl.sm_scale)
    torch.cuda.synchronize()
    for b in check_b:
        nv = None if n_valid is None else n_valid[b:b + 1].cpu().numpy()
        rs = oracle.index_full(np_bits(qi[b:b + 1]), None, np_bits(k[b:b + 1]), nv)
        ri, rt = oracle.topk(rs, None, nv, wl.K)
        assert np.array_equal(idx[b].cpu().numpy(), ri[0]), b
        assert np.array_equal(top[b].cpu().numpy().astype(np.float64), rt[0]), b
        ro, rl = oracle_attention_rows(cache, b, np_bits(q)[b], ri[0], wl.sm_scale)
        attn_close(out[b].cpu().numpy(), lse[b].cpu().numpy(), ro, rl)


@pytest.mark.parametrize("wi", [0, 1])
def test_full_mode_decode(wi):
    wl = W.WORKLOADS[wi]
    note(f"decode full: {wl.name}")
    cache = Cache(wl)
    _check_full(wl, cache, _keys(wl, wl.B), W.index_query(wl, DEV), W.attn_query(wl, DEV), range(wl.B))


def test_full_mode_decode_partial_cache():
    wl = W.WORKLOADS[1].scaled(B=3, N=5000)
    note("decode full: B=3 N=5000, n_valid 5000 / 300 / 700")
    cache = Cache(wl)
    nv = torch.tensor([5000, 300, 700], dtype=torch.int32, device=DEV)
    _check_full(wl, cache, _keys(wl, 3), W.index_query(wl, DEV), W.attn_query(wl, DEV), range(3), nv)


def test_reindex_mode_decode():
    wl = W.WORKLOADS[2]
    note(f"decode reindex: {wl.name} B=32 N=262144 (every sequence checked)")
    cache = Cache(wl)
    k = _keys(wl, wl.B)
    qi = W.index_query(wl, DEV)
    q = W.attn_query(wl, DEV)
    blk, nb = W.pool_blocks(wl, DEV)
    sc, pos = csa2.csa2_index_pool(qi, k, blk, nb, block=wl.block)
    idx, top = csa2.csa2_topk(sc, wl.K, ids=pos)
    out, lse = csa2.csa2_sparse_attn_fp4(q, cache.codes, cache.scales, cache.rope, idx, wl.sm_scale)
    torch.cuda.synchronize()
    for b in range(wl.B):
        rs, rp = oracle.index_pool(np_bits(qi[b:b + 1]), None, np_bits(k[b:b + 1]), None,
                                   blk[b:b + 1].cpu().numpy(), nb[b:b + 1].cpu().numpy(), wl.block)
        ri, rt = oracle.topk(rs, rp, None, wl.K)
        assert np.array_equal(idx[b].cpu().numpy(), ri[0]), b
        assert np.array_equal(top[b].cpu().numpy().astype(np.float64), rt[0]), b
        ro, rl = oracle_attention_rows(cache, b, np_bits(q)[b], ri[0], wl.sm_scale)
        attn_close(out[b].cpu().numpy(), lse[b].cpu().numpy(), ro, rl)


def test_reuse_mode_decode():
    wl = W.WORKLOADS[3]
    note(f"decode reuse: {wl.name} B=128 N=32768 (every sequence checked)")
    cache = Cache(wl)
    q = W.attn_query(wl, DEV)
    idx = W.reuse_index(wl, DEV)
    out, lse = csa2.csa2_sparse_attn_fp4(q, cache.codes, cache.scales, cache.rope, idx, wl.sm_scale)
    torch.cuda.synchronize()
    qb = np_bits(q)
    ih = idx.cpu().numpy()
    o = out.cpu().numpy()
    ls = lse.cpu().numpy()
    for b in range(wl.B):
        ro, rl = oracle_attention_rows(cache, b, qb[b], ih[b], wl.sm_scale)
        attn_close(o[b], ls[b], ro, rl)


def test_prefill_write_then_full_decode_1m():
    wl = W.WORKLOADS[4]
    note(f"decode prefill+full: {wl.name} append 8192 rows, B=8 N=262144 (every sequence checked)")
    cache = Cache(wl)
    chunk = W.prefill_chunk(wl, DEV)
    crope = W.prefill_rope(wl, DEV)
    r0 = wl.prefill_row0
    csa2.csa2_quantize_fp4(chunk, cache.codes[0], cache.scales[0], r0, crope, cache.rope[0])
    torch.cuda.synchronize()
    wc, ws = oracle.quantize_fp4(np_bits(chunk))
    assert np.array_equal(cache.codes[0, r0:].cpu().numpy(), wc)
    assert np.array_equal(cache.scales[0, r0:].cpu().numpy(), ws)
    # the oracle's view of sequence 0 now has the chunk in rows [r0, N)
    base_lat = cache.latents_host

    def lat0(b, rows=None):
        full = base_lat(b)
        if b == 0:
            full = full.copy()
            full[r0:] = np_bits(chunk)
        return full if rows is None else full[np.asarray(rows)]
    base_rope = cache.rope_host

    def rope0(b, rows=None):
        full = base_rope(b)
        if b == 0:
            full = full.copy()
            full[r0:] = np_bits(crope)
        return full if rows is None else full[np.asarray(rows)]
    cache.latents_host, cache.rope_host = lat0, rope0
    # scores and Top-K in the one call the step makes (the fused chunk kernel here)
    _check_full(wl, cache, _keys(wl, wl.B), W.index_query(wl, DEV), W.attn_query(wl, DEV), range(wl.B),
                fused=True)


def test_full_step_in_a_hip_graph_matches_eager():
    """The Full-mode step captured into a HIP graph and replayed several times,
    with eager work in between, reproduces the eager result bit for bit."""
    wl = W.WORKLOADS[1]
    note("decode full: HIP graph capture + 3 replays vs eager")
    cache = Cache(wl)
    k = _keys(wl, 1)
    qi = W.index_query(wl, DEV)
    q = W.attn_query(wl, DEV)
    sc = torch.empty(1, wl.N, dtype=torch.float32, device=DEV)
    idx = torch.empty(1, wl.K, dtype=torch.int32, device=DEV)
    top = torch.empty(1, wl.K, dtype=torch.float32, device=DEV)
    out = torch.empty(1, wl.H, wl.d_c, dtype=torch.float32, device=DEV)
    lse = torch.empty(1, wl.H, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(csa2.csa2_sparse_attn_workspace_bytes(1, wl.H, wl.d_c, wl.K), 16),
                     dtype=torch.uint8, device=DEV)

    def step():
        csa2.csa2_index_full(qi, k, scores=sc)
        csa2.csa2_topk(sc, wl.K, out_idx=idx, out_score=top)
        csa2.csa2_sparse_attn_fp4(q, cache.codes, cache.scales, cache.rope, idx, wl.sm_scale, out=out,
                                  lse=lse, workspace=ws)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (sc, idx, top, out, lse)]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(3):
        for t in (sc, idx, top, out, lse):
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((sc, idx, top, out, lse), ref):
            assert torch.equal(a, b), rep
        # eager work between replays
        csa2.csa2_index_full(qi, k)
        torch.cuda.synchronize()
