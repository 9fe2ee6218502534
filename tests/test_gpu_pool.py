"""Candidate-pool construction (csa2_build_pool) on the GPU against the
oracle: bit-exact pool block ids and counts over tie-heavy rows with -inf and
NaN, ragged valid lengths, both load paths (rows that are and are not a whole
number of 16-byte words), and a 1M-token context (32768 blocks, two-level
Top-K); and the hierarchical-indexer composition: Full scores -> pool ->
Reindex re-scoring with the same query gives exactly the Full Top-512."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, W, csa2, note, np_bits, oracle

pytestmark = pytest.mark.gpu


def _rows(rng, B, M, kind):
    if kind == "ties":
        s = rng.integers(0, 4, size=(B, M)).astype(np.float32)
        r = rng.random((B, M))
        s[r < 0.1] = -np.inf
        s[(r >= 0.1) & (r < 0.15)] = np.nan
    else:  # indexer-like integer sums
        s = np.maximum(rng.normal(900, 500, size=(B, M)), 0).round().astype(np.float32)
    return s


@pytest.mark.parametrize("M,block,P_max", [(1, 8, 4), (7, 8, 4), (40, 4, 5), (1001, 8, 64), (1000, 8, 64),
                                           (4099, 3, 300), (16384, 8, 2048), (50000, 8, 2048), (300, 64, 3)])
@pytest.mark.parametrize("kind", ["ties", "int"])
def test_pool_matches_oracle(M, block, P_max, kind):
    note(f"pool: M={M} block={block} P_max={P_max} {kind}")
    rng = np.random.default_rng(M + block + P_max)
    B = 4
    s = _rows(rng, B, M, kind)
    nv = np.array([M, rng.integers(0, M + 1), 0, min(M, block * 3 + 1)], dtype=np.int32)
    st = torch.from_numpy(s).to(DEV)
    nvt = torch.from_numpy(nv).to(DEV)
    pool, nb = csa2.csa2_build_pool(st, P_max, block=block, n_valid=nvt)
    torch.cuda.synchronize()
    want_p, want_n = oracle.build_pool(s.astype(np.float64), nv, block, P_max)
    assert np.array_equal(nb.cpu().numpy(), want_n)
    assert np.array_equal(pool.cpu().numpy(), want_p)


def test_pool_without_n_valid_and_all_nan_blocks():
    note("pool: n_valid NULL, NaN-only and -inf-only blocks")
    M, block, P_max = 64, 8, 8
    s = np.arange(M, dtype=np.float32)[None].repeat(2, 0)
    s[0, 8:16] = np.nan       # a NaN-only block ranks below every number
    s[0, 16:24] = -np.inf     # a -inf block ranks above it
    s[1, :] = 7.0             # all blocks tie: lower ids first
    st = torch.from_numpy(s).to(DEV)
    pool, nb = csa2.csa2_build_pool(st, P_max, block=block)
    torch.cuda.synchronize()
    want_p, want_n = oracle.build_pool(s.astype(np.float64), None, block, P_max)
    assert np.array_equal(pool.cpu().numpy(), want_p)
    assert np.array_equal(nb.cpu().numpy(), want_n)
    assert pool.cpu().numpy()[0].tolist()[-2:] == [2, 1]
    assert pool.cpu().numpy()[1].tolist() == list(range(8))


def test_pool_from_full_scores_then_reindex_reproduces_full_topk():
    """Reindex-sized context (262144 entries, 2048 blocks of 8): the pool built
    from the Full layer's own scores contains every block of its Top-512, so
    re-scoring the pool with the same indexer query returns the Full Top-512
    exactly; the pool itself matches the oracle bit for bit."""
    wl = W.WORKLOADS[2].scaled(B=2)
    note(f"pool: compose Full -> pool -> Reindex, B={wl.B} N={wl.N}")
    keys = torch.stack([W.index_keys(wl, b, DEV) for b in range(wl.B)])
    qi = W.index_query(wl, DEV)
    nv = torch.tensor([wl.N, wl.N - 12345], dtype=torch.int32, device=DEV)
    full = csa2.csa2_index_full(qi, keys, n_valid=nv)
    ref_i, ref_s = csa2.csa2_topk(full, wl.K, n_valid=nv)
    pool, nb = csa2.csa2_build_pool(full, wl.P_max, block=wl.block, n_valid=nv)
    sc, pos = csa2.csa2_index_pool(qi, keys, pool, nb, block=wl.block, n_valid=nv)
    got_i, got_s = csa2.csa2_topk(sc, wl.K, ids=pos)
    torch.cuda.synchronize()
    assert torch.equal(got_i, ref_i)
    assert torch.equal(got_s, ref_s)
    f64 = full.double().cpu().numpy()
    want_p, want_n = oracle.build_pool(f64, nv.cpu().numpy(), wl.block, wl.P_max)
    assert np.array_equal(pool.cpu().numpy(), want_p)
    assert np.array_equal(nb.cpu().numpy(), want_n)
    # and the Full scores themselves are the oracle's (integer-valued, exact)
    for b in range(wl.B):
        ok = oracle.index_full(np_bits(qi[b:b + 1]), None, np_bits(keys[b:b + 1, :4096]), None)
        assert np.array_equal(f64[b, :4096], ok[0])
