"""a3 csa2_topk on the GPU against the oracle: bit-exact ids and scores,
including heavy ties, NaN, -0, -inf, empty candidates and long rows that go
through the chunked reduction."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, csa2, note, oracle

pytestmark = pytest.mark.gpu


def _scores(rng, B, M, kind):
    if kind == "ties":
        s = rng.integers(0, 40, size=(B, M)).astype(np.float32)
    elif kind == "int_scores":      # indexer-like: integer sums, many near the top
        s = np.maximum(rng.normal(900, 500, size=(B, M)), 0).round().astype(np.float32)
    elif kind == "continuous":
        s = rng.standard_normal((B, M)).astype(np.float32)
    elif kind == "cluster":          # runs of equal scores above and at the K-th largest
        s = np.maximum(rng.normal(900, 500, size=(B, M)), 0).round().astype(np.float32)
        r = rng.random((B, M))
        s[r < 0.01] = 5000.0
        s[(r >= 0.01) & (r < 0.015)] = 2500.0
    elif kind == "outlier":          # one far-off score squeezes the rest into a bucket or two
        s = np.maximum(rng.normal(900, 500, size=(B, M)), 0).round().astype(np.float32)
        s[:, rng.integers(0, M, size=B)] = -1e30
    elif kind == "narrow":           # a tiny spread, then subnormals
        s = (1.0 + rng.random((B, M)) * 1e-6).astype(np.float32)
        if M > 1:
            s[:, ::2] = (rng.random((B, (M + 1) // 2)) * 1e-39).astype(np.float32)
    else:                            # specials sprinkled over tied integers
        s = rng.integers(-3, 4, size=(B, M)).astype(np.float32)
        r = rng.random((B, M))
        s[r < 0.05] = np.nan
        s[(r >= 0.05) & (r < 0.1)] = -0.0
        s[(r >= 0.1) & (r < 0.15)] = -np.inf
        s[(r >= 0.15) & (r < 0.17)] = np.inf
    return s


def _check(s, K, ids=None, nv=None):
    B, M = s.shape
    st = torch.from_numpy(s).to(DEV)
    it = None if ids is None else torch.from_numpy(ids).to(DEV)
    nt = None if nv is None else torch.from_numpy(nv).to(DEV)
    gi, gs = csa2.csa2_topk(st, K, ids=it, n_valid=nt)
    torch.cuda.synchronize()
    ri, rs = oracle.topk(s.astype(np.float64), ids, nv, K)
    gi = gi.cpu().numpy()
    gs = gs.cpu().numpy().astype(np.float64)
    assert np.array_equal(gi, ri), np.nonzero(gi != ri)
    assert np.array_equal(gs, rs, equal_nan=True)


# rows of one chunk, of two levels (3, 5 and 19 chunks of 16384; 8 chunks at
# K = 2048, whose winners fill the final chunk) and ragged tails
CASES = [(1, 1, 1), (2, 7, 4), (3, 1000, 64), (1, 16384, 512), (2, 16385, 512), (2, 40000, 512),
         (1, 5000, 2048), (4, 16384, 2048), (2, 100, 512), (1, 300000, 100), (2, 81920, 512),
         (1, 131072, 2048)]


@pytest.mark.parametrize("B,M,K", CASES)
@pytest.mark.parametrize("kind", ["ties", "int_scores", "continuous", "specials", "cluster", "outlier",
                                  "narrow"])
def test_topk_column_ids(B, M, K, kind):
    note(f"topk: B={B} M={M} K={K} {kind}")
    rng = np.random.default_rng(B * 7 + M + K)
    s = _scores(rng, B, M, kind)
    _check(s, K)
    nv = rng.integers(0, M + 1, size=B).astype(np.int32)
    nv[0] = M
    _check(s, K, nv=nv)


@pytest.mark.parametrize("B,M,K", [(2, 1000, 64), (2, 16384, 512), (2, 40000, 512)])
def test_topk_given_ids(B, M, K):
    note(f"topk: given ids B={B} M={M} K={K}")
    rng = np.random.default_rng(M)
    s = _scores(rng, B, M, "ties")
    ids = np.stack([rng.permutation(1 << 20)[:M] for _ in range(B)]).astype(np.int32)
    ids[rng.random((B, M)) < 0.1] = -1
    _check(s, K, ids=ids)
    # sorted pool positions (the Reindex layout) with holes
    pos = np.sort(np.stack([rng.permutation(1 << 18)[:M] for _ in range(B)]), axis=1).astype(np.int32)
    pos[:, -100:] = -1
    _check(s, K, ids=pos)


def test_topk_full_row_of_one_value_and_all_invalid():
    note("topk: constant rows, all-invalid rows")
    s = np.full((2, 20000), 7.0, dtype=np.float32)
    _check(s, 512)
    _check(s, 512, nv=np.array([0, 3], dtype=np.int32))
    ids = np.full((2, 20000), -1, dtype=np.int32)
    _check(s, 64, ids=ids)


def test_topk_indexer_workload_rows():
    note("topk: M=262144 B=8 integer indexer-like scores")
    rng = np.random.default_rng(42)
    s = _scores(rng, 8, 262144, "int_scores")
    _check(s, 512)


@pytest.mark.parametrize("M,K", [(1000, 64), (16384, 512), (40000, 512)])
def test_topk_repeated_score_id_pairs(M, K):
    note(f"topk: repeated (score, id) pairs M={M} K={K}")
    rng = np.random.default_rng(M + 5)
    s = rng.integers(0, 6, size=(2, M)).astype(np.float32)
    ids = rng.integers(0, 50, size=(2, M)).astype(np.int32)   # every id repeated many times
    _check(s, K, ids=ids)
