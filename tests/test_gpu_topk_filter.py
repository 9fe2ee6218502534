"""a3 csa2_topk on rows that take the threshold filter (K >= 64 and more
than 768 first-level chunks in all, or more than two chunk levels, in rows of
at most 2^20 columns) against the oracle: bit-exact ids and scores, and equal bit for
bit to the chunked reduction (csa2_topk_noalloc always takes it).

Besides the score families of the plain Top-K tests, the rows here are chosen
so that the filter's sample misleads: rows sorted ascending (the sample's
threshold lies above the row's K-th key), constant rows and rows whose top is
one long tie (more than 16384 keys at or above the threshold), masks that
leave fewer than K candidates.  Those rows must be reduced by their select
workgroup over the whole row; the test reads the per-row record the filter
leaves at the start of the workspace (threshold, count: the first two uint32
of each 128-byte row record) to check that they were."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, csa2, note, oracle

pytestmark = pytest.mark.gpu

CAP = 16384


def _fallback_rows(ws, B, K):
    """Rows whose kept candidates could not hold the Top-K."""
    rec = ws[: B * 128].view(torch.int32).view(B, 32).cpu().numpy().view(np.uint32)
    theta, count = rec[:, 0], rec[:, 1]
    return (count > CAP) | ((theta != 0) & (count < K))


def _run(s, K, ids=None, nv=None):
    B, M = s.shape
    need = csa2.csa2_topk_workspace_bytes(B, M, K)
    assert need == B * (128 + CAP * 8), "shape does not take the threshold filter"
    st = torch.from_numpy(s).to(DEV)
    it = None if ids is None else torch.from_numpy(ids).to(DEV)
    nt = None if nv is None else torch.from_numpy(nv).to(DEV)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    gi, gs = csa2.csa2_topk(st, K, ids=it, n_valid=nt, workspace=ws)
    ci, cs = csa2.csa2_topk_noalloc(st, K, ids=it, n_valid=nt)
    torch.cuda.synchronize()
    ri, rs = oracle.topk(s.astype(np.float64), ids, nv, K)
    gi, gs = gi.cpu().numpy(), gs.cpu().numpy()
    assert np.array_equal(gi, ri), np.nonzero(gi != ri)
    assert np.array_equal(gs.astype(np.float64), rs, equal_nan=True)
    assert np.array_equal(gi, ci.cpu().numpy())
    assert np.array_equal(gs.view(np.uint32), cs.cpu().numpy().view(np.uint32))
    return _fallback_rows(ws, B, K)


def _family(rng, B, M, kind):
    if kind == "continuous":
        return rng.standard_normal((B, M)).astype(np.float32)
    if kind == "logits":             # sampler-like: wide normal, a masked share
        s = (rng.standard_normal((B, M)) * 4).astype(np.float32)
        s[rng.random((B, M)) < 0.3] = -np.inf
        return s
    if kind == "int_scores":         # indexer-like integer sums
        return np.maximum(rng.normal(900, 500, size=(B, M)), 0).round().astype(np.float32)
    if kind == "ties":
        return rng.integers(0, 40, size=(B, M)).astype(np.float32)
    if kind == "outlier":
        s = rng.standard_normal((B, M)).astype(np.float32)
        s[:, rng.integers(0, M, size=B)] = 1e30
        s[:, rng.integers(0, M, size=B)] = -1e30
        return s
    # specials over tied integers
    s = rng.integers(-3, 4, size=(B, M)).astype(np.float32)
    r = rng.random((B, M))
    s[r < 0.05] = np.nan
    s[(r >= 0.05) & (r < 0.1)] = -0.0
    s[(r >= 0.1) & (r < 0.15)] = -np.inf
    s[(r >= 0.15) & (r < 0.17)] = np.inf
    return s


# (B, M, K): more than 768 first-level chunks (B * ceil(M / 16384) > 768), or
# three levels (19 and 64 chunks), ragged tails (an odd row length takes the
# 4-byte loads), the longest row; K from 64 to 2048
SHAPES = [(400, 20000, 1024), (20, 300001, 1024), (1, 300000, 2048), (1, 1 << 20, 2048), (100, 129280, 2048),
          (128, 129280, 512), (1, 1 << 20, 512), (300, 40000, 64), (200, 65537, 200)]


@pytest.mark.parametrize("B,M,K", SHAPES)
@pytest.mark.parametrize("kind", ["continuous", "logits", "int_scores", "ties", "outlier", "specials"])
def test_filter_families(B, M, K, kind):
    note(f"topk filter: B={B} M={M} K={K} {kind}")
    rng = np.random.default_rng(B * 31 + M + K + len(kind))
    s = _family(rng, B, M, kind)
    _run(s, K)
    nv = rng.integers(0, M + 1, size=B).astype(np.int32)
    nv[0] = M
    if B > 3:
        nv[1], nv[2], nv[3] = CAP, CAP + 1, K - 1
    _run(s, K, nv=nv)


def test_filter_misled_rows_fall_back():
    """Rows the sample misjudges: sorted ascending and descending, constant,
    a long tie at the top, fewer valid candidates than K (ids -1), all NaN,
    all -inf; beside ordinary rows."""
    B, M, K = 100, 129280, 2048
    note(f"topk filter: misled rows B={B} M={M} K={K}")
    rng = np.random.default_rng(3)
    s = rng.standard_normal((B, M)).astype(np.float32)
    s[0] = np.sort(s[0])                       # ascending: the top is the last run
    s[1] = np.sort(s[1])[::-1]                 # descending
    s[2] = 5.0                                 # constant
    s[3] = rng.standard_normal(M).astype(np.float32)
    s[3][rng.random(M) < 0.2] = 9.0            # 20% tied at the top
    s[4] = np.nan
    s[5] = -np.inf
    s[6] = np.arange(M, dtype=np.float32)      # ascending, distinct
    s[7, :] = 0.0
    s[7, ::2] = -0.0                           # +0 / -0 rank equal
    ids = np.broadcast_to(np.arange(M, dtype=np.int32), (B, M)).copy()
    ids[8, :] = -1
    ids[8, rng.integers(0, M, size=1000)] = 77  # 1000 candidates (one id repeated)
    ids[9, M // 2:] = -1                       # the sample's upper half empty
    fb = _run(s, K, ids=ids)
    assert fb[0] and fb[1] and fb[2] and fb[3] and fb[6], fb[:10]
    assert not fb[8] and not fb[9], fb[:10]
    assert not fb[10:].any(), np.nonzero(fb)


@pytest.mark.parametrize("K", [2048, 64])
def test_filter_given_ids_and_repeats(K):
    """Given ids (a permutation with holes, and ids repeated many times)."""
    B, M = 100, 131072
    note(f"topk filter: given ids B={B} M={M} K={K}")
    rng = np.random.default_rng(9)
    s = rng.integers(0, 300, size=(B, M)).astype(np.float32)
    # distinct ids per row: an odd multiplier is a bijection modulo 2^24
    off = rng.integers(0, 1 << 24, size=(B, 1))
    ids = ((np.arange(M, dtype=np.int64)[None, :] * 2654435761 + off) % (1 << 24)).astype(np.int32)
    ids[rng.random((B, M)) < 0.1] = -1
    _run(s, K, ids=ids)
    ids = rng.integers(0, 64, size=(B, M)).astype(np.int32)
    _run(s, K, ids=ids)


def test_filter_in_a_hip_graph_matches_eager():
    """Captured into a HIP graph and replayed three times (row counters reset
    by the estimate kernel each time), with eager work in between."""
    B, M, K = 100, 129280, 2048
    note(f"topk filter: HIP graph B={B} M={M} K={K}")
    rng = np.random.default_rng(21)
    st = torch.from_numpy((rng.standard_normal((B, M)) * 4).astype(np.float32)).to(DEV)
    idx = torch.empty(B, K, dtype=torch.int32, device=DEV)
    top = torch.empty(B, K, dtype=torch.float32, device=DEV)
    ws = torch.empty(csa2.csa2_topk_workspace_bytes(B, M, K), dtype=torch.uint8, device=DEV)

    def step():
        csa2.csa2_topk(st, K, out_idx=idx, out_score=top, workspace=ws)
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
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]) and torch.equal(top, ref[1]), rep
        csa2.csa2_topk(st[:2], 64)      # eager work between replays
        torch.cuda.synchronize()
