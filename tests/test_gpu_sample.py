"""The decode sampler (csa2_sample, csa2_sample_draw) on the GPU against the
oracle's sampler.

The candidates (Top-K ids) are integer work and must match bit for bit.  The
nucleus end and the drawn position are integers decided by float comparisons
of running weights; the kernel sums in float32, the oracle in float64.  Each
running weight of the kernel is within TOL = K * 2^-22 of the total weight of
its exact value (K weights, each within 2 ulp from exp2f and the scaling,
summed with K roundings of 2^-24), so a decision may differ from the oracle's
only where the oracle's running weight lies within TOL of the threshold.
The tests compare exactly everywhere else, check that every differing
decision is such a near-tie, and that near-ties stay rare on continuous
logits."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, csa2, note, oracle
from sparse_attention_decode_csa2_amd import workloads as W

pytestmark = pytest.mark.gpu


def _logits(rng, B, V, kind):
    if kind == "ties":
        return rng.integers(-6, 7, size=(B, V)).astype(np.float32)
    if kind == "neginf":
        x = (rng.standard_normal((B, V)) * 4).astype(np.float32)
        x[rng.random((B, V)) < 0.3] = -np.inf
        x[0] = -np.inf                                   # a row with no finite logit
        return x
    return (rng.standard_normal((B, V)) * 4).astype(np.float32)


def _compare(logits, K, T, top_p, u, token, prob, n_kept, max_near=None):
    """GPU (token, prob, n_kept) against the oracle, per the rules above."""
    T32, p32 = float(np.float32(T)), float(np.float32(top_p))
    rt, rp, rn, rpos, idx, w = oracle.sample(logits.astype(np.float64), K, T32, p32, u.astype(np.float64))
    B = logits.shape[0]
    tol = K * 2.0 ** -22
    near = 0
    for b in range(B):
        t, pr, n = int(token[b]), float(prob[b]), int(n_kept[b])
        if t == rt[b] and n == rn[b]:
            assert abs(pr - rp[b]) <= 1e-4 * rp[b] + 1e-7, (b, pr, rp[b])
            continue
        near += 1
        tot = w[b].sum()
        F = np.concatenate([[0.0], np.cumsum(w[b])]) / tot
        n_cand = int((idx[b] >= 0).sum())
        assert 1 <= n <= n_cand, (b, n, n_cand)
        if n != rn[b]:
            assert p32 < 1.0 and F[n] >= p32 - tol and F[n - 1] < p32 + tol, (b, n, rn[b], F[n - 1], F[n])
        hits = np.nonzero(idx[b, :n] == t)[0]
        assert hits.size == 1, (b, t, idx[b, :n])
        pos = int(hits[0])
        assert w[b, pos] > 0
        C = w[b, :n].sum()
        lo, hi = w[b, :pos].sum() / C, w[b, :pos + 1].sum() / C
        tolc = tol * tot / C
        assert lo <= u[b] + tolc and hi > u[b] - tolc, (b, pos, lo, hi, u[b])
        assert abs(pr - w[b, pos] / C) <= 1e-4 * (w[b, pos] / C) + 1e-7
    if max_near is not None:
        assert near <= max_near, f"{near} of {B} rows differ from the oracle"
    return near


def _run(logits, K, T, top_p, u, via="sample"):
    lt = torch.from_numpy(logits).to(DEV)
    ut = torch.from_numpy(u).to(DEV)
    if via == "sample":
        tok, prob, n = csa2.csa2_sample(lt, K, T, top_p, ut)
    else:
        ci, cs = csa2.csa2_topk(lt, K)
        tok, prob, n = csa2.csa2_sample_draw(ci, cs, T, top_p, ut)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), prob.cpu().numpy(), n.cpu().numpy()


CASES = [(1, 1, 1), (3, 10, 16), (4, 1000, 64), (3, 300, 65), (5, 5000, 2047), (2, 20000, 512),
         (64, 4096, 100), (2, 129280, 2048), (400, 20000, 64)]


@pytest.mark.parametrize("B,V,K", CASES)
@pytest.mark.parametrize("T,top_p", [(1.0, 1.0), (0.7, 0.9), (1.3, 0.5)])
def test_sample_vs_oracle(B, V, K, T, top_p):
    note(f"csa2_sample B={B} V={V} K={K} T={T} top_p={top_p}")
    rng = np.random.default_rng(B * 7919 + V + K)
    x = _logits(rng, B, V, "cont")
    u = rng.random(B).astype(np.float32)
    tok, prob, n = _run(x, K, T, top_p, u)
    _compare(x, K, T, top_p, u, tok, prob, n, max_near=max(1, B // 20))


@pytest.mark.parametrize("kind", ["ties", "neginf"])
@pytest.mark.parametrize("top_p", [1.0, 0.6])
def test_sample_ties_and_masked_logits(kind, top_p):
    B, V, K = 16, 3000, 256
    note(f"csa2_sample {kind} B={B} V={V} K={K} top_p={top_p}")
    rng = np.random.default_rng(17 if kind == "ties" else 18)
    x = _logits(rng, B, V, kind)
    u = rng.random(B).astype(np.float32)
    u[:3] = [0.0, np.float32(1.0) - np.float32(2.0 ** -24), 0.5]
    tok, prob, n = _run(x, K, 1.0, top_p, u)
    _compare(x, K, 1.0, top_p, u, tok, prob, n)
    if kind == "neginf":
        assert tok[0] == 0 and prob[0] == 1.0 and n[0] == 1          # no finite logit: first id


def _golden_rows():
    import oracle_pins as P
    return P._sample_records()


def test_sample_golden_rows():
    """The hand-derived draws of the oracle's fixture, on the GPU."""
    for K, T, top_p, u, logits, tok, n, pos, prob in _golden_rows():
        note(f"golden K={K} T={T} top_p={top_p} u={u} logits={logits.tolist()}")
        x = logits.astype(np.float32)[None]
        ua = np.array([u], dtype=np.float32)
        for via in ("sample", "draw"):
            t, p, nk = _run(x, K, T, top_p, ua, via)
            assert (int(t[0]), int(nk[0])) == (tok, n), (via, logits, t, nk)
            assert abs(float(p[0]) - prob) <= 1e-6, (via, p, prob)


@pytest.mark.parametrize("B,V,K,T,top_p", [(8, 50000, 1000, 0.8, 0.95), (64, 200000, 1024, 0.8, 0.95),
                                            (128, 129280, 2048, 1.0, 1.0), (100, 129280, 2048, 0.7, 0.5),
                                            (128, 129280, 64, 1.0, 1.0), (100, 129280, 200, 0.8, 0.9)])
def test_draw_on_topk_output_equals_sample(B, V, K, T, top_p):
    """csa2_sample = csa2_topk + csa2_sample_draw, bit for bit: below the
    threshold filter's shapes the draw is its own kernel; on them (the last
    five) the filter's last kernel draws from the rows it has written."""
    note(f"csa2_sample vs csa2_topk + csa2_sample_draw B={B} V={V} K={K} T={T} top_p={top_p}")
    rng = np.random.default_rng(5 + B)
    x = _logits(rng, B, V, "cont")
    x[0, :] = -np.inf                      # a row with no finite logit
    x[1, : V // 2] = -np.inf               # half the row masked
    u = rng.random(B).astype(np.float32)
    u[2] = 0.0
    u[3] = np.float32(1.0) - np.float32(2 ** -24)
    a = _run(x, K, T, top_p, u, "sample")
    b = _run(x, K, T, top_p, u, "draw")
    for ga, gb in zip(a, b):
        assert np.array_equal(ga, gb)


def test_sample_empty_batch():
    note("csa2_sample B=0")
    x = torch.empty(0, 100, dtype=torch.float32, device=DEV)
    u = torch.empty(0, dtype=torch.float32, device=DEV)
    tok, prob, n = csa2.csa2_sample(x, 8, 1.0, 1.0, u)
    torch.cuda.synchronize()
    assert tok.numel() == 0


def test_sample_full_workload():
    """The benchmarked configuration: 128 rows x 129280 logits, Top-2048,
    temperature 1, top_p 1, every row against the oracle."""
    wl = W.BY_NAME["sample-129k"]
    note(f"csa2_sample {wl.name}")
    x = W.vocab_logits(wl, DEV)
    u = W.sampler_uniforms(wl, DEV)
    tok, prob, n = csa2.csa2_sample(x, wl.K, wl.temperature, wl.top_p, u)
    torch.cuda.synchronize()
    _compare(x.cpu().numpy(), wl.K, wl.temperature, wl.top_p, u.cpu().numpy(), tok.cpu().numpy(),
             prob.cpu().numpy(), n.cpu().numpy(), max_near=2)


@pytest.mark.parametrize("B,V,K", [(16, 40000, 1024), (64, 200000, 1024)])
def test_sample_in_a_hip_graph_matches_eager(B, V, K):
    """csa2_sample captured into a HIP graph (outputs and workspace passed in)
    and replayed three times, with eager work in between, reproduces the
    eager result bit for bit (the chunk levels and the draw kernel; the
    threshold filter with the draw in its last kernel)."""
    note(f"csa2_sample: HIP graph capture + 3 replays vs eager B={B} V={V} K={K}")
    rng = np.random.default_rng(9)
    x = torch.from_numpy(_logits(rng, B, V, "cont")).to(DEV)
    u = torch.from_numpy(rng.random(B).astype(np.float32)).to(DEV)
    tok = torch.empty(B, dtype=torch.int32, device=DEV)
    prob = torch.empty(B, dtype=torch.float32, device=DEV)
    nk = torch.empty(B, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(csa2.csa2_sample_workspace_bytes(B, V, K), 16), dtype=torch.uint8, device=DEV)

    def step():
        csa2.csa2_sample(x, K, 0.9, 0.8, u, token=tok, prob=prob, n_kept=nk, workspace=ws)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (tok, prob, nk)]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(3):
        for t in (tok, prob, nk):
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((tok, prob, nk), ref):
            assert torch.equal(a, b), rep
        csa2.csa2_topk(x, 64)                       # eager work between replays
        torch.cuda.synchronize()
