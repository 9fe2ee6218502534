"""The untruncated draw (csa2_sample_full: top_p 1.0 over the whole
vocabulary) on the GPU against the oracle's sample_full.

The drawn token is an integer decided by comparing running weights with
u * sum(w); the kernel sums V float32 weights in a blocked order, the oracle
in float64.  Each float32 weight is within 2^-19 of its exact value relative
(the exponent's rounding at |logit / T| <= 64, then exp2f), and a running
weight of the kernel is a sum of positive terms of depth below 40, so every
running weight and the total lie within TOL = 2^-16 of the total weight of
their exact values.  A token may therefore differ from the oracle's only where
the oracle's running weight at one of its ends lies within TOL of the target;
the tests compare exactly everywhere else and check that every differing token
is such a near-tie of nonzero weight."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, csa2, note, oracle
from sparse_attention_decode_csa2_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = 2.0 ** -16


def _run(logits, T, u):
    lt = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to(DEV)
    ut = torch.from_numpy(np.ascontiguousarray(u, dtype=np.float32)).to(DEV)
    tok, prob = csa2.csa2_sample_full(lt, T, ut)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), prob.cpu().numpy()


def _compare(logits, T, u, token, prob, max_near):
    T32 = float(np.float32(T))
    l64 = logits.astype(np.float64)
    u64 = np.asarray(u, dtype=np.float32).astype(np.float64)
    rt, rp = oracle.sample_full(l64, T32, u64)
    near = 0
    for b in range(logits.shape[0]):
        t, pr = int(token[b]), float(prob[b])
        assert 0 <= t < logits.shape[1], (b, t)
        if t == rt[b]:
            assert abs(pr - rp[b]) <= 1e-4 * rp[b] + 1e-7, (b, pr, rp[b])
            continue
        near += 1
        lm = l64[b].max()
        w = np.where(l64[b] == -np.inf, 0.0, np.exp((l64[b] - lm) / T32))
        total = w.sum()
        C = np.concatenate([[0.0], np.cumsum(w)]) / total
        assert w[t] > 0, (b, t)
        assert C[t] <= u64[b] + TOL and C[t + 1] > u64[b] - TOL, (b, t, rt[b], C[t], C[t + 1], u64[b])
        assert abs(pr - w[t] / total) <= 1e-4 * (w[t] / total) + 1e-7
    assert near <= max_near, f"{near} of {logits.shape[0]} rows differ from the oracle"
    return near


def test_sample_full_vocabulary_workload():
    """128 rows of 129,280 logits (N(0,1) x 4), temperature 1: the sampler
    workload's own inputs."""
    wl = W.BY_NAME["sample-129k"]
    note(f"sample_full: sample-129k B={wl.B} V={wl.N} T={wl.temperature}")
    lt = W.vocab_logits(wl, DEV)
    ut = W.sampler_uniforms(wl, DEV)
    tok, prob = csa2.csa2_sample_full(lt, wl.temperature, ut)
    torch.cuda.synchronize()
    near = _compare(lt.cpu().numpy(), wl.temperature, ut.cpu().numpy(), tok.cpu().numpy(), prob.cpu().numpy(),
                    max_near=4)
    note(f"  near-ties {near} of {wl.B}")


@pytest.mark.parametrize("V", [1, 3, 5, 1001, 4096, 4097, 12289, 40000])
@pytest.mark.parametrize("kind", ["normal", "ties", "neginf"])
def test_sample_full_shapes(V, kind):
    """Vocabularies shorter than a tile, ragged last tiles (V not a multiple
    of 4: scalar loads), integer logits with ties, -inf logits and a row with
    no finite logit."""
    rng = np.random.default_rng(V * 7 + len(kind))
    B = 24
    if kind == "ties":
        x = rng.integers(-6, 7, size=(B, V)).astype(np.float32)
    else:
        x = (rng.standard_normal((B, V)) * 4).astype(np.float32)
    if kind == "neginf":
        x[rng.random((B, V)) < 0.3] = -np.inf
        x[0] = -np.inf
        x[1, :] = -np.inf
        x[1, V - 1] = 2.0                                   # only the last token is finite
    u = rng.random(B).astype(np.float32)
    u[2] = 0.0
    u[3] = np.float32(1.0 - 2.0 ** -24)
    note(f"sample_full: V={V} kind={kind} B={B}")
    tok, prob = _run(x, 1.0, u)
    _compare(x, 1.0, u, tok, prob, max_near=2)
    if kind == "neginf":
        assert tok[0] == 0 and prob[0] == 1.0                 # no finite logit: token 0
        assert tok[1] == V - 1 and prob[1] == 1.0


@pytest.mark.parametrize("T", [0.25, 0.7, 2.0, 5.0])
def test_sample_full_temperatures(T):
    rng = np.random.default_rng(int(T * 100))
    B, V = 32, 70000
    x = (rng.standard_normal((B, V)) * 3).astype(np.float32)
    u = rng.random(B).astype(np.float32)
    note(f"sample_full: T={T} B={B} V={V}")
    tok, prob = _run(x, T, u)
    _compare(x, T, u, tok, prob, max_near=2)


def test_sample_full_greedy_limit_and_largest_vocabulary():
    """A vanishing temperature draws the unique largest logit; the largest
    vocabulary the call takes (2^20 tokens) draws like the oracle."""
    rng = np.random.default_rng(5)
    B, V = 8, 9000
    x = np.round(rng.standard_normal((B, V)) * 3).astype(np.float32)
    want = np.argmax(x, axis=1)
    x[np.arange(B), want] += 0.5
    for uu in (0.0, 0.5, 0.999):
        tok, prob = _run(x, 1e-3, np.full(B, uu, np.float32))
        assert np.array_equal(tok, want) and np.all(prob == 1.0)
    V = 1 << 20
    x = (rng.standard_normal((2, V)) * 4).astype(np.float32)
    u = np.array([0.3, 0.9], np.float32)
    note(f"sample_full: V={V}")
    tok, prob = _run(x, 1.0, u)
    _compare(x, 1.0, u, tok, prob, max_near=1)


def test_sample_full_frequencies_match_softmax():
    """Over a grid of uniforms on one small row, the GPU's token frequencies
    are the softmax of the logits within one grid step (and a near-tie at
    most moves one grid point)."""
    from scipy.special import softmax
    rng = np.random.default_rng(9)
    V, G = 50, 4096
    row = (rng.standard_normal(V) * 2).astype(np.float32)
    x = np.tile(row, (G, 1))
    u = ((np.arange(G) + 0.5) / G).astype(np.float32)
    tok, _ = _run(x, 1.0, u)
    freq = np.bincount(tok, minlength=V) / G
    want = softmax(row.astype(np.float64))
    assert np.all(np.abs(freq - want) <= 2.0 / G + 1e-9), np.abs(freq - want).max()
    assert np.all(np.diff(tok) >= 0)


def test_sample_full_in_a_hip_graph_matches_eager():
    """The two launches captured into a HIP graph (outputs and workspace
    passed in) and replayed three times, with eager work in between,
    reproduce the eager result bit for bit."""
    B, V = 64, 129280
    note(f"csa2_sample_full: HIP graph capture + 3 replays vs eager B={B} V={V}")
    rng = np.random.default_rng(17)
    x = torch.from_numpy((rng.standard_normal((B, V)) * 4).astype(np.float32)).to(DEV)
    u = torch.from_numpy(rng.random(B).astype(np.float32)).to(DEV)
    tok = torch.empty(B, dtype=torch.int32, device=DEV)
    prob = torch.empty(B, dtype=torch.float32, device=DEV)
    ws = torch.empty(csa2.csa2_sample_full_workspace_bytes(B, V), dtype=torch.uint8, device=DEV)

    def step():
        csa2.csa2_sample_full(x, 1.0, u, token=tok, prob=prob, workspace=ws)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (tok, prob)]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(3):
        tok.fill_(0)
        prob.fill_(0)
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(tok, ref[0]) and torch.equal(prob, ref[1]), rep
        csa2.csa2_sample_full(x[:2], 0.5, u[:2])            # eager work between replays
        torch.cuda.synchronize()
