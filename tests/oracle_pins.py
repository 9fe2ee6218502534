"""Pins that tie the CPU oracle to things other than itself.

Each ``check_*`` function raises AssertionError when the oracle disagrees
with an independent source: a fixture derived by hand from the format
definitions (``tests/golden``), a library routine that reduces to the same
operation in a special case (torch's float8_e4m3fn cast, numpy's
round-half-even, int64 matmul, stable sorts, torch.topk, float64 SDPA), brute
force on tiny inputs, or closed-form invariants.  ``test_oracle_*.py`` run
them against the oracle; ``test_oracle_mutations.py`` plants plausible
mistakes in the oracle and checks that at least one pin catches each.
"""

import math
import os

import numpy as np
import torch

import oracle
from oracle import codec, method

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _records(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


def _all_bf16_finite_nonneg():
    b = np.arange(0x0000, 0x7F80, dtype=np.uint32).astype(np.uint16)  # +0 .. max finite
    return b, codec.bf16_bits_to_f64(b)


# ------------------------------------------------------------------ codecs


def check_e2m1_value_set():
    for code, val in _records("e2m1_values.txt"):
        c = int(code, 16)
        got = float(oracle.e2m1_decode(np.array([c]))[0])
        want = float(val)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)
    mags = sorted(set(np.abs(oracle.e2m1_decode(np.arange(16))).tolist()))
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def check_e4m3_decode():
    for code, val in _records("e4m3_values.txt"):
        got = float(oracle.e4m3_decode(np.array([int(code, 16)]))[0])
        if val == "nan":
            assert math.isnan(got), code
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), (code, got)
    v = oracle.e4m3_decode(np.arange(127))
    assert np.all(np.diff(v) > 0)                 # 127 finite non-negative codes, increasing
    assert v[0] == 0.0 and v[-1] == 448.0


def check_e4m3_encode_vs_torch():
    """RNE to E4M3 equals torch's float8_e4m3fn cast for values <= 448."""
    rng = np.random.default_rng(7)
    vals = oracle.e4m3_decode(np.arange(127))
    mids = (vals[:-1] + vals[1:]) / 2
    t = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1000),
                        rng.uniform(0, 448, 20000), rng.uniform(0, 0.02, 20000)])
    t = t.astype(np.float32).astype(np.float64)   # fp32-exact so the cast rounds once
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(t)
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, (t[bad[:5]], ref[bad[:5]], got[bad[:5]])


def check_scale_code_vs_torch():
    """Scale code for every positive finite bf16 amax below saturation equals
    torch's float8_e4m3fn cast of amax / 6."""
    _, a = _all_bf16_finite_nonneg()
    a = a[a < 6 * 448]
    ref = torch.from_numpy(a / 6.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_scale_code_for_amax(a)
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, (a[bad[:5]], ref[bad[:5]], got[bad[:5]])
    # saturation: amax/6 above 448 maps to 0x7E (the cast would give NaN there)
    _, big = _all_bf16_finite_nonneg()
    big = big[big >= 6 * 448]
    assert np.all(oracle.e4m3_scale_code_for_amax(big) == 0x7E)


def _e2m1_value_by_numpy_round(y):
    """RNE of y >= 0 onto {0,.5,1,1.5,2,3,4,6} via np.round (half-to-even) with
    the quantum of each binade, saturating at 6."""
    q = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    return np.minimum(np.round(y / q) * q, 6.0)


def check_e2m1_encode_vs_numpy_round():
    grid = oracle.e2m1_decode(np.arange(8))
    _, x = _all_bf16_finite_nonneg()
    for sigma in [1.0, 1.25, 0.75, 2.0 ** -9, 3 * 2.0 ** -9, 448.0, 1.875, 0.015625, 96.0]:
        xs = x[x < 16 * sigma]
        code = oracle.e2m1_encode_magnitude(xs, sigma)
        want = _e2m1_value_by_numpy_round(xs / sigma)
        assert np.array_equal(grid[code], want), sigma
    assert np.all(oracle.e2m1_encode_magnitude(x[:100], 0.0) == 0)


def check_bf16_decode():
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -133, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127,
             0x3E9A: 0.30078125, 0x8000: -0.0, 0x0080: 2.0 ** -126}
    for bits, val in cases.items():
        got = float(codec.bf16_bits_to_f64(np.array([bits], dtype=np.uint16))[0])
        assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(bits)


# ------------------------------------------------------------------ quantize


def check_quantize_golden():
    recs = _records("quantize_groups.txt")
    assert len(recs) % 3 == 0 and len(recs) >= 30
    rows, scales, nibs = [], [], []
    for i in range(0, len(recs), 3):
        assert recs[i][0] == "in" and recs[i + 1][0] == "scale" and recs[i + 2][0] == "codes"
        rows.append([float(v) for v in recs[i][1:]])
        scales.append(int(recs[i + 1][1], 16))
        nibs.append([int(c, 16) for c in recs[i + 2][1:]])
    # one row per group, and the same groups concatenated into one long row
    x = codec.f64_to_bf16_bits_exact(np.array(rows))
    want_n = np.array(nibs, dtype=np.uint8)
    want_c = want_n[:, 0::2] | (want_n[:, 1::2] << 4)
    c, s = oracle.quantize_fp4(x)
    assert np.array_equal(s[:, 0], np.array(scales, dtype=np.uint8)), (s[:, 0], scales)
    assert np.array_equal(c, want_c), (c, want_c)
    c2, s2 = oracle.quantize_fp4(x.reshape(1, -1))
    assert np.array_equal(c2.reshape(c.shape), c) and np.array_equal(s2.reshape(-1), s[:, 0])


def check_quantize_roundtrip_fixed_point():
    """Values already on an FP4 grid whose group holds a +-6*sigma element
    quantise back to the same codes and scale."""
    rng = np.random.default_rng(3)
    R, G = 64, 32
    S = rng.integers(0x08, 0x70, size=(R, G)).astype(np.uint8)       # normal scales
    nib = rng.integers(0, 16, size=(R, G, 16)).astype(np.uint8)
    nib[:, :, 5] = np.where(rng.random((R, G)) < 0.5, 0x7, 0xF)      # force a +-6
    codes = (nib.reshape(R, -1)[:, 0::2] | (nib.reshape(R, -1)[:, 1::2] << 4)).astype(np.uint8)
    x = oracle.dequantize_fp4(codes, S)
    bits = codec.f64_to_bf16_bits_exact(x)
    c2, s2 = oracle.quantize_fp4(bits)
    assert np.array_equal(s2, S)
    # -0 codes dequantise to -0.0 and keep their sign bit
    assert np.array_equal(c2, codes)


def check_quantize_error_bound():
    """Every non-saturated element lands within half a grid step of x, and
    the chosen scale is the nearest E4M3 value to amax/6."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((256, 512)) * np.exp(rng.uniform(-6, 6, size=(256, 1)))
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xb = codec.bf16_bits_to_f64(bits)
    c, s = oracle.quantize_fp4(bits)
    deq = oracle.dequantize_fp4(c, s)
    sig = np.repeat(oracle.e4m3_decode(s), 16, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.abs(xb) / sig
    gap = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0)) * sig
    ok = y <= 6
    assert np.all(np.abs(xb - deq)[ok] <= gap[ok] / 2 + 0.0)
    assert np.all(np.sign(deq) * np.sign(xb) >= 0)
    amax = np.abs(xb).reshape(256, 32, 16).max(-1)
    vals = oracle.e4m3_decode(np.arange(127))
    err = np.abs(oracle.e4m3_decode(s) - amax / 6)
    best = np.abs(vals[None, None, :] - (amax / 6)[..., None]).min(-1)
    assert np.allclose(err, best, rtol=0, atol=1e-12 * np.maximum(amax, 1e-30))


def check_nibble_order():
    x = np.zeros((1, 16))
    x[0, 0] = 6.0   # channel 0 -> low nibble of byte 0
    x[0, 3] = -1.0  # channel 3 -> high nibble of byte 1
    c, s = oracle.quantize_fp4(codec.f64_to_bf16_bits_exact(x))
    assert c[0, 0] == 0x07 and c[0, 1] == 0xA0 and s[0, 0] == 0x38


# ------------------------------------------------------------------ indexer


def check_index_bruteforce():
    rng = np.random.default_rng(5)
    H_I, D_I, N = 3, 8, 20
    q = rng.integers(-8, 9, size=(H_I, D_I)).astype(np.float64)
    k = rng.integers(-8, 9, size=(N, D_I)).astype(np.float64)
    w = np.array([0.5, -1.25, 2.0])
    got = oracle.index_scores(q, w, k)
    for n in range(N):
        acc = 0.0
        for h in range(H_I):
            d = sum(q[h, i] * k[n, i] for i in range(D_I))
            acc += w[h] * (d if d > 0 else 0.0)
        assert got[n] == acc, n


def check_index_full_vs_int64_matmul():
    rng = np.random.default_rng(6)
    B, H_I, D_I, N = 2, 8, 128, 300
    qi = rng.integers(-8, 9, size=(B, H_I, D_I))
    ki = rng.integers(-8, 9, size=(B, N, D_I))
    qb = codec.f64_to_bf16_bits_exact(qi.astype(np.float64))
    kb = codec.f64_to_bf16_bits_exact(ki.astype(np.float64))
    nv = np.array([N, 123])
    got = oracle.index_full(qb, None, kb, nv)
    for b in range(B):
        dots = np.matmul(ki[b], qi[b].T)                     # int64, exact
        want = np.maximum(dots, 0).sum(axis=1).astype(np.float64)
        assert np.array_equal(got[b, :nv[b]], want[:nv[b]])
        assert np.all(np.isneginf(got[b, nv[b]:]))


def check_index_pool_bruteforce():
    rng = np.random.default_rng(8)
    B, H_I, D_I, N, P_max, blk = 2, 4, 32, 96, 8, 8
    qi = rng.integers(-8, 9, size=(B, H_I, D_I)).astype(np.float64)
    ki = rng.integers(-8, 9, size=(B, N, D_I)).astype(np.float64)
    qb, kb = codec.f64_to_bf16_bits_exact(qi), codec.f64_to_bf16_bits_exact(ki)
    pool = np.array([[0, 3, 11, 5, -1, 7, 2, 9], [1, 2, 3, 4, 5, 6, 7, 8]], dtype=np.int32)
    nblk = np.array([7, 5], dtype=np.int32)
    nv = np.array([N, 50])
    sc, pos = oracle.index_pool(qb, None, kb, nv, pool, nblk, blk)
    for b in range(B):
        for i in range(P_max):
            for j in range(blk):
                slot = i * blk + j
                p = blk * int(pool[b, i]) + j
                if i < nblk[b] and pool[b, i] >= 0 and 0 <= p < nv[b]:
                    want = sum(max(0.0, float(qi[b, h] @ ki[b, p])) for h in range(H_I))
                    assert pos[b, slot] == p and sc[b, slot] == want
                else:
                    assert pos[b, slot] == -1 and np.isneginf(sc[b, slot])


# ------------------------------------------------------------------ Top-K


def _topk_brute(scores, ids, valid, K):
    cand = [(i, float(scores[i]), int(ids[i])) for i in range(len(scores)) if valid[i]]

    def key(t):
        s = t[1]
        return (1 if math.isnan(s) else 0, 0.0 if math.isnan(s) else -s, t[2])
    cand.sort(key=key)
    cand = cand[:K]
    return [c[2] for c in cand] + [-1] * (K - len(cand)), [c[1] for c in cand] + [-math.inf] * (K - len(cand))


def check_topk_bruteforce():
    rng = np.random.default_rng(9)
    for trial in range(300):
        M = int(rng.integers(1, 64))
        K = int(rng.integers(1, 70))
        s = rng.integers(-3, 4, size=M).astype(np.float64)     # heavy ties
        if trial % 5 == 0:
            s[rng.random(M) < 0.2] = np.nan
        if trial % 7 == 0:
            s[rng.random(M) < 0.3] = -np.inf
        use_ids = trial % 2 == 1
        ids = rng.permutation(1000)[:M].astype(np.int32) if use_ids else np.arange(M, dtype=np.int32)
        if use_ids:
            ids[rng.random(M) < 0.15] = -1
        nv = int(rng.integers(0, M + 1))
        gi, gs = oracle.topk(s[None], ids[None] if use_ids else None, np.array([nv]), K)
        valid = (np.arange(M) < nv) & (ids != -1)
        wi, ws = _topk_brute(s, ids, valid, K)
        assert gi[0].tolist() == wi, (trial, gi[0], wi)
        assert np.array_equal(gs[0], np.array(ws), equal_nan=True), trial


def check_topk_vs_torch_topk_distinct():
    rng = np.random.default_rng(10)
    s = rng.permutation(20000).astype(np.float64)[None, :16384] * 0.5
    gi, gs = oracle.topk(s, None, None, 512)
    tv, ti = torch.topk(torch.from_numpy(s[0]), 512, sorted=True)
    assert np.array_equal(gi[0], ti.numpy().astype(np.int32))
    assert np.array_equal(gs[0], tv.numpy())


def check_topk_ties_vs_stable_sort():
    rng = np.random.default_rng(12)
    s = rng.integers(0, 50, size=(3, 4096)).astype(np.float64)
    gi, _ = oracle.topk(s, None, None, 512)
    for b in range(3):
        order = np.argsort(-s[b], kind="stable")[:512]
        assert np.array_equal(gi[b], order.astype(np.int32))


def check_topk_invariants():
    rng = np.random.default_rng(13)
    s = rng.integers(0, 200, size=(4, 2000)).astype(np.float64)
    ids = np.stack([rng.permutation(10 ** 6)[:2000] for _ in range(4)]).astype(np.int32)
    gi, gs = oracle.topk(s, ids, None, 300)
    for b in range(4):
        sel = set(gi[b].tolist())
        assert len(sel) == 300
        pos = {int(v): i for i, v in enumerate(ids[b])}
        chosen = np.array([pos[int(v)] for v in gi[b]])
        rest = np.setdiff1d(np.arange(2000), chosen)
        assert s[b, chosen].min() >= s[b, rest].max()
        thr = s[b, chosen].min()
        tied_rest = ids[b, rest][s[b, rest] == thr]
        tied_in = ids[b, chosen][s[b, chosen] == thr]
        assert tied_rest.size == 0 or tied_in.max() < tied_rest.min()
        for a in range(299):
            assert gs[b, a] > gs[b, a + 1] or (gs[b, a] == gs[b, a + 1] and gi[b, a] < gi[b, a + 1])
    gi, _ = oracle.topk(s[:1, :100], None, None, 100)
    assert sorted(gi[0].tolist()) == list(range(100))


# ------------------------------------------------------------------ attention


def _attn_inputs(B=2, H=8, N=40, d_c=64, d_r=32, seed=14):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, d_c + d_r))
    qb = torch.from_numpy(q).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes = rng.integers(0, 256, size=(B, N, d_c // 2)).astype(np.uint8)
    scales = rng.integers(0x28, 0x40, size=(B, N, d_c // 16)).astype(np.uint8)
    rope = rng.standard_normal((B, N, d_r))
    rb = torch.from_numpy(rope).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return qb, codes, scales, rb


def check_attn_dense_vs_sdpa():
    """Top-K covering every entry reproduces dense attention (float64 SDPA)."""
    qb, codes, scales, rb = _attn_inputs()
    B, H, D = qb.shape
    N, d_c = codes.shape[1], codes.shape[2] * 2
    sm = 1.0 / math.sqrt(D)
    idx = np.tile(np.arange(N), (B, 1))
    out, lse = oracle.sparse_attn(qb, codes, scales, rb, idx, sm)
    q = torch.from_numpy(codec.bf16_bits_to_f64(qb))
    lat = torch.from_numpy(oracle.dequantize_fp4(codes, scales))
    key = torch.cat([lat, torch.from_numpy(codec.bf16_bits_to_f64(rb))], dim=-1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, key, lat, scale=sm)
    assert np.allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)
    s = sm * torch.einsum("bhd,bnd->bhn", q, key)
    assert np.allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def check_prefill_vs_causal_sdpa():
    """A prefill chunk whose query t lists every entry it may see (the first
    v_t entries of its own sequence, v_t growing with t, padded with -1)
    equals float64 SDPA with the causal mask, sequence by sequence."""
    S, T, H, N, d_c, d_r, K = 2, 6, 4, 24, 64, 32, 24
    qb, codes, scales, rb = _attn_inputs(B=S * T, H=H, N=N, d_c=d_c, d_r=d_r, seed=71)
    qb = qb.reshape(S, T, H, d_c + d_r)
    codes, scales, rb = codes[:S], scales[:S], rb[:S]              # one cache per sequence
    vis = np.array([5, 9, 12, 17, 20, 24])                          # entries query t may see
    idx = np.full((S, T, K), -1)
    for t in range(T):
        idx[:, t, :vis[t]] = np.arange(vis[t])[::-1]                # any order
    sm = 1.0 / math.sqrt(d_c + d_r)
    out, lse = oracle.prefill_sparse_attn(qb, codes, scales, rb, idx, sm)
    for s in range(S):
        q = torch.from_numpy(codec.bf16_bits_to_f64(qb[s]))          # [T, H, D]
        lat = torch.from_numpy(oracle.dequantize_fp4(codes[s], scales[s]))
        key = torch.cat([lat, torch.from_numpy(codec.bf16_bits_to_f64(rb[s]))], dim=-1)
        mask = torch.from_numpy(np.arange(N)[None, :] < vis[:, None])[:, None, :]   # [T, 1, N]
        ref = torch.nn.functional.scaled_dot_product_attention(q, key[None], lat[None], attn_mask=mask, scale=sm)
        assert np.allclose(out[s], ref.numpy(), rtol=1e-12, atol=1e-12), s
        sc = sm * torch.einsum("thd,nd->thn", q, key).masked_fill(~mask, -math.inf)
        assert np.allclose(lse[s], torch.logsumexp(sc, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def check_attn_special_cases():
    qb, codes, scales, rb = _attn_inputs(seed=15)
    B, H, D = qb.shape
    N = codes.shape[1]
    sm = 0.125
    lat = oracle.dequantize_fp4(codes, scales)
    # K = 1: the output is that entry's value row, exactly
    idx = np.array([[7], [31]])
    out, lse = oracle.sparse_attn(qb, codes, scales, rb, idx, sm)
    for b in range(B):
        assert np.array_equal(out[b], np.tile(lat[b, idx[b, 0]], (H, 1)))
    # q = 0: uniform weights -> mean of the selected values, lse = ln k
    zq = np.zeros_like(qb)
    idx = np.array([[1, 4, 9, 16, 25], [0, 2, 3, 5, 8]])
    out, lse = oracle.sparse_attn(zq, codes, scales, rb, idx, sm)
    for b in range(B):
        assert np.allclose(out[b], lat[b, idx[b]].mean(0)[None, :], rtol=1e-14, atol=1e-14)
    assert np.allclose(lse, math.log(5))
    # permutation of the index list changes nothing; masked ids are skipped
    rng = np.random.default_rng(1)
    idx = np.stack([rng.permutation(N)[:16] for _ in range(B)])
    o1, l1 = oracle.sparse_attn(qb, codes, scales, rb, idx, sm)
    o2, l2 = oracle.sparse_attn(qb, codes, scales, rb, idx[:, ::-1].copy(), sm)
    assert np.allclose(o1, o2, rtol=1e-13, atol=1e-13) and np.allclose(l1, l2, rtol=1e-13)
    idxm = np.concatenate([idx, np.full((B, 3), -1), np.full((B, 2), N + 5)], axis=1)
    o3, l3 = oracle.sparse_attn(qb, codes, scales, rb, idxm, sm)
    assert np.allclose(o1, o3, rtol=1e-13, atol=1e-13) and np.allclose(l1, l3, rtol=1e-13)
    # nothing valid -> zeros and -inf
    o4, l4 = oracle.sparse_attn(qb, codes, scales, rb, np.full((B, 4), -1), sm)
    assert np.all(o4 == 0) and np.all(np.isneginf(l4))
    # a repeated entry counts twice: same as giving it weight 2 (lse + ln of the multiplicity mix)
    o5, _ = oracle.sparse_attn(qb, codes, scales, rb, np.array([[3, 3], [6, 6]]), sm)
    for b, j in enumerate([3, 6]):
        assert np.array_equal(o5[b], np.tile(lat[b, j], (H, 1)))


def check_decode_modes_compose():
    """Full and Reindex decode are exactly index -> topk -> attention."""
    rng = np.random.default_rng(16)
    B, N, H_I, D_I = 1, 64, 2, 32
    qi = codec.f64_to_bf16_bits_exact(rng.integers(-8, 9, size=(B, H_I, D_I)).astype(float))
    ki = codec.f64_to_bf16_bits_exact(rng.integers(-8, 9, size=(B, N, D_I)).astype(float))
    qb, codes, scales, rb = _attn_inputs(B=1, N=N, seed=17)
    idx, top, out, lse = oracle.decode_full(qi, None, ki, None, qb, codes, scales, rb, 8, 0.1)
    want_i, _ = oracle.topk(oracle.index_full(qi, None, ki, None), None, None, 8)
    assert np.array_equal(idx, want_i)
    pool = np.array([[1, 3, 5, 7]], dtype=np.int32)
    idx2, _, _, _ = oracle.decode_reindex(qi, None, ki, None, pool, np.array([4]), 8,
                                          qb, codes, scales, rb, 8, 0.1)
    assert set(idx2[0].tolist()) <= set(sum(([8 * b + j for j in range(8)] for b in [1, 3, 5, 7]), []))


# ------------------------------------------------------------ pool construction

POOL_SCORES = [1, 5, 2, 2, 3, 3, 3, 3, 5, 9]


def check_pool_golden():
    """Hand-derived pools (tests/golden/pool_blocks.txt)."""
    sc = np.array([POOL_SCORES], dtype=np.float64)
    for rec in _records("pool_blocks.txt"):
        rec = [int(v) for v in rec]
        nv, P_max, nb = rec[:3]
        want = np.array(rec[3:3 + P_max], dtype=np.int32)
        pool, n_blocks = oracle.build_pool(sc, np.array([nv]), 4, P_max)
        assert np.array_equal(pool[0], want), (nv, P_max, pool[0], want)
        assert int(n_blocks[0]) == nb


def _pool_brute(scores, nv, block, P_max):
    # block scores by explicit loops, then selection by repeated scans
    cand = []
    beta = 0
    while block * beta < nv:
        best = None
        for p in range(block * beta, min(block * beta + block, nv)):
            v = float(scores[p])
            if v == v and (best is None or v > best):
                best = v
        cand.append((float("nan") if best is None else best, beta))
        beta += 1
    out = []
    left = list(cand)
    while left and len(out) < P_max:
        pick = None
        for c in left:
            if pick is None:
                pick = c
                continue
            a, b = c[0], pick[0]
            if (a == a and (b != b or a > b)) or ((a == b or (a != a and b != b)) and c[1] < pick[1]):
                pick = c
        out.append(pick[1])
        left.remove(pick)
    return out + [-1] * (P_max - len(out)), min(len(cand), P_max)


def check_pool_bruteforce():
    """Random tiny score rows full of ties (and -inf, NaN), ragged n_valid."""
    rng = np.random.default_rng(31)
    for it in range(60):
        B, M = 3, int(rng.integers(1, 41))
        block = int(rng.integers(1, 6))
        P_max = int(rng.integers(1, 9))
        sc = rng.integers(0, 4, size=(B, M)).astype(np.float64)
        sc[rng.random((B, M)) < 0.1] = -np.inf
        sc[rng.random((B, M)) < 0.05] = np.nan
        nv = rng.integers(0, M + 1, size=B)
        pool, n_blocks = oracle.build_pool(sc, nv, block, P_max)
        for b in range(B):
            want, wnb = _pool_brute(sc[b], int(nv[b]), block, P_max)
            assert pool[b].tolist() == want, (it, b, pool[b].tolist(), want)
            assert int(n_blocks[b]) == wnb


def check_pool_reindex_reproduces_full_topk():
    """With P_max >= K, re-scoring the pool built from a layer's own Full
    scores with the same indexer query selects exactly the Full-mode Top-K:
    every top-K position lies in a block whose score is at least its own."""
    rng = np.random.default_rng(32)
    for it in range(12):
        B, N, H_I, D_I, K, block = 2, 128, 2, 4, 8, 8
        P_max = int(rng.integers(K, 12))
        qi = codec.f64_to_bf16_bits_exact(rng.integers(-2, 3, size=(B, H_I, D_I)).astype(float))
        ki = codec.f64_to_bf16_bits_exact(rng.integers(-2, 3, size=(B, N, D_I)).astype(float))
        nv = np.array([N, int(rng.integers(1, N))])
        full = oracle.index_full(qi, None, ki, nv)
        want_i, want_s = oracle.topk(full, None, nv, K)
        pool, n_blocks = oracle.build_pool(full, nv, block, P_max)
        sc, pos = oracle.index_pool(qi, None, ki, nv, pool, n_blocks, block)
        got_i, got_s = oracle.topk(sc, pos, None, K)
        assert np.array_equal(got_i, want_i), (it, got_i, want_i)
        assert np.array_equal(got_s, want_s)


# ------------------------------------------------------------ sliding-window branch (FP8)


def check_fp8_golden():
    """Hand-derived FP8 rows (tests/golden/fp8_rows.txt)."""
    for rec in _records("fp8_rows.txt"):
        e = int(rec[0])
        vals = [float(v.split(":")[0]) for v in rec[1:]]
        want = [int(v.split(":")[1], 16) for v in rec[1:]]
        bits = codec.f64_to_bf16_bits_exact(np.array([vals]))
        if any(v.split(":")[0].startswith("-0") for v in rec[1:]):
            for j, v in enumerate(rec[1:]):
                if v.split(":")[0] == "-0":
                    bits[0, j] = 0x8000
        codes, sigma = oracle.quantize_fp8(bits)
        assert codes[0].tolist() == want, (rec, [hex(c) for c in codes[0]])
        assert sigma[0] == 2.0 ** e


def _fp8_rows(rng, R=64, C=512):
    x = rng.standard_normal((R, C))
    x[rng.random((R, C)) < 0.01] *= 20.0
    x[::7] *= 2.0 ** rng.integers(-40, 40, size=(len(x[::7]), 1))
    x[3] = 0.0
    return codec.f64_to_bf16_bits_exact(codec.bf16_bits_to_f64(
        (np.frombuffer(x.astype(np.float32).tobytes(), dtype=np.uint32) >> 16).astype(np.uint16).reshape(R, C)))


def check_fp8_vs_torch_cast():
    """Codes = torch's float8_e4m3fn cast of x / sigma (RNE); sigma puts the
    row's largest magnitude in (224, 448] (the top binade of E4M3), and the
    round trip is within half an E4M3 step."""
    rng = np.random.default_rng(41)
    bits = _fp8_rows(rng)
    x = codec.bf16_bits_to_f64(bits)
    codes, sigma = oracle.quantize_fp8(bits)
    amax = np.abs(x).max(axis=1)
    nz = amax > 0
    r = amax[nz] / sigma[nz]
    assert np.all((r > 224.0) & (r <= 448.0)), r.min()
    assert np.all(sigma[~nz] == 1.0)
    y = torch.from_numpy(x / sigma[:, None]).to(torch.float8_e4m3fn)
    tb = y.view(torch.uint8).numpy()
    assert np.array_equal(codes, tb)
    back = oracle.dequantize_fp8(codes, sigma)
    step = sigma[:, None] * 2.0 ** (np.floor(np.log2(np.maximum(np.abs(x) / sigma[:, None], 2.0 ** -6))) - 3)
    assert np.all(np.abs(back - x) <= step / 2 + 1e-300)


def _swa_inputs(B=2, H=8, W=24, d_c=64, d_r=32, seed=42):
    rng = np.random.default_rng(seed)
    qb = codec.f64_to_bf16_bits_exact(codec.bf16_bits_to_f64(
        (np.frombuffer(rng.standard_normal((B, H, d_c + d_r)).astype(np.float32).tobytes(),
                       dtype=np.uint32) >> 16).astype(np.uint16).reshape(B, H, d_c + d_r)))
    codes = rng.integers(0, 256, size=(B, W, d_c)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10          # no NaN codes
    sigma = 2.0 ** rng.integers(-8, -2, size=(B, W)).astype(np.float64)
    rb = (np.frombuffer(rng.standard_normal((B, W, d_r)).astype(np.float32).tobytes(),
                        dtype=np.uint32) >> 16).astype(np.uint16).reshape(B, W, d_r)
    return qb, codes, sigma, rb


def check_swa_vs_sdpa():
    """Window attention = float64 SDPA over the dequantised window rows."""
    qb, codes, sigma, rb = _swa_inputs()
    sm = 0.1
    nw = np.array([24, 17])
    out, lse = oracle.swa_attn(qb, codes, sigma, rb, nw, sm)
    q = torch.from_numpy(codec.bf16_bits_to_f64(qb))
    for b in range(2):
        lat = torch.from_numpy(codec.e4m3_decode(codes[b, :nw[b]]) * sigma[b, :nw[b], None])
        key = torch.cat([lat, torch.from_numpy(codec.bf16_bits_to_f64(rb[b, :nw[b]]))], dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(q[b][None], key[None], lat[None], scale=sm)[0]
        assert np.allclose(out[b], ref.numpy(), rtol=1e-12, atol=1e-12)
        s = sm * (q[b] @ key.T)
        assert np.allclose(lse[b], torch.logsumexp(s, dim=1).numpy(), rtol=1e-12, atol=1e-12)
    o0, l0 = oracle.swa_attn(qb, codes, sigma, rb, np.array([0, 1]), sm)
    assert np.all(o0[0] == 0) and np.all(np.isneginf(l0[0]))
    lat1 = codec.e4m3_decode(codes[1, 0]) * sigma[1, 0]
    assert np.array_equal(o0[1], np.tile(lat1, (qb.shape[1], 1)))


def check_merge_is_one_softmax_over_the_union():
    """The sparse branch (FP4 entries picked by idx) merged with the window
    branch (FP8 rows) equals one float64 SDPA over the concatenation of both
    key sets; an empty side leaves the other unchanged."""
    qb, codes, scales, rb = _attn_inputs(B=2, H=8, N=40, d_c=64, d_r=32, seed=43)
    _, c8, s8, r8 = _swa_inputs(B=2, H=8, W=24, d_c=64, d_r=32, seed=44)
    sm = 0.1
    idx = np.array([[3, 9, 11, 30, -1], [0, 1, 2, 3, 39]])
    nw = np.array([24, 5])
    o1, l1 = oracle.sparse_attn(qb, codes, scales, rb, idx, sm)
    o2, l2 = oracle.swa_attn(qb, c8, s8, r8, nw, sm)
    o, l = oracle.merge_branches(o1, l1, o2, l2)
    q = torch.from_numpy(codec.bf16_bits_to_f64(qb))
    for b in range(2):
        sel = idx[b][idx[b] >= 0]
        lat1 = oracle.dequantize_fp4(codes[b, sel], scales[b, sel])
        lat2 = codec.e4m3_decode(c8[b, :nw[b]]) * s8[b, :nw[b], None]
        lat = torch.from_numpy(np.concatenate([lat1, lat2]))
        rope = np.concatenate([codec.bf16_bits_to_f64(rb[b, sel]), codec.bf16_bits_to_f64(r8[b, :nw[b]])])
        key = torch.cat([lat, torch.from_numpy(rope)], dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(q[b][None], key[None], lat[None], scale=sm)[0]
        assert np.allclose(o[b], ref.numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(l[b], torch.logsumexp(sm * (q[b] @ key.T), dim=1).numpy(), rtol=1e-12, atol=1e-12)
    e_o, e_l = np.zeros_like(o1), np.full_like(l1, -np.inf)
    oa, la = oracle.merge_branches(o1, l1, e_o, e_l)
    assert np.array_equal(oa, o1) and np.array_equal(la, l1)
    oz, lz = oracle.merge_branches(e_o, e_l, e_o, e_l)
    assert np.all(oz == 0) and np.all(np.isneginf(lz))


# ------------------------------------------------------------------ sampler


def _sample_records():
    out = []
    for rec in _records("sampler_rows.txt"):
        a = rec.index("|")
        b = rec.index("|", a + 1)
        K, T, top_p, u = int(rec[0]), float(rec[1]), float(rec[2]), float(rec[3])
        logits = np.array([float(v) for v in rec[a + 1:b]])
        tok, n, pos, prob = int(rec[b + 1]), int(rec[b + 2]), int(rec[b + 3]), float(rec[b + 4])
        out.append((K, T, top_p, u, logits, tok, n, pos, prob))
    return out


def check_sample_golden():
    """Hand-derived draws (tests/golden/sampler_rows.txt)."""
    for K, T, top_p, u, logits, tok, n, pos, prob in _sample_records():
        t, p, nk, ps, _, _ = oracle.sample(logits[None], K, T, top_p, [u])
        assert (int(t[0]), int(nk[0]), int(ps[0])) == (tok, n, pos), (logits, K, T, top_p, u, t, nk, ps)
        assert abs(float(p[0]) - prob) <= 1e-15, (logits, p, prob)


def check_sample_frequencies_vs_softmax():
    """With every token a candidate and top_p = 1, the draws over a uniform
    grid of u give each token the share scipy's softmax of logits / T gives
    it (within one grid step), and the most likely tokens come first in u."""
    from scipy.special import softmax
    rng = np.random.default_rng(61)
    V, T, G = 12, 0.7, 6000
    logits = rng.standard_normal(V) * 2.0
    u = (np.arange(G) + 0.5) / G
    tok, _, _, _, _, _ = oracle.sample(np.tile(logits, (G, 1)), V, T, 1.0, u)
    want = softmax(logits / T)
    freq = np.bincount(tok, minlength=V) / G
    assert np.all(np.abs(freq - want) <= 1.0 / G + 1e-12), (freq, want)
    assert np.all(np.diff(want[tok]) <= 0)                  # along u: most likely first


def check_sample_nucleus_is_minimal():
    """The nucleus is the shortest most-probable prefix reaching top_p, with
    the candidate probabilities from scipy's softmax over the K largest
    logits / T (numpy sort); the reported probability is the drawn token's
    share of the nucleus."""
    from scipy.special import softmax
    rng = np.random.default_rng(62)
    B, V, K, T = 60, 40, 16, 0.8
    logits = rng.standard_normal((B, V)) * 1.5
    top_p = rng.uniform(0.05, 0.99, size=B)
    u = rng.random(B)
    for b in range(B):
        tok, prob, n, pos, _, _ = oracle.sample(logits[b][None], K, T, float(top_p[b]), u[b:b + 1])
        order = np.argsort(-logits[b], kind="stable")[:K]
        P = softmax(logits[b, order] / T)
        n, pos = int(n[0]), int(pos[0])
        assert P[:n].sum() >= top_p[b] - 1e-12 and P[:n - 1].sum() < top_p[b] + 1e-12, (b, n)
        assert 0 <= pos < n and int(tok[0]) == int(order[pos])
        assert abs(float(prob[0]) - P[pos] / P[:n].sum()) <= 1e-12
        assert P[:pos].sum() / P[:n].sum() <= u[b] + 1e-12 < P[:pos + 1].sum() / P[:n].sum() + 2e-12


def check_sample_limits():
    """K = 1 and a vanishing temperature draw the largest logit (lower id on
    ties) with probability 1, whatever u is."""
    rng = np.random.default_rng(63)
    logits = np.round(rng.standard_normal((20, 30)) * 3)      # integer logits: ties, gaps >= 1
    for u in (0.0, 0.5, 0.999999):
        uu = np.full(20, u)
        want = np.argmax(logits, axis=1)                        # first maximum = lower id
        t1, p1, n1, _, _, _ = oracle.sample(logits, 1, 1.0, 1.0, uu)
        assert np.array_equal(t1, want) and np.all(p1 == 1.0) and np.all(n1 == 1)
        distinct = logits.copy()
        distinct[np.arange(20), want] += 0.5                    # a unique maximum, gap >= 0.5
        t0, p0, _, _, _, _ = oracle.sample(distinct, 8, 1e-3, 1.0, uu)
        assert np.array_equal(t0, want) and np.all(p0 == 1.0)


def _sample_full_records():
    out = []
    for rec in _records("sampler_full_rows.txt"):
        a = rec.index("|")
        b = rec.index("|", a + 1)
        T, u = float(rec[0]), float(rec[1])
        logits = np.array([float(v) for v in rec[a + 1:b]])
        out.append((T, u, logits, int(rec[b + 1]), float(rec[b + 2])))
    return out


def check_sample_full_golden():
    """Hand-derived untruncated draws (tests/golden/sampler_full_rows.txt)."""
    for T, u, logits, tok, prob in _sample_full_records():
        t, p = oracle.sample_full(logits[None], T, [u])
        assert int(t[0]) == tok, (T, u, logits, t)
        assert abs(float(p[0]) - prob) <= 1e-15, (T, u, logits, p, prob)


def check_sample_full_frequencies_vs_softmax():
    """Over a uniform grid of u the untruncated draw gives every token of the
    vocabulary the share scipy's softmax of logits / T gives it (within one
    grid step), tokens coming in id order along u."""
    from scipy.special import softmax
    rng = np.random.default_rng(71)
    V, T, G = 40, 1.3, 20000
    logits = rng.standard_normal(V) * 2.0
    logits[[3, 17]] = -np.inf
    u = (np.arange(G) + 0.5) / G
    tok, prob = oracle.sample_full(np.tile(logits, (G, 1)), T, u)
    want = softmax(logits / T)
    freq = np.bincount(tok, minlength=V) / G
    assert np.all(np.abs(freq - want) <= 1.0 / G + 1e-12), np.abs(freq - want).max()
    assert np.all(np.diff(tok) >= 0)                        # along u: token ids ascending
    assert freq[3] == 0 and freq[17] == 0
    assert np.allclose(prob, want[tok], rtol=1e-12, atol=0)


def check_sample_full_boundary_exact_sums():
    """The drawn token t of every row satisfies C(t - 1) <= u * W < C(t), with
    C the running weights and W their total summed exactly (math.fsum), over
    random rows of a large vocabulary, temperatures and uniforms."""
    import math
    rng = np.random.default_rng(72)
    B, V = 12, 3000
    logits = rng.standard_normal((B, V)) * 4.0
    T = rng.uniform(0.3, 2.0, size=B)
    u = rng.random(B)
    for b in range(B):
        t, p = oracle.sample_full(logits[b][None], float(T[b]), u[b:b + 1])
        t = int(t[0])
        w = np.exp((logits[b] - logits[b].max()) / T[b])
        W = math.fsum(w)
        before, through = math.fsum(w[:t]), math.fsum(w[:t + 1])
        target = u[b] * W
        assert before <= target * (1 + 1e-12) and through > target * (1 - 1e-12), (b, t, before, target, through)
        assert abs(float(p[0]) - w[t] / W) <= 1e-12


def check_sample_full_limits():
    """A vanishing temperature draws the unique largest logit whatever u is,
    and a one-token vocabulary always draws token 0 with probability 1."""
    rng = np.random.default_rng(73)
    logits = np.round(rng.standard_normal((16, 50)) * 3)
    want = np.argmax(logits, axis=1)
    logits[np.arange(16), want] += 0.5                       # unique maxima, gap >= 0.5
    for uu in (0.0, 0.5, 0.999999):
        t, p = oracle.sample_full(logits, 1e-3, np.full(16, uu))
        assert np.array_equal(t, want) and np.all(p == 1.0)
    t, p = oracle.sample_full(np.array([[-2.5]]), 0.7, [0.99])
    assert int(t[0]) == 0 and float(p[0]) == 1.0


ALL_PINS = [
    check_e2m1_value_set, check_e4m3_decode, check_e4m3_encode_vs_torch, check_scale_code_vs_torch,
    check_e2m1_encode_vs_numpy_round, check_bf16_decode, check_quantize_golden,
    check_quantize_roundtrip_fixed_point, check_quantize_error_bound, check_nibble_order,
    check_index_bruteforce, check_index_full_vs_int64_matmul, check_index_pool_bruteforce,
    check_topk_bruteforce, check_topk_vs_torch_topk_distinct, check_topk_ties_vs_stable_sort,
    check_topk_invariants, check_attn_dense_vs_sdpa, check_attn_special_cases, check_decode_modes_compose,
    check_prefill_vs_causal_sdpa,
    check_pool_golden, check_pool_bruteforce, check_pool_reindex_reproduces_full_topk,
    check_fp8_golden, check_fp8_vs_torch_cast, check_swa_vs_sdpa, check_merge_is_one_softmax_over_the_union,
    check_sample_golden, check_sample_frequencies_vs_softmax, check_sample_nucleus_is_minimal,
    check_sample_limits,
    check_sample_full_golden, check_sample_full_frequencies_vs_softmax, check_sample_full_boundary_exact_sums,
    check_sample_full_limits,
]
