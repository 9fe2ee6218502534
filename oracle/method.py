"""The CSA2 decode step, written out in float64 (TEST INFRASTRUCTURE ONLY).

What the step computes, stage by stage (citations use the page keys of the
package docstring; the pages give no formulas, so where they are silent the
reading taken is stated at the function):

1. a0  ``quantize_fp4``  - the FP4 main-KV write: E2M1 values, one E4M3
       scale per 16 channels, no global scale, applied to post-RoPE values
       [P1 效率组件四件 #4; P4 CSA2 paragraph].
2. a1  ``index_full``    - Full mode: the layer's own indexer scores every
       compressed entry [P1 架构三件套 / CSA2; P3 mode paragraph; P4 CSA2 paragraph].
3. a2  ``index_pool``    - Reindex mode: the layer's own indexer query
       re-scores only the candidate pool of at most 2048 blocks x 8 positions
       chosen by an earlier Full layer [P1 Hierarchical Sparse Indexer; P4].
4. a3  ``topk``          - Top-512 selection [P1 CSA2], ties resolved so
       that the lower entry position wins.
   ``build_pool``    - the block-level candidate pool an earlier Full layer
       hands to the Reindex layers [P1 Hierarchical Sparse Indexer].
5. a4/a5 ``sparse_attn`` - gather of the selected FP4 entries, exact
       dequantisation, and softmax attention of every query head over them
       (MLA-style: one latent shared by all heads; the key is [latent ; RoPE
       part], the value is the latent).  Reuse mode is this stage alone with
       the index list handed in [P1 CSA2; P3; P4].
   ``prefill_sparse_attn`` - the same attention for a prefill chunk: many
       queries of one sequence, each with its own list [P1 inference paragraph].
   ``sample``        - the decode sampler on the same Top-K: temperature,
       top-p nucleus, inverse-CDF draw [P3 DeepSelect; P1 sampling settings].
"""

import numpy as np

from .codec import (
    bf16_bits_to_f64,
    e4m3_encode,
    e2m1_decode,
    e2m1_encode_magnitude,
    e4m3_decode,
    e4m3_scale_code_for_amax,
)

GROUP = 16  # channels per E4M3 scale [P1 效率组件四件 #4]


# ------------------------------------------------------------ a0 quantize


def quantize_fp4(x_bits):
    """Quantise bf16 rows to the FP4 cache format.

    x_bits: uint16 [R, d_c] bf16 patterns (post-RoPE latent rows), d_c % 16 == 0.
    Returns (codes uint8 [R, d_c/2], scales uint8 [R, d_c/16]).

    Per row and per group of 16 consecutive channels:
      amax  = max |x| over the group
      S     = E4M3 code nearest to amax / 6 (ties even, saturate at 448)
      sigma = value(S)
      code  = sign bit of x (bit 3) | E2M1 magnitude code nearest to |x|/sigma
              (ties even, saturating at 6; sigma == 0 gives magnitude 0)
    Byte j of a row holds channel 2j in its low nibble and 2j+1 in its high
    nibble.
    """
    x_bits = np.asarray(x_bits)
    R, d_c = x_bits.shape
    assert d_c % GROUP == 0
    x = bf16_bits_to_f64(x_bits)                       # exact
    xg = x.reshape(R, d_c // GROUP, GROUP)
    amax = np.abs(xg).max(axis=-1)                     # [R, G]
    S = e4m3_scale_code_for_amax(amax)                 # [R, G] uint8
    sigma = e4m3_decode(S)                             # [R, G]
    mag = e2m1_encode_magnitude(np.abs(xg), sigma[..., None])   # [R, G, 16]
    sign = np.signbit(xg).astype(np.uint8)
    nib = (sign << 3) | mag                            # [R, G, 16]
    nib = nib.reshape(R, d_c)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return codes, S.astype(np.uint8)


def dequantize_fp4(codes, scales):
    """Exact dequantisation: value(code) * value(scale of its group), float64."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    lead = codes.shape[:-1]
    d_c = codes.shape[-1] * 2
    nib = np.empty(lead + (d_c,), dtype=np.uint8)
    nib[..., 0::2] = codes & 0x0F
    nib[..., 1::2] = codes >> 4
    v = e2m1_decode(nib)
    sig = np.repeat(e4m3_decode(scales), GROUP, axis=-1)
    return v * sig


# ------------------------------------------------------------ a1 / a2 indexer


def index_scores(q_idx, w, keys):
    """Indexer score of every key row for one query.

    q_idx [H_I, D_I], w [H_I] (None -> all ones), keys [N, D_I], all float64.
    score[n] = sum_h w[h] * max(0, q_idx[h] . keys[n])

    Reading (the pages give no formula): several indexer heads, each gated by
    a ReLU, summed with per-head weights; one key per compressed entry shared
    by all indexer heads.
    """
    H_I = q_idx.shape[0]
    if w is None:
        w = np.ones(H_I)
    dots = keys @ q_idx.T                               # [N, H_I]
    return (np.maximum(dots, 0.0) * w[None, :]).sum(axis=1)


def index_full(q_bits, w, k_bits, n_valid):
    """Full mode: score every entry n < n_valid[b]; others get -inf.

    q_bits uint16 [B, H_I, D_I]; w float [B, H_I] or None; k_bits uint16
    [B, N, D_I]; n_valid int [B] or None (= N).  Returns float64 [B, N].
    """
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    B, N, _ = k.shape
    out = np.full((B, N), -np.inf)
    for b in range(B):
        nv = N if n_valid is None else int(min(max(int(n_valid[b]), 0), N))
        wb = None if w is None else np.asarray(w[b], dtype=np.float64)
        out[b, :nv] = index_scores(q[b], wb, k[b, :nv])
    return out


def index_pool(q_bits, w, k_bits, n_valid, pool_blocks, n_blocks, block):
    """Reindex mode: score only the positions of the candidate pool.

    Pool slot (i, j), i < n_blocks[b], j < block, is entry position
    p = block * pool_blocks[b, i] + j.  It is scored when 0 <= p < n_valid[b]
    (and the block id is non-negative); every other slot gets score -inf and
    position -1.  Returns (scores float64 [B, P_max*block],
    positions int32 [B, P_max*block]).
    """
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    B, N, _ = k.shape
    P_max = pool_blocks.shape[1]
    scores = np.full((B, P_max * block), -np.inf)
    pos = np.full((B, P_max * block), -1, dtype=np.int32)
    for b in range(B):
        nv = N if n_valid is None else int(min(max(int(n_valid[b]), 0), N))
        nb = int(min(max(int(n_blocks[b]), 0), P_max))
        blk = np.asarray(pool_blocks[b, :nb], dtype=np.int64)
        p = (block * blk[:, None] + np.arange(block)[None, :]).reshape(-1)
        ok = (np.repeat(blk, block) >= 0) & (p >= 0) & (p < nv)
        slots = np.nonzero(ok)[0]
        wb = None if w is None else np.asarray(w[b], dtype=np.float64)
        scores[b, slots] = index_scores(q[b], wb, k[b, p[slots]])
        pos[b, slots] = p[slots]
    return scores, pos


# ------------------------------------------------------------ a3 Top-K


def topk(scores, ids, n_valid, K):
    """Top-K by (score descending, id ascending) over the valid candidates.

    scores float [B, M]; ids int [B, M] or None (None -> the column index);
    n_valid int [B] or None (= M).  Candidate (b, c) is valid when
    c < n_valid[b] and its id is not -1.  The first min(K, #valid) candidates
    of that order are returned in that order; the rest is padded with id -1
    and score -inf.  NaN scores rank below every other score (numpy sorts
    NaN last).  Returns (idx int32 [B, K], score float64 [B, K]).
    """
    scores = np.asarray(scores, dtype=np.float64)
    B, M = scores.shape
    out_i = np.full((B, K), -1, dtype=np.int32)
    out_s = np.full((B, K), -np.inf)
    for b in range(B):
        nv = M if n_valid is None else int(min(max(int(n_valid[b]), 0), M))
        cid = np.arange(M, dtype=np.int64) if ids is None else np.asarray(ids[b], dtype=np.int64)
        valid = (np.arange(M) < nv) & (cid != -1)
        s = scores[b, valid]
        i = cid[valid]
        order = np.lexsort((i, -s))                   # primary: -score, then id
        take = order[:K]
        out_i[b, :take.size] = i[take]
        out_s[b, :take.size] = s[take]
    return out_i, out_s


# ------------------------------------------------------------ pool construction


def build_pool(scores, n_valid, block, P_max):
    """Block-level candidate pool built from a Full layer's indexer scores, for
    the Reindex layers after it [P1 Hierarchical Sparse Indexer; P4 CSA2
    paragraph].

    The pages say only that the decoder's first Full layer builds a pool of at
    most 2048 blocks x 8 positions and that later layers score inside it.
    Reading taken: block beta covers positions [block*beta, block*beta + block);
    it is a candidate when its first position is valid (< n_valid[b]); its
    score is the largest score among its valid positions (NaN ignored unless
    every one is NaN); the pool is the first min(P_max, #candidates) blocks in
    the Top-K order applied to blocks (block score descending, block id
    ascending), padded with -1.
    scores float [B, M]; n_valid int [B] or None (= M).
    Returns (pool_blocks int32 [B, P_max], n_blocks int32 [B]).
    """
    scores = np.asarray(scores, dtype=np.float64)
    B, M = scores.shape
    n_cand_max = (M + block - 1) // block
    block_scores = np.full((B, max(n_cand_max, 1)), -np.inf)
    n_cand = np.zeros(B, dtype=np.int64)
    for b in range(B):
        nv = M if n_valid is None else int(min(max(int(n_valid[b]), 0), M))
        n_cand[b] = (nv + block - 1) // block
        for beta in range(n_cand[b]):
            block_scores[b, beta] = np.fmax.reduce(scores[b, block * beta:min(block * beta + block, nv)])
    pool, _ = topk(block_scores, None, n_cand, P_max)
    return pool, np.minimum(n_cand, P_max).astype(np.int32)


# ------------------------------------------------------------ a4/a5 attention


def sparse_attn(q_bits, codes, scales, rope_bits, idx, sm_scale):
    """Softmax attention of every head over the selected FP4 entries.

    q_bits uint16 [B, H, d_c + d_r]; codes uint8 [B, N, d_c/2]; scales uint8
    [B, N, d_c/16]; rope_bits uint16 [B, N, d_r] (d_r may be 0); idx int
    [B, K] (entries outside [0, N), e.g. -1, are skipped; repeated entries
    count with multiplicity).

    For each b, h over the selected entries j:
      key_j   = [dequant(codes_j, scales_j) ; rope_j]
      value_j = dequant(codes_j, scales_j)
      s_j = sm_scale * q_h . key_j ;  p_j = exp(s_j - max s) ;  L = sum p
      out = sum_j p_j value_j / L ;   lse = max s + ln L
    No selected entry -> out = 0, lse = -inf.
    Returns (out float64 [B, H, d_c], lse float64 [B, H]).
    """
    q = bf16_bits_to_f64(q_bits)
    B, H, D = q.shape
    N = codes.shape[1]
    d_c = codes.shape[2] * 2
    out = np.zeros((B, H, d_c))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        sel = np.asarray(idx[b], dtype=np.int64)
        sel = sel[(sel >= 0) & (sel < N)]
        if sel.size == 0:
            continue
        lat = dequantize_fp4(codes[b, sel], scales[b, sel])          # [k, d_c]
        if D > d_c:
            key = np.concatenate([lat, bf16_bits_to_f64(rope_bits[b, sel])], axis=1)
        else:
            key = lat
        s = sm_scale * (q[b] @ key.T)                                 # [H, k]
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        L = p.sum(axis=1, keepdims=True)
        out[b] = (p @ lat) / L
        lse[b] = m[:, 0] + np.log(L[:, 0])
    return out, lse


# ------------------------------------------------------------ sliding-window branch (FP8)

E4M3_MAX = 448.0


def fp8_row_scale_exponent(amax):
    """Smallest integer e with amax <= 448 * 2^e (0 when amax = 0), clamped to
    [-126, 127] so that 2^e is a normal fp32 number."""
    amax = np.asarray(amax, dtype=np.float64)
    if not np.all(np.isfinite(amax)):
        raise ValueError("FP8 rows must be finite")
    e = np.zeros(amax.shape, dtype=np.int64)
    for idx in np.ndindex(amax.shape):
        a = float(amax[idx])
        if a == 0.0:
            continue
        k = int(np.floor(np.log2(a))) - 9          # start below, then walk up
        while E4M3_MAX * 2.0 ** k < a:
            k += 1
        while E4M3_MAX * 2.0 ** (k - 1) >= a:
            k -= 1
        e[idx] = min(max(k, -126), 127)
    return e


def quantize_fp8(x_bits):
    """FP8 write of the sliding-window KV: the window branch keeps its KV in
    FP8 [P4 CSA2 paragraph; P1 效率组件四件 #4].

    The pages give no scale granularity.  Reading taken: one power-of-two
    scale per token (row), sigma = 2^e with e the smallest integer such that
    max|x| <= 448 * sigma (sigma = 1 for an all-zero row), so x / sigma is
    exact and no element saturates; each element's code is the E4M3 value
    nearest to |x| / sigma (ties to the even code), with the sign bit copied
    from the input (-0 -> 0x80).
    x_bits uint16 bf16 [R, C].  Returns (codes uint8 [R, C], sigma float64 [R]).
    """
    bits = np.asarray(x_bits, dtype=np.uint16)
    x = bf16_bits_to_f64(bits)
    e = fp8_row_scale_exponent(np.abs(x).max(axis=1) if x.shape[1] else np.zeros(x.shape[0]))
    sigma = 2.0 ** e.astype(np.float64)
    mag = e4m3_encode(np.abs(x) / sigma[:, None])
    codes = (mag | (((bits >> 15) & 1).astype(np.uint8) << 7)).astype(np.uint8)
    return codes, sigma


def dequantize_fp8(codes, sigma):
    """Exact dequantisation of the window rows: value(code) * sigma, float64."""
    return e4m3_decode(codes) * np.asarray(sigma, dtype=np.float64)[..., None]


def swa_attn(q_bits, codes, sigma, rope_bits, n_win, sm_scale):
    """Softmax attention of every head over the sliding window (the last
    tokens, uncompressed, one FP8 entry per token) [P4 CSA2 paragraph: SWA
    branch beside the sparse one; P1 效率组件四件 #4].

    Same MLA form as the main cache: key_j = [dequant(codes_j) ; rope_j],
    value_j = dequant(codes_j).  Rows j < n_win[b] of the window are used (the
    window's order does not matter).  q_bits uint16 [B, H, d_c + d_r]; codes
    uint8 [B, W, d_c]; sigma [B, W]; rope_bits uint16 [B, W, d_r]; n_win int
    [B] or None (= W).  Returns (out float64 [B, H, d_c], lse float64 [B, H]);
    an empty window gives out = 0, lse = -inf.
    """
    q = bf16_bits_to_f64(q_bits)
    B, H, D = q.shape
    W, d_c = codes.shape[1], codes.shape[2]
    out = np.zeros((B, H, d_c))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        nw = W if n_win is None else int(min(max(int(n_win[b]), 0), W))
        if nw == 0:
            continue
        lat = dequantize_fp8(codes[b, :nw], sigma[b, :nw])
        key = np.concatenate([lat, bf16_bits_to_f64(rope_bits[b, :nw])], axis=1) if D > d_c else lat
        s = sm_scale * (q[b] @ key.T)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        L = p.sum(axis=1, keepdims=True)
        out[b] = (p @ lat) / L
        lse[b] = m[:, 0] + np.log(L[:, 0])
    return out, lse


def merge_branches(out_a, lse_a, out_b, lse_b):
    """One softmax over the union of two disjoint key sets, from each set's
    normalised output and natural-log sum-exp: the sparse branch and the
    window branch of a layer attend as one [P4 CSA2 paragraph: the sparse
    branch beside the SWA branch; reading: one softmax over the union, the
    LSE the sparse attention exports for this].

    out = (e^lse_a out_a + e^lse_b out_b) / (e^lse_a + e^lse_b),
    lse = log(e^lse_a + e^lse_b); both empty -> out = 0, lse = -inf.
    """
    la = np.asarray(lse_a, dtype=np.float64)
    lb = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(la, lb)
    safe = np.where(np.isfinite(m), m, 0.0)
    wa = np.exp(la - safe)
    wb = np.exp(lb - safe)
    tot = wa + wb
    den = np.where(tot > 0, tot, 1.0)
    out = (wa[..., None] * np.asarray(out_a, dtype=np.float64) +
           wb[..., None] * np.asarray(out_b, dtype=np.float64)) / den[..., None]
    lse = np.where(tot > 0, safe + np.log(den), -np.inf)
    return out, lse



def prefill_sparse_attn(q_bits, codes, scales, rope_bits, idx, sm_scale):
    """Sparse attention of a prefill chunk: T queries of each sequence, every
    one with its own index list into that sequence's cache [P1 inference
    paragraph: the Reuse layers also run in prefill; P4 CSA2 paragraph].

    Reading taken: a prefill query attends exactly as a decode query does
    (``sparse_attn``), over its own sequence's cache through its own list;
    causality is the lists' business (an entry a query may not see is never
    in its list), the attention adds no mask of its own.
    q_bits u16 [S, T, H, D]; codes / scales / rope_bits [S, N, ...] (one cache
    per sequence); idx int [S, T, K].  Returns (out float64 [S, T, H, d_c],
    lse float64 [S, T, H]).
    """
    S, T = q_bits.shape[:2]
    outs, lses = [], []
    for s in range(S):
        rep = lambda a: np.broadcast_to(a[s], (T,) + a.shape[1:])   # noqa: E731
        o, l = sparse_attn(q_bits[s], rep(codes), rep(scales), rep(rope_bits), np.asarray(idx[s]), sm_scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)

# ------------------------------------------------------------ the three modes


def decode_full(q_idx_bits, w, k_idx_bits, n_valid, q_bits, codes, scales, rope_bits, K, sm_scale):
    """Full mode: index every entry -> Top-K -> sparse attention [P1 CSA2; P4]."""
    sc = index_full(q_idx_bits, w, k_idx_bits, n_valid)
    idx, top = topk(sc, None, n_valid, K)
    out, lse = sparse_attn(q_bits, codes, scales, rope_bits, idx, sm_scale)
    return idx, top, out, lse


def decode_reindex(q_idx_bits, w, k_idx_bits, n_valid, pool_blocks, n_blocks, block,
                   q_bits, codes, scales, rope_bits, K, sm_scale):
    """Reindex mode: re-score the pool -> Top-K by global position -> attention."""
    sc, pos = index_pool(q_idx_bits, w, k_idx_bits, n_valid, pool_blocks, n_blocks, block)
    idx, top = topk(sc, pos, None, K)
    out, lse = sparse_attn(q_bits, codes, scales, rope_bits, idx, sm_scale)
    return idx, top, out, lse


def decode_reuse(idx, q_bits, codes, scales, rope_bits, sm_scale):
    """Reuse mode: the index list is handed in; attention only."""
    return sparse_attn(q_bits, codes, scales, rope_bits, idx, sm_scale)


# ------------------------------------------------------------ the sampler


def sample(logits, K, temperature, top_p, u):
    """One token drawn per row by the decode sampler built on the Top-K
    selection [P3 DeepSelect paragraph: one Top-K implementation serves the
    sparse attention and the sampler; P1 interface paragraph: the recommended
    sampling settings name a temperature and a top_p].

    The pages name the knobs, not their order.  Reading taken:
    1. the candidates are the row's Top-K (logit descending, token id
       ascending), as ``topk`` returns them;
    2. weight w_i = exp((l_i - l_0) / T) for the i-th candidate, l_0 the
       largest logit (a -inf logit and an empty slot weigh 0); the candidate
       probabilities are w_i / sum(w), normalised over the K candidates;
    3. the nucleus is the shortest prefix of that order whose probability
       reaches top_p; every candidate when top_p >= 1 or when no prefix
       reaches top_p;
    4. the draw takes the uniform u in [0, 1) as an input and returns the
       first position of the nucleus whose running weight exceeds u times the
       nucleus weight (if rounding leaves none, the last position of nonzero
       weight).
    A row whose largest logit is -inf draws its first candidate.

    logits float [B, V]; u float [B].  Returns (token int32 [B], prob float64
    [B] = w_pos / nucleus weight, n_kept int32 [B], pos int32 [B], idx int32
    [B, K] the candidates, w float64 [B, K] their weights).
    """
    logits = np.asarray(logits, dtype=np.float64)
    B = logits.shape[0]
    idx, s = topk(logits, None, None, K)
    u = np.asarray(u, dtype=np.float64).reshape(B)
    w = np.zeros((B, K))
    token = np.zeros(B, dtype=np.int32)
    prob = np.ones(B)
    n_kept = np.ones(B, dtype=np.int32)
    pos = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n_cand = int((idx[b] >= 0).sum())
        token[b] = idx[b, 0]
        if s[b, 0] == -np.inf:
            continue
        for i in range(n_cand):
            if s[b, i] != -np.inf:
                w[b, i] = np.exp((s[b, i] - s[b, 0]) / temperature)
        total = w[b].sum()
        n = n_cand
        if top_p < 1.0:
            mass = 0.0
            for i in range(n_cand):
                mass += w[b, i] / total
                if mass >= top_p:
                    n = i + 1
                    break
        nucleus = w[b, :n].sum()
        target = u[b] * nucleus
        run = 0.0
        p = -1
        for i in range(n):
            run += w[b, i]
            if run > target:
                p = i
                break
        if p < 0:
            p = max(i for i in range(n) if w[b, i] > 0)
        n_kept[b] = n
        pos[b] = p
        token[b] = idx[b, p]
        prob[b] = w[b, p] / nucleus
    return token, prob, n_kept, pos, idx, w


def sample_full(logits, temperature, u):
    """One token per row drawn from the softmax of logits / T over the whole
    vocabulary, untruncated: the recommended decode settings, temperature
    1.0 and top_p 1.0 [P1 interface paragraph], taken literally (top_p 1.0
    keeps every token, so no Top-K cap applies).

    The pages give only the two settings.  Reading taken:
    1. weight w_i = exp((l_i - l_max) / T) for every token i of the row (a
       -inf logit weighs 0), l_max the row's largest logit;
    2. the draw takes the uniform u in [0, 1) as an input and returns the
       first token, in token-id order, whose running weight exceeds
       u * sum(w) (if rounding leaves none, the last token of nonzero
       weight); prob = w_token / sum(w);
    3. a row whose largest logit is -inf draws token 0 with probability 1.
    Token-id order makes the draw a plain inverse CDF over the vocabulary;
    the distribution is the softmax whatever the order.

    logits float [B, V]; u float [B].  Returns (token int32 [B], prob float64 [B]).
    """
    logits = np.asarray(logits, dtype=np.float64)
    B, V = logits.shape
    u = np.asarray(u, dtype=np.float64).reshape(B)
    token = np.zeros(B, dtype=np.int32)
    prob = np.ones(B)
    for b in range(B):
        l_max = logits[b].max()
        if l_max == -np.inf:
            continue
        w = np.where(logits[b] == -np.inf, 0.0, np.exp((logits[b] - l_max) / temperature))
        run = np.cumsum(w)
        total = run[-1]
        hit = np.nonzero(run > u[b] * total)[0]
        t = int(hit[0]) if hit.size else int(np.nonzero(w > 0)[0][-1])
        token[b] = t
        prob[b] = w[t] / total
    return token, prob
