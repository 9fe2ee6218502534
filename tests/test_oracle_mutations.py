"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them.  Each mutation replaces one oracle function for the
duration of the test only."""

import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle_pins as P  # noqa: E402
import oracle  # noqa: E402
from oracle import codec, method  # noqa: E402

_orig_quantize = method.quantize_fp4
_orig_enc = codec.e2m1_encode_magnitude
_orig_scale = codec.e4m3_scale_code_for_amax
_orig_topk = method.topk
_orig_attn = method.sparse_attn
_orig_pool = method.index_pool
_orig_scores = method.index_scores
_orig_build_pool = method.build_pool
_orig_fp8_exp = method.fp8_row_scale_exponent
_orig_swa = method.swa_attn
_orig_merge = method.merge_branches
_orig_sample = method.sample
_orig_prefill = method.prefill_sparse_attn


def _swap_nibbles(x_bits):
    c, s = _orig_quantize(x_bits)
    return ((c >> 4) | (c << 4)).astype(np.uint8), s


def _ties_away(y_abs, sigma):
    code = _orig_enc(y_abs, sigma)
    grid = codec.e2m1_decode(np.arange(8))
    y = np.asarray(y_abs, dtype=np.float64)
    sg = np.broadcast_to(np.asarray(sigma, dtype=np.float64), y.shape)
    up = np.minimum(code + 1, 7)
    tie = (sg * (grid[code] + grid[up]) / 2 == y) & (code < 7)
    return np.where(tie, up, code).astype(np.uint8)


def _scale_div4(amax):
    return _orig_scale(np.asarray(amax) * 1.5)


def _fnuz_decode(codes):
    return codec_e4m3_orig(codes) / 2.0


codec_e4m3_orig = codec.e4m3_decode


def _no_relu(q_idx, w, keys):
    H_I = q_idx.shape[0]
    w = np.ones(H_I) if w is None else w
    return ((keys @ q_idx.T) * w[None, :]).sum(axis=1)


def _topk_id_desc(scores, ids, n_valid, K):
    scores = np.asarray(scores, dtype=np.float64)
    B, M = scores.shape
    out_i = np.full((B, K), -1, dtype=np.int32)
    out_s = np.full((B, K), -np.inf)
    for b in range(B):
        nv = M if n_valid is None else int(min(max(int(n_valid[b]), 0), M))
        cid = np.arange(M) if ids is None else np.asarray(ids[b], dtype=np.int64)
        valid = (np.arange(M) < nv) & (cid != -1)
        s, i = scores[b, valid], cid[valid]
        order = np.lexsort((-i, -s))[:K]
        out_i[b, :order.size] = i[order]
        out_s[b, :order.size] = s[order]
    return out_i, out_s


def _attn_no_rope(q_bits, codes, scales, rope_bits, idx, sm_scale):
    return _orig_attn(q_bits, codes, scales, np.zeros_like(rope_bits), idx, sm_scale)


def _attn_lse_log2(*a):
    out, lse = _orig_attn(*a)
    return out, lse / np.log(2.0)


def _pool_transposed(q_bits, w, k_bits, n_valid, pool_blocks, n_blocks, block):
    # plant: position = block id + block * j instead of block * id + j
    pb = np.asarray(pool_blocks)
    sc, pos = _orig_pool(q_bits, w, k_bits, n_valid, pb, n_blocks, block)
    return sc, np.where(pos >= 0, pos // block + (pos % block) * block, pos).astype(np.int32)


def _pool_block_sum(scores, n_valid, block, P_max):
    # plant: a block scored by the sum of its positions instead of the largest
    sc = np.asarray(scores, dtype=np.float64)
    B, M = sc.shape
    nb = (M + block - 1) // block
    summed = np.full((B, M), -np.inf)
    for b in range(B):
        nv = M if n_valid is None else int(min(max(int(n_valid[b]), 0), M))
        for beta in range((nv + block - 1) // block):
            summed[b, block * beta] = np.nansum(sc[b, block * beta:min(block * beta + block, nv)])
    del nb
    return _orig_build_pool(summed, n_valid, block, P_max)


def _pool_high_id_first(scores, n_valid, block, P_max):
    # plant: among blocks of equal score the higher block id wins
    sc = np.asarray(scores, dtype=np.float64)
    B, M = sc.shape
    nbk = (M + block - 1) // block
    pool = np.full((B, P_max), -1, dtype=np.int32)
    n_blocks = np.zeros(B, dtype=np.int32)
    for b in range(B):
        nv = M if n_valid is None else int(min(max(int(n_valid[b]), 0), M))
        nc = (nv + block - 1) // block
        bs = np.array([np.fmax.reduce(sc[b, block * t:min(block * t + block, nv)]) for t in range(nc)])
        order = np.lexsort((-np.arange(nc), -bs))[:P_max]
        pool[b, :order.size] = order
        n_blocks[b] = min(nc, P_max)
    del nbk
    return pool, n_blocks


def _fp8_scale_one_lower(amax):
    # plant: the row scale one binade too small (the largest elements saturate)
    e = _orig_fp8_exp(amax)
    return np.where(np.asarray(amax) > 0, e - 1, e)


def _swa_no_rope(q_bits, codes, sigma, rope_bits, n_win, sm_scale):
    return _orig_swa(q_bits, codes, sigma, np.zeros_like(rope_bits), n_win, sm_scale)


def _merge_base2(out_a, lse_a, out_b, lse_b):
    # plant: branch weights 2^lse instead of e^lse
    return _orig_merge(out_a, np.asarray(lse_a) * np.log(2.0), out_b, np.asarray(lse_b) * np.log(2.0))


def _sample_generic(logits, K, temperature, top_p, u, weight, reach, exceeds, over_vocab=False):
    """The sampler written with one step replaceable (for the plants below)."""
    logits = np.asarray(logits, dtype=np.float64)
    B = logits.shape[0]
    idx, sc = _orig_topk(logits, None, None, K)
    u = np.asarray(u, dtype=np.float64).reshape(B)
    w = np.zeros((B, K))
    tok = np.zeros(B, dtype=np.int32)
    prob = np.ones(B)
    nk = np.ones(B, dtype=np.int32)
    pos = np.zeros(B, dtype=np.int32)
    for b in range(B):
        nc = int((idx[b] >= 0).sum())
        tok[b] = idx[b, 0]
        if sc[b, 0] == -np.inf:
            continue
        w[b, :nc] = [weight(sc[b, i], sc[b, 0], temperature) if sc[b, i] != -np.inf else 0.0 for i in range(nc)]
        total = np.exp((logits[b] - sc[b, 0]) / temperature).sum() if over_vocab else w[b].sum()
        n = nc
        if top_p < 1.0:
            cum = np.cumsum(w[b, :nc]) / total
            hit = [i for i in range(nc) if reach(cum[i], top_p)]
            n = hit[0] + 1 if hit else nc
        nuc = w[b, :n].sum()
        run = np.cumsum(w[b, :n])
        hit = [i for i in range(n) if exceeds(run, i, u[b] * nuc)]
        p = hit[0] if hit else max(i for i in range(n) if w[b, i] > 0)
        nk[b], pos[b], tok[b], prob[b] = n, p, idx[b, p], w[b, p] / nuc
    return tok, prob, nk, pos, idx, w


_W = lambda l, l0, T: np.exp((l - l0) / T)          # noqa: E731
_REACH = lambda c, p: c >= p                         # noqa: E731
_EXCEEDS = lambda run, i, t: run[i] > t              # noqa: E731


def _sample_temperature_multiplies(*a):
    # plant: logits multiplied by the temperature instead of divided
    return _sample_generic(*a, lambda l, l0, T: np.exp((l - l0) * T), _REACH, _EXCEEDS)


def _sample_nucleus_strict(*a):
    # plant: the nucleus must exceed top_p instead of reaching it
    return _sample_generic(*a, _W, lambda c, p: c > p, _EXCEEDS)


def _sample_draw_exclusive(*a):
    # plant: the draw compares the weight before a position, not through it
    return _sample_generic(*a, _W, _REACH, lambda run, i, t: (run[i - 1] if i else 0.0) > t)


def _sample_probs_over_vocab(*a):
    # plant: top_p measured against the whole vocabulary instead of the K candidates
    return _sample_generic(*a, _W, _REACH, _EXCEEDS, over_vocab=True)


def _sample_unmutated(*a):
    return _sample_generic(*a, _W, _REACH, _EXCEEDS)


_orig_sample_full = method.sample_full


def _sample_full_generic(logits, temperature, u, weight, order, exceeds):
    """The untruncated draw written with one step replaceable (for the plants below)."""
    logits = np.asarray(logits, dtype=np.float64)
    B = logits.shape[0]
    u = np.asarray(u, dtype=np.float64).reshape(B)
    tok = np.zeros(B, dtype=np.int32)
    prob = np.ones(B)
    for b in range(B):
        lm = logits[b].max()
        if lm == -np.inf:
            continue
        w = np.where(logits[b] == -np.inf, 0.0, weight(logits[b], lm, temperature))
        ids = order(logits[b])
        run = np.cumsum(w[ids])
        hit = [i for i in range(len(ids)) if exceeds(run, i, u[b] * run[-1])]
        t = int(ids[hit[0]]) if hit else int(np.nonzero(w > 0)[0][-1])
        tok[b], prob[b] = t, w[t] / run[-1]
    return tok, prob


_IDS = lambda l: np.arange(len(l))                   # noqa: E731


def _sample_full_temperature_multiplies(*a):
    # plant: logits multiplied by the temperature instead of divided
    return _sample_full_generic(*a, lambda l, lm, T: np.exp((l - lm) * T), _IDS, _EXCEEDS)


def _sample_full_logit_order(*a):
    # plant: the inverse CDF walks the tokens by logit (descending), not by id
    return _sample_full_generic(*a, _W, lambda l: np.argsort(-l, kind="stable"), _EXCEEDS)


def _sample_full_boundary_inclusive(*a):
    # plant: a running weight equal to the target already selects the token
    return _sample_full_generic(*a, _W, _IDS, lambda run, i, t: run[i] >= t)


def _sample_full_unmutated(*a):
    return _sample_full_generic(*a, _W, _IDS, _EXCEEDS)


def _prefill_first_cache(q_bits, codes, scales, rope_bits, idx, sm_scale):
    # plant: every sequence of the chunk reads the first sequence's cache
    rep = lambda a: np.broadcast_to(a[:1], a.shape)   # noqa: E731
    return _orig_prefill(q_bits, rep(codes), rep(scales), rep(rope_bits), idx, sm_scale)


def _prefill_query_order(q_bits, codes, scales, rope_bits, idx, sm_scale):
    # plant: the chunk's queries paired with the lists in reverse order
    return _orig_prefill(q_bits, codes, scales, rope_bits, np.asarray(idx)[:, ::-1], sm_scale)


MUTATIONS = {
    "nibble_order_swapped": [(method, "quantize_fp4", _swap_nibbles), (oracle, "quantize_fp4", _swap_nibbles)],
    "e2m1_ties_away": [(method, "e2m1_encode_magnitude", _ties_away), (oracle, "e2m1_encode_magnitude", _ties_away)],
    "scale_wrong_divisor": [(method, "e4m3_scale_code_for_amax", _scale_div4),
                            (oracle, "e4m3_scale_code_for_amax", _scale_div4)],
    "e4m3_fnuz_bias": [(method, "e4m3_decode", _fnuz_decode), (oracle, "e4m3_decode", _fnuz_decode)],
    "indexer_without_relu": [(method, "index_scores", _no_relu), (oracle, "index_scores", _no_relu)],
    "topk_tie_id_descending": [(method, "topk", _topk_id_desc), (oracle, "topk", _topk_id_desc)],
    "attention_drops_rope": [(method, "sparse_attn", _attn_no_rope), (oracle, "sparse_attn", _attn_no_rope)],
    "attention_lse_base2": [(method, "sparse_attn", _attn_lse_log2), (oracle, "sparse_attn", _attn_lse_log2)],
    "pool_position_transposed": [(method, "index_pool", _pool_transposed), (oracle, "index_pool", _pool_transposed)],
    "pool_block_sum": [(method, "build_pool", _pool_block_sum), (oracle, "build_pool", _pool_block_sum)],
    "pool_higher_block_id_wins": [(method, "build_pool", _pool_high_id_first),
                                  (oracle, "build_pool", _pool_high_id_first)],
    "fp8_scale_one_binade_low": [(method, "fp8_row_scale_exponent", _fp8_scale_one_lower),
                                 (oracle, "fp8_row_scale_exponent", _fp8_scale_one_lower)],
    "window_drops_rope": [(method, "swa_attn", _swa_no_rope), (oracle, "swa_attn", _swa_no_rope)],
    "merge_weights_base2": [(method, "merge_branches", _merge_base2), (oracle, "merge_branches", _merge_base2)],
    "prefill_first_cache": [(method, "prefill_sparse_attn", _prefill_first_cache),
                            (oracle, "prefill_sparse_attn", _prefill_first_cache)],
    "prefill_lists_reversed": [(method, "prefill_sparse_attn", _prefill_query_order),
                               (oracle, "prefill_sparse_attn", _prefill_query_order)],
    "sample_temperature_multiplies": [(method, "sample", _sample_temperature_multiplies),
                                      (oracle, "sample", _sample_temperature_multiplies)],
    "sample_nucleus_strict": [(method, "sample", _sample_nucleus_strict), (oracle, "sample", _sample_nucleus_strict)],
    "sample_draw_exclusive": [(method, "sample", _sample_draw_exclusive), (oracle, "sample", _sample_draw_exclusive)],
    "sample_probs_over_vocab": [(method, "sample", _sample_probs_over_vocab),
                                (oracle, "sample", _sample_probs_over_vocab)],
    "sample_full_temperature_multiplies": [(method, "sample_full", _sample_full_temperature_multiplies),
                                           (oracle, "sample_full", _sample_full_temperature_multiplies)],
    "sample_full_logit_order": [(method, "sample_full", _sample_full_logit_order),
                                (oracle, "sample_full", _sample_full_logit_order)],
    "sample_full_boundary_inclusive": [(method, "sample_full", _sample_full_boundary_inclusive),
                                       (oracle, "sample_full", _sample_full_boundary_inclusive)],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    for mod, attr, fn in MUTATIONS[name]:
        monkeypatch.setattr(mod, attr, fn)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"


def test_sampler_plant_harness_is_faithful(monkeypatch):
    """The replaceable sampler above, unmutated, passes every pin (so each
    plant is caught for its planted step, not for the harness)."""
    monkeypatch.setattr(method, "sample", _sample_unmutated)
    monkeypatch.setattr(oracle, "sample", _sample_unmutated)
    monkeypatch.setattr(method, "sample_full", _sample_full_unmutated)
    monkeypatch.setattr(oracle, "sample_full", _sample_full_unmutated)
    for pin in P.ALL_PINS:
        if "sample" in pin.__name__:
            pin()
