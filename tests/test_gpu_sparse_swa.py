"""The sparse branch and the sliding window in one call (csa2_sparse_swa_attn_fp4)
on the GPU against the oracle: sparse_attn and swa_attn merged by
merge_branches, one softmax over the union of both key sets, within 2e-3.
Batches of 32+ queries at 64 heads run the window tiles inside the 32-head
kernel; smaller batches run the two kernels and merge; both are checked, over
ragged windows, empty windows, empty index lists, extreme row scales and
split queries (K > 512)."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, W, attn_close, csa2, note, np_bits, oracle

pytestmark = pytest.mark.gpu


def _cache(wl, B, N, d_r):
    codes, scales, rope = csa2.alloc_cache(B, N, 512, d_r, DEV)
    for b in range(B):
        c, s = W.random_codes(wl, b, N, DEV)
        codes[b].copy_(c)
        scales[b].copy_(s)
        if d_r:
            rope[b].copy_(W.rope_rows(wl, b, N, DEV))
    return codes, scales, rope


def _window(B, W_cap, d_r, seed, sigma_exp=(-12, -4)):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 256, size=(B, W_cap, 512)).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x31                  # E4M3 has no 0x7F / 0xFF values
    sig = (2.0 ** rng.integers(sigma_exp[0], sigma_exp[1], size=(B, W_cap))).astype(np.float32)
    rope = rng.standard_normal((B, W_cap, max(d_r, 1)))[:, :, :d_r].astype(np.float32)
    return (torch.from_numpy(c).to(DEV), torch.from_numpy(sig).to(DEV),
            torch.from_numpy(np.ascontiguousarray(rope)).to(torch.bfloat16).to(DEV))


def _reference(q, codes, scales, rope, idx, wc, ws, wr, nw, sm, rows):
    qb = np_bits(q)[rows]
    ro1, rl1 = oracle.sparse_attn(qb, codes.cpu().numpy()[rows], scales.cpu().numpy()[rows],
                                  np_bits(rope.contiguous())[rows], idx[rows], sm)
    ro2, rl2 = oracle.swa_attn(qb, wc.cpu().numpy()[rows], ws.cpu().numpy().astype(np.float64)[rows],
                               np_bits(wr.contiguous())[rows], None if nw is None else nw[rows], sm)
    return oracle.merge_branches(ro1, rl1, ro2, rl2)


def _run_case(B, H, d_r, N, K, W_cap, seed, sigma_exp=(-12, -4), check_rows=None, sm_mult=1.0):
    wl = W.WORKLOADS[3].scaled(B=B, N=N, H=H, d_r=d_r)
    codes, scales, rope = _cache(wl, B, N, d_r)
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.integers(-3, N + 3, size=K) for _ in range(B)]).astype(np.int32)
    idx[1, :] = -1                                  # no selected entry: the window alone
    nw = rng.integers(0, W_cap + 1, size=B).astype(np.int32)
    nw[0], nw[2] = W_cap, 0                         # row 2: the sparse branch alone
    if B > 3:
        nw[3] = 1
    if B > 5:
        nw[4], nw[5] = min(64, W_cap), min(65, W_cap)
    wc, ws, wr = _window(B, W_cap, d_r, seed + 1, sigma_exp)
    q = W.attn_query(wl, DEV)
    sm = wl.sm_scale * sm_mult
    idx_t = torch.from_numpy(idx).to(DEV)
    nw_t = torch.from_numpy(nw).to(DEV)
    out, lse = csa2.csa2_sparse_swa_attn_fp4(q, codes, scales, rope, idx_t, wc, ws, wr, sm, n_win=nw_t)
    # the two-call path: sparse attention, then the window merged into it
    o2, l2 = csa2.csa2_sparse_attn_fp4(q, codes, scales, rope, idx_t, sm)
    o2, l2 = csa2.csa2_swa_attn_fp8(q, wc, ws, wr, sm, n_win=nw_t, merge_out=o2, merge_lse=l2, out=o2)
    torch.cuda.synchronize()
    rows = np.arange(B) if check_rows is None else np.asarray(check_rows)
    ro, rl = _reference(q, codes, scales, rope, idx, wc, ws, wr, nw, sm, rows)
    attn_close(out.cpu().numpy()[rows], lse.cpu().numpy()[rows], ro, rl)
    attn_close(o2.cpu().numpy()[rows], l2.cpu().numpy()[rows], ro, rl)
    return out, lse


@pytest.mark.parametrize("d_r", [64, 0])
def test_fused_window_tiles_large_batch(d_r):
    """128 queries x 64 heads (the 32-head kernel with the window tiles),
    windows of 0 .. 128 rows."""
    note(f"sparse+swa fused: B=128 H=64 d_r={d_r} K=512 W_cap=128")
    _run_case(128, 64, d_r, 2048, 512, 128, 11 + d_r, check_rows=list(range(8)) + [37, 64, 101, 127])


def test_fused_window_full_256_rows_and_split_queries():
    """W_cap = 256 (four window tiles) and K = 1000 (each query split in two
    slices, the window in the first)."""
    note("sparse+swa fused: B=128 H=64 K=1000 W_cap=256")
    _run_case(128, 64, 64, 4096, 1000, 256, 23, check_rows=[0, 1, 2, 3, 4, 5, 77, 127])


@pytest.mark.parametrize("lo,hi,sm_mult", [(-40, -30, 1.0), (20, 30, 2.0 ** -25)])
def test_fused_window_extreme_row_scales(lo, hi, sm_mult):
    """Row scales far from 1 (2^-40 .. 2^30): the accumulator's division by
    the largest one and the epilogue's multiplication stay exact.  With the
    large scales the softmax scale shrinks by 2^-25 so that the logits stay
    moderate (logits of 10^11 would put fp32 rounding of the scores, not the
    kernel, above the lse bound)."""
    note(f"sparse+swa fused: row scales 2^{lo} .. 2^{hi}")
    _run_case(128, 64, 64, 2048, 512, 128, 31 + abs(lo), sigma_exp=(lo, hi), check_rows=[0, 1, 2, 3, 9, 127],
              sm_mult=sm_mult)


def test_fused_window_four_slices_per_query():
    """32 queries x 64 heads: the 32-head kernel with each query in four
    slices, the window tiles in the first, merged by the split combine."""
    note("sparse+swa fused: B=32 H=64 K=512 W_cap=128 (four slices)")
    _run_case(32, 64, 64, 2048, 512, 128, 17, check_rows=[0, 1, 2, 3, 4, 5, 17, 31])


@pytest.mark.parametrize("B,H", [(8, 64), (3, 40), (20, 40)])
def test_small_batches_run_the_two_kernels(B, H):
    """Batches the 32-head kernel does not serve (and a partial head group):
    sparse kernels, then the window kernel merging into their result."""
    note(f"sparse+swa: B={B} H={H}")
    _run_case(B, H, 64, 1024, 300, 128, 41 + B, check_rows=list(range(min(B, 8))))


def test_empty_window_is_the_sparse_attention():
    """W_cap = 0: the result is that of csa2_sparse_attn_fp4, bit for bit."""
    B, H, N, K = 128, 64, 1024, 512
    note("sparse+swa: W_cap = 0")
    wl = W.WORKLOADS[3].scaled(B=B, N=N, H=H)
    codes, scales, rope = _cache(wl, B, N, 64)
    idx = torch.from_numpy(np.random.default_rng(5).integers(0, N, size=(B, K)).astype(np.int32)).to(DEV)
    q = W.attn_query(wl, DEV)
    e = torch.empty(B, 0, 512, dtype=torch.uint8, device=DEV)
    out, lse = csa2.csa2_sparse_swa_attn_fp4(q, codes, scales, rope, idx, e, torch.empty(B, 0, device=DEV),
                                             torch.empty(B, 0, 64, dtype=torch.bfloat16, device=DEV), wl.sm_scale)
    o2, l2 = csa2.csa2_sparse_attn_fp4(q, codes, scales, rope, idx, wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)
