"""Sliding-window branch on the GPU against the oracle: csa2_quantize_fp8
bit-exact (codes and power-of-two row scales) over every finite bf16 value,
outliers, zero rows and -0; csa2_swa_attn_fp8 alone and merged with the
sparse branch (one softmax over the union) within 2e-3, over ragged windows
(empty, partial and full tiles, 256 rows), head counts with a partial head
group, with and without the RoPE part."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, W, attn_close, csa2, note, np_bits, oracle

pytestmark = pytest.mark.gpu


def _finite_bf16_rows(C=512):
    pats = np.arange(65536, dtype=np.uint32)
    exp = (pats >> 7) & 0xFF
    pats = pats[exp != 0xFF].astype(np.uint16)          # no inf / NaN
    rng = np.random.default_rng(51)
    pats = rng.permutation(pats)
    pad = (-pats.size) % C
    pats = np.concatenate([pats, np.zeros(pad, dtype=np.uint16)])
    return pats.reshape(-1, C)


def _rows_from_bits(bits):
    return torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(DEV)


def test_quantize_fp8_every_finite_bf16():
    note("fp8: every finite bf16 value, shuffled into rows of 512")
    bits = _finite_bf16_rows()
    x = _rows_from_bits(bits)
    R = bits.shape[0]
    codes = torch.zeros(R, 512, dtype=torch.uint8, device=DEV)
    sigma = torch.zeros(R, dtype=torch.float32, device=DEV)
    csa2.csa2_quantize_fp8(x, codes, sigma)
    torch.cuda.synchronize()
    wc, ws = oracle.quantize_fp8(bits)
    assert np.array_equal(sigma.cpu().numpy().astype(np.float64), ws)
    assert np.array_equal(codes.cpu().numpy(), wc)


@pytest.mark.parametrize("d_r", [64, 0])
def test_quantize_fp8_workload_rows_at_offset(d_r):
    note(f"fp8: N(0,1) rows with outliers, zero and -0 rows, row offset, d_r={d_r}")
    rng = np.random.default_rng(52 + d_r)
    R, cap, r0 = 300, 400, 77
    xf = rng.standard_normal((R, 512)).astype(np.float32)
    xf[rng.random((R, 512)) < 0.01] *= 20.0
    xf[::9] *= np.float32(2.0) ** rng.integers(-60, 60, size=(len(xf[::9]), 1)).astype(np.float32)
    xf[5] = 0.0
    xf[6] = -0.0
    x = torch.from_numpy(xf).to(torch.bfloat16).to(DEV)
    rope_src = torch.randn(R, d_r, device=DEV).to(torch.bfloat16) if d_r else None
    codes = torch.zeros(cap, 512, dtype=torch.uint8, device=DEV)
    sigma = torch.zeros(cap, dtype=torch.float32, device=DEV)
    rope = torch.zeros(cap, d_r, dtype=torch.bfloat16, device=DEV) if d_r else None
    csa2.csa2_quantize_fp8(x, codes, sigma, r0, rope_src, rope)
    torch.cuda.synchronize()
    wc, ws = oracle.quantize_fp8(np_bits(x))
    assert np.array_equal(codes[r0:r0 + R].cpu().numpy(), wc)
    assert np.array_equal(sigma[r0:r0 + R].cpu().numpy().astype(np.float64), ws)
    assert int(codes[:r0].count_nonzero()) == 0 and int(codes[r0 + R:].count_nonzero()) == 0
    if d_r:
        assert torch.equal(rope[r0:r0 + R], rope_src)


def _window(B, W_cap, d_r, seed, raw=False):
    rng = np.random.default_rng(seed)
    if raw:
        c = rng.integers(0, 256, size=(B, W_cap, 512)).astype(np.uint8)
        c[(c & 0x7F) == 0x7F] = 0x31
        codes = torch.from_numpy(c).to(DEV)
        sigma = torch.from_numpy((2.0 ** rng.integers(-12, -4, size=(B, W_cap))).astype(np.float32)).to(DEV)
    else:
        x = torch.from_numpy(rng.standard_normal((B * W_cap, 512)).astype(np.float32)).to(torch.bfloat16).to(DEV)
        codes = torch.zeros(B * W_cap, 512, dtype=torch.uint8, device=DEV)
        sigma = torch.zeros(B * W_cap, dtype=torch.float32, device=DEV)
        csa2.csa2_quantize_fp8(x, codes, sigma)
        codes, sigma = codes.view(B, W_cap, 512), sigma.view(B, W_cap)
    rope = torch.from_numpy(rng.standard_normal((B, W_cap, d_r)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    return codes, sigma, rope


@pytest.mark.parametrize("H,d_r,W_cap,raw", [(64, 64, 128, False), (16, 64, 256, True), (40, 0, 200, False),
                                             (8, 64, 64, True)])
def test_window_attention_matches_oracle(H, d_r, W_cap, raw):
    B = 6
    note(f"swa: B={B} H={H} d_r={d_r} W_cap={W_cap} raw={raw}")
    codes, sigma, rope = _window(B, W_cap, d_r, H + W_cap, raw)
    nw = np.array([W_cap, 0, 1, 63, 65, min(W_cap, 129)], dtype=np.int32)
    q = W.attn_query(W.WORKLOADS[3].scaled(B=B, H=H, d_r=d_r), DEV)
    sm = 1.0 / np.sqrt(512 + d_r)
    out, lse = csa2.csa2_swa_attn_fp8(q, codes, sigma, rope, sm, n_win=torch.from_numpy(nw).to(DEV))
    torch.cuda.synchronize()
    ro, rl = oracle.swa_attn(np_bits(q), codes.cpu().numpy(), sigma.cpu().numpy().astype(np.float64),
                             np_bits(rope.contiguous()), nw, sm)
    attn_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl)
    assert np.all(out[1].cpu().numpy() == 0) and np.all(np.isneginf(lse[1].cpu().numpy()))


@pytest.mark.parametrize("H,d_r", [(64, 64), (48, 0)])
def test_window_merged_with_sparse_branch(H, d_r):
    """Sparse branch (FP4 entries picked by an index list) then the window
    branch merged in place: one softmax over the union of both key sets."""
    B, N, K, W_cap = 5, 2048, 512, 128
    note(f"swa+sparse merge: B={B} H={H} d_r={d_r}")
    wl = W.WORKLOADS[3].scaled(B=B, N=N, H=H, d_r=d_r)
    ccodes, cscales, crope = csa2.alloc_cache(B, N, 512, d_r, DEV)
    for b in range(B):
        c, s = W.random_codes(wl, b, N, DEV)
        ccodes[b].copy_(c)
        cscales[b].copy_(s)
        if d_r:
            crope[b].copy_(W.rope_rows(wl, b, N, DEV))
    rng = np.random.default_rng(60 + H)
    idx = np.stack([np.sort(rng.permutation(N)[:K]) for _ in range(B)]).astype(np.int32)
    idx[1, :] = -1                                  # no sparse entry: the window alone
    q = W.attn_query(wl, DEV)
    sm = wl.sm_scale
    o_s, l_s = csa2.csa2_sparse_attn_fp4(q, ccodes, cscales, crope, torch.from_numpy(idx).to(DEV), sm)
    codes, sigma, rope = _window(B, W_cap, d_r, 70 + H)
    nw = np.array([128, 100, 0, 1, 64], dtype=np.int32)  # row 2: no window, the sparse result unchanged
    o_keep = o_s.clone()
    l_keep = l_s.clone()
    out, lse = csa2.csa2_swa_attn_fp8(q, codes, sigma, rope, sm, n_win=torch.from_numpy(nw).to(DEV),
                                      merge_out=o_s, merge_lse=l_s, out=o_s)
    torch.cuda.synchronize()
    ro1, rl1 = oracle.sparse_attn(np_bits(q), ccodes.cpu().numpy(), cscales.cpu().numpy(),
                                  np_bits(crope.contiguous()), idx, sm)
    ro2, rl2 = oracle.swa_attn(np_bits(q), codes.cpu().numpy(), sigma.cpu().numpy().astype(np.float64),
                               np_bits(rope.contiguous()), nw, sm)
    ro, rl = oracle.merge_branches(ro1, rl1, ro2, rl2)
    attn_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl)
    assert torch.equal(out[2], o_keep[2]) and torch.equal(lse[2], l_keep[2])


def test_window_of_zero_rows_and_full_windows_without_n_win():
    """W_cap = 0 (no window buffers at all): the merge returns the sparse
    result bit for bit; n_win omitted: every row of the window is used."""
    B, H = 3, 64
    note("swa: W_cap = 0 with merge; n_win omitted")
    q = W.attn_query(W.WORKLOADS[3].scaled(B=B, H=H), DEV)
    mo = torch.randn(B, H, 512, device=DEV)
    ml = torch.randn(B, H, device=DEV)
    empty = torch.empty(B, 0, 512, dtype=torch.uint8, device=DEV)
    out, lse = csa2.csa2_swa_attn_fp8(q, empty, torch.empty(B, 0, device=DEV),
                                      torch.empty(B, 0, 64, dtype=torch.bfloat16, device=DEV), 1 / 24,
                                      merge_out=mo, merge_lse=ml)
    torch.cuda.synchronize()
    assert torch.equal(out, mo) and torch.equal(lse, ml)
    codes, sigma, rope = _window(B, 96, 64, 81)
    out2, lse2 = csa2.csa2_swa_attn_fp8(q, codes, sigma, rope, 1 / 24)
    torch.cuda.synchronize()
    ro, rl = oracle.swa_attn(np_bits(q), codes.cpu().numpy(), sigma.cpu().numpy().astype(np.float64),
                             np_bits(rope.contiguous()), None, 1 / 24)
    attn_close(out2.cpu().numpy(), lse2.cpu().numpy(), ro, rl)
