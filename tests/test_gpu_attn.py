"""a4 + a5 csa2_sparse_attn_fp4 on the GPU against the oracle (normwise 2e-3
per (b, h) row, lse to 1e-3), over raw random caches and edge-case index lists."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, W, attn_close, csa2, note, np_bits, oracle

pytestmark = pytest.mark.gpu


def _raw_cache(wl, B, N, layout="record"):
    codes, scales, rope = csa2.alloc_cache(B, N, wl.d_c, wl.d_r, DEV, layout)
    for b in range(B):
        c, s = W.random_codes(wl, b, N, DEV)
        codes[b].copy_(c)
        scales[b].copy_(s)
        if wl.d_r:
            rope[b].copy_(W.rope_rows(wl, b, N, DEV))
    return codes, scales, rope


def _check(wl, B, N, idx, q=None, tol=2e-3, layout="record"):
    codes, scales, rope = _raw_cache(wl, B, N, layout)
    if q is None:
        q = W.attn_query(wl.scaled(B=B), DEV)
    idx_t = torch.from_numpy(np.asarray(idx, dtype=np.int32)).to(DEV)
    out, lse = csa2.csa2_sparse_attn_fp4(q, codes, scales, rope, idx_t, wl.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attn(np_bits(q), codes.cpu().numpy(), scales.cpu().numpy(),
                                np_bits(rope.contiguous()), np.asarray(idx), wl.sm_scale)
    return attn_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol)


def _rand_idx(rng, B, K, N):
    return np.stack([np.sort(rng.permutation(N)[:K]) for _ in range(B)])


@pytest.mark.parametrize("wi,B,N", [(0, 1, 1024), (1, 1, 16384), (1, 3, 4096), (3, 40, 2048), (3, 130, 1024)])
def test_attention_workload_shapes(wi, B, N):
    wl = W.WORKLOADS[wi]
    note(f"attn: {wl.name} B={B} N={N} K={wl.K} H={wl.H} d_c={wl.d_c} d_r={wl.d_r}")
    rng = np.random.default_rng(B + N)
    _check(wl, B, N, _rand_idx(rng, B, wl.K, N))


@pytest.mark.parametrize("B,K", [(300, 512), (300, 130), (260, 65), (520, 200)])
def test_attention_persistent_many_units(B, K):
    """More (query, 32-head) units than CUs with unsplit queries: the
    persistent 32-head kernel, each workgroup walking two or three units of
    8, 3, 2 or 4 tiles, each query over its own sequence; batches padded to
    a multiple of eight (300, 260); masked, repeated and empty lists."""
    wl = W.WORKLOADS[3]
    note(f"attn: persistent B={B} K={K} H={wl.H}")
    rng = np.random.default_rng(700 + B + K)
    N = 1024
    idx = _rand_idx(rng, B, K, N)
    idx[0, ::5] = -1
    idx[1, :] = idx[1, 0]
    idx[2, :] = -1
    idx[B - 1, K // 2:] = N + 7
    _check(wl, B, N, idx)


@pytest.mark.parametrize("B", [5, 9, 24, 32, 48, 96])
def test_attention_batch_sizes_and_slices(B):
    """64 heads, K = 512 at batch sizes that take different plans: the 16-head
    kernel with its slices spread over the XCDs (5), four and two slices per
    query (9, 24), the 32-head kernel with four and two slices merged by the
    combine (32, 48), and unsplit on fewer workgroups than CUs (96)."""
    wl = W.WORKLOADS[3]
    note(f"attn: B={B} H={wl.H} K={wl.K} slices per the plan")
    rng = np.random.default_rng(500 + B)
    N = 2048
    idx = _rand_idx(rng, B, wl.K, N)
    idx[0, ::9] = -1
    _check(wl, B, N, idx)


@pytest.mark.parametrize("K", [1, 5, 63, 64, 65, 200, 1000])
def test_attention_ragged_k(K):
    wl = W.WORKLOADS[1]
    note(f"attn: ragged K={K}")
    rng = np.random.default_rng(K)
    _check(wl, 2, 2048, _rand_idx(rng, 2, K, 2048))


def test_attention_masked_duplicate_and_empty_rows():
    wl = W.WORKLOADS[1]
    note("attn: masked ids, duplicates, empty rows")
    rng = np.random.default_rng(5)
    N = 1024
    idx = _rand_idx(rng, 4, 512, N)
    idx[0, ::7] = -1
    idx[1, ::5] = N + 3            # past the cache: skipped
    idx[2, 100:300] = idx[2, 0]    # repeated entry
    idx[3, :] = -1                 # nothing valid
    _check(wl, 4, N, idx)


@pytest.mark.parametrize("H", [1, 8, 17, 64, 128])
def test_attention_head_counts(H):
    wl = W.WORKLOADS[1].scaled(H=H)
    note(f"attn: H={H}")
    rng = np.random.default_rng(H)
    _check(wl, 2, 1024, _rand_idx(rng, 2, 512, 1024))


@pytest.mark.parametrize("dc,dr", [(512, 0), (128, 64)])
def test_attention_other_dims(dc, dr):
    wl = W.WORKLOADS[1].scaled(d_c=dc, d_r=dr)
    note(f"attn: d_c={dc} d_r={dr}")
    rng = np.random.default_rng(dc + dr)
    _check(wl, 2, 1024, _rand_idx(rng, 2, 512, 1024))


@pytest.mark.parametrize("wi", [0, 1])
def test_attention_separate_array_layout(wi):
    wl = W.WORKLOADS[wi]
    note(f"attn: {wl.name} with codes / scales / RoPE in three dense arrays")
    rng = np.random.default_rng(77)
    _check(wl, 3, 2048, _rand_idx(rng, 3, wl.K, 2048), layout="separate")


def test_attention_query_magnitudes():
    wl = W.WORKLOADS[1].scaled(H=16)
    note("attn: zero / huge / tiny query heads")
    rng = np.random.default_rng(9)
    q = W.attn_query(wl.scaled(B=1), DEV).float()
    q[0, 0] = 0
    q[0, 1] *= 3000.0
    q[0, 2] *= 1e-30
    q[0, 3, :512] = 0            # only the RoPE part
    q[0, 4, 512:] = 0            # only the latent part
    _check(wl, 1, 2048, _rand_idx(rng, 1, 512, 2048), q=q.to(torch.bfloat16))


def test_attention_on_quantized_cache_is_dense_attention_when_k_is_n():
    wl = W.WORKLOADS[0]
    note("attn: tiny cache built by csa2_quantize_fp4, Top-K = every entry")
    from gpu_util import Cache, oracle_attention_rows
    cache = Cache(wl)
    q = W.attn_query(wl, DEV)
    idx = torch.arange(wl.N, dtype=torch.int32, device=DEV)[None]
    out, lse = csa2.csa2_sparse_attn_fp4(q, cache.codes, cache.scales, cache.rope, idx, wl.sm_scale)
    ro, rl = oracle_attention_rows(cache, 0, np_bits(q)[0], idx.cpu().numpy()[0], wl.sm_scale)
    attn_close(out.cpu().numpy()[0], lse.cpu().numpy()[0], ro, rl)


@pytest.mark.parametrize("H,B", [(16, 2), (64, 130)])
def test_attention_every_e4m3_scale_byte(H, B):
    """Both kernels (16 heads per workgroup; 32 heads per workgroup at a
    batch that fills the GPU unsplit) over every non-NaN scale byte."""
    wl = W.WORKLOADS[1].scaled(H=H)
    note(f"attn: every non-NaN E4M3 scale byte (subnormal, negative, 448), H={H} B={B}")
    N = 1024
    codes, scales, rope = csa2.alloc_cache(B, N, wl.d_c, wl.d_r, DEV)
    for b in range(B):
        c, _ = W.random_codes(wl, b, N, DEV)
        codes[b].copy_(c)
        rope[b].copy_(W.rope_rows(wl, b, N, DEV))
    # scale bytes cycle through 0x00..0xFE, skipping the two NaN codes
    allb = torch.tensor([v for v in range(256) if v not in (0x7F, 0xFF)], dtype=torch.uint8)
    reps = (B * N * (wl.d_c // 16) + allb.numel() - 1) // allb.numel()
    sc = allb.repeat(reps)[: B * N * (wl.d_c // 16)].view(B, N, wl.d_c // 16)
    scales.copy_(sc.to(DEV))
    q = W.attn_query(wl.scaled(B=B), DEV)
    rng = np.random.default_rng(21)
    idx = _rand_idx(rng, B, 512, N)
    idx_t = torch.from_numpy(idx.astype(np.int32)).to(DEV)
    out, lse = csa2.csa2_sparse_attn_fp4(q, codes, scales, rope, idx_t, wl.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attn(np_bits(q), codes.cpu().numpy(), scales.cpu().numpy(),
                                np_bits(rope.contiguous()), idx, wl.sm_scale)
    attn_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl)


@pytest.mark.parametrize("H,dr,K", [(64, 64, 512), (64, 64, 200), (48, 64, 130), (64, 0, 512), (64, 64, 1000)])
def test_attention_32_heads_per_workgroup(H, dr, K):
    """Batches large enough for 32 heads per workgroup (score waves that
    dequantise each entry once for 32 heads, value waves on the previous
    tile): masked, out-of-range and repeated ids, an empty row, ragged K, a
    partial second head group, and K = 1000 (two slices merged by the combine)."""
    B = 260 if H == 48 else 130
    wl = W.WORKLOADS[3].scaled(H=H, d_r=dr)
    note(f"attn: 32 heads per workgroup B={B} H={H} d_r={dr} K={K}")
    rng = np.random.default_rng(H + dr + K)
    N = 1024
    idx = _rand_idx(rng, B, K, N)
    idx[0, ::7] = -1
    idx[1, ::5] = N + 3
    idx[2, K // 4:K // 2] = idx[2, 0]
    idx[3, :] = -1
    _check(wl, B, N, idx)
