"""The C-ABI library loads and exports every declared symbol; host-side
argument validation returns its status before anything reaches the GPU
(these calls never launch, so they run without one)."""

import ctypes
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from sparse_attention_decode_csa2_amd import csa2  # noqa: E402

OK, NULL, SHAPE, ALIGN, RANGE, UNSUP, HIP, WS = range(8)
A = ctypes.c_void_p(0x1000)      # 16-byte aligned fake device address (never dereferenced)
U = ctypes.c_void_p(0x1004)      # misaligned
N = None


@pytest.fixture(scope="module")
def lib():
    return csa2.load()


def test_every_declared_symbol_is_exported(lib):
    names = csa2.declared_functions()
    assert len(names) == 25
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(8):
        assert csa2.status_string(s)
    assert csa2.status_string(99) == "unknown status"
    assert lib.csa2_version() >= 100


def test_quantize_validation(lib):
    f = lib.csa2_quantize_fp4

    def call(x=A, n=4, d_c=512, rs=N, d_r=0, codes=A, cst=0, scales=A, sst=0, rd=N, rst=0, r0=0, cap=10):
        return f(x, n, d_c, rs, d_r, codes, cst, scales, sst, rd, rst, r0, cap, N)
    assert call(n=-1) == SHAPE
    assert call(d_c=500) == SHAPE
    assert call(d_r=12) == SHAPE
    assert call(cst=-16) == SHAPE
    assert call(r0=8) == RANGE
    assert call(r0=-1) == RANGE
    assert call(n=0, r0=10) == OK                    # empty append at the end: no-op
    assert call(x=N) == NULL
    assert call(d_r=64) == NULL                      # RoPE part without its buffers
    assert call(x=U) == ALIGN
    assert call(cst=520) == ALIGN                    # codes stride not a multiple of 16
    assert call(scales=ctypes.c_void_p(0x1005)) == ALIGN
    assert call(sst=33) == ALIGN                     # odd scales stride
    assert call(cst=128) == SHAPE                    # stride narrower than a row
    assert call(d_r=64, rs=A, rd=ctypes.c_void_p(0x1008), rst=512) == ALIGN


def test_index_validation(lib):
    f = lib.csa2_index_full
    assert f(A, N, A, N, 0, 8, 128, 100, A, N) == OK          # B == 0: nothing to do
    assert f(A, N, A, N, 1, 8, 128, 0, A, N) == OK            # empty cache
    assert f(A, N, A, N, -1, 8, 128, 100, A, N) == SHAPE
    assert f(A, N, A, N, 1, 17, 128, 100, A, N) == UNSUP
    assert f(A, N, A, N, 1, 8, 96, 100, A, N) == UNSUP
    assert f(N, N, A, N, 1, 8, 128, 100, A, N) == NULL
    assert f(A, U, A, N, 1, 8, 128, 100, A, N) == ALIGN
    g = lib.csa2_index_pool
    assert g(A, N, A, N, A, A, 1, 8, 128, 100, 0, 8, A, A, N) == SHAPE
    assert g(A, N, A, N, A, A, 1, 8, 128, 100, 2048, 0, A, A, N) == RANGE
    assert g(A, N, A, N, A, A, 1, 8, 128, 100, 2048, 65, A, A, N) == RANGE
    assert g(A, N, A, N, N, A, 1, 8, 128, 100, 2048, 8, A, A, N) == NULL
    assert g(A, N, A, N, A, A, 1, 8, 128, 100, 2048, 8, A, N, N) == NULL


def test_topk_validation(lib):
    f = lib.csa2_topk
    assert f(A, N, N, 1, 100, 0, A, N, N, 0, N) == RANGE
    assert f(A, N, N, 1, 100, 2049, A, N, N, 0, N) == RANGE
    assert f(A, N, N, 1, 0, 8, A, N, N, 0, N) == SHAPE
    assert f(A, N, N, -1, 100, 8, A, N, N, 0, N) == SHAPE
    assert f(A, N, N, 0, 100, 8, A, N, N, 0, N) == OK
    assert f(N, N, N, 1, 100, 8, A, N, N, 0, N) == NULL
    assert f(A, U, N, 1, 100, 8, A, N, N, 0, N) == ALIGN
    need = lib.csa2_topk_workspace_bytes(2, 40000, 512)
    assert need == 2 * 3 * 512 * 8
    assert lib.csa2_topk_workspace_bytes(2, 16384, 512) == 0
    # the threshold filter (128 bytes + 16384 keys per row): K >= 64 and
    # more than 768 first-level chunks, or more than two levels, in rows of at
    # most 2^20
    assert lib.csa2_topk_workspace_bytes(128, 129280, 512) == 128 * (128 + 16384 * 8)
    assert lib.csa2_topk_workspace_bytes(128, 129280, 64) == 128 * (128 + 16384 * 8)
    assert lib.csa2_topk_workspace_bytes(128, 129280, 32) == 128 * 8 * 32 * 8
    assert lib.csa2_topk_workspace_bytes(1, 2 ** 20, 512) == 128 + 16384 * 8
    assert lib.csa2_topk_workspace_bytes(1, 2 ** 20, 256) == 64 * 256 * 8
    assert lib.csa2_topk_workspace_bytes(128, 129280, 2048) == 128 * (128 + 16384 * 8)
    assert lib.csa2_topk_workspace_bytes(1, 300000, 2048) == 128 + 16384 * 8
    assert lib.csa2_topk_workspace_bytes(1, 300000, 512) == 19 * 512 * 8
    assert lib.csa2_topk_workspace_bytes(32, 32768, 2048) == 32 * 2 * 2048 * 8
    assert lib.csa2_topk_workspace_bytes(1, 2 ** 20 + 1, 8) == 65 * 8 * 8
    assert f(A, N, N, 2, 40000, 512, A, N, N, 0, N) == WS
    assert f(A, N, N, 2, 40000, 512, A, N, A, need - 1, N) == WS


def test_index_topk_validation(lib):
    f = lib.csa2_index_topk_full
    wsb = lib.csa2_index_topk_full_workspace_bytes
    # fused (8 x 32 chunks of 8192): the chunk winners, one later level
    assert wsb(8, 128, 262144, 512) == 8 * 32 * 512 * 8
    # fused, one row of 256 chunks: winners + the middle level's 8 chunks
    assert wsb(1, 128, 1 << 21, 512) == 256 * 512 * 8 + 8 * 512 * 8
    # too few chunks (or D_I 256): the scores, then the Top-K's workspace
    assert wsb(1, 128, 16384, 512) == 16384 * 4
    assert wsb(8, 256, 262144, 512) == 8 * 262144 * 4 + 8 * 16 * 512 * 8
    assert wsb(1, 128, 5, 4) == 32                   # scores rounded up to 16 bytes
    assert wsb(0, 128, 100, 8) == 0 and wsb(1, 96, 100, 8) == 0 and wsb(1, 128, 100, 0) == 0
    need = wsb(1, 128, 100, 8)

    def call(q=A, k=A, B=1, H_I=8, D_I=128, N_cap=100, K=8, out=A, score=N, ws=A, wsn=need, w=N, nv=N):
        return f(q, w, k, nv, B, H_I, D_I, N_cap, K, out, score, ws, wsn, N)
    assert call(B=0) == OK
    assert call(B=-1) == SHAPE
    assert call(N_cap=0) == SHAPE
    assert call(N_cap=1 << 31) == SHAPE
    assert call(K=0) == RANGE and call(K=2049) == RANGE
    assert call(H_I=17) == UNSUP and call(D_I=96) == UNSUP
    assert call(q=N) == NULL and call(k=N) == NULL and call(out=N) == NULL
    assert call(out=U) == ALIGN and call(w=U) == ALIGN and call(nv=U) == ALIGN and call(score=U) == ALIGN
    assert call(ws=N) == WS and call(wsn=need - 1) == WS
    assert call(ws=U) == ALIGN


def test_index_topk_full_append_validation(lib):
    """The fused call validates the scoring's operands as csa2_index_topk_full
    and the append's as csa2_quantize_fp4; an empty side is skipped."""
    f = lib.csa2_index_topk_full_append
    need = lib.csa2_index_topk_full_workspace_bytes(1, 128, 100, 8)

    def call(q=A, k=A, B=1, N_cap=100, K=8, out=A, ws=A, wsn=need, x=A, n=4, d_c=512, rs=N, d_r=0, codes=A,
             cst=0, scales=A, sst=0, rd=N, rst=0, r0=0, cap=10):
        return f(q, N, k, N, B, 8, 128, N_cap, K, out, N, ws, wsn, x, n, d_c, rs, d_r, codes, cst, scales, sst,
                 rd, rst, r0, cap, N)
    # the scoring's checks
    assert call(B=-1) == SHAPE and call(K=0) == RANGE and call(q=N) == NULL
    assert call(out=U) == ALIGN and call(ws=N) == WS and call(wsn=need - 1) == WS
    # the append's checks
    assert call(n=-1) == SHAPE and call(d_c=500) == SHAPE and call(r0=8) == RANGE
    assert call(x=N) == NULL and call(codes=N) == NULL and call(x=U) == ALIGN
    assert call(d_r=64, rs=A, rd=N) == NULL
    # either side empty: only the other is checked; both empty: nothing to do
    assert call(B=0, q=N, out=N, ws=N, x=N, n=0, r0=10) == OK
    assert call(B=0, q=N, out=N, ws=N, x=U) == ALIGN
    assert call(n=0, r0=10, x=N, codes=N, scales=N, q=N) == NULL



def test_sparse_swa_validation(lib):
    f = lib.csa2_sparse_swa_attn_fp4
    wsb = lib.csa2_sparse_swa_attn_workspace_bytes
    # 32-head kernel (B * ceil(H / 32) >= 256): only its split workspace; smaller
    # batches: the sparse kernels' workspace, then B x H floats of lse for the merge
    assert wsb(128, 64, 512, 512) == lib.csa2_sparse_attn_workspace_bytes(128, 64, 512, 512) == 0
    s8 = lib.csa2_sparse_attn_workspace_bytes(8, 64, 512, 512)
    assert wsb(8, 64, 512, 512) == ((s8 + 15) // 16) * 16 + 8 * 64 * 4
    assert wsb(8, 64, 128, 512) == 0 and wsb(0, 64, 512, 512) == 0
    need = wsb(8, 64, 512, 512)

    def call(q=A, codes=A, cst=0, scales=A, sst=0, rope=A, rst=0, idx=A, K=512, B=8, H=64, d_c=512, d_r=64,
             N=1000, wc=A, wcs=0, ws=A, wr=A, wrs=0, nw=N, W=128, out=A, lse=N, wsp=A, wsn=need):
        return f(q, codes, cst, scales, sst, rope, rst, idx, K, B, H, d_c, d_r, N, wc, wcs, ws, wr, wrs, nw, W,
                 0.05, out, lse, wsp, wsn, N)
    assert call(B=0) == OK
    assert call(B=-1) == SHAPE and call(K=0) == SHAPE and call(W=-1) == SHAPE and call(wcs=-16) == SHAPE
    assert call(d_c=128) == UNSUP and call(d_r=32) == UNSUP and call(H=129) == UNSUP
    assert call(W=257) == RANGE
    assert call(q=N) == NULL and call(wc=N) == NULL and call(ws=N) == NULL and call(wr=N) == NULL
    assert call(W=0, wc=N, ws=N, wr=N, K=0) == SHAPE          # no window: its buffers may be NULL
    assert call(wcs=256) == SHAPE                             # window stride narrower than a row
    assert call(wc=U) == ALIGN and call(wcs=520) == ALIGN and call(ws=ctypes.c_void_p(0x1002)) == ALIGN
    assert call(wr=U) == ALIGN and call(nw=U) == ALIGN and call(lse=U) == ALIGN
    assert call(wsp=N) == WS and call(wsn=need - 1) == WS


def test_build_pool_validation(lib):
    f = lib.csa2_build_pool
    need = lib.csa2_build_pool_workspace_bytes(2, 262144, 8, 2048)
    # block scores (2 x 32768 f32) + counts (16 B) + two-level Top-K winners (2 x 2 x 2048 u64)
    assert need == 2 * 32768 * 4 + 16 + 2 * 2 * 2048 * 8
    assert lib.csa2_build_pool_workspace_bytes(2, 262144, 0, 2048) == 0
    assert f(A, N, 2, 262144, 0, 2048, A, A, A, need, N) == RANGE
    assert f(A, N, 2, 262144, 65, 2048, A, A, A, need, N) == RANGE
    assert f(A, N, 2, 262144, 8, 2049, A, A, A, need, N) == RANGE
    assert f(A, N, 2, 0, 8, 2048, A, A, A, need, N) == SHAPE
    assert f(A, N, -1, 262144, 8, 2048, A, A, A, need, N) == SHAPE
    assert f(A, N, 0, 262144, 8, 2048, A, A, A, need, N) == OK
    assert f(N, N, 2, 262144, 8, 2048, A, A, A, need, N) == NULL
    assert f(A, N, 2, 262144, 8, 2048, N, A, A, need, N) == NULL
    assert f(A, N, 2, 262144, 8, 2048, A, A, N, need, N) == NULL
    assert f(U, N, 2, 262144, 8, 2048, A, A, A, need, N) == ALIGN
    assert f(A, U, 2, 262144, 8, 2048, A, A, A, need, N) == ALIGN
    assert f(A, N, 2, 262144, 8, 2048, A, A, A, need - 1, N) == WS


def test_window_validation(lib):
    q8 = lib.csa2_quantize_fp8
    assert q8(A, -1, 512, N, 0, A, 0, A, N, 0, 0, 10, N) == SHAPE
    assert q8(A, 4, 500, N, 0, A, 0, A, N, 0, 0, 10, N) == SHAPE
    assert q8(A, 4, 512, N, 0, A, 0, A, N, 0, 8, 10, N) == RANGE
    assert q8(A, 0, 512, N, 0, A, 0, A, N, 0, 10, 10, N) == OK
    assert q8(N, 4, 512, N, 0, A, 0, A, N, 0, 0, 10, N) == NULL
    assert q8(A, 4, 512, N, 64, A, 0, A, N, 0, 0, 10, N) == NULL
    assert q8(U, 4, 512, N, 0, A, 0, A, N, 0, 0, 10, N) == ALIGN
    assert q8(A, 4, 512, N, 0, A, 516, A, N, 0, 0, 10, N) == ALIGN
    assert q8(A, 4, 512, N, 0, A, 256, A, N, 0, 0, 10, N) == SHAPE
    sw = lib.csa2_swa_attn_fp8
    sm = ctypes.c_float(0.04)

    def call(q=A, codes=A, cst=0, sig=A, rope=A, rst=0, nw=N, B=2, H=64, d_c=512, d_r=64, W=128,
             mo=N, ml=N, out=A, lse=N):
        return sw(q, codes, cst, sig, rope, rst, nw, B, H, d_c, d_r, W, sm, mo, ml, out, lse, N)
    assert call(B=-1) == SHAPE
    assert call(d_c=128) == UNSUP
    assert call(d_r=32) == UNSUP
    assert call(H=129) == UNSUP
    assert call(W=257) == RANGE
    assert call(B=0) == OK
    assert call(q=N) == NULL
    assert call(sig=N) == NULL
    assert call(mo=A) == NULL                       # one half of the merge input
    assert call(q=U) == ALIGN
    assert call(cst=520) == ALIGN
    assert call(cst=256) == SHAPE


def test_attn_validation(lib):
    f = lib.csa2_sparse_attn_fp4
    args = dict(q=A, codes=A, cst=512, scales=A, sst=512, rope=A, rst=512, idx=A, K=512, B=1, H=64, d_c=512,
                d_r=64, N=100, sm=0.04, out=A, lse=N, ws=A, wsb=1 << 30, st=N)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return f(a["q"], a["codes"], a["cst"], a["scales"], a["sst"], a["rope"], a["rst"], a["idx"], a["K"],
                 a["B"], a["H"], a["d_c"], a["d_r"], a["N"], ctypes.c_float(a["sm"]), a["out"], a["lse"],
                 a["ws"], a["wsb"], a["st"])
    assert call(B=0) == OK
    assert call(K=0) == SHAPE
    assert call(cst=-1) == SHAPE
    assert call(d_c=256) == UNSUP
    assert call(d_r=32) == UNSUP
    assert call(H=129) == UNSUP
    assert call(q=N) == NULL
    assert call(rope=N) == NULL
    assert call(out=U) == ALIGN
    assert call(rst=520) == ALIGN
    assert call(cst=128) == SHAPE
    need = lib.csa2_sparse_attn_workspace_bytes(1, 64, 512, 512)
    assert need > 0
    assert call(ws=N) == WS
    assert call(wsb=need - 4) == WS
    assert lib.csa2_sparse_attn_workspace_bytes(128, 64, 512, 512) == 0
    # one sequence's rows must span at most 4 GiB per array (32-bit row offsets)
    RANGE = 4
    assert call(N=(1 << 32) // 512 + 1) == RANGE
    assert call(N=(1 << 32) // 1024 + 1, cst=1024) == RANGE
    assert call(N=(1 << 32) // 512, K=512, B=0) == OK


def test_sample_validation(lib):
    d = lib.csa2_sample_draw
    assert d(A, A, 0, 8, 1.0, 1.0, A, A, N, N, N) == OK            # B == 0: nothing to do
    assert d(A, A, -1, 8, 1.0, 1.0, A, A, N, N, N) == SHAPE
    assert d(A, A, 1, 0, 1.0, 1.0, A, A, N, N, N) == RANGE
    assert d(A, A, 1, 2049, 1.0, 1.0, A, A, N, N, N) == RANGE
    assert d(A, A, 1, 8, 0.0, 1.0, A, A, N, N, N) == RANGE           # temperature 0
    assert d(A, A, 1, 8, 1e-31, 1.0, A, A, N, N, N) == RANGE         # 1/T overflows float32
    assert d(A, A, 1, 8, 1.0, 0.0, A, A, N, N, N) == RANGE           # top_p 0
    assert d(A, A, 1, 8, 1.0, float("nan"), A, A, N, N, N) == RANGE
    assert d(A, A, 1, 8, float("nan"), 1.0, A, A, N, N, N) == RANGE
    assert d(A, A, 1, 8, 1.0, 1.0, N, A, N, N, N) == NULL            # no uniforms
    assert d(A, A, 1, 8, 1.0, 1.0, A, N, N, N, N) == NULL            # no token output
    assert d(U, A, 1, 8, 1.0, 1.0, A, A, N, N, N) == ALIGN
    assert d(A, A, 1, 8, 1.0, 1.0, A, A, U, N, N) == ALIGN
    s = lib.csa2_sample
    need = lib.csa2_sample_workspace_bytes(2, 129280, 2048)
    # candidates (2 x 2048 ids + 2 x 2048 logits) + the Top-K chunk winners (2 rows x 8 chunks x 2048 u64)
    assert need == 2 * 2 * 2048 * 4 + 2 * 8 * 2048 * 8
    assert lib.csa2_sample_workspace_bytes(2, 129280, 2049) == 0
    assert s(A, 0, 129280, 2048, 1.0, 1.0, A, A, N, N, N, 0, N) == OK
    assert s(A, 2, 0, 2048, 1.0, 1.0, A, A, N, N, A, need, N) == SHAPE
    assert s(A, 2, 129280, 2049, 1.0, 1.0, A, A, N, N, A, need, N) == RANGE
    assert s(A, 2, 129280, 2048, -1.0, 1.0, A, A, N, N, A, need, N) == RANGE
    assert s(N, 2, 129280, 2048, 1.0, 1.0, A, A, N, N, A, need, N) == NULL
    assert s(A, 2, 129280, 2048, 1.0, 1.0, A, A, N, N, N, need, N) == WS
    assert s(A, 2, 129280, 2048, 1.0, 1.0, A, A, N, N, A, need - 1, N) == WS
    assert s(A, 2, 129280, 2048, 1.0, 1.0, A, A, N, N, U, need, N) == ALIGN



def test_prefill_attn_validation(lib):
    f = lib.csa2_prefill_sparse_attn_fp4

    def call(q=A, S=2, T=8, K=512, H=64, d_c=512, d_r=64, Ncap=100, out=A, ws=A, wsb=1 << 30):
        return f(q, A, 512, A, 512, A, 512, A, K, S, T, H, d_c, d_r, Ncap, ctypes.c_float(0.04), out, N, ws, wsb, N)
    assert call(S=0) == OK
    assert call(T=0) == OK
    assert call(S=-1) == SHAPE
    assert call(T=-1) == SHAPE
    assert call(S=4096, T=4097) == RANGE           # more than 2^24 queries
    assert call(K=0) == SHAPE
    assert call(d_c=256) == UNSUP
    assert call(q=N) == NULL
    assert call(out=U) == ALIGN
    need = lib.csa2_sparse_attn_workspace_bytes(2 * 8, 64, 512, 512)
    assert need > 0
    assert call(ws=N) == WS
    assert call(wsb=need - 4) == WS


def test_binding_rejects_wrong_tensors(lib):
    """The binding checks dtype and contiguity before it calls the library
    (CPU tensors: nothing is launched)."""
    import torch
    f32 = torch.zeros(4, 8, dtype=torch.float32)
    i32 = torch.zeros(4, 8, dtype=torch.int32)
    u = torch.zeros(4, dtype=torch.float32)
    with pytest.raises(ValueError):
        csa2.csa2_topk(f32.double(), 2)
    with pytest.raises(ValueError):
        csa2.csa2_topk(f32.t(), 2)                       # not contiguous
    with pytest.raises(ValueError):
        csa2.csa2_sample(f32.half(), 2, 1.0, 1.0, u)
    with pytest.raises(ValueError):
        csa2.csa2_sample(f32, 2, 1.0, 1.0, u.double())
    with pytest.raises(ValueError):
        csa2.csa2_sample_draw(i32.long(), f32, 1.0, 1.0, u)
    q = torch.zeros(2, 4, 576, dtype=torch.float32)
    codes = torch.zeros(2, 16, 256, dtype=torch.uint8)
    with pytest.raises(ValueError):
        csa2.csa2_sparse_attn_fp4(q, codes, codes[..., :32], codes[..., :128], i32[:2])
    with pytest.raises(ValueError):
        csa2.csa2_prefill_sparse_attn_fp4(q.to(torch.bfloat16)[None], codes, codes[..., :32], codes[..., :128],
                                          i32[:2].long()[None])


def test_binding_rejects_caches_too_small_for_the_queries(lib):
    """Each decode query reads its own sequence of the cache, a prefill chunk
    one sequence per S: a cache with fewer sequences is refused before any
    call (CPU tensors: nothing is launched)."""
    import torch
    from sparse_attention_decode_csa2_amd import csa2 as c
    codes, scales, rope = c.alloc_cache(2, 16, 512, 64, "cpu")
    q = torch.zeros(4, 8, 576, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="sequences"):
        c.csa2_sparse_attn_fp4(q, codes, scales, rope, torch.zeros(4, 8, dtype=torch.int32))
    with pytest.raises(ValueError, match="idx"):
        c.csa2_sparse_attn_fp4(q[:2], codes, scales, rope, torch.zeros(3, 8, dtype=torch.int32))
    qp = torch.zeros(3, 5, 8, 576, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="sequences"):
        c.csa2_prefill_sparse_attn_fp4(qp, codes, scales, rope, torch.zeros(3, 5, 8, dtype=torch.int32))
    with pytest.raises(ValueError, match="idx"):
        c.csa2_prefill_sparse_attn_fp4(qp[:2], codes, scales, rope, torch.zeros(2, 4, 8, dtype=torch.int32))


def test_launches_past_2_32_work_items_are_refused(lib):
    """Sizes whose launch would hold 2^32 work-items or more return
    CSA2_ERR_RANGE from host validation (nothing is launched)."""
    # index: 16-key tiles, 4 waves of 64 threads per 64 keys -> 4 threads per key
    assert lib.csa2_index_full(A, N, A, N, 1 << 12, 8, 128, 1 << 18, A, N) == RANGE
    assert lib.csa2_index_full(A, N, A, N, 8, 8, 128, 1 << 18, A, N) != RANGE
    # Top-K: one 1024-thread workgroup per 16384 candidates in the first level
    M = 1 << 30
    assert lib.csa2_topk(A, N, N, 1 << 10, M, 512, A, N, A, 1 << 62, N) == RANGE
    # attention: 2^22 queries x 2 head groups x 512 threads = 2^32
    f = lib.csa2_sparse_attn_fp4
    sm = ctypes.c_float(0.04)
    assert f(A, A, 512, A, 512, A, 512, A, 512, 1 << 22, 64, 512, 64, 100, sm, A, N, A, 1 << 62, N) == RANGE
    # a K whose slices alone pass the limit: 2^25 tiles of 64 entries, 8 tiles a slice
    assert f(A, A, 512, A, 512, A, 512, A, (1 << 31) - 1, 1, 64, 512, 64, 100, sm, A, N, A, 1 << 62, N) == RANGE
    p = lib.csa2_prefill_sparse_attn_fp4
    assert p(A, A, 512, A, 512, A, 512, A, 512, 1 << 11, 1 << 11, 64, 512, 64, 100, sm, A, N, A, 1 << 62,
             N) == RANGE
    # sampler draw: one 256-thread workgroup per row
    assert lib.csa2_sample_draw(A, A, (1 << 31) - 1, 8, 1.0, 1.0, A, A, N, N, N) == RANGE


def test_binding_checks_index_inputs_and_output_shapes(lib):
    """The binding is the only guard on buffer sizes (the C ABI sees
    pointers): wrong dtypes, too few key sequences and output tensors of the
    wrong shape are refused before any call (CPU tensors: nothing launches)."""
    import torch
    bf = torch.bfloat16
    qi = torch.zeros(2, 8, 128, dtype=bf)
    k = torch.zeros(2, 64, 128, dtype=bf)
    with pytest.raises(ValueError):
        csa2.csa2_index_full(qi.float(), k)
    with pytest.raises(ValueError):
        csa2.csa2_index_full(qi, k.transpose(1, 2).contiguous().transpose(1, 2))   # not contiguous
    with pytest.raises(ValueError, match="k_idx"):
        csa2.csa2_index_full(qi, k[:1])                                           # fewer sequences
    with pytest.raises(ValueError, match="k_idx"):
        csa2.csa2_index_full(qi, k[..., :64].contiguous())                        # other D_I
    with pytest.raises(ValueError, match="w"):
        csa2.csa2_index_full(qi, k, w=torch.ones(2, 8, dtype=torch.float64))
    with pytest.raises(ValueError, match="n_valid"):
        csa2.csa2_index_full(qi, k, n_valid=torch.zeros(2, dtype=torch.int64))
    with pytest.raises(ValueError, match="scores"):
        csa2.csa2_index_full(qi, k, scores=torch.empty(2, 63))
    pool = torch.zeros(2, 16, dtype=torch.int32)
    nb = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="pool_blocks"):
        csa2.csa2_index_pool(qi, k, pool.long(), nb)
    with pytest.raises(ValueError, match="n_blocks"):
        csa2.csa2_index_pool(qi, k, pool, nb[:1])
    with pytest.raises(ValueError, match="positions"):
        csa2.csa2_index_pool(qi, k, pool, nb, positions=torch.empty(2, 16 * 8 - 1, dtype=torch.int32))
    sc = torch.zeros(2, 100)
    with pytest.raises(ValueError, match="ids"):
        csa2.csa2_topk(sc, 8, ids=torch.zeros(2, 99, dtype=torch.int32))
    with pytest.raises(ValueError, match="out_idx"):
        csa2.csa2_topk(sc, 8, out_idx=torch.empty(2, 7, dtype=torch.int32))
    with pytest.raises(ValueError, match="out_score"):
        csa2.csa2_topk(sc, 8, out_score=torch.empty(2, 8, dtype=torch.float64))
    with pytest.raises(ValueError, match="pool_blocks"):
        csa2.csa2_build_pool(sc, 4, pool_blocks=torch.empty(2, 5, dtype=torch.int32))
    u = torch.zeros(2)
    with pytest.raises(ValueError, match="token"):
        csa2.csa2_sample(sc, 8, 1.0, 1.0, u, token=torch.empty(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="u"):
        csa2.csa2_sample_draw(torch.zeros(2, 8, dtype=torch.int32), torch.zeros(2, 8), 1.0, 1.0, u[:1])


def test_binding_checks_cache_views_and_attention_outputs(lib):
    import torch
    codes, scales, rope = csa2.alloc_cache(2, 16, 512, 64, "cpu")
    q = torch.zeros(2, 8, 576, dtype=torch.bfloat16)
    idx = torch.zeros(2, 8, dtype=torch.int32)
    with pytest.raises(ValueError, match="scales"):
        csa2.csa2_sparse_attn_fp4(q, codes, scales[:, :8], rope, idx)              # fewer scale rows
    with pytest.raises(ValueError, match="rope"):
        csa2.csa2_sparse_attn_fp4(q, codes, scales, rope[:, :15], idx)            # fewer RoPE rows
    with pytest.raises(ValueError, match="out"):
        csa2.csa2_sparse_attn_fp4(q, codes, scales, rope, idx, out=torch.empty(2, 8, 511))
    with pytest.raises(ValueError, match="lse"):
        csa2.csa2_sparse_attn_fp4(q, codes, scales, rope, idx, lse=torch.empty(2, 7))
    with pytest.raises(ValueError, match="out"):
        csa2.csa2_prefill_sparse_attn_fp4(q[None], codes[:1], scales[:1], rope[:1], idx[None],
                                          out=torch.empty(1, 2, 8, 512, dtype=torch.float64))
    x = torch.zeros(4, 512, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="scales"):
        csa2.csa2_quantize_fp4(x, codes[0], scales[0, :8])
    with pytest.raises(ValueError, match="channels"):
        csa2.csa2_quantize_fp4(x[:, :256].contiguous(), codes[0], scales[0])
    wc, ws, wr = csa2.alloc_window(2, 16, 512, 64, "cpu")
    with pytest.raises(ValueError, match="sigma"):
        csa2.csa2_swa_attn_fp8(q, wc, ws[:, :8], wr)
    with pytest.raises(ValueError, match="merge_lse"):
        csa2.csa2_swa_attn_fp8(q, wc, ws, wr, merge_out=torch.zeros(2, 8, 512), merge_lse=torch.zeros(2, 9))
    with pytest.raises(ValueError, match="sigma"):
        csa2.csa2_quantize_fp8(x, wc[0], ws[0, :3], 0)


def test_topk_noalloc_validation(lib):
    """The no-allocation Top-K validates like csa2_topk and refuses, before
    touching the device, a call whose chunk winners exceed its 32 MiB array."""
    f = lib.csa2_topk_noalloc
    assert f(A, N, N, 0, 100, 8, A, A, N) == OK
    assert f(A, N, N, -1, 100, 8, A, A, N) == SHAPE
    assert f(A, N, N, 1, 0, 8, A, A, N) == SHAPE
    assert f(A, N, N, 1, 100, 2049, A, A, N) == RANGE
    assert f(N, N, N, 1, 100, 8, A, A, N) == NULL
    assert f(U, N, N, 1, 100, 8, A, A, N) == ALIGN
    # the chunked reduction: 4096 rows x 16 chunks x 512 winners x 8 bytes =
    # 256 MiB > 32 MiB
    assert f(A, N, N, 4096, 262144, 512, A, A, N) == RANGE


def test_sample_full_validation(lib):
    f = lib.csa2_sample_full
    wsb = lib.csa2_sample_full_workspace_bytes
    # 16 (max, sum) pairs of 8 bytes per 16384-token tile and row
    assert wsb(128, 129280) == 128 * 8 * 16 * 8 and wsb(1, 1) == 128 and wsb(0, 10) == 0
    assert wsb(2, (1 << 20) + 1) == 0
    need = wsb(2, 129280)

    def call(lg=A, B=2, V=129280, T=1.0, u=A, tok=A, prob=N, ws=A, wsn=need):
        return f(lg, B, V, T, u, tok, prob, ws, wsn, N)
    assert call(B=0, lg=N, ws=N) == OK
    assert call(B=-1) == SHAPE
    assert call(V=0) == SHAPE
    assert call(V=(1 << 20) + 1) == RANGE
    assert call(T=0.0) == RANGE
    assert call(T=float("nan")) == RANGE
    assert call(lg=N) == NULL
    assert call(tok=N) == NULL
    assert call(lg=U) == ALIGN
    assert call(prob=U) == ALIGN
    assert call(ws=N) == WS and call(wsn=need - 1) == WS
    assert call(ws=U) == ALIGN