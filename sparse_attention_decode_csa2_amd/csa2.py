"""Thin ctypes binding of libcsa2.so (declared in include/csa2.h).

Argument marshalling only: torch tensors become device pointers, the stream is
torch's current HIP stream, and a non-zero status raises ``Csa2Error``.  Every
step of the decode path runs in the library's HIP kernels; there is no
fallback of any kind.  When the library is missing the first call raises.

Functions carry the C names.  Output tensors (and workspaces) may be passed in
(the call then allocates nothing) or are allocated here with torch.
"""

import ctypes
import math
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "csa2.h")

_lib = None


class Csa2Error(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed with status {status}: {status_string(status)}")
        self.status = status


def load():
    """Load libcsa2.so (once).  Raises OSError when it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise OSError(f"{LIB_PATH} is not built: run python -m sparse_attention_decode_csa2_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "csa2_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "csa2_version": (ctypes.c_int, []),
        "csa2_quantize_fp4": (ctypes.c_int, [P, I64, I32, P, I32, P, I64, P, I64, P, I64, I64, I64, P]),
        "csa2_index_full": (ctypes.c_int, [P, P, P, P, I32, I32, I32, I64, P, P]),
        "csa2_index_pool": (ctypes.c_int, [P, P, P, P, P, P, I32, I32, I32, I64, I32, I32, P, P, P]),
        "csa2_topk_workspace_bytes": (SZ, [I32, I64, I32]),
        "csa2_topk": (ctypes.c_int, [P, P, P, I32, I64, I32, P, P, P, SZ, P]),
        "csa2_quantize_fp8": (ctypes.c_int, [P, I64, I32, P, I32, P, I64, P, P, I64, I64, I64, P]),
        "csa2_swa_attn_fp8": (ctypes.c_int, [P, P, I64, P, P, I64, P, I32, I32, I32, I32, I32, F, P, P, P, P, P]),
        "csa2_build_pool_workspace_bytes": (SZ, [I32, I64, I32, I32]),
        "csa2_build_pool": (ctypes.c_int, [P, P, I32, I64, I32, I32, P, P, P, SZ, P]),
        "csa2_sample_draw": (ctypes.c_int, [P, P, I32, I32, F, F, P, P, P, P, P]),
        "csa2_sample_workspace_bytes": (SZ, [I32, I64, I32]),
        "csa2_sample": (ctypes.c_int, [P, I32, I64, I32, F, F, P, P, P, P, P, SZ, P]),
        "csa2_sparse_attn_workspace_bytes": (SZ, [I32, I32, I32, I32]),
        "csa2_sparse_attn_fp4": (ctypes.c_int, [P, P, I64, P, I64, P, I64, P, I32, I32, I32, I32, I32, I64,
                                                F, P, P, P, SZ, P]),
        "csa2_prefill_sparse_attn_fp4": (ctypes.c_int, [P, P, I64, P, I64, P, I64, P, I32, I32, I32, I32, I32, I32,
                                                        I64, F, P, P, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def declared_functions():
    """Names of the functions include/csa2.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|int|size_t)\s+(csa2_\w+)\s*\(", text, re.M)))


def status_string(status):
    return load().csa2_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn, st):
    if st != 0:
        raise Csa2Error(fn, st)


def _need(t, dtype, name):
    if t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor")


# ------------------------------------------------------------------ the FP4 cache


def _row_stride(t, elem_bytes, name):
    """Byte distance between consecutive rows of a (possibly strided) cache view;
    rows of all sequences must be evenly spaced."""
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: the channel dimension must be contiguous")
    rs = t.stride(-2)
    if t.dim() == 3 and t.shape[0] > 1 and t.shape[1] > 0 and t.stride(0) != t.shape[1] * rs:
        raise ValueError(f"{name}: sequences must be evenly spaced rows")
    return rs * elem_bytes


def alloc_cache(B, N, d_c, d_r, device="cuda", layout="record"):
    """Allocates an FP4 cache for B sequences of N entries; returns (codes,
    scales, rope) views [B, N, *] (rope is [B, N, 0] when d_r == 0).

    layout "record": one buffer of fixed-size entry records, codes | RoPE |
    scales, record size the next power of two >= d_c/2 + 2*d_r + d_c/16 (512
    bytes for d_c = 512, d_r = 64): the attention gather then reads one
    contiguous record per entry.  layout "separate": three dense arrays.
    """
    cb, rb, sb = d_c // 2, 2 * d_r, d_c // 16
    if layout == "separate":
        codes = torch.empty(B, N, cb, dtype=torch.uint8, device=device)
        scales = torch.empty(B, N, sb, dtype=torch.uint8, device=device)
        rope = torch.empty(B, N, d_r, dtype=torch.bfloat16, device=device)
        return codes, scales, rope
    rec = 1
    while rec < cb + rb + sb:
        rec *= 2
    buf = torch.empty(B, N, rec, dtype=torch.uint8, device=device)
    codes = buf[:, :, :cb]
    rope = buf[:, :, cb:cb + rb].view(torch.bfloat16)
    scales = buf[:, :, cb + rb:cb + rb + sb]
    return codes, scales, rope


# ------------------------------------------------------------------ a0


def csa2_quantize_fp4(x, codes, scales, dst_row0=0, rope_src=None, rope_dst=None):
    """Quantise bf16 rows x [R, d_c] into rows [dst_row0, dst_row0+R) of one
    sequence's FP4 cache (codes u8 [cap, d_c/2], scales u8 [cap, d_c/16] and
    rope_dst bf16 [cap, d_r], possibly strided views of one record buffer);
    copies the RoPE part rope_src [R, d_r] when given."""
    lib = load()
    _need(x, torch.bfloat16, "x")
    R, d_c = x.shape
    d_r = 0 if rope_src is None else rope_src.shape[1]
    cs = _row_stride(codes, 1, "codes")
    ss = _row_stride(scales, 1, "scales")
    rs = _row_stride(rope_dst, 2, "rope_dst") if d_r else 0
    st = lib.csa2_quantize_fp4(_ptr(x), R, d_c, _ptr(rope_src), d_r, _ptr(codes), cs, _ptr(scales), ss,
                               _ptr(rope_dst if d_r else None), rs, int(dst_row0), codes.shape[-2],
                               _stream())
    _check("csa2_quantize_fp4", st)
    return codes, scales


# ------------------------------------------------------------------ a1 / a2


def csa2_index_full(q_idx, k_idx, scores=None, w=None, n_valid=None):
    """Full-mode indexer scores [B, N_cap] (f32)."""
    lib = load()
    B, H_I, D_I = q_idx.shape
    N_cap = k_idx.shape[1]
    if scores is None:
        scores = torch.empty(B, N_cap, dtype=torch.float32, device=k_idx.device)
    st = lib.csa2_index_full(_ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(n_valid), B, H_I, D_I, N_cap,
                             _ptr(scores), _stream())
    _check("csa2_index_full", st)
    return scores


def csa2_index_pool(q_idx, k_idx, pool_blocks, n_blocks, block=8, scores=None, positions=None, w=None,
                    n_valid=None):
    """Reindex-mode pool scores and global positions, both [B, P_max*block]."""
    lib = load()
    B, H_I, D_I = q_idx.shape
    N_cap = k_idx.shape[1]
    P_max = pool_blocks.shape[1]
    M = P_max * block
    if scores is None:
        scores = torch.empty(B, M, dtype=torch.float32, device=k_idx.device)
    if positions is None:
        positions = torch.empty(B, M, dtype=torch.int32, device=k_idx.device)
    st = lib.csa2_index_pool(_ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(n_valid), _ptr(pool_blocks),
                             _ptr(n_blocks), B, H_I, D_I, N_cap, P_max, block, _ptr(scores),
                             _ptr(positions), _stream())
    _check("csa2_index_pool", st)
    return scores, positions


# ------------------------------------------------------------------ a3


def csa2_topk_workspace_bytes(B, M, K):
    return int(load().csa2_topk_workspace_bytes(B, M, K))


def csa2_topk(scores, K, ids=None, n_valid=None, out_idx=None, out_score=None, workspace=None,
              want_score=True):
    """Top-K (score desc, id asc): returns (idx i32 [B, K], score f32 [B, K] or None)."""
    lib = load()
    _need(scores, torch.float32, "scores")
    if ids is not None:
        _need(ids, torch.int32, "ids")
    if n_valid is not None:
        _need(n_valid, torch.int32, "n_valid")
    B, M = scores.shape
    dev = scores.device
    if out_idx is None:
        out_idx = torch.empty(B, K, dtype=torch.int32, device=dev)
    if out_score is None and want_score:
        out_score = torch.empty(B, K, dtype=torch.float32, device=dev)
    need = csa2_topk_workspace_bytes(B, M, K)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.csa2_topk(_ptr(scores), _ptr(ids), _ptr(n_valid), B, M, K, _ptr(out_idx), _ptr(out_score),
                       _ptr(workspace), ws_bytes, _stream())
    _check("csa2_topk", st)
    return out_idx, out_score


# ------------------------------------------------------------------ sampler


def csa2_sample_draw(cand_idx, cand_score, temperature, top_p, u, token=None, prob=None, n_kept=None):
    """Draw over Top-K candidates: cand_idx i32 [B, K], cand_score f32 [B, K],
    u f32 [B] -> (token i32 [B], prob f32 [B], n_kept i32 [B])."""
    lib = load()
    _need(cand_idx, torch.int32, "cand_idx")
    _need(cand_score, torch.float32, "cand_score")
    _need(u, torch.float32, "u")
    B, K = cand_idx.shape
    dev = cand_idx.device
    token = torch.empty(B, dtype=torch.int32, device=dev) if token is None else token
    prob = torch.empty(B, dtype=torch.float32, device=dev) if prob is None else prob
    n_kept = torch.empty(B, dtype=torch.int32, device=dev) if n_kept is None else n_kept
    st = lib.csa2_sample_draw(_ptr(cand_idx), _ptr(cand_score), B, K, float(temperature), float(top_p), _ptr(u),
                              _ptr(token), _ptr(prob), _ptr(n_kept), _stream())
    _check("csa2_sample_draw", st)
    return token, prob, n_kept


def csa2_sample_workspace_bytes(B, V, K):
    return int(load().csa2_sample_workspace_bytes(B, V, K))


def csa2_sample(logits, K, temperature, top_p, u, token=None, prob=None, n_kept=None, workspace=None):
    """Top-K over logits f32 [B, V], then the draw: (token, prob, n_kept)."""
    lib = load()
    _need(logits, torch.float32, "logits")
    _need(u, torch.float32, "u")
    B, V = logits.shape
    dev = logits.device
    token = torch.empty(B, dtype=torch.int32, device=dev) if token is None else token
    prob = torch.empty(B, dtype=torch.float32, device=dev) if prob is None else prob
    n_kept = torch.empty(B, dtype=torch.int32, device=dev) if n_kept is None else n_kept
    if workspace is None:
        workspace = torch.empty(max(csa2_sample_workspace_bytes(B, V, K), 16), dtype=torch.uint8, device=dev)
    st = lib.csa2_sample(_ptr(logits), B, V, K, float(temperature), float(top_p), _ptr(u), _ptr(token),
                         _ptr(prob), _ptr(n_kept), _ptr(workspace), workspace.numel(), _stream())
    _check("csa2_sample", st)
    return token, prob, n_kept


# ------------------------------------------------------------------ a4 / a5


def alloc_window(B, W_cap, d_c, d_r, device="cuda"):
    """Sliding-window FP8 cache: codes u8 [B, W_cap, d_c], sigma f32 [B, W_cap],
    rope bf16 [B, W_cap, d_r] (dense rows)."""
    codes = torch.zeros(B, W_cap, d_c, dtype=torch.uint8, device=device)
    sigma = torch.ones(B, W_cap, dtype=torch.float32, device=device)
    rope = torch.zeros(B, W_cap, d_r, dtype=torch.bfloat16, device=device)
    return codes, sigma, rope


def csa2_quantize_fp8(x, codes, sigma, dst_row0=0, rope_src=None, rope_dst=None):
    """FP8 write of window rows: x bf16 [R, d_c] -> rows [dst_row0, dst_row0 + R)
    of codes u8 [cap, d_c] / sigma f32 [cap] (and the RoPE part, copied)."""
    lib = load()
    _need(x, torch.bfloat16, "x")
    R, d_c = x.shape
    d_r = 0 if rope_src is None else rope_src.shape[1]
    cap = codes.shape[0]
    cs = _row_stride(codes, 1, "codes")
    rs = _row_stride(rope_dst, 2, "rope_dst") if d_r > 0 else 0
    st = lib.csa2_quantize_fp8(_ptr(x), R, d_c, _ptr(rope_src), d_r, _ptr(codes), cs, _ptr(sigma),
                               _ptr(rope_dst if d_r > 0 else None), rs, dst_row0, cap, _stream())
    _check("csa2_quantize_fp8", st)


def csa2_swa_attn_fp8(q, codes, sigma, rope, sm_scale=None, n_win=None, merge_out=None, merge_lse=None,
                      out=None, lse=None):
    """Window attention over codes [B, W_cap, d_c] (E4M3) with row scales sigma
    [B, W_cap], merged with (merge_out, merge_lse) when given: returns
    (out f32 [B, H, d_c], lse f32 [B, H])."""
    lib = load()
    _need(q, torch.bfloat16, "q")
    B, H, D = q.shape
    W_cap, d_c = codes.shape[1], codes.shape[2]
    d_r = D - d_c
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    dev = q.device
    if out is None:
        out = torch.empty(B, H, d_c, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(B, H, dtype=torch.float32, device=dev)
    cs = _row_stride(codes, 1, "codes")
    rs = _row_stride(rope, 2, "rope") if d_r > 0 else 0
    st = lib.csa2_swa_attn_fp8(_ptr(q), _ptr(codes), cs, _ptr(sigma), _ptr(rope if d_r > 0 else None), rs,
                               _ptr(n_win), B, H, d_c, d_r, W_cap, float(sm_scale), _ptr(merge_out),
                               _ptr(merge_lse), _ptr(out), _ptr(lse), _stream())
    _check("csa2_swa_attn_fp8", st)
    return out, lse


def csa2_build_pool_workspace_bytes(B, M, block, P_max):
    return int(load().csa2_build_pool_workspace_bytes(B, M, block, P_max))


def csa2_build_pool(scores, P_max, block=8, n_valid=None, pool_blocks=None, n_blocks=None, workspace=None):
    """Block-level candidate pool from a Full layer's scores f32 [B, M]:
    returns (pool_blocks i32 [B, P_max], n_blocks i32 [B])."""
    lib = load()
    B, M = scores.shape
    dev = scores.device
    _need(scores, torch.float32, "scores")
    if pool_blocks is None:
        pool_blocks = torch.empty(B, P_max, dtype=torch.int32, device=dev)
    if n_blocks is None:
        n_blocks = torch.empty(B, dtype=torch.int32, device=dev)
    need = csa2_build_pool_workspace_bytes(B, M, block, P_max)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.csa2_build_pool(_ptr(scores), _ptr(n_valid), B, M, block, P_max, _ptr(pool_blocks),
                             _ptr(n_blocks), _ptr(workspace), ws_bytes, _stream())
    _check("csa2_build_pool", st)
    return pool_blocks, n_blocks


def csa2_sparse_attn_workspace_bytes(B, H, d_c, K):
    return int(load().csa2_sparse_attn_workspace_bytes(B, H, d_c, K))


def csa2_sparse_attn_fp4(q, codes, scales, rope, idx, sm_scale=None, out=None, lse=None, workspace=None,
                         want_lse=True):
    """Sparse attention over the selected FP4 entries of the cache (codes,
    scales, rope: [B, N_cap, *] views as from alloc_cache): returns
    (out f32 [B, H, d_c], lse f32 [B, H])."""
    lib = load()
    _need(q, torch.bfloat16, "q")
    B, H, D = q.shape
    N_cap = codes.shape[1]
    d_c = codes.shape[2] * 2
    d_r = D - d_c
    _need(idx, torch.int32, "idx")
    K = idx.shape[1]
    if idx.dim() != 2 or idx.shape[0] != B:
        raise ValueError(f"idx must be [B={B}, K], got {tuple(idx.shape)}")
    if codes.shape[0] < B or scales.shape[0] < B or (d_r > 0 and rope.shape[0] < B):
        raise ValueError(f"the cache holds {codes.shape[0]} sequences, {B} queries need one each")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    dev = q.device
    if out is None:
        out = torch.empty(B, H, d_c, dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(B, H, dtype=torch.float32, device=dev)
    need = csa2_sparse_attn_workspace_bytes(B, H, d_c, K)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    cs = _row_stride(codes, 1, "codes")
    ss = _row_stride(scales, 1, "scales")
    rs = _row_stride(rope, 2, "rope") if d_r > 0 else 0
    st = lib.csa2_sparse_attn_fp4(_ptr(q), _ptr(codes), cs, _ptr(scales), ss,
                                  _ptr(rope if d_r > 0 else None), rs, _ptr(idx), K, B, H, d_c, d_r, N_cap,
                                  float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream())
    _check("csa2_sparse_attn_fp4", st)
    return out, lse


def csa2_prefill_sparse_attn_fp4(q, codes, scales, rope, idx, sm_scale=None, out=None, lse=None, workspace=None,
                                 want_lse=True):
    """Prefill sparse attention: q bf16 [S, T, H, D], idx i32 [S, T, K], one
    cache per sequence (codes, scales, rope: [S, N_cap, *] views as from
    alloc_cache): returns (out f32 [S, T, H, d_c], lse f32 [S, T, H])."""
    lib = load()
    _need(q, torch.bfloat16, "q")
    _need(idx, torch.int32, "idx")
    S, T, H, D = q.shape
    N_cap = codes.shape[1]
    d_c = codes.shape[2] * 2
    d_r = D - d_c
    K = idx.shape[2]
    if tuple(idx.shape[:2]) != (S, T):
        raise ValueError(f"idx must be [S={S}, T={T}, K], got {tuple(idx.shape)}")
    if codes.shape[0] < S or scales.shape[0] < S or (d_r > 0 and rope.shape[0] < S):
        raise ValueError(f"the cache holds {codes.shape[0]} sequences, the chunk needs {S}")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    dev = q.device
    if out is None:
        out = torch.empty(S, T, H, d_c, dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(S, T, H, dtype=torch.float32, device=dev)
    need = csa2_sparse_attn_workspace_bytes(S * T, H, d_c, K)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    cs = _row_stride(codes, 1, "codes")
    ss = _row_stride(scales, 1, "scales")
    rs = _row_stride(rope, 2, "rope") if d_r > 0 else 0
    st = lib.csa2_prefill_sparse_attn_fp4(_ptr(q), _ptr(codes), cs, _ptr(scales), ss,
                                          _ptr(rope if d_r > 0 else None), rs, _ptr(idx), K, S, T, H, d_c, d_r,
                                          N_cap, float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                          _stream())
    _check("csa2_prefill_sparse_attn_fp4", st)
    return out, lse
