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
# CSA2_LIBRARY names another build of the same library (e.g. the host-ASan
# build the CPU tests make of the validation layer); the default is the
# in-tree libcsa2.so
LIB_PATH = os.environ.get("CSA2_LIBRARY") or os.path.join(_HERE, "libcsa2.so")
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
        "csa2_topk_noalloc": (ctypes.c_int, [P, P, P, I32, I64, I32, P, P, P]),
        "csa2_index_topk_full_workspace_bytes": (SZ, [I32, I32, I64, I32]),
        "csa2_index_topk_full": (ctypes.c_int, [P, P, P, P, I32, I32, I32, I64, I32, P, P, P, SZ, P]),
        "csa2_index_topk_full_append": (ctypes.c_int, [P, P, P, P, I32, I32, I32, I64, I32, P, P, P, SZ,
                                                       P, I64, I32, P, I32, P, I64, P, I64, P, I64, I64, I64, P]),
        "csa2_quantize_fp8": (ctypes.c_int, [P, I64, I32, P, I32, P, I64, P, P, I64, I64, I64, P]),
        "csa2_swa_attn_fp8": (ctypes.c_int, [P, P, I64, P, P, I64, P, I32, I32, I32, I32, I32, F, P, P, P, P, P]),
        "csa2_build_pool_workspace_bytes": (SZ, [I32, I64, I32, I32]),
        "csa2_build_pool": (ctypes.c_int, [P, P, I32, I64, I32, I32, P, P, P, SZ, P]),
        "csa2_sample_draw": (ctypes.c_int, [P, P, I32, I32, F, F, P, P, P, P, P]),
        "csa2_sample_workspace_bytes": (SZ, [I32, I64, I32]),
        "csa2_sample": (ctypes.c_int, [P, I32, I64, I32, F, F, P, P, P, P, P, SZ, P]),
        "csa2_sample_full_workspace_bytes": (SZ, [I32, I64]),
        "csa2_sample_full": (ctypes.c_int, [P, I32, I64, F, P, P, P, P, SZ, P]),
        "csa2_sparse_attn_workspace_bytes": (SZ, [I32, I32, I32, I32]),
        "csa2_sparse_swa_attn_workspace_bytes": (SZ, [I32, I32, I32, I32]),
        "csa2_sparse_swa_attn_fp4": (ctypes.c_int, [P, P, I64, P, I64, P, I64, P, I32, I32, I32, I32, I32, I64,
                                                    P, I64, P, P, I64, P, I32, F, P, P, P, SZ, P]),
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


def _need(t, dtype, name, shape=None):
    """Input check: a contiguous tensor of `dtype` (and of `shape` when given;
    None in `shape` accepts any size in that dimension)."""
    if t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor")
    if shape is not None and (t.dim() != len(shape) or
                              any(w is not None and d != w for d, w in zip(t.shape, shape))):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _out(t, shape, dtype, device, name):
    """An output buffer: allocated when None, else checked to be exactly the
    contiguous `shape` / `dtype` the kernels write (the C ABI sees only a
    pointer, so this is the only guard on its size)."""
    if t is None:
        return torch.empty(*shape, dtype=dtype, device=device)
    _need(t, dtype, name, shape)
    return t


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


def _cache_views(codes, scales, rope, d_r, dims):
    """The three views of an FP4 cache: codes u8 [..., d_c/2], scales u8
    [..., d_c/16], rope bf16 [..., d_r] with the same leading (sequence, row)
    shape, so that every row the kernels address exists in all three."""
    if codes.dtype != torch.uint8 or scales.dtype != torch.uint8:
        raise ValueError("codes and scales must be uint8 views")
    if dims == 2 and codes.dim() == 3 and codes.shape[0] == 1:
        dims = 3   # one sequence's cache, as [1, cap, *] views
    if codes.dim() != dims or scales.dim() != dims:
        raise ValueError(f"codes and scales must have {dims} dimensions")
    if tuple(scales.shape[:-1]) != tuple(codes.shape[:-1]) or scales.shape[-1] * 8 != codes.shape[-1]:
        raise ValueError(f"scales {tuple(scales.shape)} do not match codes {tuple(codes.shape)} "
                         f"(one scale byte per 16 channels, the same rows)")
    if d_r > 0:
        if rope is None or rope.dtype != torch.bfloat16 or rope.dim() != dims:
            raise ValueError(f"rope must be a bf16 view with {dims} dimensions")
        if tuple(rope.shape[:-1]) != tuple(codes.shape[:-1]) or rope.shape[-1] != d_r:
            raise ValueError(f"rope {tuple(rope.shape)} does not match codes {tuple(codes.shape)} with "
                             f"{d_r} RoPE channels")


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
    if x.dim() != 2:
        raise ValueError(f"x must be [R, d_c], got {tuple(x.shape)}")
    R, d_c = x.shape
    d_r = 0 if rope_src is None else rope_src.shape[-1]
    if rope_src is not None:
        _need(rope_src, torch.bfloat16, "rope_src", (R, None))
    _cache_views(codes, scales, rope_dst, d_r, 2)
    if codes.shape[1] * 2 != d_c:
        raise ValueError(f"codes rows hold {codes.shape[1] * 2} channels, x has {d_c}")
    cs = _row_stride(codes, 1, "codes")
    ss = _row_stride(scales, 1, "scales")
    rs = _row_stride(rope_dst, 2, "rope_dst") if d_r else 0
    st = lib.csa2_quantize_fp4(_ptr(x), R, d_c, _ptr(rope_src), d_r, _ptr(codes), cs, _ptr(scales), ss,
                               _ptr(rope_dst if d_r else None), rs, int(dst_row0), codes.shape[-2],
                               _stream())
    _check("csa2_quantize_fp4", st)
    return codes, scales


# ------------------------------------------------------------------ a1 / a2


def _index_inputs(q_idx, k_idx, w, n_valid):
    _need(q_idx, torch.bfloat16, "q_idx")
    if q_idx.dim() != 3:
        raise ValueError(f"q_idx must be [B, H_I, D_I], got {tuple(q_idx.shape)}")
    B, H_I, D_I = q_idx.shape
    _need(k_idx, torch.bfloat16, "k_idx")
    if k_idx.dim() != 3 or k_idx.shape[0] < B or k_idx.shape[2] != D_I:
        raise ValueError(f"k_idx must be [>= {B}, N_cap, {D_I}], got {tuple(k_idx.shape)}")
    if w is not None:
        _need(w, torch.float32, "w", (B, H_I))
    if n_valid is not None:
        _need(n_valid, torch.int32, "n_valid", (B,))
    return B, H_I, D_I, k_idx.shape[1]


def csa2_index_full(q_idx, k_idx, scores=None, w=None, n_valid=None):
    """Full-mode indexer scores [B, N_cap] (f32)."""
    lib = load()
    B, H_I, D_I, N_cap = _index_inputs(q_idx, k_idx, w, n_valid)
    scores = _out(scores, (B, N_cap), torch.float32, k_idx.device, "scores")
    st = lib.csa2_index_full(_ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(n_valid), B, H_I, D_I, N_cap,
                             _ptr(scores), _stream())
    _check("csa2_index_full", st)
    return scores


def csa2_index_pool(q_idx, k_idx, pool_blocks, n_blocks, block=8, scores=None, positions=None, w=None,
                    n_valid=None):
    """Reindex-mode pool scores and global positions, both [B, P_max*block]."""
    lib = load()
    B, H_I, D_I, N_cap = _index_inputs(q_idx, k_idx, w, n_valid)
    _need(pool_blocks, torch.int32, "pool_blocks", (B, None))
    _need(n_blocks, torch.int32, "n_blocks", (B,))
    P_max = pool_blocks.shape[1]
    M = P_max * block
    scores = _out(scores, (B, M), torch.float32, k_idx.device, "scores")
    positions = _out(positions, (B, M), torch.int32, k_idx.device, "positions")
    st = lib.csa2_index_pool(_ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(n_valid), _ptr(pool_blocks),
                             _ptr(n_blocks), B, H_I, D_I, N_cap, P_max, block, _ptr(scores),
                             _ptr(positions), _stream())
    _check("csa2_index_pool", st)
    return scores, positions


def csa2_index_topk_full_workspace_bytes(B, D_I, N_cap, K):
    return int(load().csa2_index_topk_full_workspace_bytes(B, D_I, N_cap, K))


def csa2_index_topk_full(q_idx, k_idx, K, w=None, n_valid=None, out_idx=None, out_score=None, workspace=None,
                         want_score=True):
    """Full-mode indexer scores and their Top-K in one call: (idx i32 [B, K],
    score f32 [B, K] or None), as csa2_topk(csa2_index_full(...), K, n_valid)."""
    lib = load()
    B, H_I, D_I, N_cap = _index_inputs(q_idx, k_idx, w, n_valid)
    dev = k_idx.device
    out_idx = _out(out_idx, (B, K), torch.int32, dev, "out_idx")
    if out_score is not None or want_score:
        out_score = _out(out_score, (B, K), torch.float32, dev, "out_score")
    need = csa2_index_topk_full_workspace_bytes(B, D_I, N_cap, K)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.csa2_index_topk_full(_ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(n_valid), B, H_I, D_I, N_cap, K,
                                  _ptr(out_idx), _ptr(out_score), _ptr(workspace), ws_bytes, _stream())
    _check("csa2_index_topk_full", st)
    return out_idx, out_score


def csa2_index_topk_full_append(q_idx, k_idx, K, x, codes, scales, dst_row0=0, rope_src=None, rope_dst=None,
                                w=None, n_valid=None, out_idx=None, out_score=None, workspace=None,
                                want_score=True):
    """csa2_index_topk_full and csa2_quantize_fp4 (x rows into rows dst_row0..
    of one sequence's cache views, as csa2_quantize_fp4 takes them) in one
    call: returns (idx, score) of the scoring; the cache views are written."""
    lib = load()
    B, H_I, D_I, N_cap = _index_inputs(q_idx, k_idx, w, n_valid)
    dev = k_idx.device
    out_idx = _out(out_idx, (B, K), torch.int32, dev, "out_idx")
    if out_score is not None or want_score:
        out_score = _out(out_score, (B, K), torch.float32, dev, "out_score")
    need = csa2_index_topk_full_workspace_bytes(B, D_I, N_cap, K)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError(f"x must be [R, d_c], got {tuple(x.shape)}")
    R, d_c = x.shape
    d_r = 0 if rope_src is None else rope_src.shape[-1]
    if rope_src is not None:
        _need(rope_src, torch.bfloat16, "rope_src", (R, None))
    _cache_views(codes, scales, rope_dst, d_r, 2)
    if codes.shape[1] * 2 != d_c:
        raise ValueError(f"codes rows hold {codes.shape[1] * 2} channels, x has {d_c}")
    cs = _row_stride(codes, 1, "codes")
    ss = _row_stride(scales, 1, "scales")
    rs = _row_stride(rope_dst, 2, "rope_dst") if d_r else 0
    st = lib.csa2_index_topk_full_append(_ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(n_valid), B, H_I, D_I, N_cap, K,
                                         _ptr(out_idx), _ptr(out_score), _ptr(workspace), ws_bytes,
                                         _ptr(x), R, d_c, _ptr(rope_src), d_r, _ptr(codes), cs, _ptr(scales), ss,
                                         _ptr(rope_dst if d_r else None), rs, int(dst_row0), codes.shape[-2],
                                         _stream())
    _check("csa2_index_topk_full_append", st)
    return out_idx, out_score


# ------------------------------------------------------------------ a3


def csa2_topk_workspace_bytes(B, M, K):
    return int(load().csa2_topk_workspace_bytes(B, M, K))


def csa2_topk(scores, K, ids=None, n_valid=None, out_idx=None, out_score=None, workspace=None,
              want_score=True):
    """Top-K (score desc, id asc): returns (idx i32 [B, K], score f32 [B, K] or None)."""
    lib = load()
    _need(scores, torch.float32, "scores")
    if scores.dim() != 2:
        raise ValueError(f"scores must be [B, M], got {tuple(scores.shape)}")
    B, M = scores.shape
    if ids is not None:
        _need(ids, torch.int32, "ids", (B, M))
    if n_valid is not None:
        _need(n_valid, torch.int32, "n_valid", (B,))
    dev = scores.device
    out_idx = _out(out_idx, (B, K), torch.int32, dev, "out_idx")
    if out_score is not None or want_score:
        out_score = _out(out_score, (B, K), torch.float32, dev, "out_score")
    need = csa2_topk_workspace_bytes(B, M, K)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.csa2_topk(_ptr(scores), _ptr(ids), _ptr(n_valid), B, M, K, _ptr(out_idx), _ptr(out_score),
                       _ptr(workspace), ws_bytes, _stream())
    _check("csa2_topk", st)
    return out_idx, out_score


def csa2_topk_noalloc(scores, K, ids=None, n_valid=None, out_idx=None, out_score=None, want_score=True):
    """csa2_topk with its scratch in the library's static device array (no
    workspace; the library allocates nothing).  Pass out_idx / out_score to
    allocate nothing here either.  Calls that overlap on one GPU race."""
    lib = load()
    _need(scores, torch.float32, "scores")
    if scores.dim() != 2:
        raise ValueError(f"scores must be [B, M], got {tuple(scores.shape)}")
    B, M = scores.shape
    if ids is not None:
        _need(ids, torch.int32, "ids", (B, M))
    if n_valid is not None:
        _need(n_valid, torch.int32, "n_valid", (B,))
    dev = scores.device
    out_idx = _out(out_idx, (B, K), torch.int32, dev, "out_idx")
    if out_score is not None or want_score:
        out_score = _out(out_score, (B, K), torch.float32, dev, "out_score")
    st = lib.csa2_topk_noalloc(_ptr(scores), _ptr(ids), _ptr(n_valid), B, M, K, _ptr(out_idx), _ptr(out_score),
                               _stream())
    _check("csa2_topk_noalloc", st)
    return out_idx, out_score


# ------------------------------------------------------------------ sampler


def csa2_sample_draw(cand_idx, cand_score, temperature, top_p, u, token=None, prob=None, n_kept=None):
    """Draw over Top-K candidates: cand_idx i32 [B, K], cand_score f32 [B, K],
    u f32 [B] -> (token i32 [B], prob f32 [B], n_kept i32 [B])."""
    lib = load()
    _need(cand_idx, torch.int32, "cand_idx")
    if cand_idx.dim() != 2:
        raise ValueError(f"cand_idx must be [B, K], got {tuple(cand_idx.shape)}")
    B, K = cand_idx.shape
    _need(cand_score, torch.float32, "cand_score", (B, K))
    _need(u, torch.float32, "u", (B,))
    dev = cand_idx.device
    token = _out(token, (B,), torch.int32, dev, "token")
    prob = _out(prob, (B,), torch.float32, dev, "prob")
    n_kept = _out(n_kept, (B,), torch.int32, dev, "n_kept")
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
    if logits.dim() != 2:
        raise ValueError(f"logits must be [B, V], got {tuple(logits.shape)}")
    B, V = logits.shape
    _need(u, torch.float32, "u", (B,))
    dev = logits.device
    token = _out(token, (B,), torch.int32, dev, "token")
    prob = _out(prob, (B,), torch.float32, dev, "prob")
    n_kept = _out(n_kept, (B,), torch.int32, dev, "n_kept")
    if workspace is None:
        workspace = torch.empty(max(csa2_sample_workspace_bytes(B, V, K), 16), dtype=torch.uint8, device=dev)
    st = lib.csa2_sample(_ptr(logits), B, V, K, float(temperature), float(top_p), _ptr(u), _ptr(token),
                         _ptr(prob), _ptr(n_kept), _ptr(workspace), workspace.numel(), _stream())
    _check("csa2_sample", st)
    return token, prob, n_kept


def csa2_sample_full_workspace_bytes(B, V):
    return int(load().csa2_sample_full_workspace_bytes(B, V))


def csa2_sample_full(logits, temperature, u, token=None, prob=None, workspace=None):
    """The untruncated draw (top_p 1.0 over the whole vocabulary): logits f32
    [B, V], u f32 [B] -> (token i32 [B], prob f32 [B])."""
    lib = load()
    _need(logits, torch.float32, "logits")
    if logits.dim() != 2:
        raise ValueError(f"logits must be [B, V], got {tuple(logits.shape)}")
    B, V = logits.shape
    _need(u, torch.float32, "u", (B,))
    dev = logits.device
    token = _out(token, (B,), torch.int32, dev, "token")
    prob = _out(prob, (B,), torch.float32, dev, "prob")
    need = csa2_sample_full_workspace_bytes(B, V)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.csa2_sample_full(_ptr(logits), B, V, float(temperature), _ptr(u), _ptr(token), _ptr(prob),
                              _ptr(workspace), ws_bytes, _stream())
    _check("csa2_sample_full", st)
    return token, prob


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
    if x.dim() != 2:
        raise ValueError(f"x must be [R, d_c], got {tuple(x.shape)}")
    R, d_c = x.shape
    d_r = 0 if rope_src is None else rope_src.shape[-1]
    if rope_src is not None:
        _need(rope_src, torch.bfloat16, "rope_src", (R, None))
    if codes.dtype != torch.uint8 or codes.dim() != 2 or codes.shape[1] != d_c:
        raise ValueError(f"codes must be a uint8 [cap, {d_c}] view, got {tuple(codes.shape)}")
    cap = codes.shape[0]
    _need(sigma, torch.float32, "sigma", (cap,))
    if d_r > 0 and (rope_dst is None or rope_dst.dtype != torch.bfloat16 or tuple(rope_dst.shape) != (cap, d_r)):
        raise ValueError(f"rope_dst must be a bf16 [{cap}, {d_r}] view")
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
    if q.dim() != 3:
        raise ValueError(f"q must be [B, H, D], got {tuple(q.shape)}")
    B, H, D = q.shape
    if codes.dtype != torch.uint8 or codes.dim() != 3 or codes.shape[0] != B:
        raise ValueError(f"codes must be a uint8 [{B}, W_cap, d_c] view, got {tuple(codes.shape)}")
    W_cap, d_c = codes.shape[1], codes.shape[2]
    d_r = D - d_c
    _need(sigma, torch.float32, "sigma", (B, W_cap))
    if d_r > 0 and (rope is None or rope.dtype != torch.bfloat16 or tuple(rope.shape) != (B, W_cap, d_r)):
        raise ValueError(f"rope must be a bf16 [{B}, {W_cap}, {d_r}] view")
    if n_win is not None:
        _need(n_win, torch.int32, "n_win", (B,))
    if merge_out is not None:
        _need(merge_out, torch.float32, "merge_out", (B, H, d_c))
    if merge_lse is not None:
        _need(merge_lse, torch.float32, "merge_lse", (B, H))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    dev = q.device
    out = _out(out, (B, H, d_c), torch.float32, dev, "out")
    lse = _out(lse, (B, H), torch.float32, dev, "lse")
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
    _need(scores, torch.float32, "scores")
    if scores.dim() != 2:
        raise ValueError(f"scores must be [B, M], got {tuple(scores.shape)}")
    B, M = scores.shape
    dev = scores.device
    if n_valid is not None:
        _need(n_valid, torch.int32, "n_valid", (B,))
    pool_blocks = _out(pool_blocks, (B, P_max), torch.int32, dev, "pool_blocks")
    n_blocks = _out(n_blocks, (B,), torch.int32, dev, "n_blocks")
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
    if q.dim() != 3:
        raise ValueError(f"q must be [B, H, D], got {tuple(q.shape)}")
    B, H, D = q.shape
    N_cap = codes.shape[1]
    d_c = codes.shape[2] * 2
    d_r = D - d_c
    _cache_views(codes, scales, rope, d_r, 3)
    _need(idx, torch.int32, "idx")
    if idx.dim() != 2 or idx.shape[0] != B:
        raise ValueError(f"idx must be [B={B}, K], got {tuple(idx.shape)}")
    K = idx.shape[1]
    if codes.shape[0] < B:
        raise ValueError(f"the cache holds {codes.shape[0]} sequences, {B} queries need one each")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    dev = q.device
    out = _out(out, (B, H, d_c), torch.float32, dev, "out")
    if lse is not None or want_lse:
        lse = _out(lse, (B, H), torch.float32, dev, "lse")
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


def csa2_sparse_swa_attn_workspace_bytes(B, H, d_c, K):
    return int(load().csa2_sparse_swa_attn_workspace_bytes(B, H, d_c, K))


def csa2_sparse_swa_attn_fp4(q, codes, scales, rope, idx, w_codes, w_sigma, w_rope, sm_scale=None, n_win=None,
                             out=None, lse=None, workspace=None, want_lse=True):
    """Sparse attention over the selected FP4 entries and the FP8 window rows
    (w_codes [B, W_cap, d_c] E4M3, w_sigma [B, W_cap], w_rope [B, W_cap, d_r]
    as from alloc_window) in one softmax: returns (out f32 [B, H, d_c],
    lse f32 [B, H])."""
    lib = load()
    _need(q, torch.bfloat16, "q")
    if q.dim() != 3:
        raise ValueError(f"q must be [B, H, D], got {tuple(q.shape)}")
    B, H, D = q.shape
    N_cap = codes.shape[1]
    d_c = codes.shape[2] * 2
    d_r = D - d_c
    _cache_views(codes, scales, rope, d_r, 3)
    _need(idx, torch.int32, "idx")
    if idx.dim() != 2 or idx.shape[0] != B:
        raise ValueError(f"idx must be [B={B}, K], got {tuple(idx.shape)}")
    K = idx.shape[1]
    if codes.shape[0] < B:
        raise ValueError(f"the cache holds {codes.shape[0]} sequences, {B} queries need one each")
    if w_codes.dtype != torch.uint8 or w_codes.dim() != 3 or w_codes.shape[0] != B or w_codes.shape[2] != d_c:
        raise ValueError(f"w_codes must be a uint8 [{B}, W_cap, {d_c}] view, got {tuple(w_codes.shape)}")
    W_cap = w_codes.shape[1]
    _need(w_sigma, torch.float32, "w_sigma", (B, W_cap))
    if d_r > 0 and (w_rope is None or w_rope.dtype != torch.bfloat16 or tuple(w_rope.shape) != (B, W_cap, d_r)):
        raise ValueError(f"w_rope must be a bf16 [{B}, {W_cap}, {d_r}] view")
    if n_win is not None:
        _need(n_win, torch.int32, "n_win", (B,))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    dev = q.device
    out = _out(out, (B, H, d_c), torch.float32, dev, "out")
    if lse is not None or want_lse:
        lse = _out(lse, (B, H), torch.float32, dev, "lse")
    need = csa2_sparse_swa_attn_workspace_bytes(B, H, d_c, K)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    cs = _row_stride(codes, 1, "codes")
    ss = _row_stride(scales, 1, "scales")
    rs = _row_stride(rope, 2, "rope") if d_r > 0 else 0
    wcs = _row_stride(w_codes, 1, "w_codes")
    wrs = _row_stride(w_rope, 2, "w_rope") if d_r > 0 else 0
    st = lib.csa2_sparse_swa_attn_fp4(_ptr(q), _ptr(codes), cs, _ptr(scales), ss, _ptr(rope if d_r > 0 else None),
                                      rs, _ptr(idx), K, B, H, d_c, d_r, N_cap, _ptr(w_codes), wcs, _ptr(w_sigma),
                                      _ptr(w_rope if d_r > 0 else None), wrs, _ptr(n_win), W_cap, float(sm_scale),
                                      _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream())
    _check("csa2_sparse_swa_attn_fp4", st)
    return out, lse


def csa2_prefill_sparse_attn_fp4(q, codes, scales, rope, idx, sm_scale=None, out=None, lse=None, workspace=None,
                                 want_lse=True):
    """Prefill sparse attention: q bf16 [S, T, H, D], idx i32 [S, T, K], one
    cache per sequence (codes, scales, rope: [S, N_cap, *] views as from
    alloc_cache): returns (out f32 [S, T, H, d_c], lse f32 [S, T, H])."""
    lib = load()
    _need(q, torch.bfloat16, "q")
    _need(idx, torch.int32, "idx")
    if q.dim() != 4:
        raise ValueError(f"q must be [S, T, H, D], got {tuple(q.shape)}")
    S, T, H, D = q.shape
    N_cap = codes.shape[1]
    d_c = codes.shape[2] * 2
    d_r = D - d_c
    _cache_views(codes, scales, rope, d_r, 3)
    if idx.dim() != 3 or tuple(idx.shape[:2]) != (S, T):
        raise ValueError(f"idx must be [S={S}, T={T}, K], got {tuple(idx.shape)}")
    K = idx.shape[2]
    if codes.shape[0] < S:
        raise ValueError(f"the cache holds {codes.shape[0]} sequences, the chunk needs {S}")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    dev = q.device
    out = _out(out, (S, T, H, d_c), torch.float32, dev, "out")
    if lse is not None or want_lse:
        lse = _out(lse, (S, T, H), torch.float32, dev, "lse")
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
