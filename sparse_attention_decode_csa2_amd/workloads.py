"""Seeded synthetic inputs for the CSA2 decode step.

This module only draws random inputs of the shapes, value distributions and
structure the decode workloads use.  It holds none of the method's arithmetic
(no quantisation, no scoring, no selection, no attention), so both the HIP
path and the CPU oracle may take their inputs from it.

Every tensor is drawn from its own ``torch.Generator`` whose seed is derived
from the workload seed, the tensor's name and (for per-sequence tensors) the
sequence index, so any one tensor can be regenerated alone.  Draws made on
``cuda`` and on ``cpu`` differ (different generator engines); a test always
hands the oracle a host copy of the tensors the GPU path consumed.

Workloads (the five decode configurations; entry counts are tokens / 4, one
compressed entry per 4 tokens):

0. tiny-full      B=1,   N=1024,   latent 128 (no RoPE part), 8 heads,
                  indexer 4 x 64, Top-64
1. full-64k       B=1,   N=16384,  latent 512 + RoPE 64, 64 heads,
                  indexer 8 x 128, Top-512
2. reindex-1m     B=32,  N=262144, pool 2048 blocks x 8 positions, Top-512
3. reuse-128k     B=128, N=32768,  index lists handed in (512 unique, sorted)
4. prefill-full-1m  an 8192-row post-RoPE chunk (N(0,1), 1% of elements
                  x20) appended to sequence 0 at rows [253952, 262144), then
                  B=8 Full-mode decode over 262144 entries
5. pool-build-1m  the shapes of reindex-1m, for the layer before it: Full
                  indexer scores over 262144 entries, then the pool of 2048
                  blocks x 8 positions built from them (no attention)
6. reuse-swa-128k reuse-128k plus the sliding-window branch: 128 FP8 window
                  rows per sequence (RMS-normalised N(0,1) latents, one
                  power-of-two scale per row) merged with the sparse result
8. prefill-reuse-1m  a Reuse layer in prefill: an 8192-token chunk at the end
                  of a 1M-token context (262144 entries), every chunk token a
                  query (64 heads) with its own list of 512 entries, unique
                  and uniform over the entries it may see (sorted)
7. sample-129k    the decode sampler: B=128 rows of f32 logits over a
                  129280-token vocabulary (N(0,1) x 4), Top-2048, temperature
                  1 and top_p 1 (the recommended sampling settings), one
                  uniform per row
9. sample-full-129k  the same rows and uniforms (same seed), drawn without a
                  Top-K cap: temperature 1 and top_p 1 over the whole
                  vocabulary
"""

from dataclasses import dataclass
import hashlib
import math

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    mode: str            # "full" | "reindex" | "reuse" | "prefill_full" | "pool_build" | "reuse_swa" | "sample"
                         # | "prefill_reuse" | "sample_full"
    B: int               # decode queries (sequences) per step
    N: int               # compressed entries per sequence (cache capacity)
    d_c: int             # FP4 latent channels
    d_r: int             # bf16 RoPE channels (0 = none)
    H: int               # attention query heads
    H_I: int             # indexer heads
    D_I: int             # indexer dimension
    K: int               # Top-K
    seed: int
    block: int = 8       # positions per pool block
    P_max: int = 2048    # pool capacity in blocks
    n_blocks: int = 2048  # pool blocks drawn per sequence
    prefill_rows: int = 0
    prefill_row0: int = 0
    window: int = 0      # sliding-window rows per sequence (FP8)
    temperature: float = 1.0  # sampler: logits are divided by it
    top_p: float = 1.0   # sampler: nucleus mass

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_c + self.d_r)

    @property
    def D(self) -> int:
        return self.d_c + self.d_r

    def scaled(self, **kw) -> "Workload":
        """Same recipe with some sizes replaced (small parity cases)."""
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = [
    Workload("tiny-full", "full", B=1, N=1024, d_c=128, d_r=0, H=8, H_I=4, D_I=64, K=64, seed=0),
    Workload("full-64k", "full", B=1, N=16384, d_c=512, d_r=64, H=64, H_I=8, D_I=128, K=512, seed=1),
    Workload("reindex-1m", "reindex", B=32, N=262144, d_c=512, d_r=64, H=64, H_I=8, D_I=128, K=512, seed=2),
    Workload("reuse-128k", "reuse", B=128, N=32768, d_c=512, d_r=64, H=64, H_I=8, D_I=128, K=512, seed=3),
    Workload("prefill-full-1m", "prefill_full", B=8, N=262144, d_c=512, d_r=64, H=64, H_I=8, D_I=128,
             K=512, seed=4, prefill_rows=8192, prefill_row0=262144 - 8192),
    Workload("pool-build-1m", "pool_build", B=32, N=262144, d_c=512, d_r=64, H=64, H_I=8, D_I=128, K=512,
             seed=5),
    Workload("reuse-swa-128k", "reuse_swa", B=128, N=32768, d_c=512, d_r=64, H=64, H_I=8, D_I=128, K=512,
             seed=6, window=128),
    Workload("sample-129k", "sample", B=128, N=129280, d_c=0, d_r=0, H=0, H_I=0, D_I=0, K=2048, seed=7),
    Workload("prefill-reuse-1m", "prefill_reuse", B=1, N=262144, d_c=512, d_r=64, H=64, H_I=8, D_I=128, K=512,
             seed=8, prefill_rows=8192),
    Workload("sample-full-129k", "sample_full", B=128, N=129280, d_c=0, d_r=0, H=0, H_I=0, D_I=0, K=0, seed=7),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def _gen(wl: Workload, name: str, b: int, device) -> torch.Generator:
    h = hashlib.sha256(f"{wl.seed}/{name}/{b}".encode()).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
    return g


def latent_rows(wl: Workload, b: int, n: int, device="cpu", name="latent") -> torch.Tensor:
    """bf16 [n, d_c]: N(0,1) rows scaled to unit RMS (the RMSNorm'd latent)."""
    g = _gen(wl, name, b, device)
    x = torch.randn(n, wl.d_c, generator=g, device=device, dtype=torch.float32)
    x = x * torch.rsqrt((x * x).mean(dim=1, keepdim=True))
    return x.to(torch.bfloat16)


def rope_rows(wl: Workload, b: int, n: int, device="cpu") -> torch.Tensor:
    """bf16 [n, d_r]: N(0,1) post-RoPE part (empty when d_r == 0)."""
    g = _gen(wl, "rope", b, device)
    return torch.randn(n, wl.d_r, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def _ints(g, shape, device):
    return torch.randint(-8, 9, shape, generator=g, device=device, dtype=torch.int32).to(torch.bfloat16)


def index_keys(wl: Workload, b: int, device="cpu") -> torch.Tensor:
    """bf16 [N, D_I]: indexer keys, integers uniform in [-8, 8]."""
    return _ints(_gen(wl, "index_keys", b, device), (wl.N, wl.D_I), device)


def index_query(wl: Workload, device="cpu") -> torch.Tensor:
    """bf16 [B, H_I, D_I]: indexer queries, integers uniform in [-8, 8]."""
    return _ints(_gen(wl, "index_query", 0, device), (wl.B, wl.H_I, wl.D_I), device)


def attn_query(wl: Workload, device="cpu") -> torch.Tensor:
    """bf16 [B, H, d_c + d_r]: attention queries, N(0,1)."""
    g = _gen(wl, "attn_query", 0, device)
    return torch.randn(wl.B, wl.H, wl.D, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def _unique_sorted(g, B, k, n, device):
    out = torch.empty(B, k, dtype=torch.int32, device=device)
    for b in range(B):
        out[b] = torch.randperm(n, generator=g, device=device)[:k].sort().values.to(torch.int32)
    return out


def pool_blocks(wl: Workload, device="cpu"):
    """int32 [B, P_max] pool block ids (n_blocks unique, sorted, uniform over
    the N/block blocks; unused slots -1) and int32 [B] block counts."""
    g = _gen(wl, "pool", 0, device)
    blk = torch.full((wl.B, wl.P_max), -1, dtype=torch.int32, device=device)
    blk[:, :wl.n_blocks] = _unique_sorted(g, wl.B, wl.n_blocks, wl.N // wl.block, device)
    nb = torch.full((wl.B,), wl.n_blocks, dtype=torch.int32, device=device)
    return blk, nb


def reuse_index(wl: Workload, device="cpu") -> torch.Tensor:
    """int32 [B, K]: handed-in index lists (unique, sorted, uniform over N)."""
    return _unique_sorted(_gen(wl, "reuse_idx", 0, device), wl.B, wl.K, wl.N, device)


def prefill_chunk(wl: Workload, device="cpu") -> torch.Tensor:
    """bf16 [prefill_rows, d_c]: N(0,1), each element x20 with probability 0.01."""
    g = _gen(wl, "prefill", 0, device)
    x = torch.randn(wl.prefill_rows, wl.d_c, generator=g, device=device, dtype=torch.float32)
    hit = torch.rand(wl.prefill_rows, wl.d_c, generator=g, device=device) < 0.01
    return torch.where(hit, x * 20.0, x).to(torch.bfloat16)


def prefill_rope(wl: Workload, device="cpu") -> torch.Tensor:
    g = _gen(wl, "prefill_rope", 0, device)
    return torch.randn(wl.prefill_rows, wl.d_r, generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def random_codes(wl: Workload, b: int, n: int, device="cpu", scale_lo=0x20, scale_hi=0x48):
    """Raw cache bytes for attention-only tests: uniform FP4 code bytes and
    E4M3 scale bytes uniform in [scale_lo, scale_hi] (finite, positive)."""
    g = _gen(wl, "raw_codes", b, device)
    codes = torch.randint(0, 256, (n, wl.d_c // 2), generator=g, device=device, dtype=torch.int32)
    scales = torch.randint(scale_lo, scale_hi + 1, (n, wl.d_c // 16), generator=g, device=device,
                           dtype=torch.int32)
    return codes.to(torch.uint8), scales.to(torch.uint8)


def bf16_bits(t: torch.Tensor):
    """Host numpy uint16 view of a bf16 tensor (for the oracle)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")


def vocab_logits(wl: Workload, device="cpu", name="logits") -> torch.Tensor:
    """f32 [B, N]: next-token logits, N(0,1) x 4 (a peaked distribution: at
    temperature 1 the 2048 largest of 129280 hold 95-97 % of the mass)."""
    g = _gen(wl, name, 0, device)
    return torch.randn(wl.B, wl.N, generator=g, device=device, dtype=torch.float32) * 4.0


def sampler_uniforms(wl: Workload, device="cpu", name="uniforms") -> torch.Tensor:
    """f32 [B]: the sampler's uniforms in [0, 1)."""
    return torch.rand(wl.B, generator=_gen(wl, name, 0, device), device=device, dtype=torch.float32)


def chunk_visible(wl: Workload, t) -> torch.Tensor:
    """Entries query t of a prefill chunk may see: the chunk is the last T =
    prefill_rows tokens of a context of 4 N tokens, and entry e (tokens 4e ..
    4e + 3) is visible once its last token is at or before the query's."""
    T = wl.prefill_rows
    p0 = 4 * wl.N - T
    return (p0 + torch.as_tensor(t) + 1) // 4


def chunk_index(wl: Workload, device="cpu") -> torch.Tensor:
    """int32 [B, T, K]: each chunk query's list, K unique entries uniform over
    the entries it may see, sorted (all of them, padded with -1, when it sees
    fewer than K).  Drawn as the first K distinct values of i.i.d. uniform
    draws, which is a uniform K-subset (a random permutation's first K when
    the range is at most 4 K)."""
    T, K = wl.prefill_rows, wl.K
    out = torch.full((wl.B, T, K), -1, dtype=torch.int32)
    vis = chunk_visible(wl, torch.arange(T))
    for b in range(wl.B):
        g = _gen(wl, "chunk_idx", b, "cpu")
        D = K + K // 2 + 64
        draws = (torch.rand(T, D, generator=g, dtype=torch.float64) * vis[:, None]).floor().long()
        srt, order = torch.sort(draws, dim=1, stable=True)
        dup_sorted = torch.zeros_like(srt, dtype=torch.bool)
        dup_sorted[:, 1:] = srt[:, 1:] == srt[:, :-1]
        dup = torch.zeros_like(dup_sorted).scatter_(1, order, dup_sorted)   # later repeats, in draw order
        rank = torch.cumsum((~dup).long(), dim=1)
        keep = (~dup) & (rank <= K)
        for t in range(T):
            v = int(vis[t])
            if v <= K:
                out[b, t, :v] = torch.arange(v, dtype=torch.int32)
                continue
            if v <= 4 * K:        # a small range: the draws may hold fewer than K distinct values
                out[b, t] = torch.sort(torch.randperm(v, generator=g)[:K]).values.to(torch.int32)
                continue
            sel = draws[t][keep[t]]
            assert sel.numel() == K, "too few distinct draws"
            out[b, t] = torch.sort(sel).values.to(torch.int32)
    return out.to(device)
