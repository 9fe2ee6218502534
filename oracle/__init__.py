"""CPU oracle for the CSA2 FP4 sparse-attention decode step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The product path (the HIP library and its Python binding) never imports,
calls or links it, and this package never imports the product path.

Everything here is plain NumPy in float64 (integer work in int64 / uint8),
written from the format definitions and from the method as the pages
describe it.  Nothing is blocked, fused or reordered beyond what the
definitions state, so each function can be checked against its source by eye.

Page keys used in citations (the pages are secondary write-ups of the
DeepSeek-V4.1-Flash technical report, arXiv 2609.19969):

* [P1] "DeepSeek-V4.1-Flash：把 KV Cache 压缩到极限的百万上下文 MoE（技术报告全系统解读）"
  (ai-engineering-6yk.pages.dev, ch01/059)
* [P2] "DeepSeek-V4.1-Flash：突破 KV Cache 压缩极限的长上下文 MoE 模型"
  (papers.ananclaw.com explainer 2609-19969)
* [P3] "552B参数干掉1.6T：DeepSeek V4.1 Flash技术深度解析" (55zb.com)
* [P4] "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
  (agihunt.info paper page 2609.19969)

Parity status per function (the pins live in ``tests/test_oracle_*.py``):

* codec (bf16 / E2M1 / E4M3 decode and encode): pinned (closed forms, the
  E2M1 value set, torch's float8_e4m3fn cast, numpy's round-half-even).
* quantize_fp4 / dequantize_fp4: pinned (hand-derived fixtures, invariants).
* index_full / index_pool: pinned (int64 matmul, brute-force loops).
* topk: pinned (brute-force sort, torch.topk / stable sort special cases).
* quantize_fp8 / swa_attn / merge_branches: pinned (hand-derived scales and
  codes, torch's float8_e4m3fn cast, float64 SDPA over the window and over the
  union of the selected entries and the window).
* build_pool: pinned (hand-derived fixture, brute-force selection, and Reindex
  over the built pool reproducing the Full-mode Top-K).
* sparse_attn: pinned (dense float64 SDPA when Top-K covers every entry,
  closed-form special cases, logsumexp).
* prefill_sparse_attn: pinned (float64 SDPA with a causal mask over two
  sequences with different caches, every visible entry selected).
* sample: pinned (hand-derived draws, the token frequencies over a grid of
  uniforms against scipy's softmax, the nucleus' minimality, greedy and
  single-candidate limits).
* sample_full: pinned (hand-derived draws, token frequencies against scipy's
  softmax over the whole vocabulary, the inverse-CDF boundary checked with
  exactly rounded sums, the vanishing-temperature limit).
"""

from .codec import (  # noqa: F401
    bf16_bits_to_f64,
    f64_to_bf16_bits_exact,
    e2m1_decode,
    e2m1_encode_magnitude,
    e4m3_decode,
    e4m3_encode,
    e4m3_scale_code_for_amax,
)
from .method import (  # noqa: F401
    quantize_fp4,
    dequantize_fp4,
    index_scores,
    index_full,
    index_pool,
    topk,
    build_pool,
    sparse_attn,
    prefill_sparse_attn,
    fp8_row_scale_exponent,
    quantize_fp8,
    dequantize_fp8,
    swa_attn,
    merge_branches,
    sample,
    sample_full,
    decode_full,
    decode_reindex,
    decode_reuse,
)
