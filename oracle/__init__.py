"""CPU oracle for sparse Multi-head Latent Attention over a paged latent KV cache.

TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library and its Python binding never
do, and nothing here imports them. It shares no code with the HIP path: the only
thing both sides consume in common is the seeded input generator in `workloads`.

It is plain numpy in float64: every step is the textbook definition of what the
pages describe, written out without blocking, fusion or reordering:

  * slot resolution through a page table, with page size 1 as the "virtual block
    table" (The Virtual Block Table: Reusing Triton MLA for Sparse Attention on
    Blackwell GPUs, sections "The Investigation" and "Assumptions and Reasoning");
  * absorbed-MLA attention of every head over its own gathered 576-wide rows,
    value = the first 512 columns of the same row (vLLM PR 63104, bench_shardq_rank.py
    and "Details");
  * the log-sum-exp combine of split partial results (IBM Triton paged-attention
    explainer, section 4 table, "Parallel Tiled Softmax");
  * per-group top-k unions with per-query membership bits in bits 24.. of each entry
    (vLLM PR 63104, "Tests" and "Changes");
  * the cache write, bf16 or fp8 e4m3 with a per-token scale (The Assertion That
    Changed Everything, "The Message" and "Why This Message Was Written").

Every function is pinned by tests against facts the pages or mathematics fix
(closed forms, library routines, brute force, the fp8 format definition).
"""
from .formats import (bf16_bits_to_f64, f32_to_bf16_rne, e4m3_decode, e4m3_encode, E4M3_MAX)
from .reference import (Pool, resolve_slots, attended_slots, attention, sparse_decode,
                        lse_combine, split_attention, group_union, membership_lists,
                        grouped_prefill, kv_write, KV_F32, KV_BF16, KV_FP8, ROW, LATENT, ROPE,
                        ROW_BITS)

__all__ = [n for n in dir() if not n.startswith("_")]
