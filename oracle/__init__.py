"""CPU oracle for the indexer -> Top-K -> sparse-attention hot path.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, double-precision
statement of what the hot path computes.  Only the test-suite, the smoke check
of the package entry point and the CPU-baseline leg of the benchmark may import
it.  The product (the HIP library and its Python binding) never imports, links
or calls anything in here, and nothing in here imports the product: the two
share no code, tables or helpers.  Inputs come from the separate seeded
generators in ``workloads``; nothing in here ever consumes a value produced by
the GPU path.

Sources (the method is defined in prose only; no page prints code or a worked
numeric example for any step):

* Baidu AI Cloud, "Day0 Inference Support and Performance Optimization for New
  Architecture LLMs":
  - section 2.2: an indexer scores each query against all historical
    positions, the per-head scores are aggregated with head weights, the
    Top-K positions are selected, and the attention core reads only those KV
    rows;
  - section 4.1: the indexer operator reads the paged K cache directly;
  - section 4.2: the attention core gathers the selected rows of the main KV
    cache from the indexer's position list;
  - section 4.3: the fused call takes the quantised query, the index keys and
    the head weights and returns the selected positions; before it, the
    indexer prolog projects q and the head weights, normalises the new key
    and quantises q per group (``prolog.py``);
  - section 5.1 / 5.2: FP8 storage for the indexer and the KV cache; the
    indexer's MXFP8 format (one shared scale per group of 32); the KV cache's
    per-token tiles of 128 elements with one scale each.
* vLLM's DeepSeek-V4.1-Flash article, "Kernels": later indexer layers score
  only a fixed set of candidate positions and take their top-k from it.
* "Bandwidth-Aware LLM Inference on Heterogeneous Many-Core Supercomputers"
  (THInfer), eq. 9: softmax attention softmax(Q K^T / sqrt(d)) V, used here as
  the dense reference; section III.B.4: fp32 (here: fp64) accumulation.
* "SPLASH: Switching Parallel Layouts of Attention with Seamless Handoff for
  LLM Serving" (summary page), section 2 and appendix E: one KV latent shared
  by every query head; two layouts give the same result up to floating-point
  reduction order.

Readings of points the pages leave open (ReLU gate, tie rule, output order,
latent V = leading D_v columns of the K row, history inclusive of the current
token) are stated where each function uses them.

Two routes state the same definitions: this numpy package, and the plain C++
file ``cpp/dsa_oracle.cpp`` (its own decoders, binary64 loops, a full sort,
the softmax definition), loaded through ``oracle.cpp``.  They share no code;
the tests pin each against the other and run every closed-form pin on both.

Parity status: every function here is pinned by tests under ``tests/`` that do
not re-type its formula (closed forms, brute force, library routines,
invariants).  The constants the pages never fix (ReLU gate, K, block size 64,
head dims, attention scale) are readings, not values the pages confirm.
"""

from .formats import E4M3_TABLE, KV_TILE, e4m3_to_f64, e8m0_to_f64, bf16_to_f64, kv_fp8_to_f64, kv_tiles
from .dsa import (
    resolve_rows,
    gather_positions,
    row_history,
    indexer_scores_row,
    score_keys,
    topk_row,
    sparse_attn_row,
    sparse_attn_values,
    masked_dense_attn_row,
    dense_causal_attn_row,
    decode_step,
)
from .prolog import (
    MX_GROUP,
    bf16_round,
    e4m3_round,
    mx_quantize,
    mx_dequantize,
    rms_norm,
    indexer_prolog,
)

__all__ = [
    "E4M3_TABLE", "KV_TILE", "e4m3_to_f64", "e8m0_to_f64", "bf16_to_f64", "kv_fp8_to_f64",
    "kv_tiles", "resolve_rows", "gather_positions", "row_history", "indexer_scores_row",
    "score_keys", "topk_row", "sparse_attn_row", "sparse_attn_values", "masked_dense_attn_row",
    "dense_causal_attn_row", "decode_step", "MX_GROUP", "bf16_round", "e4m3_round",
    "mx_quantize", "mx_dequantize", "rms_norm", "indexer_prolog",
]
