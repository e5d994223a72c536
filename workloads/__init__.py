"""Seeded synthetic inputs for the indexer -> Top-K -> sparse-attention path.

Shared by the oracle's tests, the GPU parity tests, the smoke check and the
benchmark.  This module only draws random numbers and lays them out in the
buffers the library reads; it holds none of the method's arithmetic (no
scoring, selection or attention).  FP8 and bf16 encodings go through torch's
own dtype conversions.

Workloads stand in for the long-context serving workloads the pages measure
(SPLASH's 128K-256K contexts, the agentic serving benchmark of the vLLM
DeepSeek-V4.1-Flash post); none of those suites' items is reproduced.
"""

from .configs import Workload, CONFIGS, BENCH_WORKLOAD, small_workload
from .gen import Batch, make_batch, oracle_arrays, row_positions, kv_fp8_split, kv_scale_rows
from .prolog import PROLOG_D_X, PrologInputs, make_prolog_inputs, prolog_arrays

__all__ = ["Workload", "CONFIGS", "BENCH_WORKLOAD", "small_workload", "kv_fp8_split", "kv_scale_rows",
           "Batch", "make_batch", "oracle_arrays", "row_positions", "PROLOG_D_X", "PrologInputs",
           "make_prolog_inputs", "prolog_arrays"]
