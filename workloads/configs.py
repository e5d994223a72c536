"""Named workload shapes.

Five shapes of decode and prefill for a DeepSeek/GLM-style sparse-attention
layer: an FP8 indexer of 64 heads x 128 dims over one shared index key per
position, Top-2048 selection, and 128 query heads over one shared bf16 KV
latent of 576 columns (the first 512 of which serve as V).  Page size 64.
"""

from dataclasses import dataclass, replace
import math


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int                      # sequences
    context: int = 0                # tokens per sequence (0: ragged)
    ragged: tuple = ()              # (lo, hi): lengths uniform on [lo, hi]
    lengths: tuple = ()             # explicit per-sequence lengths
    prefill_rows: int = 0           # 0: decode, one row per sequence at its last token
    H_I: int = 64
    D_I: int = 128
    H_q: int = 128
    D_qk: int = 576
    D_v: int = 512
    K: int = 2048
    scale: float = 1.0 / math.sqrt(576.0)
    mode: str = "gauss"             # "int": q/k integers in [-8, 8], w in {0..3}
    latent: bool = True             # V = first D_v columns of the K row
    table: str = "identity"         # "identity" or "shuffled" block table
    seed: int = 0
    # indexer operands: "e4m3" unscaled codes, or "mxfp8" codes with one E8M0
    # scale per 32 dims (integer mode: codes in [-4, 4], scales 2**-1 .. 2**1)
    indexer_fmt: str = "e4m3"
    # candidate-restricted indexer: each row scores only n_cand of its
    # positions (a seeded uniform subset, ascending; rows shorter than n_cand
    # take every position); 0: the whole history
    n_cand: int = 0
    # KV cache: "bf16" rows, or "fp8": E4M3 codes with one float32 scale per
    # tile of 128 elements of each row (latent layout only)
    kv_fmt: str = "bf16"

    @property
    def rows(self) -> int:
        return self.prefill_rows if self.prefill_rows else self.batch

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


CONFIGS = {
    # batch 1, context 1024; 4 x 64 integer indexer; Top-64; 8 query heads
    # over separate K and V of head dim 64
    "tiny_decode_1x1k": Workload(
        name="tiny_decode_1x1k", batch=1, context=1024, H_I=4, D_I=64, H_q=8,
        D_qk=64, D_v=64, K=64, scale=1.0 / 8.0, mode="int", latent=False, seed=1),
    # batch 32 x 32768
    "decode_32x32k": Workload(name="decode_32x32k", batch=32, context=32768, seed=2),
    # 4096 new query tokens on a 61440-token prefix: one sequence of 65536,
    # rows at positions 61440 .. 65535
    "prefill_4096_on_61440": Workload(
        name="prefill_4096_on_61440", batch=1, context=65536, prefill_rows=4096, seed=3),
    # batch 4 x 131072: the bandwidth-bound long-context decode step
    "long_decode_4x128k": Workload(name="long_decode_4x128k", batch=4, context=131072, seed=4),
    # 64 requests, lengths uniform on [1024, 131072], shuffled block table
    "ragged_64_1k_128k": Workload(
        name="ragged_64_1k_128k", batch=64, ragged=(1024, 131072), table="shuffled", seed=5),
}

#: the workload the benchmark's headline number is quoted on
BENCH_WORKLOAD = "long_decode_4x128k"


def small_workload(name, batch=3, context=0, lengths=None, **kw) -> Workload:
    """A reduced shape for oracle-speed tests (same dims as the large ones
    unless overridden)."""
    if lengths is not None:
        kw["lengths"] = tuple(int(x) for x in lengths)
        batch = len(kw["lengths"])
    return Workload(name=name, batch=batch, context=context).with_(**kw)
