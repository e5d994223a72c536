"""Shared test plumbing: run the oracle on the arrays ``workloads`` produced."""

import numpy as np

import oracle


def run_oracle(arr, keep_scores=True):
    """Oracle decode step over every row held in ``arr`` (see workloads.oracle_arrays)."""
    return oracle.decode_step(
        qI=arr["qI"], w=arr["w"], kI_cache=arr["kI_cache"], q=arr["q"],
        k_cache=arr["k_cache"], v_cache=arr["v_cache"], block_table=arr["block_table"],
        seq_lens=arr["seq_lens"], K=arr["K"], scale=arr["scale"], D_v=arr["D_v"],
        row_seq=arr["row_seq"], row_pos=arr["row_pos"], keep_scores=keep_scores,
        qI_scale=arr.get("qI_scale"), kI_scale_cache=arr.get("kI_scale_cache"),
        cand=arr.get("cand"), cand_len=arr.get("cand_len"))


def f32_bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)
