"""Shared test plumbing: run the oracle on the arrays ``workloads`` produced."""

import os

import numpy as np

import oracle
import oracle.cpp

#: the two oracle routes: the numpy statement and the plain C++ one
ORACLES = {"numpy": oracle, "cpp": oracle.cpp}

#: host threads the C++ oracle may use
HOST_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def run_oracle(arr, keep_scores=True, impl=None, rows=None):
    """Oracle decode step over the rows held in ``arr`` (see
    workloads.oracle_arrays).  ``impl``: a module of ORACLES or its name
    (default: the C++ oracle, on HOST_THREADS threads)."""
    if impl is None or isinstance(impl, str):
        impl = ORACLES[impl or "cpp"]
    kw = dict(
        qI=arr["qI"], w=arr["w"], kI_cache=arr["kI_cache"], q=arr["q"],
        k_cache=arr["k_cache"], v_cache=arr["v_cache"], block_table=arr["block_table"],
        seq_lens=arr["seq_lens"], K=arr["K"], scale=arr["scale"], D_v=arr["D_v"],
        row_seq=arr["row_seq"], row_pos=arr["row_pos"], keep_scores=keep_scores, rows=rows,
        qI_scale=arr.get("qI_scale"), kI_scale_cache=arr.get("kI_scale_cache"),
        cand=arr.get("cand"), cand_len=arr.get("cand_len"), k_scale_cache=arr.get("k_scale_cache"))
    if impl is oracle.cpp:
        kw["threads"] = HOST_THREADS
    return impl.decode_step(**kw)


def f32_bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)
