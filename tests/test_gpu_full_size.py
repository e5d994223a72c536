"""GPU parity at the full workload sizes, through dsa_decode_step as the
benchmark launches it (one call over the whole batch, workspace from
dsa_workspace_size, the default stream).

Every row is checked for what holds at any size: the count is min(K, L),
the kept positions are ascending, distinct and inside the history, the
rest is -1, and the output is finite with no device error.  Sampled rows
(the first, the last, the longest and shortest history, and a seeded
random pick) are compared element by element with the oracle: integer
mode -- indices bit-exact and attention within tolerance; Gaussian mode
(every workload shape) -- Top-K recall >= 0.999 and attention within
tolerance against the oracle's attention over the GPU's own indices."""

import numpy as np
import pytest
import torch

from tests.gpu_helpers import (RECALL_MIN, check_attention, fp8_kv_lse_slack, gpu_decode, np_,
                               oracle_attention_on, recall, say)
from tests.helpers import run_oracle
from workloads import BENCH_WORKLOAD, CONFIGS, make_batch, oracle_arrays, row_positions

pytestmark = pytest.mark.gpu


def _sample_rows(batch, seed):
    n = batch.rows
    lens = [p + 1 for _, p in row_positions(batch)]
    rows = {0, n - 1, int(np.argmax(lens)), int(np.argmin(lens))}
    if n > 2:
        rows.add(int(np.random.default_rng(seed).integers(1, n - 1)))
    return sorted(rows)


def _check_every_row(batch, res):
    K = batch.wl.K
    gi = np_(res["indices"])
    cnt = np_(res["counts"])
    for i, (_, p) in enumerate(row_positions(batch)):
        n = min(K, p + 1)
        assert int(cnt[i]) == n, f"row {i}: count {cnt[i]} != {n}"
        sel = gi[i, :n]
        assert (np.diff(sel) > 0).all(), f"row {i}: not ascending"
        assert sel[0] >= 0 and sel[-1] <= p, f"row {i}: outside the history"
        assert (gi[i, n:] == -1).all(), f"row {i}: padding"
    assert torch.isfinite(res["out"].float()).all()


@pytest.mark.parametrize("name", list(CONFIGS))
def test_full_size_integer_mode(name):
    wl = CONFIGS[name]
    say(f"full size {name}: {wl.batch} sequences, integer mode, seed {wl.seed}")
    batch = make_batch(wl, device="cuda", seed=wl.seed, mode="int")
    res = gpu_decode(batch)
    _check_every_row(batch, res)
    rows = _sample_rows(batch, wl.seed)
    say(f"  oracle rows {rows}")
    orc = run_oracle(oracle_arrays(batch, rows=rows), keep_scores=False)
    assert (np_(res["counts"])[rows] == orc["counts"]).all()
    gi = np_(res["indices"])[rows]
    for j, r in enumerate(rows):
        assert (gi[j] == orc["indices"][j]).all(), f"row {r}: indices differ"
    check_attention(res["out"][rows], res["lse"][rows], orc["out"], orc["lse"])


# Gaussian mode: the GPU's fp32 scores may order near-equal positions
# differently from the binary64 oracle, so the selection is held to a recall
# bound, and every checked row's attention is compared with the oracle's
# attention over the positions the GPU itself selected.
GAUSS = [(BENCH_WORKLOAD, None), ("decode_32x32k", 8), ("ragged_64_1k_128k", 8),
         ("prefill_4096_on_61440", 6)]


@pytest.mark.parametrize("name,n_rows", GAUSS, ids=[g[0] for g in GAUSS])
def test_full_size_gaussian(name, n_rows):
    wl = CONFIGS[name]
    say(f"full size {name}: Gaussian mode, seed {wl.seed}")
    batch = make_batch(wl, device="cuda", seed=wl.seed, mode="gauss")
    res = gpu_decode(batch)
    _check_every_row(batch, res)
    if n_rows is None:
        rows = list(range(batch.rows))
    else:
        rows = set(_sample_rows(batch, wl.seed))
        pick = np.random.default_rng(wl.seed + 1).permutation(batch.rows)
        rows = sorted(rows | set(int(x) for x in pick[:max(0, n_rows - len(rows))]))
    say(f"  oracle rows {rows}")
    arr = oracle_arrays(batch, rows=rows)
    orc = run_oracle(arr, keep_scores=False)
    gi = np_(res["indices"])[rows]
    gc = np_(res["counts"])[rows]
    assert (gc == orc["counts"]).all()
    rec, worst = recall(gi, orc["indices"], orc["counts"])
    say(f"  recall {rec:.6f} (worst row {worst:.6f})")
    assert rec >= RECALL_MIN
    o_ref, l_ref = oracle_attention_on(arr, gi, gc)
    e_max, e_mean = check_attention(res["out"][rows], res["lse"][rows], o_ref, l_ref)
    say(f"  attention on the GPU's own indices: max {e_max:.3g} mean {e_mean:.3g}")


def test_full_size_mxfp8_indexer_bench_shape():
    # the 4 x 128k decode step with MXFP8 indexer operands (one E8M0 scale
    # per 32 dims of every query head and key row), integer mode: every row's
    # indices bit-exact against the oracle, attention within tolerance
    wl = CONFIGS[BENCH_WORKLOAD].with_(indexer_fmt="mxfp8")
    say(f"full size {BENCH_WORKLOAD}: MXFP8 indexer, integer mode, seed {wl.seed}")
    batch = make_batch(wl, device="cuda", seed=wl.seed, mode="int")
    res = gpu_decode(batch)
    _check_every_row(batch, res)
    rows = list(range(batch.rows))
    orc = run_oracle(oracle_arrays(batch, rows=rows), keep_scores=False)
    assert (np_(res["counts"]) == orc["counts"]).all()
    assert (np_(res["indices"]) == orc["indices"]).all()
    check_attention(res["out"], res["lse"], orc["out"], orc["lse"])


def test_full_size_candidates_bench_shape():
    # the 4 x 128k decode step scoring 16384 candidate positions per row
    # (the candidate-restricted indexer), integer mode: every row's indices
    # bit-exact against the oracle, attention within tolerance
    wl = CONFIGS[BENCH_WORKLOAD].with_(n_cand=16384)
    say(f"full size {BENCH_WORKLOAD}: 16384 candidates per row, integer mode, seed {wl.seed}")
    batch = make_batch(wl, device="cuda", seed=wl.seed, mode="int")
    res = gpu_decode(batch)
    _check_every_row(batch, res)
    rows = list(range(batch.rows))
    orc = run_oracle(oracle_arrays(batch, rows=rows), keep_scores=False)
    assert (np_(res["counts"]) == orc["counts"]).all()
    assert (np_(res["indices"]) == orc["indices"]).all()
    check_attention(res["out"], res["lse"], orc["out"], orc["lse"])


def test_full_size_fp8_kv_bench_shape():
    # the 4 x 128k decode step over an FP8 KV cache (E4M3 latent rows, one
    # float32 scale per tile of 128 elements), integer-mode indexer: every
    # row's indices bit-exact against the oracle, attention within tolerance
    wl = CONFIGS[BENCH_WORKLOAD].with_(kv_fmt="fp8")
    say(f"full size {BENCH_WORKLOAD}: FP8 KV cache, integer mode, seed {wl.seed}")
    batch = make_batch(wl, device="cuda", seed=wl.seed, mode="int")
    res = gpu_decode(batch)
    _check_every_row(batch, res)
    rows = list(range(batch.rows))
    arr = oracle_arrays(batch, rows=rows)
    orc = run_oracle(arr, keep_scores=False)
    assert (np_(res["counts"]) == orc["counts"]).all()
    assert (np_(res["indices"]) == orc["indices"]).all()
    slack = fp8_kv_lse_slack(arr, orc["indices"], orc["counts"])
    e_max, e_mean = check_attention(res["out"], res["lse"], orc["out"], orc["lse"],
                                    lse_slack=slack)
    say(f"  attention: max {e_max:.3g} mean {e_mean:.3g}; lse slack up to {slack.max():.3g}")
