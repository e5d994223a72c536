"""The allocation-free fused step, dsa_decode_step_static, against
dsa_decode_step with a workspace, through the C ABI.

Two calls in a row share the library's scratch: the 4 x 131072 decode batch
(Gaussian), then a smaller ragged batch whose rows take every selection
route (histories shorter than K, full-row and summary selections).  Both
entry points run the same kernels on the same inputs, so indices, counts,
outputs and lse must agree bit for bit, and no device error may be raised."""

import pytest
import torch

from indexer_top_sparse_score_amd import binding as B
from tests.gpu_helpers import gpu_decode, kv_and_v, say
from workloads import BENCH_WORKLOAD, CONFIGS, make_batch, small_workload

pytestmark = pytest.mark.gpu


def _static(batch):
    prob = B.problem_for_batch(batch)
    wl = batch.wl
    out = torch.full((batch.rows, wl.H_q, wl.D_v), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((batch.rows, wl.H_q), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((batch.rows, wl.K), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((batch.rows,), -7, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    k, v = kv_and_v(batch)
    B.dsa_decode_step_static(prob, batch.qI, batch.w, batch.kI, batch.q, k, v, out, lse=lse,
                             indices=idx, counts=cnt, err=err)
    torch.cuda.synchronize()
    return {"out": out, "lse": lse, "indices": idx, "counts": cnt, "err": int(err.item())}


def _same(a, b, what):
    assert a["err"] == 0, f"{what}: device error {a['err']:#x}"
    for key in ("indices", "counts"):
        assert torch.equal(a[key], b[key]), f"{what}: {key} differ"
    for key in ("out", "lse"):
        x, y = a[key].float(), b[key].float()
        same = (x == y) | (torch.isnan(x) & torch.isnan(y))
        assert bool(same.all()), f"{what}: {key} differ"


def test_static_scratch_matches_workspace_entry_point():
    big = CONFIGS[BENCH_WORKLOAD]
    small = small_workload("no_alloc_small", lengths=[1, 700, 2048, 5000, 20000, 70000],
                           mode="gauss", table="shuffled")
    for wl, seed in ((big, 31), (small, 32)):
        say(f"static scratch: {wl.name}, {wl.batch} sequences, seed {seed}")
        batch = make_batch(wl, device="cuda", seed=seed)
        got = _static(batch)
        want = gpu_decode(batch)
        _same(got, want, wl.name)
        del batch
