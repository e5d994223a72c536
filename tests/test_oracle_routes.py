"""The two oracle routes pinned against each other.

The numpy statement (oracle/dsa.py) and the plain C++ one
(oracle/cpp/dsa_oracle.cpp) are written separately from the same
definitions; neither calls the other.  On every workload shape they must give
the same float32 scores (both round one binary64 sum; the sums differ only in
order, so a rare one-ulp split next to a rounding boundary is allowed), the
same indices and counts, and attention equal to binary64 noise.  A slip in
either (a dropped term, a wrong index, a transposed operand, a wrong tie rule)
shows up here as well as in the closed-form pins that both routes run.
"""

import numpy as np
import pytest

import oracle
import oracle.cpp
from tests.helpers import run_oracle
from workloads import make_batch, oracle_arrays, small_workload

CASES = [
    small_workload("int", lengths=[1, 700, 2100, 5000], mode="int", seed=11, K=256),
    small_workload("gauss", lengths=[1, 700, 2100, 5000], seed=12, K=256),
    small_workload("mxfp8", lengths=[300, 4000], seed=13, K=512, indexer_fmt="mxfp8"),
    small_workload("mxfp8_int", lengths=[300, 2000], seed=17, K=128, indexer_fmt="mxfp8",
                   mode="int"),
    small_workload("cand", lengths=[300, 4000], seed=14, K=128, n_cand=1000),
    small_workload("prefill", lengths=[3000], prefill_rows=5, seed=15, K=256),
    small_workload("separate_v", lengths=[100, 3000], seed=16, K=64, latent=False, D_qk=64,
                   D_v=64, H_q=8, table="shuffled", mode="int"),
    small_workload("fp8_kv", lengths=[100, 3000], seed=18, K=256, kv_fmt="fp8", mode="int",
                   table="shuffled"),
]


@pytest.mark.parametrize("wl", CASES, ids=[c.name for c in CASES])
def test_numpy_and_cpp_routes_agree(wl):
    arr = oracle_arrays(make_batch(wl, seed=wl.seed))
    a = run_oracle(arr, impl="numpy")
    c = run_oracle(arr, impl="cpp")
    split = 0
    for sa, sc in zip(a["scores"], c["scores"]):
        assert len(sa) == len(sc)
        d = sa.view(np.uint32).astype(np.int64) - sc.view(np.uint32).astype(np.int64)
        assert np.abs(d).max(initial=0) <= 1
        split += int((d != 0).sum())
    assert split <= 2
    if split == 0:
        assert (a["indices"] == c["indices"]).all()
    assert (a["counts"] == c["counts"]).all()
    same = (a["indices"] == c["indices"]).all(axis=1)
    assert np.abs(a["out"][same] - c["out"][same]).max(initial=0) <= 1e-12
    assert np.abs(a["lse"][same] - c["lse"][same]).max(initial=0) <= 1e-12
    if wl.mode == "int":
        # integer inputs: scores are integers, so both routes are exact
        assert split == 0 and (a["indices"] == c["indices"]).all()


def test_cpp_thread_count_does_not_change_the_result():
    wl = CASES[1]
    arr = oracle_arrays(make_batch(wl, seed=wl.seed))
    one = run_oracle(arr, impl="cpp")
    kw = {k: arr.get(k) for k in ("qI", "w", "q", "block_table", "seq_lens", "row_seq",
                                  "row_pos")}
    many = oracle.cpp.decode_step(kI_cache=arr["kI_cache"], k_cache=arr["k_cache"],
                                  v_cache=arr["v_cache"], K=arr["K"], scale=arr["scale"],
                                  D_v=arr["D_v"], threads=7, **kw)
    single = oracle.cpp.decode_step(kI_cache=arr["kI_cache"], k_cache=arr["k_cache"],
                                    v_cache=arr["v_cache"], K=arr["K"], scale=arr["scale"],
                                    D_v=arr["D_v"], threads=1, **kw)
    for r in (one, many):
        assert (r["indices"] == single["indices"]).all()
        assert np.array_equal(r["out"], single["out"]) and np.array_equal(r["lse"], single["lse"])
        assert all(np.array_equal(x, y) for x, y in zip(r["scores"], single["scores"]))


@pytest.mark.parametrize("impl", ["numpy", "cpp"])
def test_topk_membership_by_counting(impl):
    # the definition read as a count: position i is kept iff fewer than K
    # positions beat it (a larger score, or an equal score at a lower
    # position).  No sort involved.
    orc = oracle if impl == "numpy" else oracle.cpp
    rng = np.random.default_rng(77)
    for trial in range(20):
        L = int(rng.integers(1, 120))
        K = int(rng.integers(1, 40))
        vals = rng.choice(np.array([-np.inf, -1.5, -0.0, 0.0, 0.5, 2.0, np.inf, np.nan],
                                   np.float32), L)
        if trial % 2:
            vals = rng.standard_normal(L).astype(np.float32)
        # NaN ranks below every number; -0 and +0 are equal
        rank = [(0, 0.0) if np.isnan(x) else (1, 0.0 if x == 0 else float(x)) for x in vals]
        kept = []
        for i in range(L):
            beaten = sum(1 for j in range(L)
                         if rank[j] > rank[i] or (rank[j] == rank[i] and j < i))
            if beaten < K:
                kept.append(i)
        idx, n = orc.topk_row(vals, K)
        assert n == min(K, L) == len(kept)
        assert idx[:n].tolist() == kept and (idx[n:] == -1).all()
