"""GPU parity at oracle-speed sizes: every entry point against the oracle,
element by element, on shapes that span several tiles and ragged tails.

Bars: integer mode -- scores and indices bit-exact; Gaussian mode -- scores
within the float32 forward-error bound, Top-K recall >= 0.999, and Top-K
bit-exact when both sides select from the same scores; attention -- max
|error| <= 2e-2 and mean |error| <= 2e-3 against the oracle on the same
indices."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from indexer_top_sparse_score_amd import binding as B
from tests.gpu_helpers import (RECALL_MIN, check_attention, check_scores_exact, fp8_kv_lse_slack,
                               gpu_attn, gpu_decode, gpu_scores, gpu_topk, np_,
                               oracle_attention_on, recall, say, score_bound, score_ld)
from tests.helpers import run_oracle
from workloads import CONFIGS, make_batch, oracle_arrays, row_positions, small_workload

pytestmark = pytest.mark.gpu

# lengths chosen to hit: a single position, a partial first page, exact page
# and tile edges, L < K, L == K, L == K + 1, several 1024-position tiles and
# ragged last pages
LENGTHS = [1, 63, 64, 65, 1000, 2048, 2049, 4097, 5000]
MLA = dict(H_I=64, D_I=128, H_q=128, D_qk=576, D_v=512, K=2048, scale=576 ** -0.5)
TINY = dict(H_I=4, D_I=64, H_q=8, D_qk=64, D_v=64, K=64, scale=0.125, latent=False)

CASES = {
    "mla_int": dict(lengths=LENGTHS, mode="int", **MLA),
    "mla_int_shuffled": dict(lengths=LENGTHS, mode="int", table="shuffled", **MLA),
    "tiny_int": dict(lengths=[1, 50, 64, 1024, 3000], mode="int", **TINY),
    "mla_int_k100": dict(lengths=[99, 100, 101, 3000], mode="int", **{**MLA, "K": 100}),
    "mla_int_k1": dict(lengths=[1, 2, 700], mode="int", **{**MLA, "K": 1}),
    "h48_d64": dict(lengths=[777, 2500], mode="int", **{**MLA, "H_I": 48, "D_I": 64, "H_q": 80}),
    # 576/512 with a separate V cache (not the latent layout)
    "mla_sepv": dict(lengths=[1, 777, 3000], mode="int", latent=False, **MLA),
    # histories on both sides of the Top-K's split threshold (16384 in one
    # workgroup, 16385 over slices) and long enough for summary segments of
    # 32 and 64 positions
    "mla_int_grouped": dict(lengths=[9000, 16384, 16385, 20000, 40000], mode="int", **MLA),
    # MXFP8 indexer operands (one E8M0 scale per 32 dims), both head dims
    "mla_mx_int": dict(lengths=LENGTHS, mode="int", indexer_fmt="mxfp8", **MLA),
    "h48_d64_mx": dict(lengths=[777, 2500], mode="int", indexer_fmt="mxfp8",
                       **{**MLA, "H_I": 48, "D_I": 64, "H_q": 80}),
    # candidate-restricted rows: short lists (one workgroup per row; rows up
    # to 1500 positions take every position), lists long enough to split
    # (a length that is not a multiple of 4, then one that is, with MXFP8)
    "mla_cand_int": dict(lengths=LENGTHS, mode="int", n_cand=1500, **MLA),
    "mla_cand_split": dict(lengths=[20000, 70000, 131072], mode="int", n_cand=17001, **MLA),
    "mla_mx_cand": dict(lengths=[5000, 40000], mode="int", indexer_fmt="mxfp8", n_cand=16388,
                        **MLA),
    "tiny_cand": dict(lengths=[1, 50, 64, 1024, 3000], mode="int", n_cand=700, **TINY),
    # FP8 KV cache: E4M3 latent rows with one float32 scale per tile of 128
    "mla_fp8kv": dict(lengths=LENGTHS, mode="int", kv_fmt="fp8", table="shuffled", **MLA),
    # 16 rows and more: bf16 latent rows take the 64-head attention workgroups
    # (no key split), also with a head count that leaves the second workgroup
    # of a row 16 heads; FP8 rows keep the 32-head kernel
    "mla_wide": dict(lengths=LENGTHS * 2, mode="int", table="shuffled", **MLA),
    "h80_wide": dict(lengths=[777, 2500] * 8 + [3000], mode="int",
                     **{**MLA, "H_I": 48, "D_I": 64, "H_q": 80}),
    "mla_fp8kv_wide": dict(lengths=LENGTHS * 2, mode="int", kv_fmt="fp8", **MLA),
}


def _batch(name, seed=21, **over):
    kw = dict(CASES[name])
    kw.update(over)
    lengths = kw.pop("lengths")
    wl = small_workload(name, lengths=lengths, **kw)
    say(f"case {name} seed {seed} lengths {lengths}")
    return make_batch(wl, device="cuda", seed=seed)


@pytest.mark.parametrize("name", list(CASES))
def test_scores_exact_integer_mode(name):
    batch = _batch(name)
    arr = oracle_arrays(batch)
    orc = run_oracle(arr)
    check_scores_exact(gpu_scores(batch), orc, row_positions(batch))


@pytest.mark.parametrize("name", ["mla_int", "mla_mx_int"])
def test_scores_gaussian_within_fp32_bound(name):
    batch = _batch(name, mode="gauss", seed=22)
    arr = oracle_arrays(batch)
    orc = run_oracle(arr)
    g = np_(gpu_scores(batch))
    for i, (_, p) in enumerate(row_positions(batch)):
        want = orc["scores"][i].astype(np.float64)
        got = g[i, :p + 1].astype(np.float64)
        ulp = np.spacing(np.abs(orc["scores"][i])).astype(np.float64)
        bound = score_bound(arr, i, p) + ulp
        assert (np.abs(got - want) <= bound).all(), f"row {i}"
        assert np.isnan(g[i, p + 1:]).all()


@pytest.mark.parametrize("name", list(CASES))
def test_topk_exact_on_oracle_scores(name):
    # both sides select from the same float32 scores: indices must be identical
    batch = _batch(name, mode="gauss", seed=23)
    arr = oracle_arrays(batch)
    orc = run_oracle(arr)
    ld = score_ld(batch)
    sc = np.full((batch.rows, ld), np.nan, np.float32)
    for i, s in enumerate(orc["scores"]):
        sc[i, :len(s)] = s
    idx, cnt = gpu_topk(batch, torch.from_numpy(sc).cuda())
    assert (np_(cnt) == orc["counts"]).all()
    assert (np_(idx) == orc["indices"]).all()


def test_topk_ties_and_special_values():
    # heavy ties, signed zeros, infinities, all-equal rows: exact vs the oracle
    # (rows of more than 16384 positions split over slices unless their ties
    # or NaNs send them down the streamed path; shorter rows select on their
    # keys in one workgroup)
    wl = small_workload("ties", lengths=[5000, 5000, 5000, 5000, 3000, 2049, 20000, 40000,
                                         40000, 9000, 131072, 131072, 70000], **MLA)
    batch = make_batch(wl, device="cuda", seed=24)
    rng = np.random.default_rng(24)
    ld = 64 * batch.max_blocks
    sc = np.full((batch.rows, ld), np.nan, np.float32)
    L = batch.lengths
    sc[0, :L[0]] = rng.integers(0, 7, L[0])                        # 7 distinct values
    sc[1, :L[1]] = 3.0                                              # all equal
    sc[2, :L[2]] = rng.choice(np.array([-0.0, 0.0, 1.0, -1.0], np.float32), L[2])
    sc[3, :L[3]] = rng.choice(np.array([-np.inf, np.inf, 5.0, -2.0], np.float32), L[3])
    sc[4, :L[4]] = rng.standard_normal(L[4]).astype(np.float32) * 1e-30  # subnormal-ish range
    sc[5, :L[5]] = -np.arange(L[5], dtype=np.float32)              # K+1 distinct, descending
    sc[6, :L[6]] = rng.integers(0, 3, L[6])                        # 3 distinct values: streamed
    sc[7, :L[7]] = 1.5                                              # all equal: streamed
    sc[8, :L[8]] = np.where(rng.random(L[8]) < 0.99, np.nan,       # mostly NaN: t = 0
                            rng.standard_normal(L[8])).astype(np.float32)
    x = rng.standard_normal(L[9]).astype(np.float32)                # a few exact ties near
    x[rng.choice(L[9], 300, replace=False)] = np.sort(x)[-2100]     # the threshold (one workgroup)
    sc[9, :L[9]] = x
    # 32 slices of 4096 positions: scores on a 1/64 grid tie some 80 ways at
    # the threshold, so the budget of keys equal to T spans several slices
    sc[10, :L[10]] = np.round(rng.standard_normal(L[10]) * 64) / 64
    # the best keys packed into a few thousand recent positions: one slice
    # holds far more candidates than its share, and the finish reloads
    # them densely
    x = rng.standard_normal(L[11]).astype(np.float32)
    x[-3000:] += 10.0
    sc[11, :L[11]] = x
    x = rng.standard_normal(L[12]).astype(np.float32)
    x[30000:32500] += 6.0
    sc[12, :L[12]] = x
    idx, cnt = gpu_topk(batch, torch.from_numpy(sc).cuda())
    for i in range(batch.rows):
        want, n = oracle.topk_row(sc[i, :L[i]], wl.K)
        assert int(np_(cnt)[i]) == n
        assert (np_(idx)[i] == want).all(), f"row {i}"


@pytest.mark.parametrize("name", ["mla_int", "tiny_int", "mla_int_k100", "h48_d64", "mla_sepv",
                                  "mla_fp8kv", "mla_wide", "h80_wide", "mla_fp8kv_wide"])
def test_sparse_attn_on_oracle_indices(name):
    batch = _batch(name, mode="gauss", seed=25)
    arr = oracle_arrays(batch)
    orc = run_oracle(arr)
    out, lse = gpu_attn(batch, torch.from_numpy(orc["indices"]).cuda())
    slack = None
    if batch.wl.kv_fmt == "fp8":
        slack = fp8_kv_lse_slack(arr, orc["indices"], orc["counts"])
    mx, mean = check_attention(out, lse, orc["out"], orc["lse"], lse_slack=slack)
    say(f"attention {name}: max {mx:.3g} mean {mean:.3g}")


@pytest.mark.parametrize("name", ["mla_int", "mla_fp8kv", "mla_wide"])
def test_sparse_attn_skips_padding_and_handles_empty_rows(name):
    _padding_case(name)


# a zero or negative logit scale must not turn the masked (absent) keys into
# NaN or +inf: the kernels mask after scaling (regression test)
@pytest.mark.parametrize("scale", [0.0, -1.0 / 24.0])
@pytest.mark.parametrize("name", ["mla_int", "tiny_int", "mla_fp8kv", "mla_wide"])
def test_sparse_attn_padding_with_zero_and_negative_scale(name, scale):
    _padding_case(name, scale=scale)


def _padding_case(name, **over):
    batch = _batch(name, mode="gauss", seed=26, **over)
    arr = oracle_arrays(batch)
    K = batch.wl.K
    rng = np.random.default_rng(26)
    idx = np.full((batch.rows, K), -1, np.int32)
    for i, (_, p) in enumerate(row_positions(batch)):
        if i == 2:
            continue                                                # no valid index: out 0, lse -inf
        n = int(rng.integers(1, min(K, p + 1) + 1))
        sel = np.sort(rng.choice(p + 1, n, replace=False))
        slots = np.sort(rng.choice(K, n, replace=False))            # scattered among -1 pads
        idx[i, slots] = sel
    out, lse = gpu_attn(batch, torch.from_numpy(idx).cuda())
    want_o = np.zeros((batch.rows, batch.wl.H_q, batch.wl.D_v))
    want_l = np.full((batch.rows, batch.wl.H_q), -np.inf)
    for i, (b, p) in enumerate(row_positions(batch)):
        sel = np.sort(idx[i][idx[i] >= 0])
        if len(sel) == 0:
            continue
        k_rows = oracle.gather_positions(arr["k_cache"], arr["block_table"][b], sel)
        D_v = batch.wl.D_v
        if arr["k_scale_cache"] is not None:
            kv = oracle.kv_fp8_to_f64(
                k_rows, oracle.gather_positions(arr["k_scale_cache"], arr["block_table"][b], sel))
            want_o[i], want_l[i] = oracle.sparse_attn_values(
                oracle.bf16_to_f64(arr["q"][i]), kv, kv[:, :D_v], batch.wl.scale)
        elif arr["v_cache"] is not None:
            v_rows = oracle.gather_positions(arr["v_cache"], arr["block_table"][b], sel)
            want_o[i], want_l[i] = oracle.sparse_attn_row(arr["q"][i], k_rows, v_rows,
                                                          batch.wl.scale)
        else:
            want_o[i], want_l[i] = oracle.sparse_attn_row(arr["q"][i], k_rows, k_rows[:, :D_v],
                                                          batch.wl.scale)
    slack = None
    if batch.wl.kv_fmt == "fp8":
        packed = np.full_like(idx, -1)
        cnt = np.zeros(batch.rows, np.int64)
        for i in range(batch.rows):
            sel = np.sort(idx[i][idx[i] >= 0])
            packed[i, :len(sel)], cnt[i] = sel, len(sel)
        slack = fp8_kv_lse_slack(arr, packed, cnt)
    check_attention(out, lse, want_o, want_l, lse_slack=slack)
    assert (np_(out.float())[2] == 0).all() and np.isneginf(np_(lse)[2]).all()


@pytest.mark.parametrize("name", ["mla_int", "mla_int_shuffled", "tiny_int", "mla_int_k100",
                                  "mla_sepv", "mla_int_grouped", "mla_mx_int", "mla_cand_int",
                                  "mla_cand_split", "mla_mx_cand", "tiny_cand", "mla_fp8kv",
                                  "mla_wide", "h80_wide", "mla_fp8kv_wide"])
def test_decode_step_integer_mode(name):
    batch = _batch(name, seed=27)
    arr = oracle_arrays(batch)
    orc = run_oracle(arr, keep_scores=False)
    res = gpu_decode(batch)
    assert (np_(res["counts"]) == orc["counts"]).all()
    assert (np_(res["indices"]) == orc["indices"]).all()
    slack = None
    if batch.wl.kv_fmt == "fp8":
        slack = fp8_kv_lse_slack(arr, orc["indices"], orc["counts"])
    check_attention(res["out"], res["lse"], orc["out"], orc["lse"], lse_slack=slack)


def test_decode_step_gaussian_mode():
    batch = _batch("mla_int", mode="gauss", seed=28)
    arr = oracle_arrays(batch)
    orc = run_oracle(arr, keep_scores=False)
    res = gpu_decode(batch)
    gi = np_(res["indices"])
    rec, worst = recall(gi, orc["indices"], orc["counts"])
    say(f"recall {rec:.6f} (worst row {worst:.6f})")
    assert rec >= RECALL_MIN
    same = [i for i in range(batch.rows) if (gi[i] == orc["indices"][i]).all()]
    assert len(same) >= batch.rows - 1
    check_attention(res["out"], res["lse"], orc["out"], orc["lse"], rows=same)
    # every row, against the oracle's attention over the GPU's own selection
    o_ref, l_ref = oracle_attention_on(arr, gi, np_(res["counts"]))
    check_attention(res["out"], res["lse"], o_ref, l_ref)
    # every selection is valid: ascending, distinct, inside the history, -1 padded
    for i, (_, p) in enumerate(row_positions(batch)):
        n = int(orc["counts"][i])
        sel = gi[i, :n]
        assert (np.diff(sel) > 0).all() and sel.min() >= 0 and sel.max() <= p
        assert (gi[i, n:] == -1).all()


def test_decode_step_prefill_rows():
    wl = small_workload("prefill", lengths=[6000], prefill_rows=48, mode="int", **MLA)
    batch = make_batch(wl, device="cuda", seed=29)
    arr = oracle_arrays(batch)
    orc = run_oracle(arr, keep_scores=False)
    res = gpu_decode(batch)
    assert (np_(res["indices"]) == orc["indices"]).all()
    check_attention(res["out"], res["lse"], orc["out"], orc["lse"])


def test_decode_step_rows_of_mixed_sequences():
    # an explicit row -> sequence map whose neighbouring rows mix sequences
    # (and an odd row count): the chunked-prefill scan shares a workgroup's
    # key loads only between rows of one sequence and loads its own keys for
    # the others; scores bit-exact, indices exact, attention within bounds
    wl = small_workload("mixed", lengths=[3000, 5000, 700, 4097, 1, 2500, 1200], mode="int",
                        **MLA)
    batch = make_batch(wl, device="cuda", seed=33)
    L = batch.lengths
    seq = [0, 0, 1, 3, 3, 5, 2]
    pos = [L[0] - 1, L[0] // 2, L[1] - 1, L[3] - 1, L[3] - 3, L[5] - 1, L[2] - 1]
    batch = dataclasses.replace(
        batch, row_seq_host=seq, row_pos_host=pos,
        row_seq=torch.tensor(seq, dtype=torch.int32, device="cuda"),
        row_pos=torch.tensor(pos, dtype=torch.int32, device="cuda"))
    say(f"rows -> sequences {seq}, positions {pos}")
    arr = oracle_arrays(batch)
    orc = run_oracle(arr)
    check_scores_exact(gpu_scores(batch), orc, row_positions(batch))
    res = gpu_decode(batch)
    assert (np_(res["counts"]) == orc["counts"]).all()
    assert (np_(res["indices"]) == orc["indices"]).all()
    check_attention(res["out"], res["lse"], orc["out"], orc["lse"])


@pytest.mark.parametrize("table", ["identity", "shuffled"])
def test_decode_step_prefill_rows_with_candidates(table):
    # chunked-prefill rows (one sequence, 48 consecutive positions) each with
    # its own candidate list, through a shuffled table too
    wl = small_workload("prefill_cand", lengths=[24000], prefill_rows=48, mode="int",
                        n_cand=16500, table=table, **MLA)
    batch = make_batch(wl, device="cuda", seed=31)
    arr = oracle_arrays(batch)
    orc = run_oracle(arr, keep_scores=False)
    res = gpu_decode(batch)
    assert (np_(res["counts"]) == orc["counts"]).all()
    assert (np_(res["indices"]) == orc["indices"]).all()
    check_attention(res["out"], res["lse"], orc["out"], orc["lse"])


def test_decode_step_deterministic_and_matches_unfused_calls():
    batch = _batch("mla_int", mode="gauss", seed=30)
    a = gpu_decode(batch)
    b = gpu_decode(batch)
    for key in ("out", "lse", "indices", "counts"):
        assert torch.equal(a[key].view(torch.uint8) if a[key].dtype == torch.bfloat16 else a[key],
                           b[key].view(torch.uint8) if b[key].dtype == torch.bfloat16 else b[key])
    sc = gpu_scores(batch)
    idx, cnt = gpu_topk(batch, sc)
    assert torch.equal(idx, a["indices"]) and torch.equal(cnt, a["counts"])
    out, lse = gpu_attn(batch, idx)
    assert torch.equal(out.view(torch.int16), a["out"].view(torch.int16))
    assert torch.equal(lse, a["lse"])


def test_tiny_workload_matches_golden_fixture():
    import json
    import os
    wl = CONFIGS["tiny_decode_1x1k"]
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_decode_1x1k_seed1.json")
    want = json.load(open(path))
    batch = make_batch(wl, device="cpu", seed=wl.seed)
    for name in ("seq_lens", "block_table", "qI", "w", "kI", "q", "kv", "v"):
        setattr(batch, name, getattr(batch, name).cuda())
    res = gpu_decode(batch)
    assert np_(res["indices"])[0].tolist() == want["indices"]
    assert int(np_(res["counts"])[0]) == want["count"]


def test_decode_step_timed_matches_decode_step():
    # the timed entry launches the same kernels: identical results, and the
    # eight events it stamps give ordered, non-negative stage times
    batch = _batch("mla_int", seed=29)
    prob = B.problem_for_batch(batch)
    ref = gpu_decode(batch)
    wl = batch.wl
    out = torch.full_like(ref["out"], float("nan"))
    lse = torch.full_like(ref["lse"], float("nan"))
    idx = torch.full_like(ref["indices"], -7)
    cnt = torch.full_like(ref["counts"], -7)
    ws = B.workspace(prob, B.DSA_OP_DECODE_STEP)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    v = batch.v if batch.v is not None else batch.kv
    B.dsa_decode_step_timed(prob, batch.qI, batch.w, batch.kI, batch.q, batch.kv, v, out, ws, ev,
                            lse=lse, indices=idx, counts=cnt)
    torch.cuda.synchronize()
    assert B.device_errors(ws) == 0
    assert torch.equal(idx, ref["indices"]) and torch.equal(cnt, ref["counts"])
    assert torch.equal(out.view(torch.int16), ref["out"].view(torch.int16))
    assert torch.equal(lse.view(torch.int32), ref["lse"].view(torch.int32))
    t = [ev[i].elapsed_time(ev[i + 1]) for i in range(7)]
    say(f"stage times and gaps (ms) {t}")
    assert all(x >= 0 for x in t) and t[0] > 0 and t[2] > 0 and t[4] > 0
    assert wl.K == idx.shape[1]
