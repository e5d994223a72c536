"""Plumbing shared by the GPU tests: run the HIP entry points on a seeded
batch and compare with the oracle at the stated tolerances."""

import math

import numpy as np
import torch

from indexer_top_sparse_score_amd import binding as B

# attention output tolerance (bf16 output, fp32 softmax): max and mean |error|
ATT_MAX_ABS = 2e-2
ATT_MEAN_ABS = 2e-3
RECALL_MIN = 0.999
U32 = 2.0 ** -24


def say(*a):
    print(*a, flush=True)


def kv_and_v(batch):
    return batch.kv, (batch.v if batch.v is not None else batch.kv)


def gpu_scores(batch):
    """dsa_indexer_scores into a NaN-filled [rows, ld] buffer (ld: the longest
    history, or the candidate lists' length)."""
    prob = B.problem_for_batch(batch)
    ld = score_ld(batch)
    scores = torch.full((batch.rows, ld), float("nan"), dtype=torch.float32, device="cuda")
    ws = B.workspace(prob, B.DSA_OP_INDEXER_SCORES)
    B.dsa_indexer_scores(prob, batch.qI, batch.w, batch.kI, scores, ws)
    torch.cuda.synchronize()
    assert B.device_errors(ws) == 0
    return scores


def score_ld(batch):
    return batch.cand.shape[1] if batch.cand is not None else 64 * batch.max_blocks


def gpu_topk(batch, scores):
    prob = B.problem_for_batch(batch)
    idx = torch.full((batch.rows, batch.wl.K), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((batch.rows,), -7, dtype=torch.int32, device="cuda")
    ws = B.workspace(prob, B.DSA_OP_TOPK)
    B.dsa_topk(prob, scores, idx, ws, counts=cnt)
    torch.cuda.synchronize()
    assert B.device_errors(ws) == 0
    return idx, cnt


def gpu_attn(batch, indices):
    prob = B.problem_for_batch(batch)
    wl = batch.wl
    out = torch.full((batch.rows, wl.H_q, wl.D_v), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((batch.rows, wl.H_q), float("nan"), dtype=torch.float32, device="cuda")
    ws = B.workspace(prob, B.DSA_OP_SPARSE_ATTN)
    k, v = kv_and_v(batch)
    B.dsa_sparse_attn(prob, batch.q, k, v, indices, out, ws, lse=lse)
    torch.cuda.synchronize()
    assert B.device_errors(ws) == 0
    return out, lse


def gpu_decode(batch, ws=None, stream=None):
    prob = B.problem_for_batch(batch)
    wl = batch.wl
    out = torch.full((batch.rows, wl.H_q, wl.D_v), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((batch.rows, wl.H_q), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((batch.rows, wl.K), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((batch.rows,), -7, dtype=torch.int32, device="cuda")
    if ws is None:
        ws = B.workspace(prob, B.DSA_OP_DECODE_STEP)
    k, v = kv_and_v(batch)
    B.dsa_decode_step(prob, batch.qI, batch.w, batch.kI, batch.q, k, v, out, ws, lse=lse,
                      indices=idx, counts=cnt, stream=stream)
    torch.cuda.synchronize()
    assert B.device_errors(ws) == 0
    return {"out": out, "lse": lse, "indices": idx, "counts": cnt}


def np_(t):
    return t.detach().cpu().numpy()


def check_scores_exact(gpu_scores_t, orc, rows_pos):
    # the oracle's row holds one score per position (or per candidate)
    g = np_(gpu_scores_t)
    for i, _ in enumerate(rows_pos):
        want = orc["scores"][i]
        n = len(want)
        got = g[i, :n]
        assert (got.view(np.uint32) == want.view(np.uint32)).all(), \
            f"row {i}: {int((got != want).sum())} score mismatches"
        assert np.isnan(g[i, n:]).all(), f"row {i}: wrote past its score row"


def score_bound(arr, i, p):
    """Forward-error bound of a float32 head-weighted, ReLU-gated FP8 dot
    product against the correctly rounded value: 2 * gamma_n * sum_h |w_h| *
    sum_d |q_hd k_sd| + 1 ulp, n = D_I + H_I + 1 (per-position array)."""
    import oracle
    b = arr["row_seq"][i]
    q = np.abs(oracle.e4m3_to_f64(arr["qI"][i]))
    rows = oracle.gather_positions(arr["kI_cache"], arr["block_table"][b], np.arange(p + 1))
    D = q.shape[1]
    k = np.abs(oracle.e4m3_to_f64(rows[:, :D]))
    if arr.get("qI_scale") is not None:  # MXFP8: fold each group's scales in
        G = D // 32
        sq = np.repeat(oracle.e8m0_to_f64(arr["qI_scale"][i]), 32, axis=1)
        srows = oracle.gather_positions(arr["kI_scale_cache"], arr["block_table"][b],
                                        np.arange(p + 1))
        sk = np.repeat(oracle.e8m0_to_f64(srows[:, :G]), 32, axis=1)
        q, k = q * sq, k * sk
    mag = np.abs(arr["w"][i].astype(np.float64)) @ (q @ k.T)
    n = q.shape[1] + q.shape[0] + 1
    gamma = n * U32 / (1 - n * U32)
    return 2 * gamma * mag


def recall(gpu_idx, orc_idx, counts):
    hit = tot = 0
    per_row = []
    for g, o, n in zip(gpu_idx, orc_idx, counts):
        sg = set(int(x) for x in g[:n])
        so = set(int(x) for x in o[:n])
        hit += len(sg & so)
        tot += len(so)
        per_row.append(len(sg & so) / max(1, len(so)))
    return hit / max(1, tot), min(per_row) if per_row else 1.0


def check_attention(out_t, lse_t, orc_out, orc_lse, rows=None, lse_slack=None):
    """Attention within ATT_MAX_ABS / ATT_MEAN_ABS on the output and lse to
    rtol 1e-4 + atol 1e-3, plus ``lse_slack`` [rows, H_q] where the kernel's
    arithmetic adds a derived error (see fp8_kv_lse_slack)."""
    o = np_(out_t.float()).astype(np.float64)
    l = np_(lse_t).astype(np.float64)
    if rows is not None:
        o, l = o[rows], l[rows]
        orc_out, orc_lse = orc_out[rows], orc_lse[rows]
        if lse_slack is not None and len(lse_slack) != len(rows):
            lse_slack = lse_slack[rows]
    err = np.abs(o - orc_out)
    assert np.isfinite(o).all()
    assert err.max() <= ATT_MAX_ABS, f"max abs error {err.max():.3g}"
    assert err.mean() <= ATT_MEAN_ABS, f"mean abs error {err.mean():.3g}"
    fin = np.isfinite(orc_lse)
    assert (np.isfinite(l) == fin).all()
    tol = 1e-3 + 1e-4 * np.abs(orc_lse[fin])
    if lse_slack is not None:
        tol = tol + lse_slack[fin]
    assert (np.abs(l[fin] - orc_lse[fin]) <= tol).all(), \
        f"lse error {np.abs(l[fin] - orc_lse[fin]).max():.3g}"
    return float(err.max()), float(err.mean())


def log2ceil(x):
    return int(math.ceil(math.log2(max(1, x))))


def oracle_attention_on(arr, indices, counts, threads=None):
    """The oracle's sparse attention of every row held in ``arr`` over the
    positions the GPU selected for it (indices [rows, K], counts [rows]):
    the selected rows are gathered through the block table and attended by
    the C++ oracle.  Returns (out [rows, H_q, D_v], lse [rows, H_q])."""
    import oracle
    import oracle.cpp
    from tests.helpers import HOST_THREADS

    D_v = int(arr["D_v"])
    outs, lses = [], []
    for i in range(len(arr["qI"])):
        b = arr["row_seq"][i]
        sel = np.asarray(indices[i][:int(counts[i])], dtype=np.int64)
        k_rows = oracle.gather_positions(arr["k_cache"], arr["block_table"][b], sel)
        if arr.get("k_scale_cache") is not None:  # FP8 KV: decode the rows (C++ route)
            kv = oracle.cpp.kv_fp8_to_f64(
                k_rows, oracle.gather_positions(arr["k_scale_cache"], arr["block_table"][b], sel))
            o, l = oracle.sparse_attn_values(oracle.bf16_to_f64(arr["q"][i]), kv, kv[:, :D_v],
                                             arr["scale"])
            outs.append(o)
            lses.append(l)
            continue
        if arr["v_cache"] is None:
            v_rows = k_rows[:, :D_v]
        else:
            v_rows = oracle.gather_positions(arr["v_cache"], arr["block_table"][b], sel)
        o, l = oracle.cpp.sparse_attn_row(arr["q"][i], k_rows, v_rows, arr["scale"],
                                          threads=threads or HOST_THREADS)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def fp8_kv_lse_slack(arr, indices, counts):
    """Added lse tolerance for an FP8 KV cache [rows, H_q].  The kernel rounds
    each decoded element (code * tile scale) to bf16 before the bf16 products:
    a relative change of at most 2**-9 per K element, so each logit moves by at
    most scale * 2**-9 * sum_d |q[h, d]| |k[j, d]|, and lse (a smooth maximum
    of the logits) by at most the largest of those over the selected rows."""
    import oracle
    out = np.zeros((len(arr["qI"]), arr["q"].shape[1]))
    for i in range(len(arr["qI"])):
        b = arr["row_seq"][i]
        sel = np.asarray(indices[i][:int(counts[i])], dtype=np.int64)
        if len(sel) == 0:
            continue
        k = oracle.kv_fp8_to_f64(
            oracle.gather_positions(arr["k_cache"], arr["block_table"][b], sel),
            oracle.gather_positions(arr["k_scale_cache"], arr["block_table"][b], sel))
        q = np.abs(oracle.bf16_to_f64(arr["q"][i]))
        out[i] = abs(arr["scale"]) * 2.0 ** -9 * (q @ np.abs(k).T).max(axis=1)
    return out
