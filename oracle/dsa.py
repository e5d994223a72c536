"""The indexer -> Top-K -> sparse-attention step, written out in binary64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Each function follows one step of the method as Baidu AI Cloud's "Day0
Inference Support and Performance Optimization for New Architecture LLMs"
describes it in section 2.2 (score every historical position, aggregate the
per-head scores with head weights, keep the Top-K positions, attend over only
those rows), with the paged caches of sections 4.1-4.2.  Library primitives
(a matrix product, a sort, exp/log) serve as steps; there is no blocking,
fusion or reordering beyond the definitions.

Array conventions (raw storage bits, exactly what the GPU reads):

* ``qI``  uint8 E4M3 codes   [rows, H_I, D_I]   indexer queries
* ``w``   float32            [rows, H_I]        head weights
* ``kI_cache`` uint8 E4M3    [num_blocks, 64, D_I]  paged index keys
* ``q``   uint16 bf16 bits   [rows, H_q, D_qk]  attention queries
* ``k_cache`` uint16 bf16    [num_blocks, 64, D_qk] paged keys (latent rows)
* ``v_cache`` uint16 bf16    [num_blocks, 64, D_v] or None (latent layout:
  V is the first D_v columns of the K row)
* ``block_table`` int32 [num_seqs, max_blocks]; ``seq_lens`` int32 [num_seqs]
* ``cand`` int32 [rows, n_cand], ``cand_len`` int32 [rows] (optional): a
  row's candidate positions, ascending, the first cand_len[r] entries valid
"""

import numpy as np

from .formats import bf16_to_f64, e4m3_to_f64, e8m0_to_f64, kv_fp8_to_f64

#: dims per shared scale of the MXFP8 indexer format (Day0 article, section 5.1)
MX_GROUP = 32

#: tokens per page of every paged cache
BLOCK = 64


def resolve_rows(seq_lens, num_rows=None, row_seq=None, row_pos=None):
    """Sequence and position of every query row.

    Decode (no row arrays): row r belongs to sequence r and sits at that
    sequence's last position seq_lens[r] - 1.  Chunked prefill passes
    ``row_seq`` / ``row_pos`` explicitly.  Reading of "all historical
    positions" (Day0 article, section 2.2): row r's history is positions
    0 .. p_r inclusive -- the current token's key is already in the cache.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    if num_rows is None:
        num_rows = len(row_seq) if row_seq is not None else len(seq_lens)
    rs = np.arange(num_rows) if row_seq is None else np.asarray(row_seq, np.int64)
    rp = seq_lens[rs] - 1 if row_pos is None else np.asarray(row_pos, np.int64)
    return rs.astype(np.int64), rp.astype(np.int64)


def gather_positions(cache, table_row, positions, block=BLOCK):
    """Rows of a paged cache for logical positions of one sequence.

    Position s lives in physical block table_row[s // block], row s % block
    (paged K cache read directly by the indexer, Day0 article section 4.1;
    selected KV rows gathered from the main cache, section 4.2).
    """
    positions = np.asarray(positions, dtype=np.int64)
    phys = np.asarray(table_row, dtype=np.int64)[positions // block]
    return cache[phys, positions % block]


def indexer_scores_row(qI_codes, w, kI_rows, qI_scale=None, kI_scale=None):
    """Index score of one query row against the given key rows.

    I[s] = sum_h w[h] * max(0, sum_d qI[h, d] * kI[s, d])

    Scoring against every historical position, then aggregating the per-head
    scores with head weights (Day0 article, section 2.2; the fused call of
    section 4.3 takes exactly these three inputs: the quantised query, the
    index keys and the head weights).  Readings: the per-head score passes a ReLU gate before the
    weighting; one shared index key per position serves every indexer head.

    The per-head dot products are exact in binary64: E4M3 products carry at
    most 8 significant bits, lie between 2**-18 and 448**2, so a sum of a few
    hundred of them needs far fewer than 53 bits.  The weighted head sum is
    formed in binary64 and rounded once to float32; a zero score is stored as
    +0.

    MXFP8 (Day0 article, section 5.1: Q and K quantised per group of 32 with
    one shared scale per group): given ``qI_scale`` [H_I, D_I/32] and
    ``kI_scale`` [L, D_I/32] E8M0 bytes, each group's partial dot product is
    multiplied by the two groups' scales before the groups are summed,

    dot[h, s] = sum_g sq[h, g] * sk[s, g] * sum_{d in group g} qI[h, d] * kI[s, d].

    Each group's sum is exact as above and the power-of-two scales keep it
    exact; the groups are summed in binary64.
    """
    q = e4m3_to_f64(qI_codes)                       # [H_I, D_I]
    k = e4m3_to_f64(kI_rows)                        # [L, D_I]
    if qI_scale is None:
        dot = q @ k.T                               # [H_I, L]
    else:
        sq = e8m0_to_f64(qI_scale)                  # [H_I, D_I / 32]
        sk = e8m0_to_f64(kI_scale)                  # [L, D_I / 32]
        dot = np.zeros((q.shape[0], k.shape[0]))
        for g in range(q.shape[1] // MX_GROUP):
            dims = slice(MX_GROUP * g, MX_GROUP * (g + 1))
            dot += (q[:, dims] @ k[:, dims].T) * sq[:, g][:, None] * sk[:, g][None, :]
    gated = np.maximum(dot, 0.0)                    # ReLU gate, per head
    weights = np.asarray(w, dtype=np.float32).astype(np.float64)
    total = weights @ gated                         # head-weighted sum, [L]
    return (total.astype(np.float32) + np.float32(0.0)).astype(np.float32)


def score_keys(scores):
    """Order-preserving unsigned 32-bit key of each float32 score.

    Larger score -> larger key.  -0 and +0 share one key.  NaN gets key 0 and
    so ranks below every number (reading: the pages say nothing about NaN;
    generated inputs never produce one).
    """
    s = np.array(scores, dtype=np.float32, copy=True)
    s[s == 0] = np.float32(0.0)
    u = s.view(np.uint32)
    negative = (u >> np.uint32(31)) == 1
    key = np.where(negative, ~u, u | np.uint32(0x80000000)).astype(np.uint32)
    key[np.isnan(s)] = 0
    return key


def topk_row(scores, K):
    """Top-K positions of one row's scores.

    Keeps the min(K, L) positions with the largest score (Day0 article,
    section 2.2).  Readings: equal scores go to the lower position; the kept
    positions are returned in ascending order, padded with -1 up to K.
    Returns (indices int32 [K], count).
    """
    L = len(scores)
    keys = score_keys(scores).astype(np.int64)
    positions = np.arange(L, dtype=np.int64)
    order = np.lexsort((positions, -keys))          # key descending, then position ascending
    count = min(int(K), L)
    out = np.full(int(K), -1, dtype=np.int32)
    out[:count] = np.sort(order[:count])
    return out, count


def sparse_attn_row(q_bits, k_rows_bits, v_rows_bits, scale):
    """Softmax attention of one query row over the gathered rows only.

    For every query head h and selected row j:
      logit[h, j] = scale * sum_d q[h, d] * k[j, d]
      o[h] = sum_j exp(logit[h, j] - m_h) v[j] / sum_j exp(logit[h, j] - m_h)
    with m_h the largest logit; lse[h] = m_h + log(sum_j exp(logit[h, j] - m_h)).
    The sparse core reads only the selected KV rows (Day0 article, section
    2.2); one KV head serves every query head (SPLASH summary, section 2).
    With no rows selected the output is 0 and lse is -inf.
    Returns (o float64 [H_q, D_v], lse float64 [H_q]).
    """
    return sparse_attn_values(bf16_to_f64(q_bits), bf16_to_f64(k_rows_bits),
                              bf16_to_f64(v_rows_bits), scale)


def sparse_attn_values(q, k, v, scale):
    """``sparse_attn_row`` on decoded values: q [H_q, D_qk], k [n, D_qk],
    v [n, D_v], all binary64."""
    H_q, D_v = q.shape[0], v.shape[1]
    if k.shape[0] == 0:
        return np.zeros((H_q, D_v)), np.full(H_q, -np.inf)
    logits = scale * (q @ k.T)                      # [H_q, n]
    m = logits.max(axis=1)
    p = np.exp(logits - m[:, None])
    l = p.sum(axis=1)
    o = (p @ v) / l[:, None]
    return o, m + np.log(l)


def masked_dense_attn_row(q_bits, k_all_bits, v_all_bits, selected, scale):
    """Dense attention over every history row, with unselected rows masked out.

    Computes logits against all rows 0..L-1, sets the unselected ones to -inf
    and normalises over the whole row: the brute-force counterpart of
    ``sparse_attn_row`` (no gather).  Returns (o [H_q, D_v], lse [H_q]).
    """
    q = bf16_to_f64(q_bits)
    k = bf16_to_f64(k_all_bits)
    v = bf16_to_f64(v_all_bits)
    mask = np.asarray(selected, dtype=bool)
    logits = scale * (q @ k.T)
    logits[:, ~mask] = -np.inf
    m = logits.max(axis=1)
    e = np.exp(logits - m[:, None])
    l = e.sum(axis=1)
    return (e @ v) / l[:, None], m + np.log(l)


def dense_causal_attn_row(q_bits, k_all_bits, v_all_bits, scale):
    """softmax(scale * q K^T) V over the whole history of one row.

    The dense attention of THInfer ("Bandwidth-Aware LLM Inference on
    Heterogeneous Many-Core Supercomputers"), eq. 9, with the scale as an
    argument; causal because the history stops at the row's own position.
    """
    q = bf16_to_f64(q_bits)
    k = bf16_to_f64(k_all_bits)
    v = bf16_to_f64(v_all_bits)
    s = scale * (q @ k.T)
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v


def row_history(p, cand_row=None, cand_len=None):
    """Positions a row's indexer scores.

    Without candidates: every position 0 .. p (Day0 article, section 2.2).
    With a candidate list (vLLM's DeepSeek-V4.1-Flash article, "Kernels":
    later indexer layers choose their top-k from a fixed set of candidate
    positions and score only those): the first cand_len entries of the
    row's list, which the caller gives in ascending order, each in 0 .. p.
    """
    if cand_row is None:
        return np.arange(p + 1)
    h = np.asarray(cand_row[:int(cand_len)], dtype=np.int64)
    if len(h) and (h[0] < 0 or h[-1] > p or (np.diff(h) <= 0).any()):
        raise ValueError("candidates must be ascending positions in 0..p")
    return h


def decode_step(*, qI, w, kI_cache, q, k_cache, v_cache, block_table, seq_lens,
                K, scale, D_v, row_seq=None, row_pos=None, rows=None,
                keep_scores=True, qI_scale=None, kI_scale_cache=None,
                cand=None, cand_len=None, k_scale_cache=None):
    """The whole step for the chosen query rows (default: all rows).

    Row by row: index scores over positions 0..p_r, Top-K, gather of the
    selected KV rows, sparse softmax attention.  With ``qI_scale`` [rows,
    H_I, D_I/32] and ``kI_scale_cache`` [num_blocks, 64, D_I/32] (paged like
    ``kI_cache``) the indexer is MXFP8.  With ``cand`` / ``cand_len`` each
    row scores only its candidate positions (row_history) and keeps the
    Top-K among them; ``scores`` then holds one entry per candidate.  With
    ``k_scale_cache`` float32 [num_blocks, 64, ceil(D_qk / 128)] the KV cache
    is FP8 (Day0 article, section 5.2): ``k_cache`` holds E4M3 codes
    [num_blocks, 64, D_qk] in the latent layout (``v_cache`` None) and each
    gathered row is decoded by ``kv_fp8_to_f64``.
    Returns a dict with
    ``scores`` (list of float32 arrays, or None), ``indices`` int32 [R, K],
    ``counts`` int64 [R], ``out`` float64 [R, H_q, D_v], ``lse`` float64
    [R, H_q] and ``rows`` (the row ids, in order).
    """
    num_rows = qI.shape[0]
    rs, rp = resolve_rows(seq_lens, num_rows, row_seq, row_pos)
    rows = np.arange(num_rows) if rows is None else np.asarray(rows, np.int64)
    H_q = q.shape[1]
    out = np.zeros((len(rows), H_q, D_v))
    lse = np.zeros((len(rows), H_q))
    indices = np.full((len(rows), int(K)), -1, dtype=np.int32)
    counts = np.zeros(len(rows), dtype=np.int64)
    scores = [] if keep_scores else None
    for i, r in enumerate(rows):
        b, p = rs[r], rp[r]
        history = row_history(p, None if cand is None else cand[r],
                              None if cand is None else cand_len[r])
        k_index = gather_positions(kI_cache, block_table[b], history)
        if qI_scale is None:
            sc = indexer_scores_row(qI[r], w[r], k_index)
        else:
            k_scale = gather_positions(kI_scale_cache, block_table[b], history)
            sc = indexer_scores_row(qI[r], w[r], k_index, qI_scale[r], k_scale)
        idx, n = topk_row(sc, K)
        # candidate slots are in position order: ties to the lower slot are
        # ties to the lower position, and ascending slots ascending positions
        idx = idx.copy()
        idx[:n] = history[idx[:n]]
        chosen = idx[:n]
        k_rows = gather_positions(k_cache, block_table[b], chosen)
        if k_scale_cache is not None:
            if v_cache is not None:
                raise ValueError("the FP8 KV cache takes the latent layout")
            k_vals = kv_fp8_to_f64(k_rows, gather_positions(k_scale_cache, block_table[b], chosen))
            out[i], lse[i] = sparse_attn_values(bf16_to_f64(q[r]), k_vals, k_vals[:, :D_v], scale)
        else:
            if v_cache is None:
                v_rows = k_rows[:, :D_v]
            else:
                v_rows = gather_positions(v_cache, block_table[b], chosen)
            out[i], lse[i] = sparse_attn_row(q[r], k_rows, v_rows, scale)
        indices[i], counts[i] = idx, n
        if keep_scores:
            scores.append(sc)
    return {"scores": scores, "indices": indices, "counts": counts,
            "out": out, "lse": lse, "rows": rows}
