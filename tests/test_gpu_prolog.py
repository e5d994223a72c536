"""GPU parity of the indexer prolog (dsa_indexer_prolog) against the oracle.

Bars:
* integer mode (x, weights small integers: every projection sum is an
  integer, exact in float32 in any order) -- qI, qI_scale and w bit-exact;
* Gaussian mode -- each MXFP8 value within half an E4M3 step of the exact
  value plus bf16 rounding and the float32 accumulation bound (or saturated
  at 448 scale units), scales within one of the oracle's and equal except
  where the group maximum sits next to a power of two, and at least 99 % of
  the codes equal to the oracle's;
* the new keys: written at exactly each row's slot of the MXFP8 cache (every
  other byte of the cache unchanged); bit-exact for keys of exact RMS, else
  as the Gaussian bar;
* fed to the fused step, the prolog's outputs give the oracle's indices bit
  for bit (integer mode, keys of exact RMS).
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from indexer_top_sparse_score_amd import binding as B
from tests.gpu_helpers import check_attention, gpu_decode, np_, say
from tests.helpers import HOST_THREADS, run_oracle
from workloads import make_batch, make_prolog_inputs, oracle_arrays, prolog_arrays, small_workload

pytestmark = pytest.mark.gpu

EPS = 1e-6
MLA = dict(H_q=128, D_qk=576, D_v=512, K=2048, scale=576 ** -0.5)

# name: (history lengths (one decode row each), H_I, D_I, D_x, mode, table)
CASES = {
    # the headline's indexer shape: 4 decode rows over a 4096-wide input
    "decode4_int": ([3000, 64, 65, 2049], 64, 128, 4096, "int", "identity"),
    "decode4_gauss": ([3000, 64, 65, 2049], 64, 128, 4096, "gauss", "shuffled"),
    # one row, the narrowest input, the smallest indexer
    "one_row_tiny": ([1], 4, 64, 32, "int", "identity"),
    # 4 rows are the vector-ALU kernel's largest batch; 5, 8 and 16 rows take
    # the 16-row MFMA tile, and 17 the first of the 64-row tiles
    "rows5_gauss": ([7, 300, 64, 65, 1], 64, 128, 4096, "gauss", "identity"),
    "rows8_int": ([1 + 97 * i for i in range(8)], 64, 64, 512, "int", "shuffled"),
    "rows16_gauss": ([5 + 37 * i for i in range(16)], 64, 128, 1024, "gauss", "shuffled"),
    "rows17_int": ([1 + 61 * i for i in range(17)], 8, 128, 96, "int", "identity"),
    # ragged row tiles, 48 heads (a half-filled head-weight tile), 64-dim heads
    "rows100_h48_int": ([1 + (37 * i) % 900 for i in range(100)], 48, 64, 160, "int", "shuffled"),
    # several tiles of 64 rows with a ragged last one, at the full width
    "rows300_gauss": ([1 + (53 * i) % 700 for i in range(300)], 64, 128, 4096, "gauss",
                      "shuffled"),
}


def _setup(lengths, H_I, D_I, mode, table, seed):
    wl = small_workload("prolog", lengths=lengths, H_I=H_I, D_I=D_I, mode="int",
                        indexer_fmt="mxfp8", table=table, **MLA)
    return make_batch(wl, device="cuda", seed=seed)


def _run_prolog(batch, inp, eps=EPS):
    wl = batch.wl
    rows = batch.rows
    prob = B.problem_for_batch(batch)
    qI = torch.full((rows, wl.H_I, wl.D_I), 0xAA, dtype=torch.uint8, device="cuda")
    qs = torch.full((rows, wl.H_I, wl.D_I // 32), 0xAA, dtype=torch.uint8, device="cuda")
    w = torch.full((rows, wl.H_I), float("nan"), dtype=torch.float32, device="cuda")
    ws = B.workspace(prob, B.DSA_OP_INDEXER_PROLOG)
    B.dsa_indexer_prolog(prob, inp.x, inp.w_q, inp.w_g, inp.k_new, inp.k_gamma, qI, qs, w,
                         batch.kI, ws, eps=eps)
    torch.cuda.synchronize()
    return qI, qs, w, B.device_errors(ws)


def _slots(batch):
    """(block, row) of each row's own position in the caches."""
    bt = np_(batch.block_table)
    out = []
    for b, p in zip(batch.row_seq_host, batch.row_pos_host):
        out.append((int(bt[b, p // 64]), p % 64))
    return out


def _f32_bound(W_bits, x_bits):
    """Float32 accumulation bound of W x per output: n 2^-24 sum |W||x|."""
    Wf = np.abs(oracle.formats.bf16_to_f64(W_bits))
    xf = np.abs(oracle.formats.bf16_to_f64(x_bits))
    return xf.shape[1] * 2.0 ** -24 * (xf @ Wf.T)


def _check_mx_close(codes_g, scales_g, codes_o, scales_o, exact, err_abs, what):
    """codes/scales [..., n] and [..., n/32]; exact binary64 values [..., n]."""
    cg = np.asarray(codes_g).reshape(-1, 32)
    sg = np.asarray(scales_g).reshape(-1).astype(np.int64)
    so = np.asarray(scales_o).reshape(-1).astype(np.int64)
    v = np.asarray(exact, np.float64).reshape(-1, 32)
    e = np.broadcast_to(np.asarray(err_abs, np.float64), np.asarray(exact).shape).reshape(-1, 32)
    assert np.all(np.abs(sg - so) <= 1), what
    diff = np.nonzero(sg != so)[0]
    if len(diff):
        amax = np.abs(v[diff]).max(axis=1)
        near = np.abs(amax / np.exp2(np.round(np.log2(amax))) - 1.0)
        assert np.all(near <= 2.0 ** -7), (what, "scale differs away from a power of two")
    X = np.exp2(sg - 127.0)[:, None]
    deq = oracle.formats.E4M3_TABLE[cg] * X
    sat = np.abs(v) >= 448 * X * (1 - 2.0 ** -7)
    bound = 2.0 ** -4 * np.abs(v) * (1 + 2.0 ** -6) + 2.0 ** -10 * X + np.abs(v) * 2.0 ** -8 + e
    ok = (np.abs(deq - v) <= bound) | (sat & (np.abs(deq) == 448 * X))
    assert ok.all(), (what, int((~ok).sum()), float(np.abs(deq - v)[~ok].max()))
    same = (cg == np.asarray(codes_o).reshape(-1, 32)).mean()
    assert same >= 0.99, (what, same)
    return same


@pytest.mark.parametrize("name", sorted(CASES))
def test_prolog_on_oracle(name):
    lengths, H_I, D_I, D_x, mode, table = CASES[name]
    say(f"[prolog] {name}: rows {len(lengths)} H_I {H_I} D_I {D_I} D_x {D_x} {mode}")
    batch = _setup(lengths, H_I, D_I, mode, table, seed=11)
    inp = make_prolog_inputs(batch.rows, H_I, D_I, D_x=D_x, mode=mode, seed=12, device="cuda")
    kI_before = np_(batch.kI).copy()
    qI, qs, w, errs = _run_prolog(batch, inp)
    assert errs == 0
    arr = prolog_arrays(inp)
    res = oracle.cpp.indexer_prolog(**arr, eps=EPS, H_I=H_I, D_I=D_I, threads=HOST_THREADS)
    kI_after = np_(batch.kI)
    slots = _slots(batch)
    # the cache: only each row's code row and scale bytes changed
    expect_same = np.ones(kI_after.shape, bool)
    got_k = np.empty((batch.rows, D_I), np.uint8)
    got_ks = np.empty((batch.rows, D_I // 32), np.uint8)
    for i, (blk, row) in enumerate(slots):
        expect_same[blk, row, :] = False
        flat = kI_after[blk, 64:].reshape(-1)
        got_k[i] = kI_after[blk, row]
        got_ks[i] = flat[row * (D_I // 32):(row + 1) * (D_I // 32)]
        m = expect_same[blk, 64:].reshape(-1)
        m[row * (D_I // 32):(row + 1) * (D_I // 32)] = False
        expect_same[blk, 64:] = m.reshape(expect_same[blk, 64:].shape)
    assert np.array_equal(kI_after[expect_same], kI_before[expect_same])

    if mode == "int":
        assert np.array_equal(np_(qI), res["qI"])
        assert np.array_equal(np_(qs), res["qI_scale"])
        assert np.array_equal(np_(w), res["w"])
    else:
        eb = _f32_bound(arr["w_q"], arr["x"])
        same = _check_mx_close(np_(qI), np_(qs), res["qI"], res["qI_scale"], res["q"], eb, "q")
        say(f"  q codes equal to the oracle's: {same:.6f}")
        g = oracle.formats.bf16_to_f64(arr["x"]) @ oracle.formats.bf16_to_f64(arr["w_g"]).T
        gb = _f32_bound(arr["w_g"], arr["x"])
        assert np.all(np.abs(np_(w) - g) <= np.abs(g) * 2.0 ** -8 + gb)
    y = oracle.rms_norm(oracle.formats.bf16_to_f64(arr["k_new"]),
                        oracle.formats.bf16_to_f64(arr["k_gamma"]), EPS)
    same = _check_mx_close(got_k, got_ks, res["kI"], res["kI_scale"], y, np.abs(y) * 2.0 ** -20,
                           "k")
    say(f"  key codes equal to the oracle's: {same:.6f}")


def test_prolog_exact_keys_and_the_step_it_feeds():
    """Integer inputs and keys of exact RMS: every prolog output bit-exact;
    the fused step on them selects exactly what the oracle's step selects on
    the oracle's prolog outputs."""
    lengths = [1, 64, 65, 3000, 5000]
    say("[prolog] exact keys, then the fused step")
    batch = _setup(lengths, 64, 128, "int", "shuffled", seed=21)
    inp = make_prolog_inputs(batch.rows, 64, 128, D_x=4096, mode="int", seed=22, device="cuda",
                             key_pm4=True)
    arr_before = oracle_arrays(batch)
    qI, qs, w, errs = _run_prolog(batch, inp, eps=0.0)
    assert errs == 0
    res = oracle.cpp.indexer_prolog(**prolog_arrays(inp), eps=0.0, H_I=64, D_I=128,
                                    threads=HOST_THREADS)
    assert np.array_equal(np_(qI), res["qI"]) and np.array_equal(np_(qs), res["qI_scale"])
    assert np.array_equal(np_(w), res["w"])
    # the oracle's view of the caches after its own prolog
    kc = arr_before["kI_cache"].copy()
    ksc = arr_before["kI_scale_cache"].copy()
    bt = arr_before["block_table"]
    for i, (b, p) in enumerate(zip(arr_before["row_seq"], arr_before["row_pos"])):
        kc[bt[b, p // 64], p % 64] = res["kI"][i]
        ksc[bt[b, p // 64], p % 64] = res["kI_scale"][i]
    got = oracle_arrays(batch)
    assert np.array_equal(got["kI_cache"], kc) and np.array_equal(got["kI_scale_cache"], ksc)
    # the step on the prolog's outputs
    b2 = dataclasses.replace(batch, qI=qI, qI_scale=qs, w=w)
    g = gpu_decode(b2)
    arr = dict(arr_before, qI=res["qI"], qI_scale=res["qI_scale"], w=res["w"], kI_cache=kc,
               kI_scale_cache=ksc, K=batch.wl.K, scale=batch.wl.scale, D_v=batch.wl.D_v)
    o = run_oracle(arr, keep_scores=False)
    assert np.array_equal(np_(g["indices"]), o["indices"])
    check_attention(g["out"], g["lse"], o["out"], o["lse"])


def test_prolog_bad_rows_write_no_key():
    """A row whose sequence is out of range, and a row whose page id is out
    of range, set their error bits and leave the cache alone; their q and w
    are still written."""
    say("[prolog] bad rows")
    batch = _setup([100, 200, 300], 64, 128, "int", "identity", seed=31)
    inp = make_prolog_inputs(3, 64, 128, D_x=256, mode="int", seed=32, device="cuda")
    prob = B.problem_for_batch(batch)
    row_seq = torch.tensor([0, 7, 2], dtype=torch.int32, device="cuda")   # sequence 7: none
    row_pos = torch.tensor([99, 0, 299], dtype=torch.int32, device="cuda")
    bt = batch.block_table.clone()
    bt[2, 299 // 64] = 1 << 20                                          # page out of range
    prob = B.problem(seq_lens=batch.seq_lens, block_table=bt, num_rows=3, row_seq=row_seq,
                     row_pos=row_pos, H_I=64, D_I=128, indexer_format=B.DSA_INDEXER_MXFP8)
    kI_before = np_(batch.kI).copy()
    qI = torch.zeros((3, 64, 128), dtype=torch.uint8, device="cuda")
    qs = torch.zeros((3, 64, 4), dtype=torch.uint8, device="cuda")
    w = torch.zeros((3, 64), dtype=torch.float32, device="cuda")
    ws = B.workspace(prob, B.DSA_OP_INDEXER_PROLOG)
    B.dsa_indexer_prolog(prob, inp.x, inp.w_q, inp.w_g, inp.k_new, inp.k_gamma, qI, qs, w,
                         batch.kI, ws)
    torch.cuda.synchronize()
    assert B.device_errors(ws) == (B.DSA_DEVERR_ROW | B.DSA_DEVERR_BLOCK)
    after = np_(batch.kI)
    blk0 = int(np_(bt)[0, 99 // 64])
    changed = np.argwhere(np.any(after != kI_before, axis=-1))
    assert {tuple(x) for x in changed} <= {(blk0, 99 % 64), (blk0, 64), (blk0, 65)}
    res = oracle.cpp.indexer_prolog(**prolog_arrays(inp), eps=EPS, H_I=64, D_I=128)
    assert np.array_equal(np_(qI), res["qI"]) and np.array_equal(np_(w), res["w"])
