"""The C ABI on the host: the library loads, exports every symbol its header
declares, sizes workspaces, and rejects bad arguments synchronously with the
documented status codes.  Nothing here launches a kernel."""

import ctypes
import os
import re

import pytest

from indexer_top_sparse_score_amd import binding as B
from workloads import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # an aligned address that host code never dereferences


def header_symbols():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    return sorted(set(re.findall(r"DSA_API\s+[\w\s\*]+?\b(dsa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return B.load()


def test_exports_every_header_symbol(lib):
    syms = header_symbols()
    assert len(syms) == 10 and sorted(B.EXPORTS) == syms
    for s in syms:
        assert getattr(lib, s) is not None
    assert lib.dsa_abi_version() == B.ABI_VERSION


def test_status_strings():
    assert B.status_string(0) == "ok"
    assert B.status_string(-3).startswith("workspace")
    assert B.status_string(99) == "unknown status"


def prob(**kw):
    base = dict(num_seqs=4, num_rows=4, seq_lens=FAKE, block_table=FAKE + 4096, max_blocks=2048,
                block_size=64, row_seq=None, row_pos=None, H_I=64, D_I=128, H_q=128, D_qk=576,
                D_v=512, K=2048, scale=576 ** -0.5)
    base.update(kw)
    return B.DsaProblem(**base)


def paged(base=FAKE + (1 << 30), row=128, nb=8192):
    return B.DsaPaged(base, 64 * row, row, nb)


def ws_size(p, op):
    return B.load().dsa_workspace_size(ctypes.byref(p), op)


def test_workspace_sizes_for_every_workload():
    for name, wl in CONFIGS.items():
        max_blocks = -(-(wl.context or wl.ragged[1]) // 64)
        p = prob(num_seqs=wl.batch, num_rows=wl.rows, max_blocks=max_blocks, H_I=wl.H_I,
                 D_I=wl.D_I, H_q=wl.H_q, D_qk=wl.D_qk, D_v=wl.D_v, K=wl.K, scale=wl.scale,
                 row_seq=FAKE if wl.prefill_rows else None, row_pos=FAKE if wl.prefill_rows else None)
        for op in range(4):
            n = ws_size(p, op)
            assert n >= 256 and n % 256 == 0, (name, op, n)
        # the fused step keeps its scores in the workspace: at least one row's worth
        assert ws_size(p, B.DSA_OP_DECODE_STEP) >= 64 * max_blocks * 4


@pytest.mark.parametrize("field,value", [
    ("num_seqs", 0), ("num_rows", -1), ("max_blocks", 0), ("seq_lens", None),
    ("block_table", None), ("H_I", 0), ("K", 0), ("seq_lens", FAKE + 2)])
def test_invalid_problem_has_no_workspace(field, value):
    assert ws_size(prob(**{field: value}), B.DSA_OP_DECODE_STEP) == 0


@pytest.mark.parametrize("field,value", [("block_size", 32), ("H_I", 65), ("D_I", 96),
                                         ("H_q", 129), ("D_qk", 128), ("D_v", 256)])
def test_unsupported_shapes(field, value):
    assert ws_size(prob(**{field: value}), B.DSA_OP_DECODE_STEP) == 0


def call_scores(p, *, qI=FAKE, w=FAKE, kI=None, scores=FAKE, ld=131072, ws=FAKE, ws_bytes=256):
    return B.raw_call("dsa_indexer_scores", ctypes.byref(p), ctypes.c_void_p(qI),
                      ctypes.c_void_p(w), kI or paged(), ctypes.c_void_p(scores),
                      ctypes.c_int64(ld), ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes), None)


def test_indexer_scores_rejections():
    p = prob()
    assert call_scores(prob(block_size=16)) == B.DSA_ERR_UNSUPPORTED
    assert call_scores(prob(D_I=256)) == B.DSA_ERR_UNSUPPORTED
    assert call_scores(prob(H_I=0)) == B.DSA_ERR_INVALID
    assert call_scores(p, qI=0) == B.DSA_ERR_INVALID
    assert call_scores(p, qI=FAKE + 8) == B.DSA_ERR_INVALID          # misaligned
    assert call_scores(p, ld=1000) == B.DSA_ERR_INVALID              # ld < 64 * max_blocks
    assert call_scores(p, kI=paged(row=64)) == B.DSA_ERR_INVALID     # row shorter than D_I
    assert call_scores(p, kI=B.DsaPaged(FAKE, 8200, 128, 4)) == B.DSA_ERR_INVALID  # stride % 16
    assert call_scores(p, kI=B.DsaPaged(FAKE, 8192, 128, 0)) == B.DSA_ERR_INVALID  # no blocks
    assert call_scores(p, ws=0) == B.DSA_ERR_WORKSPACE
    assert call_scores(p, ws_bytes=255) == B.DSA_ERR_WORKSPACE
    assert call_scores(p, ws=FAKE + 16) == B.DSA_ERR_INVALID         # workspace alignment
    assert call_scores(None if False else prob(num_rows=0)) == B.DSA_OK  # empty: nothing runs
    assert B.raw_call("dsa_indexer_scores", None, None, None, paged(), None, 0, None, 0,
                      None) == B.DSA_ERR_INVALID


def test_indexer_format_rejections():
    # MXFP8: scales for qI are required, and each key block must hold its 64
    # code rows and then 2 * D_I bytes of row scales
    mx = dict(indexer_format=B.DSA_INDEXER_MXFP8, qI_scale=FAKE + (2 << 30))
    kb = lambda row, extra: B.DsaPaged(FAKE + (1 << 30), 64 * row + extra, row, 8192)
    assert call_scores(prob(num_rows=0, **mx), kI=kb(128, 256)) == B.DSA_OK
    assert call_scores(prob(num_rows=0, D_I=64, **mx), kI=kb(64, 128)) == B.DSA_OK
    assert call_scores(prob(num_rows=0, **mx), kI=kb(144, 256)) == B.DSA_OK  # padded rows
    assert call_scores(prob(**mx), kI=kb(128, 0)) == B.DSA_ERR_INVALID     # no room for scales
    assert call_scores(prob(**mx), kI=kb(128, 240)) == B.DSA_ERR_INVALID   # too little room
    assert call_scores(prob(indexer_format=B.DSA_INDEXER_MXFP8)) == B.DSA_ERR_INVALID  # no qI_scale
    assert call_scores(prob(qI_scale=FAKE)) == B.DSA_ERR_INVALID             # E4M3 with scales
    assert call_scores(prob(indexer_format=2)) == B.DSA_ERR_INVALID          # unknown format
    assert ws_size(prob(indexer_format=2), B.DSA_OP_INDEXER_SCORES) == 0
    assert ws_size(prob(**mx), B.DSA_OP_DECODE_STEP) > 0


def test_candidate_list_rejections():
    # candidates need both arrays, a row length >= 1, 16-byte aligned lists;
    # the score rows are then n_cand long
    cand = dict(cand=FAKE + (3 << 30), cand_len=FAKE + (3 << 30) + 4096, n_cand=16384)
    assert call_scores(prob(num_rows=0, **cand), ld=16384) == B.DSA_OK
    assert call_scores(prob(**cand), ld=16383) == B.DSA_ERR_INVALID        # ld < n_cand
    assert call_scores(prob(cand=FAKE), ld=16384) == B.DSA_ERR_INVALID     # no cand_len
    assert call_scores(prob(cand_len=FAKE), ld=16384) == B.DSA_ERR_INVALID # no cand
    assert call_scores(prob(**{**cand, "n_cand": 0})) == B.DSA_ERR_INVALID
    assert call_scores(prob(**{**cand, "cand": FAKE + 4}), ld=16384) == B.DSA_ERR_INVALID
    # sized by slots, not positions: 8192 candidates need no summary, a
    # 131072-position history does
    small = ws_size(prob(**{**cand, "n_cand": 8192}), B.DSA_OP_TOPK)
    assert 0 < small < ws_size(prob(), B.DSA_OP_TOPK)
    assert ws_size(prob(**cand), B.DSA_OP_DECODE_STEP) > 0


def test_topk_rejections():
    def call(p, scores=FAKE, ld=131072, idx=FAKE, counts=None, ws=FAKE, nbytes=256):
        return B.raw_call("dsa_topk", ctypes.byref(p), ctypes.c_void_p(scores),
                          ctypes.c_int64(ld), ctypes.c_void_p(idx), ctypes.c_void_p(counts),
                          ctypes.c_void_p(ws), ctypes.c_size_t(nbytes), None)
    assert call(prob(K=0)) == B.DSA_ERR_INVALID
    assert call(prob(), idx=0) == B.DSA_ERR_INVALID
    assert call(prob(), counts=FAKE + 2) == B.DSA_ERR_INVALID
    assert call(prob(), ld=10) == B.DSA_ERR_INVALID
    assert call(prob(), nbytes=0) == B.DSA_ERR_WORKSPACE
    assert call(prob(num_rows=0)) == B.DSA_OK


def test_sparse_attn_rejections():
    def call(p, q=FAKE, k=None, v=None, idx=FAKE, out=FAKE, lse=None, ws=FAKE, nbytes=1 << 30):
        return B.raw_call("dsa_sparse_attn", ctypes.byref(p), ctypes.c_void_p(q),
                          k or paged(row=1152), v or paged(row=1152), ctypes.c_void_p(idx),
                          ctypes.c_void_p(out), ctypes.c_void_p(lse), ctypes.c_void_p(ws),
                          ctypes.c_size_t(nbytes), None)
    assert call(prob(D_qk=128, D_v=128)) == B.DSA_ERR_UNSUPPORTED
    assert call(prob(K=16385)) == B.DSA_ERR_UNSUPPORTED              # above DSA_MAX_ATTN_K
    assert call(prob(K=16384), nbytes=0) == B.DSA_ERR_WORKSPACE      # shape accepted
    assert call(prob(scale=float("nan"))) == B.DSA_ERR_INVALID
    assert call(prob(), k=paged(row=1024)) == B.DSA_ERR_INVALID      # K row < 576 bf16
    assert call(prob(), q=FAKE + 4) == B.DSA_ERR_INVALID
    assert call(prob(), idx=0) == B.DSA_ERR_INVALID
    assert call(prob(), lse=FAKE + 1) == B.DSA_ERR_INVALID
    need = ws_size(prob(), B.DSA_OP_SPARSE_ATTN)
    assert call(prob(), nbytes=need - 256) == B.DSA_ERR_WORKSPACE
    assert call(prob(num_rows=0)) == B.DSA_OK
    # a latent cache (v aliases k) may span at most 64 GiB; separate V may not
    big = paged(row=1152, nb=1 << 20)                                 # 72 GiB
    assert call(prob(), k=big, v=big) == B.DSA_ERR_UNSUPPORTED
    sep_v = paged(base=FAKE + (1 << 40), row=1024, nb=1 << 20)
    assert call(prob(), k=big, v=sep_v, nbytes=0) == B.DSA_ERR_WORKSPACE
    edge = paged(row=1152, nb=(1 << 36) // (64 * 1152))               # just below 64 GiB
    assert call(prob(), k=edge, v=edge, nbytes=0) == B.DSA_ERR_WORKSPACE


def test_fp8_kv_rejections():
    def call(p, k=None, v=None, nbytes=0):
        k = k or fp8()
        return B.raw_call("dsa_sparse_attn", ctypes.byref(p), ctypes.c_void_p(FAKE), k, v or k,
                          ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None,
                          ctypes.c_void_p(FAKE), ctypes.c_size_t(nbytes), None)

    def fp8(row=576, extra=1280, nb=8192, base=FAKE + (1 << 30)):
        return B.DsaPaged(base, 64 * row + extra, row, nb)

    fp8p = prob(kv_format=B.DSA_KV_FP8)
    assert call(fp8p) == B.DSA_ERR_WORKSPACE                          # accepted up to the workspace
    assert ws_size(fp8p, B.DSA_OP_SPARSE_ATTN) == ws_size(prob(), B.DSA_OP_SPARSE_ATTN)
    assert ws_size(prob(kv_format=2), B.DSA_OP_SPARSE_ATTN) == 0
    assert call(prob(kv_format=2)) == B.DSA_ERR_INVALID
    assert call(prob(kv_format=B.DSA_KV_FP8, D_qk=64, D_v=64, H_q=8)) == B.DSA_ERR_UNSUPPORTED
    assert call(fp8p, k=fp8(extra=1264)) == B.DSA_ERR_INVALID          # no room for the scales
    assert call(fp8p, k=fp8(row=560)) == B.DSA_ERR_INVALID             # row < 576 codes
    assert call(fp8p, k=fp8(), v=fp8(base=FAKE + (1 << 31))) == B.DSA_ERR_INVALID  # not latent
    # the 64 GiB limit of the bf16 latent kernel does not apply
    assert call(fp8p, k=fp8(nb=1 << 22)) == B.DSA_ERR_WORKSPACE


def test_decode_step_rejections():
    def call(p, kI=None, k=None, nbytes=None, ws=FAKE, indices=None):
        nbytes = ws_size(prob(), 3) if nbytes is None else nbytes
        return B.raw_call("dsa_decode_step", ctypes.byref(p), ctypes.c_void_p(FAKE),
                          ctypes.c_void_p(FAKE), kI or paged(), ctypes.c_void_p(FAKE),
                          k or paged(row=1152), k or paged(row=1152), ctypes.c_void_p(FAKE),
                          None, ctypes.c_void_p(indices), None, ctypes.c_void_p(ws),
                          ctypes.c_size_t(nbytes), None)
    assert call(prob(H_I=100)) == B.DSA_ERR_UNSUPPORTED
    assert call(prob(), kI=paged(row=16)) == B.DSA_ERR_INVALID
    assert call(prob(), nbytes=1024) == B.DSA_ERR_WORKSPACE
    assert call(prob(), indices=FAKE + 2) == B.DSA_ERR_INVALID
    assert call(prob(num_rows=0), nbytes=256) == B.DSA_OK


def test_decode_step_static_rejections():
    # validation runs before the scratch is looked up, so every case here
    # returns without touching a GPU
    def call(p, kI=None, k=None, indices=None, err=None):
        return B.raw_call("dsa_decode_step_static", ctypes.byref(p), ctypes.c_void_p(FAKE),
                          ctypes.c_void_p(FAKE), kI or paged(), ctypes.c_void_p(FAKE),
                          k or paged(row=1152), k or paged(row=1152), ctypes.c_void_p(FAKE),
                          None, ctypes.c_void_p(indices), None, ctypes.c_void_p(err), None)
    assert call(prob(H_I=100)) == B.DSA_ERR_UNSUPPORTED
    assert call(prob(), kI=paged(row=16)) == B.DSA_ERR_INVALID
    assert call(prob(), indices=FAKE + 2) == B.DSA_ERR_INVALID
    assert call(prob(), err=FAKE + 2) == B.DSA_ERR_INVALID
    assert call(prob(num_rows=0)) == B.DSA_OK
    # a layout that cannot fit DSA_STATIC_SCRATCH_BYTES even one row per pass:
    # a history of 2^24 blocks needs a 4 GiB score row
    assert call(prob(max_blocks=1 << 24)) == B.DSA_ERR_WORKSPACE


def test_decode_step_timed_rejections():
    # the events are checked first, then everything dsa_decode_step checks;
    # no case here reaches a launch
    def call(p, events, ws_bytes=1 << 40):
        ev = None if events is None else (ctypes.c_void_p * 8)(*events)
        return B.raw_call("dsa_decode_step_timed", ctypes.byref(p), ctypes.c_void_p(FAKE),
                          ctypes.c_void_p(FAKE), paged(), ctypes.c_void_p(FAKE),
                          paged(row=1152), paged(row=1152), ctypes.c_void_p(FAKE), None, None,
                          None, ctypes.c_void_p(FAKE), ws_bytes, ev, None)
    eight = [FAKE + 256 * i for i in range(8)]
    assert call(prob(), None) == B.DSA_ERR_INVALID
    assert call(prob(), eight[:7] + [None]) == B.DSA_ERR_INVALID
    assert call(prob(H_I=100), eight) == B.DSA_ERR_UNSUPPORTED
    assert call(prob(), eight, ws_bytes=0) == B.DSA_ERR_WORKSPACE
    assert call(prob(num_rows=0), eight) == B.DSA_OK


def call_prolog(p, D_x=4096, eps=1e-6, x=FAKE, w_q=FAKE + (1 << 28), w_g=FAKE + (2 << 28),
                k_new=FAKE + (3 << 28), k_gamma=FAKE + (4 << 28), qI=FAKE + (5 << 28),
                qI_scale=FAKE + (6 << 28), w=FAKE + (7 << 28), kI=None, ws=FAKE + (8 << 28),
                ws_bytes=256):
    V = ctypes.c_void_p
    return B.raw_call("dsa_indexer_prolog", ctypes.byref(p), ctypes.c_int32(D_x),
                      ctypes.c_float(eps), V(x), V(w_q), V(w_g), V(k_new), V(k_gamma), V(qI),
                      V(qI_scale), V(w), kI or B.DsaPaged(FAKE + (1 << 30), 64 * 128 + 256, 128, 8192),
                      V(ws), ctypes.c_size_t(ws_bytes), None)


def test_indexer_prolog_rejections():
    mx = dict(indexer_format=B.DSA_INDEXER_MXFP8)
    p = prob(**mx)
    assert ws_size(p, B.DSA_OP_INDEXER_PROLOG) == 256
    assert ws_size(prob(), B.DSA_OP_INDEXER_PROLOG) == 0               # not MXFP8
    assert call_prolog(prob(num_rows=0, **mx)) == B.DSA_OK              # empty: nothing runs
    assert call_prolog(prob(num_rows=0, D_I=64, **mx),
                       kI=B.DsaPaged(FAKE, 64 * 64 + 128, 64, 4)) == B.DSA_OK
    assert call_prolog(prob()) == B.DSA_ERR_INVALID                     # E4M3 format
    assert call_prolog(prob(D_I=96, **mx)) == B.DSA_ERR_UNSUPPORTED
    assert call_prolog(prob(H_I=65, **mx)) == B.DSA_ERR_UNSUPPORTED
    assert call_prolog(p, D_x=0) == B.DSA_ERR_INVALID
    assert call_prolog(p, D_x=4016) == B.DSA_ERR_INVALID                # not a multiple of 32
    assert call_prolog(p, D_x=65536 + 32) == B.DSA_ERR_UNSUPPORTED
    assert call_prolog(p, eps=-1.0) == B.DSA_ERR_INVALID
    assert call_prolog(p, eps=float("nan")) == B.DSA_ERR_INVALID
    for arg in ("x", "w_q", "w_g", "k_new", "k_gamma", "qI", "qI_scale", "w"):
        assert call_prolog(p, **{arg: 0}) == B.DSA_ERR_INVALID, arg
    for arg, off in (("x", 8), ("w_q", 8), ("w_g", 8), ("qI", 8), ("k_new", 2),
                     ("k_gamma", 2), ("w", 2)):
        assert call_prolog(p, **{arg: FAKE + off}) == B.DSA_ERR_INVALID, arg   # misaligned
    assert call_prolog(p, kI=B.DsaPaged(FAKE, 64 * 128, 128, 8)) == B.DSA_ERR_INVALID  # no scale room
    assert call_prolog(p, ws=0) == B.DSA_ERR_WORKSPACE
    assert call_prolog(p, ws_bytes=255) == B.DSA_ERR_WORKSPACE
    assert call_prolog(prob(seq_lens=None, **mx)) == B.DSA_ERR_INVALID
