"""Thin ctypes binding of libdsa.so (see include/dsa.h for the contract).

Argument marshalling only: torch tensors supply device memory and the
current stream; every step of the path runs in the HIP kernels of the
library.  There is no fallback: a missing or stale library raises.
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

DSA_OK = 0
DSA_ERR_INVALID = -1
DSA_ERR_UNSUPPORTED = -2
DSA_ERR_WORKSPACE = -3
DSA_ERR_HIP = -4

DSA_DEVERR_ROW = 1
DSA_DEVERR_BLOCK = 2
DSA_DEVERR_INDEX = 4

DSA_OP_INDEXER_SCORES = 0
DSA_OP_TOPK = 1
DSA_OP_SPARSE_ATTN = 2
DSA_OP_DECODE_STEP = 3
DSA_OP_INDEXER_PROLOG = 4

ABI_VERSION = 8
DSA_INDEXER_E4M3 = 0
DSA_INDEXER_MXFP8 = 1
DSA_KV_BF16 = 0
DSA_KV_FP8 = 1
BLOCK = 64

#: every symbol include/dsa.h declares
EXPORTS = ("dsa_workspace_size", "dsa_indexer_scores", "dsa_topk", "dsa_sparse_attn",
           "dsa_decode_step", "dsa_decode_step_timed", "dsa_decode_step_static",
           "dsa_indexer_prolog", "dsa_status_string", "dsa_abi_version")


class DsaPaged(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("block_stride", ctypes.c_int64),
                ("row_stride", ctypes.c_int64), ("num_blocks", ctypes.c_int64)]


class DsaProblem(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_rows", ctypes.c_int32),
                ("seq_lens", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("max_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("row_seq", ctypes.c_void_p), ("row_pos", ctypes.c_void_p),
                ("H_I", ctypes.c_int32), ("D_I", ctypes.c_int32), ("H_q", ctypes.c_int32),
                ("D_qk", ctypes.c_int32), ("D_v", ctypes.c_int32), ("K", ctypes.c_int32),
                ("scale", ctypes.c_float), ("indexer_format", ctypes.c_int32),
                ("qI_scale", ctypes.c_void_p),
                ("cand", ctypes.c_void_p), ("cand_len", ctypes.c_void_p), ("n_cand", ctypes.c_int32),
                ("kv_format", ctypes.c_int32)]


class DsaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what} failed: {status_string(status)} ({status})")


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdsa.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m indexer_top_sparse_score_amd.build`")
    lib = ctypes.CDLL(path)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    prob = ctypes.POINTER(DsaProblem)
    lib.dsa_workspace_size.argtypes = [prob, ctypes.c_int]
    lib.dsa_workspace_size.restype = sz
    lib.dsa_indexer_scores.argtypes = [prob, P, P, DsaPaged, P, i64, P, sz, P]
    lib.dsa_topk.argtypes = [prob, P, i64, P, P, P, sz, P]
    lib.dsa_sparse_attn.argtypes = [prob, P, DsaPaged, DsaPaged, P, P, P, P, sz, P]
    lib.dsa_decode_step.argtypes = [prob, P, P, DsaPaged, P, DsaPaged, DsaPaged, P, P, P, P, P,
                                    sz, P]
    lib.dsa_decode_step_timed.argtypes = [prob, P, P, DsaPaged, P, DsaPaged, DsaPaged, P, P, P,
                                          P, P, sz, ctypes.POINTER(P), P]
    lib.dsa_decode_step_static.argtypes = [prob, P, P, DsaPaged, P, DsaPaged, DsaPaged, P, P, P,
                                           P, P, P]
    lib.dsa_indexer_prolog.argtypes = [prob, i32, ctypes.c_float, P, P, P, P, P, P, P, P,
                                       DsaPaged, P, sz, P]
    for f in ("dsa_indexer_scores", "dsa_topk", "dsa_sparse_attn", "dsa_decode_step",
              "dsa_decode_step_timed", "dsa_decode_step_static", "dsa_indexer_prolog"):
        getattr(lib, f).restype = ctypes.c_int
    lib.dsa_status_string.argtypes = [ctypes.c_int]
    lib.dsa_status_string.restype = ctypes.c_char_p
    lib.dsa_abi_version.argtypes = []
    lib.dsa_abi_version.restype = ctypes.c_int
    if lib.dsa_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path} has ABI {lib.dsa_abi_version()}, expected {ABI_VERSION}")
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().dsa_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def paged(cache: torch.Tensor) -> DsaPaged:
    """Descriptor of a [num_blocks, 64, ...] cache tensor (any row stride).
    An MXFP8 index-key cache is [num_blocks, 66, D_I]: two more D_I-byte rows
    per block hold the 64 rows' scales.  An FP8 KV cache is uint8
    [num_blocks, 64 + n, D_qk]: the rows after the 64 code rows hold the 64
    rows' float32 tile scales."""
    if cache.dim() < 3 or cache.shape[1] < BLOCK or (cache.shape[1] > BLOCK and
                                                     cache.dtype != torch.uint8):
        raise ValueError("paged cache must be [num_blocks, 64, row] (uint8 [num_blocks, 64 + n, "
                         "row] with the block's scales in the extra rows)")
    es = cache.element_size()
    return DsaPaged(cache.data_ptr(), cache.stride(0) * es, cache.stride(1) * es, cache.shape[0])


def problem(*, seq_lens, block_table, num_rows=None, row_seq=None, row_pos=None, H_I=64,
            D_I=128, H_q=128, D_qk=576, D_v=512, K=2048, scale=576 ** -0.5,
            qI_scale=None, cand=None, cand_len=None, kv_format=DSA_KV_BF16,
            indexer_format=None) -> DsaProblem:
    """Problem descriptor; device tensors are referenced, not copied.  With
    ``qI_scale`` (uint8 E8M0 [rows, H_I, D_I/32]) the indexer runs in MXFP8
    format and each index-key block carries its rows' scales after the code rows.
    With ``cand`` (int32 [rows, n_cand], ascending positions) and ``cand_len``
    (int32 [rows]) each row scores only its candidate positions.  ``kv_format``
    DSA_KV_FP8: the KV cache holds E4M3 rows with float32 tile scales.
    ``indexer_format`` overrides the format ``qI_scale`` implies (the prolog
    writes MXFP8 operands and takes no ``qI_scale`` here)."""
    num_seqs = int(seq_lens.shape[0])
    if num_rows is None:
        num_rows = int(row_seq.shape[0]) if row_seq is not None else num_seqs
    p = DsaProblem(num_seqs, num_rows, seq_lens.data_ptr(), block_table.data_ptr(),
                   int(block_table.shape[1]), BLOCK,
                   None if row_seq is None else row_seq.data_ptr(),
                   None if row_pos is None else row_pos.data_ptr(),
                   H_I, D_I, H_q, D_qk, D_v, K, scale,
                   (DSA_INDEXER_E4M3 if qI_scale is None else DSA_INDEXER_MXFP8)
                   if indexer_format is None else int(indexer_format),
                   None if qI_scale is None else qI_scale.data_ptr(),
                   None if cand is None else cand.data_ptr(),
                   None if cand_len is None else cand_len.data_ptr(),
                   0 if cand is None else int(cand.shape[1]), int(kv_format))
    p._keep = (seq_lens, block_table, row_seq, row_pos, qI_scale, cand, cand_len)  # keep alive
    return p


def problem_for_batch(batch) -> DsaProblem:
    """Problem descriptor for an object with ``seq_lens``, ``block_table``,
    ``row_seq``, ``row_pos``, ``qI`` tensors and a ``wl`` carrying the dims."""
    wl = batch.wl
    return problem(seq_lens=batch.seq_lens, block_table=batch.block_table,
                   num_rows=int(batch.qI.shape[0]), row_seq=batch.row_seq,
                   row_pos=batch.row_pos, H_I=wl.H_I, D_I=wl.D_I, H_q=wl.H_q, D_qk=wl.D_qk,
                   D_v=wl.D_v, K=wl.K, scale=wl.scale,
                   qI_scale=getattr(batch, "qI_scale", None), cand=getattr(batch, "cand", None),
                   cand_len=getattr(batch, "cand_len", None),
                   kv_format=DSA_KV_FP8 if getattr(wl, "kv_fmt", "bf16") == "fp8" else DSA_KV_BF16)


def dsa_workspace_size(prob: DsaProblem, op: int) -> int:
    return int(load().dsa_workspace_size(ctypes.byref(prob), op))


def workspace(prob: DsaProblem, op: int, device="cuda") -> torch.Tensor:
    """A zeroed workspace of the size `op` needs (its error word starts clear)."""
    n = dsa_workspace_size(prob, op)
    if n == 0:
        raise DsaError(DSA_ERR_UNSUPPORTED, "dsa_workspace_size")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def device_errors(ws: torch.Tensor) -> int:
    """The sticky DSA_DEVERR_* bits (synchronises the workspace's stream)."""
    return int(ws[:4].view(torch.int32).item()) & 0xFFFFFFFF


def _check(st, what):
    if st != DSA_OK:
        raise DsaError(st, what)


def dsa_indexer_scores(prob, qI, w, kI, scores, ws, stream=None):
    """scores[r, s] = sum_h w[r,h] max(0, qI[r,h] . kI[s]) for s <= p_r."""
    _check(load().dsa_indexer_scores(ctypes.byref(prob), _ptr(qI), _ptr(w), paged(kI),
                                     _ptr(scores), scores.stride(0), _ptr(ws), ws.numel(),
                                     _stream(stream)), "dsa_indexer_scores")


def dsa_topk(prob, scores, indices, ws, counts=None, stream=None):
    """indices[r] = ascending Top-K positions of scores[r, :p_r+1], -1 padded."""
    _check(load().dsa_topk(ctypes.byref(prob), _ptr(scores), scores.stride(0), _ptr(indices),
                           _ptr(counts), _ptr(ws), ws.numel(), _stream(stream)), "dsa_topk")


def dsa_sparse_attn(prob, q, k, v, indices, out, ws, lse=None, stream=None):
    """Softmax attention of each row over the KV rows named in indices (v may be k)."""
    _check(load().dsa_sparse_attn(ctypes.byref(prob), _ptr(q), paged(k), paged(v),
                                  _ptr(indices), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                  _stream(stream)), "dsa_sparse_attn")


def dsa_decode_step(prob, qI, w, kI, q, k, v, out, ws, lse=None, indices=None, counts=None,
                    stream=None):
    """The fused indexer -> Top-K -> sparse attention step."""
    _check(load().dsa_decode_step(ctypes.byref(prob), _ptr(qI), _ptr(w), paged(kI), _ptr(q),
                                  paged(k), paged(v), _ptr(out), _ptr(lse), _ptr(indices),
                                  _ptr(counts), _ptr(ws), ws.numel(), _stream(stream)),
           "dsa_decode_step")


def dsa_decode_step_timed(prob, qI, w, kI, q, k, v, out, ws, events, lse=None, indices=None,
                          counts=None, stream=None):
    """dsa_decode_step, stamping eight torch.cuda.Event objects with the start
    and end of its stages (scan, selection, attention, merge).  Each event is
    recorded once first if it has no HIP event yet (torch creates them
    lazily)."""
    if len(events) != 8:
        raise ValueError("eight events")
    handles = []
    for e in events:
        if not e.cuda_event:
            e.record()
        handles.append(e.cuda_event)
    arr = (ctypes.c_void_p * 8)(*handles)
    _check(load().dsa_decode_step_timed(ctypes.byref(prob), _ptr(qI), _ptr(w), paged(kI), _ptr(q),
                                        paged(k), paged(v), _ptr(out), _ptr(lse), _ptr(indices),
                                        _ptr(counts), _ptr(ws), ws.numel(), arr,
                                        _stream(stream)), "dsa_decode_step_timed")


def dsa_decode_step_static(prob, qI, w, kI, q, k, v, out, lse=None, indices=None, counts=None,
                           err=None, stream=None):
    """The fused step on the library's own scratch (no workspace argument)."""
    _check(load().dsa_decode_step_static(ctypes.byref(prob), _ptr(qI), _ptr(w), paged(kI),
                                         _ptr(q), paged(k), paged(v), _ptr(out), _ptr(lse),
                                         _ptr(indices), _ptr(counts), _ptr(err),
                                         _stream(stream)), "dsa_decode_step_static")


def dsa_indexer_prolog(prob, x, w_q, w_g, k_new, k_gamma, qI, qI_scale, w, kI, ws, eps=1e-6,
                       stream=None):
    """The indexer prolog: MXFP8 qI / qI_scale = quant(W_q x), w = W_g x, and
    each row's normalised, quantised new key written into the MXFP8 cache kI
    ([num_blocks, 66, D_I] uint8).  x [rows, D_x], w_q [H_I * D_I, D_x], w_g
    [H_I, D_x], k_new [rows, D_I], k_gamma [D_I], all bf16."""
    _check(load().dsa_indexer_prolog(ctypes.byref(prob), int(x.shape[1]), float(eps), _ptr(x),
                                     _ptr(w_q), _ptr(w_g), _ptr(k_new), _ptr(k_gamma), _ptr(qI),
                                     _ptr(qI_scale), _ptr(w), paged(kI), _ptr(ws), ws.numel(),
                                     _stream(stream)), "dsa_indexer_prolog")


def raw_call(name, *args):
    """Call an entry point with raw ctypes arguments (for boundary tests)."""
    return getattr(load(), name)(*args)
