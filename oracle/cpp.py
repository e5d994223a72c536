"""ctypes front end of the plain C++ oracle (oracle/cpp/dsa_oracle.cpp).

TEST INFRASTRUCTURE ONLY (see the package docstring).  The C++ oracle states
the same definitions as the numpy one in this package, written separately:
its own E4M3 / E8M0 / bfloat16 decoders, binary64 arithmetic, a full sort for
Top-K and the softmax definition for attention.  The two are independent
routes to one result and the tests pin each against the other and against
closed forms and brute force.  It exists because it is fast enough to check
long rows and to time as the CPU baseline; the numpy route stays the
readable statement.

``build()`` compiles it with the host compiler (g++ -O2, no GPU code); the
loader builds it on first use when the library is missing.
"""

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cpp", "dsa_oracle.cpp")
LIB = os.path.join(HERE, "cpp", "libdsa_oracle.so")

_lock = threading.Lock()
_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


class _Step(ctypes.Structure):
    _fields_ = [
        ("num_rows", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
        ("seq_lens", _i32p), ("block_table", _i32p), ("row_seq", _i32p), ("row_pos", _i32p),
        ("H_I", ctypes.c_int32), ("D_I", ctypes.c_int32),
        ("qI", _u8p), ("w", _f32p), ("kI", _u8p), ("qI_scale", _u8p), ("kI_scale", _u8p),
        ("cand", _i32p), ("cand_len", _i32p), ("n_cand", ctypes.c_int32),
        ("H_q", ctypes.c_int32), ("D_qk", ctypes.c_int32), ("D_v", ctypes.c_int32),
        ("K", ctypes.c_int32), ("scale", ctypes.c_double),
        ("q", _u16p), ("k", _u16p), ("v", _u16p), ("k8", _u8p), ("k8_scale", _f32p),
    ]


def build(verbose=False):
    """Compile libdsa_oracle.so from source (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def lib():
    """The loaded oracle library (built first if it is missing)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
                build()
            L = ctypes.CDLL(LIB)
            L.orc_e4m3_table.argtypes = [_f64p]
            L.orc_score_keys.argtypes = [_f32p, ctypes.c_int64, ctypes.POINTER(ctypes.c_uint32)]
            L.orc_indexer_scores.argtypes = [_u8p, _f32p, _u8p, _u8p, _u8p, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int64, _f32p, ctypes.c_int]
            L.orc_topk.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int64, _i32p]
            L.orc_topk.restype = ctypes.c_int64
            L.orc_attention.argtypes = [_u16p, _u16p, _u16p, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_double, _f64p, _f64p,
                                        ctypes.c_int]
            L.orc_masked_dense_attention.argtypes = [_u16p, _u16p, _u16p, _u8p, ctypes.c_int64,
                                                     ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                     ctypes.c_double, _f64p, _f64p]
            L.orc_decode_step.argtypes = [ctypes.POINTER(_Step), _i32p, ctypes.c_int, _i32p,
                                          _i64p, _f64p, _f64p, _f32p, ctypes.c_int64,
                                          ctypes.c_int]
            L.orc_decode_step.restype = ctypes.c_int
            L.orc_kv_fp8_decode.argtypes = [_u8p, _f32p, ctypes.c_int64, ctypes.c_int, _f64p]
            L.orc_bf16_round.argtypes = [_f64p, ctypes.c_int64, _u16p]
            L.orc_e4m3_round.argtypes = [_f64p, ctypes.c_int64, _u8p]
            L.orc_mx_quantize.argtypes = [_f64p, ctypes.c_int64, ctypes.c_int, _u8p, _u8p]
            L.orc_prolog.argtypes = [_u16p, _u16p, _u16p, _u16p, _u16p, ctypes.c_double,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     _f64p, _u16p, _u8p, _u8p, _f32p, _u16p, _u8p, _u8p,
                                     ctypes.c_int]
            _lib = L
    return _lib


def _arr(x, dtype):
    return np.ascontiguousarray(np.asarray(x), dtype=dtype)


def _ptr(a, ctype):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctype))


def e4m3_table():
    """Value of every E4M3 code as the C++ decoder gives it."""
    out = np.empty(256, np.float64)
    lib().orc_e4m3_table(_ptr(out, ctypes.c_double))
    return out


def score_keys(scores):
    s = _arr(scores, np.float32).ravel()
    keys = np.empty(len(s), np.uint32)
    lib().orc_score_keys(_ptr(s, ctypes.c_float), len(s), _ptr(keys, ctypes.c_uint32))
    return keys


def indexer_scores_row(qI_codes, w, kI_rows, qI_scale=None, kI_scale=None, threads=1):
    """Index scores of one row; same contract as the numpy oracle's."""
    q = _arr(qI_codes, np.uint8)
    k = _arr(kI_rows, np.uint8).reshape(-1, q.shape[1])
    wv = _arr(w, np.float32)
    qs = None if qI_scale is None else _arr(qI_scale, np.uint8)
    ks = None if kI_scale is None else _arr(kI_scale, np.uint8)
    out = np.empty(k.shape[0], np.float32)
    lib().orc_indexer_scores(_ptr(q, ctypes.c_uint8), _ptr(wv, ctypes.c_float),
                             _ptr(k, ctypes.c_uint8), _ptr(qs, ctypes.c_uint8),
                             _ptr(ks, ctypes.c_uint8), q.shape[0], q.shape[1], k.shape[0],
                             _ptr(out, ctypes.c_float), int(threads))
    return out


def topk_row(scores, K):
    s = _arr(scores, np.float32).ravel()
    out = np.empty(int(K), np.int32)
    n = lib().orc_topk(_ptr(s, ctypes.c_float), len(s), int(K), _ptr(out, ctypes.c_int32))
    return out, int(n)


def sparse_attn_row(q_bits, k_rows_bits, v_rows_bits, scale, threads=1):
    q = _arr(q_bits, np.uint16)
    k = _arr(k_rows_bits, np.uint16).reshape(-1, q.shape[1])
    v = _arr(v_rows_bits, np.uint16)
    v = v.reshape(k.shape[0], v.shape[-1])
    H, D_v = q.shape[0], v.shape[1]
    o = np.empty((H, D_v), np.float64)
    lse = np.empty(H, np.float64)
    lib().orc_attention(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                        _ptr(v, ctypes.c_uint16), k.shape[0], H, q.shape[1], D_v, float(scale),
                        _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double), int(threads))
    return o, lse


def kv_fp8_to_f64(codes, scales):
    """Decoded FP8 KV rows (codes uint8 [..., D], scales float32 [..., ceil(D/128)])
    -> float64 [..., D]; the C++ route's counterpart of ``oracle.kv_fp8_to_f64``."""
    c = _arr(codes, np.uint8)
    D = c.shape[-1]
    n = c.size // D if D else 0
    s = _arr(scales, np.float32)
    if s.shape[-1] != (D + 127) // 128 or s.size != n * s.shape[-1]:
        raise ValueError("one scale per tile of 128 elements")
    out = np.empty(c.shape, np.float64)
    lib().orc_kv_fp8_decode(_ptr(c, ctypes.c_uint8), _ptr(s, ctypes.c_float), n, D,
                            _ptr(out, ctypes.c_double))
    return out


def bf16_round(values):
    """bf16 bits of binary64 values, nearest even (the C++ route)."""
    v = _arr(values, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().orc_bf16_round(_ptr(v, ctypes.c_double), v.size, _ptr(out, ctypes.c_uint16))
    return out


def e4m3_round(values):
    """E4M3 codes of binary64 values (the C++ route): nearest, ties to even,
    saturated at 448, sign kept."""
    v = _arr(values, np.float64)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e4m3_round(_ptr(v, ctypes.c_double), v.size, _ptr(out, ctypes.c_uint8))
    return out


def mx_quantize(values, group=32):
    """MXFP8 codes and E8M0 scales along the last axis (the C++ route)."""
    if group != 32:
        raise ValueError("groups of 32")
    v = _arr(values, np.float64)
    n = v.shape[-1]
    if n % 32:
        raise ValueError("length must be a multiple of the group")
    rows = v.size // n if n else 0
    codes = np.empty(v.shape, np.uint8)
    scales = np.empty(v.shape[:-1] + (n // 32,), np.uint8)
    lib().orc_mx_quantize(_ptr(v, ctypes.c_double), rows, n, _ptr(codes, ctypes.c_uint8),
                          _ptr(scales, ctypes.c_uint8))
    return codes, scales


def indexer_prolog(*, x, w_q, w_g, k_new, k_gamma, eps, H_I, D_I, threads=1):
    """The indexer prolog; same contract and result dict as
    ``oracle.indexer_prolog`` (the numpy route)."""
    xa = _arr(x, np.uint16)
    rows, D_x = xa.shape
    wq = _arr(w_q, np.uint16)
    wg = _arr(w_g, np.uint16)
    kn = _arr(k_new, np.uint16)
    ga = _arr(k_gamma, np.uint16)
    F = H_I * D_I
    if wq.shape != (F, D_x) or wg.shape != (H_I, D_x) or kn.shape != (rows, D_I) \
            or ga.shape != (D_I,) or D_I % 32:
        raise ValueError("prolog shapes")
    q = np.empty((rows, F), np.float64)
    q16 = np.empty((rows, F), np.uint16)
    qI = np.empty((rows, F), np.uint8)
    qs = np.empty((rows, F // 32), np.uint8)
    w = np.empty((rows, H_I), np.float32)
    k16 = np.empty((rows, D_I), np.uint16)
    kI = np.empty((rows, D_I), np.uint8)
    ks = np.empty((rows, D_I // 32), np.uint8)
    P = ctypes.c_uint16, ctypes.c_uint8
    lib().orc_prolog(_ptr(xa, P[0]), _ptr(wq, P[0]), _ptr(wg, P[0]), _ptr(kn, P[0]),
                     _ptr(ga, P[0]), float(eps), rows, D_x, H_I, D_I, _ptr(q, ctypes.c_double),
                     _ptr(q16, P[0]), _ptr(qI, P[1]), _ptr(qs, P[1]), _ptr(w, ctypes.c_float),
                     _ptr(k16, P[0]), _ptr(kI, P[1]), _ptr(ks, P[1]), int(threads))
    return {"q": q, "q_bf16": q16, "qI": qI.reshape(rows, H_I, D_I),
            "qI_scale": qs.reshape(rows, H_I, D_I // 32), "w": w,
            "k_bf16": k16, "kI": kI, "kI_scale": ks}


def masked_dense_attn_row(q_bits, k_all_bits, v_all_bits, selected, scale):
    q = _arr(q_bits, np.uint16)
    k = _arr(k_all_bits, np.uint16).reshape(-1, q.shape[1])
    v = _arr(v_all_bits, np.uint16)
    v = v.reshape(k.shape[0], v.shape[-1])
    sel = _arr(selected, np.uint8)
    H, D_v = q.shape[0], v.shape[1]
    o = np.empty((H, D_v), np.float64)
    lse = np.empty(H, np.float64)
    lib().orc_masked_dense_attention(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                                     _ptr(v, ctypes.c_uint16), _ptr(sel, ctypes.c_uint8),
                                     k.shape[0], H, q.shape[1], D_v, float(scale),
                                     _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double))
    return o, lse


def decode_step(*, qI, w, kI_cache, q, k_cache, v_cache, block_table, seq_lens, K, scale,
                D_v, row_seq=None, row_pos=None, rows=None, keep_scores=True, qI_scale=None,
                kI_scale_cache=None, cand=None, cand_len=None, k_scale_cache=None, threads=1):
    """The whole step for the chosen rows; same contract and result dict as
    the numpy oracle's ``decode_step``, plus ``threads`` host threads."""
    keep = {}

    def hold(x, dtype):
        if x is None:
            return None
        a = _arr(x, dtype)
        keep[id(a)] = a
        return a

    qI_a = hold(qI, np.uint8)
    num_rows, H_I, D_I = qI_a.shape
    q_a = hold(q, np.uint16)
    H_q, D_qk = q_a.shape[1], q_a.shape[2]
    kI_a = hold(kI_cache, np.uint8)
    bt = hold(block_table, np.int32)
    sl = hold(seq_lens, np.int32)
    st = _Step()
    st.num_rows, st.num_seqs = num_rows, len(sl)
    st.max_blocks, st.num_blocks = bt.shape[1], kI_a.shape[0]
    st.seq_lens, st.block_table = _ptr(sl, ctypes.c_int32), _ptr(bt, ctypes.c_int32)
    st.row_seq = _ptr(hold(row_seq, np.int32), ctypes.c_int32)
    st.row_pos = _ptr(hold(row_pos, np.int32), ctypes.c_int32)
    st.H_I, st.D_I = H_I, D_I
    st.qI, st.w = _ptr(qI_a, ctypes.c_uint8), _ptr(hold(w, np.float32), ctypes.c_float)
    st.kI = _ptr(kI_a, ctypes.c_uint8)
    st.qI_scale = _ptr(hold(qI_scale, np.uint8), ctypes.c_uint8)
    st.kI_scale = _ptr(hold(kI_scale_cache, np.uint8), ctypes.c_uint8)
    if cand is not None:
        ca = hold(cand, np.int32)
        st.cand, st.n_cand = _ptr(ca, ctypes.c_int32), ca.shape[1]
        st.cand_len = _ptr(hold(cand_len, np.int32), ctypes.c_int32)
    st.H_q, st.D_qk, st.D_v, st.K, st.scale = H_q, D_qk, int(D_v), int(K), float(scale)
    st.q = _ptr(q_a, ctypes.c_uint16)
    if k_scale_cache is not None:  # FP8 KV cache: E4M3 codes and tile scales, latent layout
        if v_cache is not None:
            raise ValueError("the FP8 KV cache takes the latent layout")
        st.k8 = _ptr(hold(k_cache, np.uint8), ctypes.c_uint8)
        st.k8_scale = _ptr(hold(k_scale_cache, np.float32), ctypes.c_float)
    else:
        st.k = _ptr(hold(k_cache, np.uint16), ctypes.c_uint16)
        st.v = _ptr(hold(v_cache, np.uint16), ctypes.c_uint16)

    rows = np.arange(num_rows) if rows is None else np.asarray(rows, np.int64)
    rows32 = _arr(rows, np.int32)
    n = len(rows32)
    indices = np.empty((n, int(K)), np.int32)
    counts = np.empty(n, np.int64)
    out = np.empty((n, H_q, int(D_v)), np.float64)
    lse = np.empty((n, H_q), np.float64)
    scores = None
    if keep_scores:
        if cand is not None:
            ld = int(np.asarray(cand).shape[1])
        else:
            ld = int(bt.shape[1]) * 64
        scores = np.empty((max(n, 1), max(ld, 1)), np.float32)
    rc = lib().orc_decode_step(ctypes.byref(st), _ptr(rows32, ctypes.c_int32), n,
                               _ptr(indices, ctypes.c_int32), _ptr(counts, ctypes.c_int64),
                               _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double),
                               _ptr(scores, ctypes.c_float), 0 if scores is None else scores.shape[1],
                               int(threads))
    if rc != 0:
        raise ValueError("a row's sequence, position or candidate list is out of range")
    score_list = None
    if keep_scores:
        score_list = []
        for i in range(n):
            length = _history_length(rows[i], sl, row_seq, row_pos, cand_len)
            score_list.append(scores[i, :length].copy())
    return {"scores": score_list, "indices": indices, "counts": counts, "out": out, "lse": lse,
            "rows": rows}


def _history_length(r, seq_lens, row_seq, row_pos, cand_len):
    if cand_len is not None:
        return int(np.asarray(cand_len)[r])
    b = int(r if row_seq is None else np.asarray(row_seq)[r])
    p = int(seq_lens[b] - 1 if row_pos is None else np.asarray(row_pos)[r])
    return p + 1
