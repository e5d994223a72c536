"""Seeded generation of one batch of inputs, on any torch device.

Two generators per batch: a CPU one for the structure (sequence lengths,
block-table permutation), so every device sees the same structure for a seed,
and one on the target device for the bulk values.  Large tensors are filled
chunk by chunk to bound temporary memory.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

from .configs import Workload

BLOCK = 64
_CHUNK = 1 << 26          # elements per generation chunk


@dataclass
class Batch:
    wl: Workload
    lengths: list            # host copy of seq_lens
    row_seq_host: list       # host copy of each row's sequence
    row_pos_host: list       # host copy of each row's position
    max_blocks: int
    num_blocks: int
    seq_lens: torch.Tensor   # int32 [B]
    block_table: torch.Tensor  # int32 [B, max_blocks], -1 past each sequence's blocks
    row_seq: Optional[torch.Tensor]  # int32 [rows] or None (decode)
    row_pos: Optional[torch.Tensor]
    qI: torch.Tensor         # uint8 E4M3 [rows, H_I, D_I]
    w: torch.Tensor          # float32 [rows, H_I]
    kI: torch.Tensor         # uint8 E4M3 [num_blocks, 64, D_I] (MXFP8: [num_blocks, 66,
                             # D_I], the 64 rows' D_I/32 E8M0 scales each, in row order,
                             # in the last two D_I-byte rows of the block)
    q: torch.Tensor          # bfloat16 [rows, H_q, D_qk]
    kv: torch.Tensor         # bfloat16 [num_blocks, 64, D_qk] (FP8 KV: uint8 [num_blocks,
                             # 64 + KV_SCALE_ROWS, D_qk], E4M3 code rows, then the 64 rows'
                             # float32 tile scales, row after row, from row 64 on)
    v: Optional[torch.Tensor] = None   # bfloat16 [num_blocks, 64, D_v] (separate V)
    qI_scale: Optional[torch.Tensor] = None  # MXFP8: uint8 E8M0 [rows, H_I, D_I/32]
    cand: Optional[torch.Tensor] = None      # int32 [rows, n_cand]: candidate positions, -1 past
    cand_len: Optional[torch.Tensor] = None  # int32 [rows]: valid candidates of each row
    extra: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.qI.shape[0]


def _fill(out: torch.Tensor, draw):
    flat = out.view(-1)
    n = flat.numel()
    for i in range(0, n, _CHUNK):
        j = min(n, i + _CHUNK)
        flat[i:j] = draw(j - i)
    return out


def _fp8_codes(shape, mode, gen, device):
    out = torch.empty(shape, dtype=torch.uint8, device=device)
    if mode == "int":
        def draw(n):
            x = torch.randint(-8, 9, (n,), generator=gen, device=device, dtype=torch.int32)
            return x.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
    else:
        def draw(n):
            x = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
            return x.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return _fill(out, draw)


MX_GROUP = 32


def _mx_codes_scales(shape, mode, gen, device):
    """MXFP8 operands of the given shape (last dim a multiple of 32): E4M3
    codes and one E8M0 scale byte per group of 32.  Integer mode: codes are
    integers in [-4, 4] and scales 2**-1, 1 or 2**1 (every score stays exact
    in float32).  Gaussian mode: N(0, 1) values quantised the OCP way, shared
    exponent floor(log2(max |x|)) - 8 per group, codes saturated to +-448."""
    *lead, D = shape
    codes = torch.empty(shape, dtype=torch.uint8, device=device)
    scales = torch.empty((*lead, D // MX_GROUP), dtype=torch.uint8, device=device)
    flat_c = codes.view(-1, D)
    flat_s = scales.view(-1, D // MX_GROUP)
    rows = flat_c.shape[0]
    step = max(1, _CHUNK // D)
    for i in range(0, rows, step):
        j = min(rows, i + step)
        n = j - i
        if mode == "int":
            x = torch.randint(-4, 5, (n, D), generator=gen, device=device, dtype=torch.int32)
            flat_c[i:j] = x.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
            flat_s[i:j] = torch.randint(126, 129, (n, D // MX_GROUP), generator=gen,
                                        device=device, dtype=torch.int32).to(torch.uint8)
        else:
            x = torch.randn(n, D // MX_GROUP, MX_GROUP, generator=gen, device=device,
                            dtype=torch.float32)
            amax = x.abs().amax(dim=2, keepdim=True).clamp_min(2.0 ** -100)
            e = torch.floor(torch.log2(amax)) - 8.0
            y = (x * torch.exp2(-e)).clamp_(-448.0, 448.0)
            flat_c[i:j] = y.to(torch.float8_e4m3fn).view(torch.uint8).view(n, D)
            flat_s[i:j] = (e.view(n, -1) + 127.0).to(torch.int32).to(torch.uint8)
    return codes, scales


KV_TILE = 128


def kv_scale_rows(D):
    """Rows of D bytes after a block's 64 FP8 KV code rows that hold the 64
    rows' float32 tile scales (4 * ceil(D / 128) bytes per row)."""
    tiles = (D + KV_TILE - 1) // KV_TILE
    return (BLOCK * 4 * tiles + D - 1) // D


def _kv_fp8_pages(num_blocks, D, gen, device):
    """FP8 KV pages of N(0, 1) rows: every tile of 128 elements (the last one
    shorter when 128 does not divide D) is scaled by amax / 448 and rounded
    to E4M3; the float32 scales follow the block's code rows."""
    tiles = (D + KV_TILE - 1) // KV_TILE
    srows = kv_scale_rows(D)
    pages = torch.zeros((num_blocks, BLOCK + srows, D), dtype=torch.uint8, device=device)
    step = max(1, _CHUNK // (BLOCK * D))
    for i in range(0, num_blocks, step):
        j = min(num_blocks, i + step)
        n = j - i
        x = torch.randn(n, BLOCK, D, generator=gen, device=device, dtype=torch.float32)
        pad = torch.zeros(n, BLOCK, tiles * KV_TILE, device=device, dtype=torch.float32)
        pad[..., :D] = x
        t = pad.view(n, BLOCK, tiles, KV_TILE)
        scale = (t.abs().amax(dim=3) / 448.0).clamp_min(2.0 ** -100)      # [n, 64, tiles]
        codes = (t / scale[..., None]).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
        pages[i:j, :BLOCK] = codes.view(torch.uint8).view(n, BLOCK, tiles * KV_TILE)[..., :D]
        sb = scale.contiguous().view(torch.uint8).view(n, BLOCK * 4 * tiles)
        pages[i:j, BLOCK:].view(n, srows * D)[:, :BLOCK * 4 * tiles] = sb
    return pages


def kv_fp8_split(pages, D):
    """(codes uint8 [..., 64, D], scales float32 [..., 64, ceil(D / 128)]) of
    FP8 KV pages laid out by ``_kv_fp8_pages`` (any leading dims)."""
    tiles = (D + KV_TILE - 1) // KV_TILE
    lead = pages.shape[:-2]
    codes = pages[..., :BLOCK, :]
    tail = pages[..., BLOCK:, :].reshape(*lead, -1)[..., :BLOCK * 4 * tiles]
    if isinstance(tail, torch.Tensor):
        scales = tail.contiguous().view(torch.float32).view(*lead, BLOCK, tiles)
    else:
        scales = np.ascontiguousarray(tail).view(np.float32).reshape(*lead, BLOCK, tiles)
    return codes, scales


def _bf16_normal(shape, gen, device):
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    return _fill(out, lambda n: torch.randn(n, generator=gen, device=device,
                                            dtype=torch.float32).to(torch.bfloat16))


def _weights(shape, mode, gen, device):
    if mode == "int":
        return torch.randint(0, 4, shape, generator=gen, device=device,
                             dtype=torch.int32).to(torch.float32)
    return torch.rand(shape, generator=gen, device=device, dtype=torch.float32) * 3.0


def make_batch(wl: Workload, device="cpu", seed=None, mode=None, table=None,
               lengths=None) -> Batch:
    """Draw one batch for workload ``wl``.

    ``seed``, ``mode`` ("int"/"gauss") and ``table`` ("identity"/"shuffled")
    override the workload's own.  Integer mode: indexer q and k are integers
    in [-8, 8] (exact in E4M3) and head weights integers in [0, 3].  Gaussian
    mode: q and k are N(0, 1) rounded to E4M3, weights uniform on [0, 3).
    Attention q and the KV rows are N(0, 1) rounded to bf16 in both modes.
    """
    seed = wl.seed if seed is None else seed
    mode = wl.mode if mode is None else mode
    table = wl.table if table is None else table
    device = torch.device(device)
    gs = torch.Generator(device="cpu")
    gs.manual_seed(seed)
    gd = torch.Generator(device=device)
    gd.manual_seed(seed * 7919 + 17)

    if lengths is not None:
        lens = [int(x) for x in lengths]
    elif wl.lengths:
        lens = list(wl.lengths)
    elif wl.context:
        lens = [wl.context] * wl.batch
    else:
        lo, hi = wl.ragged
        lens = torch.randint(lo, hi + 1, (wl.batch,), generator=gs).tolist()
    B = len(lens)
    nblk = [(L + BLOCK - 1) // BLOCK for L in lens]
    max_blocks = max(nblk)
    num_blocks = sum(nblk)
    if table == "shuffled":
        phys = torch.randperm(num_blocks, generator=gs)
    else:
        phys = torch.arange(num_blocks)
    bt = torch.full((B, max_blocks), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        bt[b, :nblk[b]] = phys[off:off + nblk[b]].to(torch.int32)
        off += nblk[b]

    if wl.prefill_rows:
        # one chunk of new tokens at the end of sequence 0
        R = wl.prefill_rows
        first = lens[0] - R
        row_seq_h = [0] * R
        row_pos_h = list(range(first, lens[0]))
        row_seq = torch.tensor(row_seq_h, dtype=torch.int32, device=device)
        row_pos = torch.tensor(row_pos_h, dtype=torch.int32, device=device)
    else:
        R = B
        row_seq_h = list(range(B))
        row_pos_h = [L - 1 for L in lens]
        row_seq = row_pos = None

    qI_scale = None
    if wl.indexer_fmt == "mxfp8":
        qI, qI_scale = _mx_codes_scales((R, wl.H_I, wl.D_I), mode, gd, device)
        w = _weights((R, wl.H_I), mode, gd, device)
        k_codes, k_scales = _mx_codes_scales((num_blocks, BLOCK, wl.D_I), mode, gd, device)
        kI = torch.empty((num_blocks, BLOCK + 2, wl.D_I), dtype=torch.uint8, device=device)
        kI[:, :BLOCK] = k_codes
        kI[:, BLOCK:] = k_scales.reshape(num_blocks, 2, wl.D_I)
        del k_codes, k_scales
    else:
        qI = _fp8_codes((R, wl.H_I, wl.D_I), mode, gd, device)
        w = _weights((R, wl.H_I), mode, gd, device)
        kI = _fp8_codes((num_blocks, BLOCK, wl.D_I), mode, gd, device)
    q = _bf16_normal((R, wl.H_q, wl.D_qk), gd, device)
    if wl.kv_fmt == "fp8":
        if not wl.latent:
            raise ValueError("the FP8 KV cache takes the latent layout")
        kv = _kv_fp8_pages(num_blocks, wl.D_qk, gd, device)
    else:
        kv = _bf16_normal((num_blocks, BLOCK, wl.D_qk), gd, device)
    v = None if wl.latent else _bf16_normal((num_blocks, BLOCK, wl.D_v), gd, device)

    cand = cand_len = None
    if wl.n_cand:
        # each row's candidates: a uniform subset of its history, ascending
        C = wl.n_cand
        ch = torch.full((R, C), -1, dtype=torch.int32)
        cl = torch.zeros(R, dtype=torch.int32)
        for i, p in enumerate(row_pos_h):
            n = min(C, p + 1)
            pick = torch.randperm(p + 1, generator=gs)[:n] if n < p + 1 else torch.arange(p + 1)
            ch[i, :n] = torch.sort(pick).values.to(torch.int32)
            cl[i] = n
        cand, cand_len = ch.to(device), cl.to(device)

    return Batch(wl=wl, lengths=lens, row_seq_host=row_seq_h, row_pos_host=row_pos_h,
                 max_blocks=max_blocks, num_blocks=num_blocks,
                 seq_lens=torch.tensor(lens, dtype=torch.int32, device=device),
                 block_table=bt.to(device), row_seq=row_seq, row_pos=row_pos,
                 qI=qI, w=w, kI=kI, q=q, kv=kv, v=v, qI_scale=qI_scale,
                 cand=cand, cand_len=cand_len)


def row_positions(batch: Batch):
    """(sequence, position) of every row, as recorded when the batch was drawn."""
    return list(zip(batch.row_seq_host, batch.row_pos_host))


def _np(t):
    return t.detach().cpu().numpy()


def _kv_host(kv):
    if kv.dtype == torch.uint8:  # FP8 KV pages
        return _np(kv)
    return _np(kv.view(torch.int16)).view(np.uint16)


def oracle_arrays(batch: Batch, rows=None) -> dict:
    """The batch as plain numpy arrays of raw storage bits.

    The per-row arrays hold the chosen ``rows`` (default: all) in order, with
    their sequences and positions in ``row_seq`` / ``row_pos`` and their ids
    in the batch in ``row_ids``.  With ``rows`` given, only the cache blocks
    those rows' sequences own are copied to the host and the block table is
    renumbered to the copied blocks (whole blocks move; no value is touched).
    """
    wl = batch.wl
    if rows is None:
        rows = np.arange(batch.rows)
        bt = _np(batch.block_table)
        kI, kv = _np(batch.kI), _kv_host(batch.kv)
        v = None if batch.v is None else _np(batch.v.view(torch.int16)).view(np.uint16)
        seqs = None
    else:
        rows = np.asarray(rows, dtype=np.int64)
        seqs = sorted({batch.row_seq_host[r] for r in rows})
        bt_full = batch.block_table.cpu()
        ids = []
        for b in seqs:
            nb = (batch.lengths[b] + BLOCK - 1) // BLOCK
            ids.append(bt_full[b, :nb].to(torch.int64))
        ids_t = torch.cat(ids)
        idx_dev = ids_t.to(batch.kI.device)
        kI = _np(batch.kI.index_select(0, idx_dev))
        kv = _kv_host(batch.kv.index_select(0, idx_dev))
        v = None if batch.v is None else \
            _np(batch.v.index_select(0, idx_dev).view(torch.int16)).view(np.uint16)
        bt = np.full(_np(bt_full).shape, -1, dtype=np.int32)
        off = 0
        for b in seqs:
            nb = (batch.lengths[b] + BLOCK - 1) // BLOCK
            bt[b, :nb] = np.arange(off, off + nb, dtype=np.int32)
            off += nb
    sel = torch.as_tensor(rows, dtype=torch.int64).to(batch.qI.device)
    k_scale = None
    if wl.kv_fmt == "fp8":  # FP8 KV: E4M3 code rows and their float32 tile scales
        kv, k_scale = kv_fp8_split(kv, wl.D_qk)
        kv = np.ascontiguousarray(kv)
    kI_scale = None
    if batch.qI_scale is not None:  # MXFP8: split each block into code rows and row scales
        kI_scale = np.ascontiguousarray(kI[:, BLOCK:]).reshape(kI.shape[0], BLOCK, -1)
        kI = kI[:, :BLOCK]
    return {
        "qI_scale": None if batch.qI_scale is None else _np(batch.qI_scale.index_select(0, sel)),
        "kI_scale_cache": kI_scale,
        "cand": None if batch.cand is None else _np(batch.cand.index_select(0, sel)),
        "cand_len": None if batch.cand is None else _np(batch.cand_len.index_select(0, sel)),
        "qI": _np(batch.qI.index_select(0, sel)),
        "w": _np(batch.w.index_select(0, sel)),
        "q": _np(batch.q.index_select(0, sel).view(torch.int16)).view(np.uint16),
        "kI_cache": kI, "k_cache": kv, "v_cache": v, "k_scale_cache": k_scale,
        "block_table": bt, "seq_lens": np.asarray(batch.lengths, np.int32),
        "row_seq": np.asarray(batch.row_seq_host, np.int64)[rows],
        "row_pos": np.asarray(batch.row_pos_host, np.int64)[rows],
        "row_ids": np.asarray(rows, np.int64),
        "K": wl.K, "scale": wl.scale, "D_v": wl.D_v,
    }
