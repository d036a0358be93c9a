"""CPU oracle for packed-sequence (THD) varlen-attention metadata.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``varlen_attention_metadata_amd``) never imports it, and it imports nothing
from the product path: the two share no code.

The arithmetic lives in ``psq_oracle.c`` (plain C, one loop per step of the
pages' definitions, built with gcc).  This module only marshals numpy arrays
into it and returns plain numpy results.

Pages followed:
  * NeMo AutoModel API reference, ``nemo_automodel.components.datasets.packed_seq``
    (``packed_seq_params_from_doc_ids``) -> :func:`doc_segments`.
  * NeMo AutoModel 0.5 API reference, ``nemo_automodel.components.distributed.thd_utils``
    (``process_input_for_thd``, ``_thd_padding_mask``) -> :func:`thd_tables`,
    :func:`copy_rows`.
    ``split_batch_into_thd_chunks`` -> :func:`split_thd`;
    ``thd_padding_mask_from_token_ids`` -> :func:`pad_mask_from_ids`.
  * "Who packs the sequences: the loader, or the trainer?" (Trainer packs /
    Loader packs) -> :func:`pack`, :func:`pack_rect`, :func:`trainer_width`.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "psq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BAD_LENGTH = 1
TABLE_MISMATCH = 2
ROW_OVERFLOW = 4
EMPTY_ROW = 8
PACK_OVERFLOW = 16
EMPTY_PACK = 32
BAD_INDEX = 64
PAD_IS_CONTENT = 256

_lib = None


def build() -> str:
    """Compile the oracle with gcc (plain -O2, single thread)."""
    subprocess.run(
        ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared",
         "-o", _LIB, _SRC],
        check=True)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.orc_doc_segments.restype = i64
    lib.orc_doc_segments.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.orc_thd_tables.restype = ctypes.c_uint32
    lib.orc_thd_tables.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp]
    lib.orc_copy_rows.restype = None
    lib.orc_copy_rows.argtypes = [vp, vp, i64, i64, i64]
    lib.orc_pack.restype = ctypes.c_uint32
    lib.orc_pack.argtypes = [vp, i64, vp, vp, i64, i32, vp, vp, i64, i32,
                             ctypes.c_int, i64, vp, vp, vp, vp]
    lib.orc_pack_rect.restype = ctypes.c_uint32
    lib.orc_pack_rect.argtypes = [vp, i64, vp, i64, i32, vp, vp, i64, i32,
                                  ctypes.c_int, i64, vp, vp, vp, vp]
    lib.orc_pad_mask_from_ids.restype = ctypes.c_uint32
    lib.orc_pad_mask_from_ids.argtypes = [vp, i64, i64, vp, vp]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def doc_segments(doc_ids, want_mask: bool = True) -> dict:
    """``packed_seq_params_from_doc_ids`` on a ``[B, S]`` integer map.

    Returns ``cu_seqlens`` (int32, exact length), ``num_segments``,
    ``max_seqlen`` and (optionally) ``padding_mask`` (uint8 0/1, ``[B*S]``).
    """
    d = np.ascontiguousarray(np.asarray(doc_ids), dtype=np.int64)
    assert d.ndim == 2
    B, S = d.shape
    T = B * S
    if T >= 2 ** 31:
        raise OverflowError("B*S does not fit int32 cu_seqlens")
    cu = np.empty(T + 1, dtype=np.int32)
    mx = np.zeros(1, dtype=np.int32)
    mask = np.empty(T, dtype=np.uint8) if want_mask else None
    nseg = _load().orc_doc_segments(_ptr(d), B, S, _ptr(cu), _ptr(mx), _ptr(mask))
    out = {"cu_seqlens": cu[: nseg + 1].copy(), "num_segments": int(nseg),
           "max_seqlen": int(mx[0])}
    if want_mask:
        out["padding_mask"] = mask
    return out


def thd_tables(seq_lens, seq_lens_padded, S: int, pad_value: int = -1000) -> dict:
    """``process_input_for_thd`` metadata from ``[B, P]`` length tables.

    Returns ``status`` (0 = ok); on success also ``cu_seqlens``,
    ``cu_seqlens_padded`` (int32, exact length), ``num_seqs``, ``max_seqlen``,
    ``pad_between_seqs`` and ``padding_mask`` (uint8 0/1, ``[B*S]``).
    """
    L = np.ascontiguousarray(np.asarray(seq_lens), dtype=np.int64)
    assert L.ndim == 2
    B, P = L.shape
    Lp = None
    if seq_lens_padded is not None:
        Lp = np.ascontiguousarray(np.asarray(seq_lens_padded), dtype=np.int64)
        assert Lp.shape == L.shape
    T = B * S
    if T >= 2 ** 31 or B * P + 1 >= 2 ** 31:
        raise OverflowError("sizes do not fit int32 boundaries")
    cu = np.zeros(B * P + 1, dtype=np.int32)
    cp = np.zeros(B * P + 1, dtype=np.int32)
    n = np.zeros(1, dtype=np.int64)
    mx = np.zeros(1, dtype=np.int32)
    pb = np.zeros(1, dtype=np.int32)
    mask = np.empty(T, dtype=np.uint8)
    st = _load().orc_thd_tables(_ptr(L), _ptr(Lp), B, P, S, pad_value, _ptr(cu),
                                _ptr(cp), _ptr(n), _ptr(mx), _ptr(pb), _ptr(mask))
    if st != 0:
        return {"status": int(st)}
    k = int(n[0])
    return {"status": 0, "cu_seqlens": cu[: k + 1].copy(),
            "cu_seqlens_padded": cp[: k + 1].copy(), "num_seqs": k,
            "max_seqlen": int(mx[0]), "pad_between_seqs": int(pb[0]),
            "padding_mask": mask}


def copy_rows(src, rows: int, row_bytes: int, src_row_stride_bytes: int) -> np.ndarray:
    """The THD collapse of one tensor: a byte copy of ``rows`` rows."""
    s = np.ascontiguousarray(np.asarray(src)).view(np.uint8).reshape(-1)
    if rows > 0:
        assert s.size >= (rows - 1) * src_row_stride_bytes + row_bytes
    dst = np.empty(rows * row_bytes, dtype=np.uint8)
    _load().orc_copy_rows(_ptr(s), _ptr(dst), rows, row_bytes, src_row_stride_bytes)
    return dst


def pack(src, src_off, real_len, q: int, pack_start, capacity: int, fold: bool = True,
         pad_token: int = 0, order=None) -> dict:
    """The squeeze of padded sources into ``P`` packs of ``capacity`` slots.

    Returns ``status``; on success also ``packed`` (int64 ``[P, C]``),
    ``token_mask`` (uint8 ``[P, C]``) and ``cu_seqlens`` / ``cu_seqlens_padded``
    as the flat per-pack CSR (pack ``p`` at ``pack_start[p] + p``).
    """
    src = np.ascontiguousarray(np.asarray(src), dtype=np.int64)
    so = np.ascontiguousarray(np.asarray(src_off), dtype=np.int64)
    rl = np.ascontiguousarray(np.asarray(real_len), dtype=np.int32)
    ps = np.ascontiguousarray(np.asarray(pack_start), dtype=np.int64)
    od = None if order is None else np.ascontiguousarray(np.asarray(order), dtype=np.int32)
    N = rl.size
    P = ps.size - 1
    assert so.size == N and P >= 0
    csr = (N if od is None else od.size) + P
    packed = np.empty((P, capacity), dtype=np.int64)
    tm = np.empty((P, capacity), dtype=np.uint8)
    cu = np.zeros(max(csr, 1), dtype=np.int32)
    cp = np.zeros(max(csr, 1), dtype=np.int32)
    st = _load().orc_pack(_ptr(src), src.size, _ptr(so), _ptr(rl), N, q, _ptr(od),
                          _ptr(ps), P, capacity, int(bool(fold)), pad_token,
                          _ptr(packed), _ptr(tm), _ptr(cu), _ptr(cp))
    if st != 0:
        return {"status": int(st)}
    used = int(ps[-1]) + P if P > 0 else 0
    return {"status": 0, "packed": packed, "token_mask": tm,
            "cu_seqlens": cu[:used], "cu_seqlens_padded": cp[:used]}


def pack_csr_slices(cu_csr, pack_start):
    """Split a per-pack CSR boundary array into one array per pack."""
    ps = np.asarray(pack_start, dtype=np.int64)
    out = []
    for p in range(ps.size - 1):
        a, b = int(ps[p]), int(ps[p + 1])
        out.append(np.asarray(cu_csr)[a + p: b + p + 1])
    return out


def split_thd(seq_lens, seq_lens_padded, S: int, num_chunks: int,
              pad_value: int = -1000) -> dict:
    """``split_batch_into_thd_chunks`` on ``[B, P]`` length tables.

    The batch is cut along rows into ``num_chunks`` equal groups, each group
    goes through :func:`thd_tables` on its own, and the results are stacked:
    ``cu_seqlens`` / ``cu_seqlens_padded`` become ``[num_chunks, L]`` with
    every row filled up to ``L`` (the longest) with ``pad_value``;
    ``max_seqlen``, ``num_seqs`` and ``pad_between_seqs`` become
    ``[num_chunks]``; ``padding_mask`` becomes ``[num_chunks, B/num_chunks*S]``.
    Returns ``status`` (OR over chunks) and, on success, those arrays.
    """
    L = np.asarray(seq_lens)
    Lp = None if seq_lens_padded is None else np.asarray(seq_lens_padded)
    B = L.shape[0]
    if num_chunks < 1 or B % num_chunks != 0:
        raise ValueError("num_chunks must evenly divide the batch size")
    rows = B // num_chunks
    parts = []
    status = 0
    for c in range(num_chunks):
        part = thd_tables(L[c * rows:(c + 1) * rows],
                          None if Lp is None else Lp[c * rows:(c + 1) * rows],
                          S, pad_value)
        status |= part["status"]
        parts.append(part)
    if status != 0:
        return {"status": status}
    width = max(p["cu_seqlens"].size for p in parts)

    def stacked(key):
        out = np.full((num_chunks, width), pad_value, dtype=np.int32)
        for c, p in enumerate(parts):
            out[c, :p[key].size] = p[key]
        return out

    return {"status": 0,
            "cu_seqlens": stacked("cu_seqlens"),
            "cu_seqlens_padded": stacked("cu_seqlens_padded"),
            "num_seqs": np.array([p["num_seqs"] for p in parts], dtype=np.int32),
            "max_seqlen": np.array([p["max_seqlen"] for p in parts], dtype=np.int32),
            "pad_between_seqs": np.array([p["pad_between_seqs"] for p in parts],
                                         dtype=np.int32),
            "padding_mask": np.stack([p["padding_mask"] for p in parts])}


def pad_mask_from_ids(input_ids, pad_id: int) -> dict:
    """``thd_padding_mask_from_token_ids`` on a flat ``[T]`` id stream.

    Returns ``status`` (``PAD_IS_CONTENT`` when the pad id occurs before the
    pad tail), ``padding_mask`` (uint8 0/1) and ``num_content`` (index of the
    first pad slot, ``T`` when there is none).
    """
    ids = np.ascontiguousarray(np.asarray(input_ids), dtype=np.int64).reshape(-1)
    mask = np.empty(ids.size, dtype=np.uint8)
    nc = np.zeros(1, dtype=np.int64)
    st = _load().orc_pad_mask_from_ids(_ptr(ids), ids.size, pad_id, _ptr(mask), _ptr(nc))
    return {"status": int(st), "padding_mask": mask, "num_content": int(nc[0])}


def bins_to_csr(bins):
    """Bin membership lists -> (pack_order int32 [sum], pack_start int64 [P+1])."""
    order = np.array([i for b in bins for i in b], dtype=np.int32)
    start = np.zeros(len(bins) + 1, dtype=np.int64)
    start[1:] = np.cumsum([len(b) for b in bins])
    return order, start


def trainer_width(real_len, bins, q: int) -> int:
    """Trainer packs: the row width is the largest padded fill over the bins."""
    rl = np.asarray(real_len, dtype=np.int64)
    widths = [sum(-(-int(rl[i]) // q) * q for i in b) for b in bins]
    return max(widths) if widths else 0


def pack_rect(rows, real_len, q: int, bins, width: int | None = None,
              fold: bool = False, pad_token: int = 0) -> dict:
    """Trainer packs: squeeze the padded rectangle ``rows [N, W]`` into bins.

    ``bins`` lists the member row indices of each bin (chosen on the host).
    ``width`` defaults to :func:`trainer_width`.  Returns the same keys as
    :func:`pack` plus ``width``.
    """
    r = np.ascontiguousarray(np.asarray(rows), dtype=np.int64)
    assert r.ndim == 2
    N, W = r.shape
    rl = np.ascontiguousarray(np.asarray(real_len), dtype=np.int32)
    assert rl.size == N
    order, start = bins_to_csr(bins)
    C = trainer_width(rl, bins, q) if width is None else int(width)
    P = len(bins)
    csr = order.size + P
    packed = np.empty((P, C), dtype=np.int64)
    tm = np.empty((P, C), dtype=np.uint8)
    cu = np.zeros(max(csr, 1), dtype=np.int32)
    cp = np.zeros(max(csr, 1), dtype=np.int32)
    st = _load().orc_pack_rect(_ptr(r), W, _ptr(rl), N, q, _ptr(order), _ptr(start), P,
                               C, int(bool(fold)), pad_token, _ptr(packed), _ptr(tm),
                               _ptr(cu), _ptr(cp))
    if st != 0:
        return {"status": int(st)}
    return {"status": 0, "packed": packed, "token_mask": tm, "width": C,
            "cu_seqlens": cu[:csr], "cu_seqlens_padded": cp[:csr],
            "pack_order": order, "pack_start": start}
