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
  * "Who packs the sequences: the loader, or the trainer?" (Trainer packs /
    Loader packs) -> :func:`pack`.
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
