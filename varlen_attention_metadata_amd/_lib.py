"""ctypes binding of ``libpsq.so`` (the C ABI of ``include/psq.h``).

Functions here carry the C names and take plain integers (device addresses,
sizes, a stream handle); they only marshal arguments.  Every step of the
computation runs in the HIP kernels behind them.  Loading fails loudly when
the library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpsq.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "psq.h")

# constants of include/psq.h
I32, I64 = 0, 1
OK, ERR_ARG, ERR_OVERFLOW, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
DATA_BAD_LENGTH = 1
DATA_TABLE_MISMATCH = 2
DATA_ROW_OVERFLOW = 4
DATA_EMPTY_ROW = 8
DATA_PACK_OVERFLOW = 16
DATA_EMPTY_PACK = 32
DATA_BAD_INDEX = 64
DATA_WORKSPACE = 128
DATA_PAD_IS_CONTENT = 256
LAYOUT_SEQ_LENS, LAYOUT_DOC_IDS = 0, 1
MAX_COPIES = 8


class PsqCopy(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("dst", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("row_bytes", ctypes.c_int64),
                ("src_row_stride_bytes", ctypes.c_int64),
                ("dst_row_stride_bytes", ctypes.c_int64)]


class PsqThdLayout(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("seq_lens", ctypes.c_void_p),
                ("seq_lens_padded", ctypes.c_void_p), ("lens_dtype", ctypes.c_int),
                ("P", ctypes.c_int64), ("pad_value", ctypes.c_int64),
                ("doc_ids", ctypes.c_void_p), ("doc_dtype", ctypes.c_int)]


class PsqError(RuntimeError):
    """A host-side PSQ_ERR_* return code."""

    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {status_string(code, False)} (code {code})")
        self.code = code


_lib = None


def header_functions() -> list:
    """Names of the functions ``include/psq.h`` declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(psq_\w+)\s*\(", text)))


def load():
    """Load ``libpsq.so``; raises if it is missing (build it first)."""
    global _lib
    if _lib is None:
        _lib = open_library(LIB_PATH)
    return _lib


def open_library(path: str):
    """A ctypes handle on a build of the library at ``path`` (``libpsq.so``,
    or the race-test build ``libpsq_jitter.so``) with every prototype set."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    ci = ctypes.c_int
    lib.psq_status_string.restype = ctypes.c_char_p
    lib.psq_status_string.argtypes = [ci, ci]
    lib.psq_workspace_init.restype = ci
    lib.psq_workspace_init.argtypes = [vp, sz, vp]
    lib.psq_params_from_doc_ids_workspace.restype = sz
    lib.psq_params_from_doc_ids_workspace.argtypes = [i64, i64]
    lib.psq_params_from_doc_ids.restype = ci
    lib.psq_params_from_doc_ids.argtypes = [vp, ci, i64, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.psq_params_from_doc_ids_noalloc.restype = ci
    lib.psq_params_from_doc_ids_noalloc.argtypes = [vp, ci, i64, i64, vp, vp, vp, vp, vp, vp]
    lib.psq_process_thd_workspace.restype = sz
    lib.psq_process_thd_workspace.argtypes = [ctypes.POINTER(PsqThdLayout), i64, i64]
    lib.psq_process_thd.restype = ci
    lib.psq_process_thd.argtypes = [ctypes.POINTER(PsqThdLayout), i64, i64, vp, vp, vp, vp,
                                    vp, vp, ctypes.POINTER(PsqCopy), ci, vp, vp, sz, vp]
    lib.psq_split_thd_workspace.restype = sz
    lib.psq_split_thd_workspace.argtypes = [ctypes.POINTER(PsqThdLayout), i64, i64, i64]
    lib.psq_split_thd.restype = ci
    lib.psq_split_thd.argtypes = [ctypes.POINTER(PsqThdLayout), i64, i64, i64, vp, vp, vp, vp,
                                  vp, vp, vp, ctypes.POINTER(PsqCopy), ci, vp, vp, sz, vp]
    lib.psq_padding_mask_from_token_ids_workspace.restype = sz
    lib.psq_padding_mask_from_token_ids_workspace.argtypes = [i64]
    lib.psq_padding_mask_from_token_ids.restype = ci
    lib.psq_padding_mask_from_token_ids.argtypes = [vp, ci, i64, i64, vp, vp, vp, vp, sz, vp]
    lib.psq_pack_padded_rows.restype = ci
    lib.psq_pack_padded_rows.argtypes = [vp, i64, vp, i64, i32, vp, vp, i64, i32, ci, i64,
                                         vp, vp, vp, vp, vp, vp, sz, vp]
    lib.psq_pack_rows_workspace.restype = sz
    lib.psq_pack_rows_workspace.argtypes = [i64, i64, i32]
    lib.psq_pack_rows.restype = ci
    lib.psq_pack_rows.argtypes = [vp, i64, vp, vp, i64, i32, vp, vp, i64, i32, ci, i64,
                                  vp, vp, vp, vp, vp, vp, sz, vp]
    return lib


def status_string(code: int, is_status: bool) -> str:
    return load().psq_status_string(int(code), int(bool(is_status))).decode()


def _check(rc: int, what: str) -> int:
    if rc != OK:
        raise PsqError(rc, what)
    return rc


def psq_workspace_init(workspace: int, nbytes: int, stream: int) -> int:
    return _check(load().psq_workspace_init(workspace, nbytes, stream), "psq_workspace_init")


def psq_params_from_doc_ids_workspace(B: int, S: int) -> int:
    return load().psq_params_from_doc_ids_workspace(B, S)


def psq_params_from_doc_ids(doc_ids, doc_dtype, B, S, cu_seqlens, num_segments, max_seqlen,
                            padding_mask, status, workspace, workspace_bytes, stream,
                            check=True) -> int:
    rc = load().psq_params_from_doc_ids(doc_ids, doc_dtype, B, S, cu_seqlens, num_segments,
                                        max_seqlen, padding_mask, status, workspace,
                                        workspace_bytes, stream)
    return _check(rc, "psq_params_from_doc_ids") if check else rc


def psq_params_from_doc_ids_noalloc(doc_ids, doc_dtype, B, S, cu_seqlens, num_segments,
                                    max_seqlen, padding_mask, status, stream,
                                    check=True) -> int:
    rc = load().psq_params_from_doc_ids_noalloc(doc_ids, doc_dtype, B, S, cu_seqlens,
                                                num_segments, max_seqlen, padding_mask, status,
                                                stream)
    return _check(rc, "psq_params_from_doc_ids_noalloc") if check else rc


def make_layout(kind, seq_lens=None, seq_lens_padded=None, lens_dtype=I64, P=0,
                pad_value=-1000, doc_ids=None, doc_dtype=I32) -> PsqThdLayout:
    return PsqThdLayout(kind, seq_lens, seq_lens_padded, lens_dtype, P, pad_value, doc_ids,
                        doc_dtype)


def make_copies(copies) -> tuple:
    """``copies``: list of (src, dst, rows, row_bytes, src_row_stride_bytes
    [, dst_row_stride_bytes]); a missing or 0 destination stride is dense."""
    arr = (PsqCopy * max(len(copies), 1))()
    for i, c in enumerate(copies):
        arr[i] = PsqCopy(*(tuple(c) + (0,) * (6 - len(c))))
    return arr, len(copies)


def psq_process_thd_workspace(layout: PsqThdLayout, B: int, S: int) -> int:
    return load().psq_process_thd_workspace(ctypes.byref(layout), B, S)


def psq_process_thd(layout, B, S, cu_seqlens, cu_seqlens_padded, num_seqs, max_seqlen,
                    pad_between_seqs, padding_mask, copies, n_copies, status, workspace,
                    workspace_bytes, stream, check=True) -> int:
    rc = load().psq_process_thd(ctypes.byref(layout), B, S, cu_seqlens, cu_seqlens_padded,
                                num_seqs, max_seqlen, pad_between_seqs, padding_mask, copies,
                                n_copies, status, workspace, workspace_bytes, stream)
    return _check(rc, "psq_process_thd") if check else rc


def psq_pack_rows_workspace(N: int, P: int, capacity: int) -> int:
    return load().psq_pack_rows_workspace(N, P, capacity)


def psq_pack_rows(src_tokens, src_len, src_offsets, real_len, N, pad_to, pack_order,
                  pack_start, P, capacity, fold, pad_token, packed, token_mask, cu_seqlens,
                  cu_seqlens_padded, status, workspace, workspace_bytes, stream,
                  check=True) -> int:
    rc = load().psq_pack_rows(src_tokens, src_len, src_offsets, real_len, N, pad_to,
                              pack_order, pack_start, P, capacity, fold, pad_token, packed,
                              token_mask, cu_seqlens, cu_seqlens_padded, status, workspace,
                              workspace_bytes, stream)
    return _check(rc, "psq_pack_rows") if check else rc


def psq_split_thd_workspace(layout: PsqThdLayout, B: int, S: int, num_chunks: int) -> int:
    return load().psq_split_thd_workspace(ctypes.byref(layout), B, S, num_chunks)


def psq_split_thd(layout, B, S, num_chunks, cu_seqlens, cu_seqlens_padded, cu_width, num_seqs,
                  max_seqlen, pad_between_seqs, padding_mask, copies, n_copies, status,
                  workspace, workspace_bytes, stream, check=True) -> int:
    rc = load().psq_split_thd(ctypes.byref(layout), B, S, num_chunks, cu_seqlens,
                              cu_seqlens_padded, cu_width, num_seqs, max_seqlen,
                              pad_between_seqs, padding_mask, copies, n_copies, status,
                              workspace, workspace_bytes, stream)
    return _check(rc, "psq_split_thd") if check else rc


def psq_padding_mask_from_token_ids_workspace(T: int) -> int:
    return load().psq_padding_mask_from_token_ids_workspace(T)


def psq_padding_mask_from_token_ids(input_ids, ids_dtype, T, pad_id, padding_mask, num_content,
                                    status, workspace, workspace_bytes, stream,
                                    check=True) -> int:
    rc = load().psq_padding_mask_from_token_ids(input_ids, ids_dtype, T, pad_id, padding_mask,
                                                num_content, status, workspace,
                                                workspace_bytes, stream)
    return _check(rc, "psq_padding_mask_from_token_ids") if check else rc


def psq_pack_padded_rows(rows, W, real_len, N, pad_to, pack_order, pack_start, P, capacity,
                         fold, pad_token, packed, token_mask, cu_seqlens, cu_seqlens_padded,
                         status, workspace, workspace_bytes, stream, check=True) -> int:
    rc = load().psq_pack_padded_rows(rows, W, real_len, N, pad_to, pack_order, pack_start, P,
                                     capacity, fold, pad_token, packed, token_mask, cu_seqlens,
                                     cu_seqlens_padded, status, workspace, workspace_bytes,
                                     stream)
    return _check(rc, "psq_pack_padded_rows") if check else rc
