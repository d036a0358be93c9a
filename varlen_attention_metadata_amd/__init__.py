"""Packed-sequence (THD) varlen-attention metadata on MI355X (gfx950).

Torch-facing API with the names of the pages it follows.  Tensors are only
containers here: every step runs in the HIP kernels of ``libpsq.so``,
reached through the C ABI (``include/psq.h``, bound in :mod:`._lib`).  The
functions synchronize once at the end, because they return exact-length
boundary arrays and Python scalars, as the pages' functions do; callers that
must not synchronize use the C ABI (or :mod:`._lib`) directly.

* :func:`packed_seq_params_from_doc_ids`, :class:`PackedSeqParams`,
  :func:`to_flash_attention_kwargs` -- NeMo AutoModel API,
  ``nemo_automodel.components.datasets.packed_seq``.
* :func:`process_input_for_thd`, :func:`split_batch_into_thd_chunks`,
  :func:`thd_padding_mask_from_token_ids` -- NeMo AutoModel 0.5 API,
  ``nemo_automodel.components.distributed.thd_utils`` (with
  ``_thd_padding_mask``).
* :func:`pack_rows` (Loader packs) and :func:`pack_padded_rows` (Trainer
  packs, from the padded rectangle) -- "Who packs the sequences: the loader,
  or the trainer?".
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib

__all__ = ["PackedSeqParams", "packed_seq_params_from_doc_ids", "to_flash_attention_kwargs",
           "process_input_for_thd", "split_batch_into_thd_chunks",
           "thd_padding_mask_from_token_ids", "pack_rows", "pack_padded_rows",
           "workspace_for"]

_DTYPES = {torch.int32: _lib.I32, torch.int64: _lib.I64}
_WORKSPACES: dict = {}


@dataclass
class PackedSeqParams:
    """Packed-sequence metadata of a neat-packing document map.

    ``cu_seqlens``: int32 ``[num_segments + 1]`` over the flattened
    ``[batch * sequence]`` axis, ending at ``batch * sequence``.
    ``max_seqlen``: length of the longest segment.  ``doc_ids``: the
    caller's map, unchanged.
    """
    cu_seqlens: torch.Tensor
    max_seqlen: int
    doc_ids: torch.Tensor


def _require_gpu(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the HIP kernels are the only path)")


def _int_dtype(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"{name} must be int32 or int64, got {t.dtype}")
    return _DTYPES[t.dtype]


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def workspace_for(device: torch.device, nbytes: int) -> torch.Tensor:
    """A zero-filled workspace of at least ``nbytes`` bytes for the current
    stream of ``device``.  Calls on one stream are ordered, so they share it;
    every call leaves it zero-filled again."""
    stream = _stream(device)
    key = (device.index, stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        _lib.psq_workspace_init(ws.data_ptr(), ws.numel(), stream)
        _WORKSPACES[key] = ws
    return ws


def _raise_status(code: int, what: str, device: torch.device) -> None:
    """Raise on a nonzero status word (read back, so the stream has drained).
    A call that reports DATA_WORKSPACE may leave records in the workspace,
    so the stream's cached one is dropped and the next call zero-fills a
    fresh one."""
    if code == 0:
        return
    if code & _lib.DATA_WORKSPACE:
        _WORKSPACES.pop((device.index, _stream(device)), None)
    raise ValueError(f"{what}: {_lib.status_string(code, True)} (status bits {code:#x})")


def packed_seq_params_from_doc_ids(doc_ids: torch.Tensor) -> PackedSeqParams:
    """Segment boundaries and the longest segment of a ``[B, S]`` document map.

    A segment ends wherever the document index changes and at the end of
    every row; a run of padding (index 0) counts as a segment like any other.
    """
    _require_gpu(doc_ids, "doc_ids")
    dt = _int_dtype(doc_ids, "doc_ids")
    if doc_ids.dim() != 2:
        raise ValueError(f"doc_ids must be [batch, sequence], got {tuple(doc_ids.shape)}")
    if not doc_ids.is_contiguous():
        raise ValueError("doc_ids must be contiguous (row-major)")
    B, S = doc_ids.shape
    dev = doc_ids.device
    cu = torch.empty(B * S + 1, dtype=torch.int32, device=dev)
    scal = torch.empty(4, dtype=torch.int32, device=dev)   # n, max, status, -
    ws = workspace_for(dev, _lib.psq_params_from_doc_ids_workspace(B, S))
    sp = scal.data_ptr()
    _lib.psq_params_from_doc_ids(doc_ids.data_ptr(), dt, B, S, cu.data_ptr(), sp, sp + 4, None,
                                 sp + 8, ws.data_ptr(), ws.numel(), _stream(dev))
    n, mx, st, _ = scal.cpu().tolist()
    _raise_status(st, "packed_seq_params_from_doc_ids", dev)
    return PackedSeqParams(cu_seqlens=cu[: n + 1], max_seqlen=int(mx), doc_ids=doc_ids)


def to_flash_attention_kwargs(params: PackedSeqParams) -> dict:
    """HuggingFace ``FlashAttentionKwargs`` of a packed batch (self-attention:
    the query and key entries are the same objects)."""
    return {"cu_seq_lens_q": params.cu_seqlens, "cu_seq_lens_k": params.cu_seqlens,
            "max_length_q": params.max_seqlen, "max_length_k": params.max_seqlen}


def _table_layout(batch: dict, B: int, seq_lens_padding_value: int):
    """(layout, P, has_padded) of a ``seq_lens`` / ``seq_lens_padded`` batch."""
    L = batch["seq_lens"]
    Lp = batch.get("seq_lens_padded")
    _require_gpu(L, "seq_lens")
    lt = _int_dtype(L, "seq_lens")
    if L.dim() != 2 or L.shape[0] != B or not L.is_contiguous():
        raise ValueError("seq_lens must be a contiguous [B, num_packs] tensor")
    P = int(L.shape[1])
    if Lp is not None:
        _require_gpu(Lp, "seq_lens_padded")
        if Lp.shape != L.shape or Lp.dtype != L.dtype or not Lp.is_contiguous():
            raise ValueError("seq_lens_padded must match seq_lens in shape and dtype")
    layout = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, L.data_ptr(),
                              Lp.data_ptr() if Lp is not None else None, lt, P,
                              seq_lens_padding_value)
    return layout, P, Lp is not None


def _copy_desc(src: torch.Tensor, dst: torch.Tensor, name: str) -> tuple:
    """(src, dst, rows, row_bytes, src_row_stride_bytes) of one collapse."""
    esz = src.element_size()
    if src.is_contiguous():
        nb = src.numel() * esz
        return (src.data_ptr(), dst.data_ptr(), 1, nb, nb)
    inner = src[0] if src.dim() > 1 else None
    if inner is not None and inner.is_contiguous():
        rows = src.shape[0]
        return (src.data_ptr(), dst.data_ptr(), rows, inner.numel() * esz, src.stride(0) * esz)
    raise ValueError(f"{name}: only row-strided layouts are supported, got strides {src.stride()}")


def process_input_for_thd(batch: dict, seq_lens_padding_value: int = -1000,
                          padding_token_id: int = 0) -> dict:
    """Convert a BSHD batch to THD: collapsed tensors plus varlen metadata.

    ``batch`` holds ``input_ids`` ``[B, S]`` (or ``[B, S, H]`` embeddings),
    ``labels`` ``[B, S]``, ``position_ids`` ``[B, S]`` (or mRoPE
    ``[n_rope, B, S]``), and the pack layout: ``seq_lens`` (with optional
    ``seq_lens_padded``) ``[B, num_packs]`` whose ``seq_lens_padding_value``
    entries are unused, or a document map ``doc_ids`` ``[B, S]``.
    ``padding_token_id`` is accepted for signature parity only: the padding
    mask comes from the layout, never from token values.
    """
    del padding_token_id
    input_ids = batch["input_ids"]
    position_ids = batch["position_ids"]
    labels = batch.get("labels")
    _require_gpu(input_ids, "input_ids")
    dev = input_ids.device
    if input_ids.dim() not in (2, 3):
        raise ValueError("input_ids must be [B, S] or [B, S, H]")
    B, S = int(input_ids.shape[0]), int(input_ids.shape[1])
    T = B * S
    stream = _stream(dev)

    out = {}
    copies = []
    flat_ids = torch.empty((T,) + tuple(input_ids.shape[2:]), dtype=input_ids.dtype, device=dev)
    copies.append(_copy_desc(input_ids, flat_ids, "input_ids"))
    out["input_ids"] = flat_ids
    if labels is not None:
        _require_gpu(labels, "labels")
        if tuple(labels.shape[:2]) != (B, S):
            raise ValueError("labels must be [B, S]")
        flat_labels = torch.empty((T,) + tuple(labels.shape[2:]), dtype=labels.dtype, device=dev)
        copies.append(_copy_desc(labels, flat_labels, "labels"))
        out["labels"] = flat_labels
    _require_gpu(position_ids, "position_ids")
    if position_ids.dim() == 3:       # mRoPE [n_rope, B, S] -> [n_rope, 1, T]
        n_rope = int(position_ids.shape[0])
        if tuple(position_ids.shape[1:]) != (B, S):
            raise ValueError("mRoPE position_ids must be [n_rope, B, S]")
        flat_pos = torch.empty((n_rope, 1, T), dtype=position_ids.dtype, device=dev)
    else:
        if tuple(position_ids.shape) != (B, S):
            raise ValueError("position_ids must be [B, S]")
        flat_pos = torch.empty(T, dtype=position_ids.dtype, device=dev)
    copies.append(_copy_desc(position_ids, flat_pos, "position_ids"))
    out["position_ids"] = flat_pos

    has_padded = False
    if "seq_lens" in batch:
        layout, P, has_padded = _table_layout(batch, B, seq_lens_padding_value)
        cap = B * P + 1
    elif "doc_ids" in batch:
        d = batch["doc_ids"]
        _require_gpu(d, "doc_ids")
        dt = _int_dtype(d, "doc_ids")
        if tuple(d.shape) != (B, S) or not d.is_contiguous():
            raise ValueError("doc_ids must be a contiguous [B, S] tensor")
        layout = _lib.make_layout(_lib.LAYOUT_DOC_IDS, doc_ids=d.data_ptr(), doc_dtype=dt)
        cap = T + 1
    else:
        raise ValueError("batch needs a pack layout: seq_lens (+ seq_lens_padded) or doc_ids")

    cu = torch.empty(cap, dtype=torch.int32, device=dev)
    cp = torch.empty(cap, dtype=torch.int32, device=dev) if has_padded else None
    mask = torch.empty(T, dtype=torch.bool, device=dev)
    scal = torch.empty(4, dtype=torch.int32, device=dev)   # n, max, pad_between, status
    sp = scal.data_ptr()
    arr, n_copies = _lib.make_copies(copies)
    ws = workspace_for(dev, _lib.psq_process_thd_workspace(layout, B, S))
    _lib.psq_process_thd(layout, B, S, cu.data_ptr(), cp.data_ptr() if cp is not None else None,
                         sp, sp + 4, sp + 8, mask.data_ptr(), arr, n_copies, sp + 12,
                         ws.data_ptr(), ws.numel(), stream)
    n, _, pad_between, st = scal.cpu().tolist()
    _raise_status(st, "process_input_for_thd", dev)
    out["cu_seqlens"] = cu[: n + 1]
    if cp is not None:
        out["cu_seqlens_padded"] = cp[: n + 1]
    out["pad_between_seqs"] = bool(pad_between)
    out["max_seqlen"] = scal[1]
    out["padding_mask"] = mask
    for key, value in batch.items():
        if not isinstance(value, torch.Tensor) and key not in out:
            out[key] = value
    return out


def pack_rows(src_tokens: torch.Tensor, src_offsets: torch.Tensor, real_len: torch.Tensor,
              pack_start, capacity: int, pad_to: int, fold: bool = True, pad_token: int = 0,
              pack_order: torch.Tensor | None = None) -> dict:
    """Squeeze padded sources end to end into ``P`` packs of ``capacity`` slots.

    Source ``i`` is ``src_tokens[src_offsets[i] : src_offsets[i] + real_len[i]]``,
    padded to a multiple of ``pad_to``; pack ``p`` holds the sources
    ``pack_start[p] .. pack_start[p+1]-1`` (of ``pack_order`` when given).
    With ``fold`` the last padded boundary of every pack is the capacity.
    Returns ``input_ids`` int64 ``[P, capacity]``, ``token_mask`` uint8
    ``[P, capacity]`` and per-pack ``cu_seqlens`` / ``cu_seqlens_padded``
    lists (views of flat CSR arrays, also returned as ``*_flat``).
    """
    for t, name in ((src_tokens, "src_tokens"), (src_offsets, "src_offsets"), (real_len, "real_len")):
        _require_gpu(t, name)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if src_tokens.dtype != torch.int64 or src_offsets.dtype != torch.int64 or real_len.dtype != torch.int32:
        raise TypeError("src_tokens/src_offsets must be int64 and real_len int32")
    dev = src_tokens.device
    ps_host = torch.as_tensor(pack_start, dtype=torch.int64).cpu()
    ps_dev = ps_host.to(dev)
    P = ps_host.numel() - 1
    N = real_len.numel()
    order_ptr = None
    if pack_order is not None:
        _require_gpu(pack_order, "pack_order")
        if pack_order.dtype != torch.int32 or pack_order.numel() != N:
            raise ValueError("pack_order must be int32 [N]")
        order_ptr = pack_order.data_ptr()
    packed = torch.empty((P, capacity), dtype=torch.int64, device=dev)
    tmask = torch.empty((P, capacity), dtype=torch.uint8, device=dev)
    csr = max(N + P, 1)
    cu = torch.empty(csr, dtype=torch.int32, device=dev)
    cp = torch.empty(csr, dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    ws = workspace_for(dev, _lib.psq_pack_rows_workspace(N, P, capacity))
    _lib.psq_pack_rows(src_tokens.data_ptr(), src_tokens.numel(), src_offsets.data_ptr(),
                       real_len.data_ptr(), N, pad_to, order_ptr, ps_dev.data_ptr(), P,
                       capacity, int(bool(fold)), pad_token, packed.data_ptr(), tmask.data_ptr(),
                       cu.data_ptr(), cp.data_ptr(), status.data_ptr(), ws.data_ptr(),
                       ws.numel(), _stream(dev))
    _raise_status(int(status.item()), "pack_rows", dev)
    psl = ps_host.tolist()
    used = (psl[-1] + P) if P > 0 else 0
    cu_list = [cu[psl[p] + p: psl[p + 1] + p + 1] for p in range(P)]
    cp_list = [cp[psl[p] + p: psl[p + 1] + p + 1] for p in range(P)]
    return {"input_ids": packed, "token_mask": tmask, "cu_seqlens": cu_list,
            "cu_seqlens_padded": cp_list, "cu_seqlens_flat": cu[:used],
            "cu_seqlens_padded_flat": cp[:used]}


def split_batch_into_thd_chunks(batch: dict, num_chunks: int, seq_lens_padding_value: int = -1000,
                                padding_token_id: int = 0) -> dict:
    """Split the batch along rows into ``num_chunks`` equal groups, convert
    each group to THD as :func:`process_input_for_thd` does, and stack.

    One kernel launch converts every group (each with its own boundaries,
    absorption, ``max_seqlen`` and mask).  Returned tensors gain a leading
    chunk axis: ``input_ids`` ``[num_chunks, B/num_chunks*S(, H)]``,
    ``position_ids`` likewise (mRoPE: ``[num_chunks, n_rope, 1, ...]``),
    ``cu_seqlens`` / ``cu_seqlens_padded`` ``[num_chunks, L]`` with every
    chunk filled up to the longest with ``seq_lens_padding_value``,
    ``max_seqlen`` int32 ``[num_chunks]``, ``pad_between_seqs`` bool
    ``[num_chunks]``, ``padding_mask`` ``[num_chunks, B/num_chunks*S]``.
    ``num_chunks <= 1`` returns :func:`process_input_for_thd` unchanged.
    Needs the table layout (``seq_lens``).
    """
    if num_chunks <= 1:
        return process_input_for_thd(batch, seq_lens_padding_value, padding_token_id)
    input_ids = batch["input_ids"]
    position_ids = batch["position_ids"]
    labels = batch.get("labels")
    _require_gpu(input_ids, "input_ids")
    dev = input_ids.device
    if input_ids.dim() not in (2, 3):
        raise ValueError("input_ids must be [B, S] or [B, S, H]")
    B, S = int(input_ids.shape[0]), int(input_ids.shape[1])
    if B % num_chunks != 0:
        raise ValueError(f"num_chunks ({num_chunks}) must evenly divide the batch size ({B})")
    if "seq_lens" not in batch:
        raise ValueError("split_batch_into_thd_chunks needs seq_lens (+ seq_lens_padded)")
    G = int(num_chunks)
    Bc = B // G
    Tc = Bc * S
    stream = _stream(dev)

    out = {}
    copies = []
    ids_out = torch.empty((G, Tc) + tuple(input_ids.shape[2:]), dtype=input_ids.dtype,
                          device=dev)
    copies.append(_copy_desc(input_ids, ids_out, "input_ids"))
    out["input_ids"] = ids_out
    if labels is not None:
        _require_gpu(labels, "labels")
        if tuple(labels.shape[:2]) != (B, S):
            raise ValueError("labels must be [B, S]")
        lab_out = torch.empty((G, Tc) + tuple(labels.shape[2:]), dtype=labels.dtype, device=dev)
        copies.append(_copy_desc(labels, lab_out, "labels"))
        out["labels"] = lab_out
    _require_gpu(position_ids, "position_ids")
    if position_ids.dim() == 3:       # mRoPE [n_rope, B, S] -> [G, n_rope, 1, Tc]
        n_rope = int(position_ids.shape[0])
        if tuple(position_ids.shape[1:]) != (B, S) or not position_ids.is_contiguous():
            raise ValueError("mRoPE position_ids must be a contiguous [n_rope, B, S] tensor")
        pos_out = torch.empty((G, n_rope, 1, Tc), dtype=position_ids.dtype, device=dev)
        esz = position_ids.element_size()
        for k in range(n_rope):       # rope k of every group, written at a stride
            copies.append((position_ids.data_ptr() + k * B * S * esz,
                           pos_out.data_ptr() + k * Tc * esz, G, Tc * esz, Tc * esz,
                           n_rope * Tc * esz))
    else:
        if tuple(position_ids.shape) != (B, S):
            raise ValueError("position_ids must be [B, S]")
        pos_out = torch.empty((G, Tc), dtype=position_ids.dtype, device=dev)
        copies.append(_copy_desc(position_ids, pos_out, "position_ids"))
    out["position_ids"] = pos_out
    if len(copies) > _lib.MAX_COPIES:
        raise ValueError(f"at most {_lib.MAX_COPIES} collapse copies per call")

    layout, P, has_padded = _table_layout(batch, B, seq_lens_padding_value)
    cap = G * (Bc * P + 1)
    cu = torch.empty(cap, dtype=torch.int32, device=dev)
    cp = torch.empty(cap, dtype=torch.int32, device=dev) if has_padded else None
    mask = torch.empty((G, Tc), dtype=torch.bool, device=dev)
    per = torch.empty((3, G), dtype=torch.int32, device=dev)    # n, max, pad_between
    scal = torch.empty(2, dtype=torch.int32, device=dev)        # width, status
    pp, sp = per.data_ptr(), scal.data_ptr()
    arr, n_copies = _lib.make_copies(copies)
    ws = workspace_for(dev, _lib.psq_split_thd_workspace(layout, B, S, G))
    _lib.psq_split_thd(layout, B, S, G, cu.data_ptr(), cp.data_ptr() if cp is not None else None,
                       sp, pp, pp + 4 * G, pp + 8 * G, mask.data_ptr(), arr, n_copies, sp + 4,
                       ws.data_ptr(), ws.numel(), stream)
    width, st = scal.cpu().tolist()
    _raise_status(st, "split_batch_into_thd_chunks", dev)
    out["cu_seqlens"] = cu[: G * width].view(G, width)
    if cp is not None:
        out["cu_seqlens_padded"] = cp[: G * width].view(G, width)
    out["pad_between_seqs"] = per[2].bool()
    out["max_seqlen"] = per[1]
    out["padding_mask"] = mask
    for key, value in batch.items():
        if not isinstance(value, torch.Tensor) and key not in out:
            out[key] = value
    return out


def thd_padding_mask_from_token_ids(input_ids: torch.Tensor, padding_token_id: int) -> torch.Tensor:
    """The padding mask from token values alone, when no pack layout is at hand.

    ``input_ids`` ``[total_tokens]``; returns bool ``[total_tokens]``, True on
    padding.  Raises ``ValueError`` when ``padding_token_id`` also occurs as
    content, i.e. when the pad slots are not a right-padded tail.
    """
    _require_gpu(input_ids, "input_ids")
    dt = _int_dtype(input_ids, "input_ids")
    if input_ids.dim() != 1 or not input_ids.is_contiguous():
        raise ValueError("input_ids must be a contiguous [total_tokens] tensor")
    dev = input_ids.device
    T = input_ids.numel()
    mask = torch.empty(T, dtype=torch.bool, device=dev)
    scal = torch.empty(2, dtype=torch.int32, device=dev)        # num_content, status
    sp = scal.data_ptr()
    ws = workspace_for(dev, _lib.psq_padding_mask_from_token_ids_workspace(T))
    _lib.psq_padding_mask_from_token_ids(input_ids.data_ptr(), dt, T, int(padding_token_id),
                                         mask.data_ptr(), sp, sp + 4, ws.data_ptr(), ws.numel(),
                                         _stream(dev))
    _raise_status(int(scal[1].item()), "thd_padding_mask_from_token_ids", dev)
    return mask


def pack_padded_rows(input_ids: torch.Tensor, input_lengths, bins, pad_to: int, width: int,
                     fold: bool = False, pad_token: int = 0) -> dict:
    """Trainer packs: squeeze the padded rectangle ``input_ids [N, W]`` into bins.

    ``bins`` lists each bin's row indices (chosen on the host, e.g. by token
    budget).  Row ``i`` holds ``input_lengths[i]`` real tokens; each is padded
    to a multiple of ``pad_to`` and a bin's rows are laid end to end in an
    output row of ``width`` slots.  The host packer that chose the bins knows
    the width the batch needs (its fullest bin's padded sum); a bin that does
    not fit raises ``ValueError``.  The trainer path leaves ``fold`` off.
    Returns the keys of :func:`pack_rows` plus ``width``.
    """
    _require_gpu(input_ids, "input_ids")
    if input_ids.dtype != torch.int64 or input_ids.dim() != 2 or not input_ids.is_contiguous():
        raise TypeError("input_ids must be a contiguous int64 [N, W] tensor")
    dev = input_ids.device
    N, W = int(input_ids.shape[0]), int(input_ids.shape[1])
    lens_host = torch.as_tensor(input_lengths, dtype=torch.int64).cpu()
    if lens_host.numel() != N:
        raise ValueError("input_lengths must hold one length per row")
    if N and (int(lens_host.min()) < -(1 << 31) or int(lens_host.max()) >= (1 << 31)):
        raise ValueError("input_lengths must fit int32")
    bins = [list(map(int, b)) for b in bins]
    width = int(width)
    if width < 1:
        raise ValueError("the packed row width must be at least 1")
    P = len(bins)
    members = [i for b in bins for i in b]
    order_host = torch.zeros(max(N, 1), dtype=torch.int32)
    if len(members) > N:
        raise ValueError("the bins hold more members than there are rows")
    order_host[: len(members)] = torch.as_tensor(members, dtype=torch.int32)
    ps_host = torch.zeros(P + 1, dtype=torch.int64)
    ps_host[1:] = torch.as_tensor([len(b) for b in bins], dtype=torch.int64).cumsum(0)
    order_dev = order_host.to(dev)
    ps_dev = ps_host.to(dev)
    lens_dev = lens_host.to(torch.int32).to(dev)
    packed = torch.empty((P, width), dtype=torch.int64, device=dev)
    tmask = torch.empty((P, width), dtype=torch.uint8, device=dev)
    csr = max(N + P, 1)
    cu = torch.empty(csr, dtype=torch.int32, device=dev)
    cp = torch.empty(csr, dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    ws = workspace_for(dev, _lib.psq_pack_rows_workspace(N, P, width))
    _lib.psq_pack_padded_rows(input_ids.data_ptr(), W, lens_dev.data_ptr(), N, pad_to,
                              order_dev.data_ptr(), ps_dev.data_ptr(), P, width, int(bool(fold)),
                              pad_token, packed.data_ptr(), tmask.data_ptr(), cu.data_ptr(),
                              cp.data_ptr(), status.data_ptr(), ws.data_ptr(), ws.numel(),
                              _stream(dev))
    _raise_status(int(status.item()), "pack_padded_rows", dev)
    psl = ps_host.tolist()
    used = (psl[-1] + P) if P > 0 else 0
    return {"input_ids": packed, "token_mask": tmask, "width": width,
            "cu_seqlens": [cu[psl[p] + p: psl[p + 1] + p + 1] for p in range(P)],
            "cu_seqlens_padded": [cp[psl[p] + p: psl[p + 1] + p + 1] for p in range(P)],
            "cu_seqlens_flat": cu[:used], "cu_seqlens_padded_flat": cp[:used]}
