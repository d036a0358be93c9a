"""Seeded synthetic inputs for the packed-sequence metadata path.

This module only *draws* inputs: document maps, length tables, token
streams and the host-side bin assignment that decides which sources share a
pack.  It computes none of the metadata (boundaries, maxima, masks, packed
rows); both the HIP library and the CPU oracle receive its arrays as inputs.

Every generator is a pure function of its seed (numpy ``default_rng`` over a
``SeedSequence``, one spawned stream for lengths and one for token values).
The five workloads are:

  1. ``doc_map_small``   doc_ids int32 [4, 64]:  docs of length U{1..24},
     indices 1, 2, ... restarting per row, trailing pad U{0..16}.
  2. ``doc_map_medium``  doc_ids int32 [8, 4096]: one row (about 5 % of 8)
     is a single document filling the row; the others carry docs of
     lognormal length (median 300, sigma 1.0, clipped 1..4096) and a trailing
     pad U{0..512}.
  3. ``thd_tables``      seq_lens / seq_lens_padded int64 [16, 64] for rows of
     8192 slots: lognormal lengths (median 100, sigma 1.0, clipped 1..2048),
     padded up to a multiple of 8, a row closes when the next padded length
     would overflow it or its 64 slots are used, -1000 fills unused slots;
     input_ids / labels int64 [16, 8192] uniform over 0..151935 in every slot
     (so 0 occurs as content), position_ids 0..real-1 on real slots, 0 on pad.
  4. ``pack_sources``    65536 sources of lognormal length (median 400,
     sigma 1.2, clipped 1..8192), stored end to end; pad multiple 64; in-order
     next-fit into packs of 16384 slots.
  5. ``stage_embedding`` doc_ids int32 [32, 32768] drawn like workload 1, and
     int64 position_ids counting from 0 inside every run (padding runs too);
     the bf16 [32, 32768, 4096] N(0, 1) hidden tensor is drawn on the device
     by :func:`stage_hidden` with a seeded torch generator.

Inputs of the steps around the workloads:

  * ``pad_tail_stream``   a flat int64 token stream of workload 3's size
    (131072 ids, uniform over 0..151935) whose last U{0..8192} slots hold a
    pad id outside the token range: the metadata-free padding mask.
  * ``trainer_rectangle`` a trainer micro-batch: 256 conversations of
    workload 4's length law in a padded [N, max_len] rectangle (0 past each
    length), bins chosen by first-fit decreasing on a 16384-token budget
    (:func:`token_budget_bins`), pad multiple 64.
"""
from __future__ import annotations

import numpy as np

TOKEN_HIGH = 151935          # token ids are uniform over 0..TOKEN_HIGH
PAD_VALUE = -1000            # unused-slot sentinel of the length tables


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    a, b = ss.spawn(2)
    return np.random.default_rng(a), np.random.default_rng(b)


def _lognormal_int(rng, median: float, sigma: float, lo: int, hi: int, size=None):
    z = rng.standard_normal(size)
    return np.clip(np.rint(np.exp(np.log(median) + sigma * z)), lo, hi).astype(np.int64)


def _round_up(x, m):
    return (x + m - 1) // m * m


def _fill_row_uniform(rng, S: int, doc_lo: int, doc_hi: int, pad_hi: int) -> np.ndarray:
    row = np.zeros(S, dtype=np.int32)
    pad = int(rng.integers(0, pad_hi + 1))
    end = max(S - pad, 0)
    t, idx = 0, 1
    while t < end:
        n = int(rng.integers(doc_lo, doc_hi + 1))
        n = min(n, end - t)
        row[t:t + n] = idx
        t += n
        idx += 1
    return row


def doc_map_small(seed: int = 1, B: int = 4, S: int = 64) -> np.ndarray:
    """Workload 1 generator (also used by workload 5)."""
    rng, _ = _streams(seed)
    return np.stack([_fill_row_uniform(rng, S, 1, 24, 16) for _ in range(B)])


def doc_map_medium(seed: int = 2, B: int = 8, S: int = 4096) -> np.ndarray:
    """Workload 2: lognormal docs, a few single-document rows."""
    rng, _ = _streams(seed)
    k = max(1, int(round(0.05 * B)))
    single = set(int(x) for x in rng.choice(max(B - 1, 1), size=min(k, max(B - 1, 1)),
                                            replace=False))
    rows = []
    for r in range(B):
        row = np.zeros(S, dtype=np.int32)
        if r in single:
            row[:] = 1
        else:
            pad = int(rng.integers(0, 513))
            end = max(S - pad, 0)
            t, idx = 0, 1
            while t < end:
                n = int(_lognormal_int(rng, 300.0, 1.0, 1, 4096))
                n = min(n, end - t)
                row[t:t + n] = idx
                t += n
                idx += 1
        rows.append(row)
    return np.stack(rows)


def thd_tables(seed: int = 3, B: int = 16, S: int = 8192, P: int = 64) -> dict:
    """Workload 3: per-row sequence tables plus the token tensors they describe."""
    rng_len, rng_tok = _streams(seed)
    L = np.full((B, P), PAD_VALUE, dtype=np.int64)
    Lp = np.full((B, P), PAD_VALUE, dtype=np.int64)
    pos = np.zeros((B, S), dtype=np.int64)
    for r in range(B):
        used, j = 0, 0
        while j < P:
            real = int(_lognormal_int(rng_len, 100.0, 1.0, 1, 2048))
            padded = int(_round_up(real, 8))
            if used + padded > S:
                break
            L[r, j], Lp[r, j] = real, padded
            # the collate writes positions 0..real-1 where the sequence sits
            pos[r, used:used + real] = np.arange(real)
            used += padded
            j += 1
    input_ids = rng_tok.integers(0, TOKEN_HIGH + 1, size=(B, S), dtype=np.int64)
    labels = rng_tok.integers(0, TOKEN_HIGH + 1, size=(B, S), dtype=np.int64)
    return {"seq_lens": L, "seq_lens_padded": Lp, "input_ids": input_ids,
            "labels": labels, "position_ids": pos, "S": S}


def next_fit(padded_len: np.ndarray, capacity: int) -> np.ndarray:
    """In-order next-fit bin assignment on the host; returns ``pack_start``.

    Walk the sources in order; close the open pack when the next padded
    source no longer fits and the pack already holds something.
    """
    starts = [0]
    cur = 0
    for i, n in enumerate(np.asarray(padded_len).tolist()):
        if n > capacity:
            raise ValueError(f"source {i} ({n} slots) exceeds capacity {capacity}")
        if cur + n > capacity and i > starts[-1]:
            starts.append(i)
            cur = 0
        cur += n
    starts.append(len(padded_len))
    if len(padded_len) == 0:
        starts = [0]
    return np.asarray(starts, dtype=np.int64)


def pack_sources(seed: int = 4, N: int = 65536, capacity: int = 16384, q: int = 64,
                 median: float = 400.0, sigma: float = 1.2, max_len: int = 8192) -> dict:
    """Workload 4: sources stored end to end and their next-fit packs."""
    rng_len, rng_tok = _streams(seed)
    real = _lognormal_int(rng_len, median, sigma, 1, max_len, size=N)
    src_off = np.zeros(N, dtype=np.int64)
    if N > 1:
        src_off[1:] = np.cumsum(real[:-1])
    total = int(real.sum())
    tokens = rng_tok.integers(0, TOKEN_HIGH + 1, size=total, dtype=np.int64)
    pack_start = next_fit(_round_up(real, q), capacity)
    return {"src": tokens, "src_off": src_off, "real_len": real.astype(np.int32),
            "pack_start": pack_start, "q": q, "capacity": capacity}


def token_budget_bins(padded_len, budget: int) -> tuple:
    """First-fit decreasing on the host: longest padded source first, each
    into the first bin with room for it.  Returns each bin's source indices
    in the order they were placed, and each bin's fill (the padded slots it
    holds, from the packer's own room bookkeeping)."""
    padded = np.asarray(padded_len, dtype=np.int64)
    order = sorted(range(padded.size), key=lambda i: (-int(padded[i]), i))
    bins, room = [], []
    for i in order:
        n = int(padded[i])
        if n > budget:
            raise ValueError(f"source {i} ({n} slots) exceeds the budget {budget}")
        for b in range(len(bins)):
            if room[b] >= n:
                bins[b].append(i)
                room[b] -= n
                break
        else:
            bins.append([i])
            room.append(budget - n)
    return bins, [budget - r for r in room]


def trainer_rectangle(seed: int = 6, N: int = 256, q: int = 64, budget: int = 16384,
                      median: float = 400.0, sigma: float = 1.2, max_len: int = 8192) -> dict:
    """A trainer micro-batch: padded rectangle, lengths, token-budget bins,
    and the packed row width the packer chose: the padded fill of its
    fullest bin, so no row is wider than that bin requires."""
    rng_len, rng_tok = _streams(seed)
    real = _lognormal_int(rng_len, median, sigma, 1, max_len, size=N)
    W = int(real.max()) if N > 0 else 0
    rows = np.zeros((N, W), dtype=np.int64)
    for i in range(N):
        rows[i, :real[i]] = rng_tok.integers(0, TOKEN_HIGH + 1, size=int(real[i]))
    bins, fill = token_budget_bins(_round_up(real, q), budget)
    return {"rows": rows, "real_len": real.astype(np.int32), "bins": bins, "q": q,
            "budget": budget, "width": max(fill, default=0)}


def pad_tail_stream(seed: int = 7, T: int = 131072, tail_hi: int = 8192) -> dict:
    """A flat token stream with a right-padded tail of a non-content pad id."""
    rng_len, rng_tok = _streams(seed)
    tail = int(rng_len.integers(0, tail_hi + 1))
    ids = rng_tok.integers(0, TOKEN_HIGH + 1, size=T, dtype=np.int64)
    pad_id = TOKEN_HIGH + 1
    ids[T - tail:] = pad_id
    return {"input_ids": ids, "pad_id": pad_id, "tail": tail}


def run_positions(doc_ids: np.ndarray) -> np.ndarray:
    """Position ids counting from 0 inside every run of one index in a row.

    This is input construction for workload 5 (a collate's position ids),
    done with a plain per-row loop.
    """
    d = np.asarray(doc_ids)
    B, S = d.shape
    pos = np.zeros((B, S), dtype=np.int64)
    for r in range(B):
        row = d[r]
        change = np.ones(S, dtype=bool)
        change[1:] = row[1:] != row[:-1]
        start_idx = np.maximum.accumulate(np.where(change, np.arange(S), 0))
        pos[r] = np.arange(S) - start_idx
    return pos


def stage_embedding(seed: int = 5, B: int = 32, S: int = 32768) -> dict:
    """Workload 5 host side: the doc map (drawn like workload 1) and positions."""
    doc = doc_map_small(seed, B, S)
    return {"doc_ids": doc, "position_ids": run_positions(doc)}


def stage_hidden(seed: int, B: int, S: int, H: int, device):
    """Workload 5 device side: bf16 N(0, 1) hidden states, drawn on ``device``."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((B, S, H), dtype=torch.bfloat16, device=device, generator=g)


WORKLOADS = {
    1: "doc_map_small: doc_ids int32 [4,64] -> cu_seqlens, max_seqlen",
    2: "doc_map_medium: doc_ids int32 [8,4096] -> cu_seqlens, max_seqlen",
    3: "thd_tables: seq_lens int64 [16,64], S=8192 -> THD metadata, mask, 3 collapsed int64 tensors",
    4: "pack_sources: 65536 sources, q=64, next-fit at 16384 -> packed int64 [P,16384], token_mask, CSR",
    5: "stage_embedding: doc_ids int32 [32,32768], hidden bf16 [32,32768,4096] -> THD [1048576,4096]",
}
