"""Pins for the oracle's THD conversion from length tables (CPU only).

The oracle follows the NeMo AutoModel 0.5 API page
``nemo_automodel.components.distributed.thd_utils`` (``process_input_for_thd``
and ``_thd_padding_mask``).  Pinned here by the page's printed Example values,
the printed ``split_batch_into_thd_chunks`` Example, hand cases of the readings
the page leaves open (row fold, absorption gate, max after absorption), brute
force over every small table against an independent slot-grid simulation, and
invariants on the seeded workload.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth
from conftest import load_golden

V = -1000


def grid_formulation(L, Lp, S, v=V):
    """Independent formulation by writing sequences into the [B, S] slot grid.

    Each row's valid sequences are written left to right, each taking its
    padded width, and the last sequence of a row owns every slot to the end
    of the row.  Boundaries are then *counted* off the grid: the physical
    boundary before sequence i is the number of slots owned by sequences
    < i, the real boundary the number of token slots owned by them.
    """
    L = np.asarray(L)
    Lp = L if Lp is None else np.asarray(Lp)
    B, P = L.shape
    owner = np.full((B, S), -1, dtype=np.int64)
    is_tok = np.zeros((B, S), dtype=bool)
    n = 0
    for r in range(B):
        entries = [(int(L[r, j]), int(Lp[r, j])) for j in range(P) if L[r, j] != v]
        col = 0
        for idx, (real, padded) in enumerate(entries):
            width = (S - col) if idx == len(entries) - 1 else padded
            for c in range(col, col + width):
                owner[r, c] = n
                is_tok[r, c] = (c - col) < real
            col += width
            n += 1
    own = owner.reshape(-1)
    tok = is_tok.reshape(-1)
    cp = [int(np.sum(own < i)) for i in range(n + 1)]
    cu = [int(np.sum(tok & (own < i))) for i in range(n + 1)]
    T = B * S
    # Absorption reading: the pack-pad is purely trailing when no interior
    # real boundary departs from its physical one.
    if all(cu[i] == cp[i] for i in range(1, n)) and cu[n] < T:
        cu[n] = T
    pad_between = int(any(a != b for a, b in zip(cu, cp)))
    mx = max((cu[i + 1] - cu[i] for i in range(n)), default=0)
    return {"cu_seqlens": cu, "cu_seqlens_padded": cp, "max_seqlen": mx,
            "pad_between_seqs": pad_between, "padding_mask": (~tok).astype(int).tolist()}


def test_page_example_printed_values():
    g = load_golden("thd_example.json")
    inp = g["input"]
    out = oracle.thd_tables(inp["seq_lens"], inp["seq_lens_padded"], inp["S"])
    assert out["status"] == 0
    pr = g["printed"]
    assert out["cu_seqlens"].tolist() == pr["cu_seqlens"]
    assert out["cu_seqlens_padded"].tolist() == pr["cu_seqlens_padded"]
    assert out["max_seqlen"] == pr["max_seqlen"]
    assert out["padding_mask"].size == pr["flat_length"]
    d = g["derived"]
    assert out["padding_mask"].tolist() == d["padding_mask"]
    assert out["pad_between_seqs"] == d["pad_between_seqs"]
    # The masked slot is the one holding token 99 at position 0.
    flat_ids = np.array(inp["input_ids"]).reshape(-1)
    assert flat_ids[out["padding_mask"].astype(bool)].tolist() == [99]


def test_chunks_example_printed_values():
    # split_batch_into_thd_chunks: every chunk of 2 rows gives [0, 6, 12].
    g = load_golden("thd_chunks_example.json")
    inp = g["input"]
    L = np.array(inp["seq_lens"])
    Lp = np.array(inp["seq_lens_padded"])
    per = len(L) // inp["num_chunks"]
    for c in range(inp["num_chunks"]):
        out = oracle.thd_tables(L[c * per:(c + 1) * per], Lp[c * per:(c + 1) * per], inp["S"])
        assert out["cu_seqlens"].tolist() == g["printed"]["cu_seqlens_per_chunk"][c]
        assert out["cu_seqlens_padded"].tolist() == g["derived"]["cu_seqlens_padded_per_chunk"][c]
        assert out["max_seqlen"] == g["derived"]["max_seqlen"]
        assert out["pad_between_seqs"] == g["derived"]["pad_between_seqs"]
        assert out["padding_mask"].sum() == 0


def test_split_chunks_example_printed_values():
    # split_batch_into_thd_chunks Example: input_ids [2, 12], cu_seqlens [2, 3],
    # each chunk [0, 6, 12].
    g = load_golden("thd_chunks_example.json")
    inp = g["input"]
    out = oracle.split_thd(inp["seq_lens"], inp["seq_lens_padded"], inp["S"],
                           inp["num_chunks"])
    assert out["status"] == 0
    pr = g["printed"]
    assert list(out["cu_seqlens"].shape) == pr["cu_seqlens_shape"]
    assert out["cu_seqlens"].tolist() == pr["cu_seqlens_per_chunk"]
    assert list(out["padding_mask"].shape) == pr["input_ids_shape"]
    assert out["cu_seqlens_padded"].tolist() == g["derived"]["cu_seqlens_padded_per_chunk"]
    assert out["max_seqlen"].tolist() == [g["derived"]["max_seqlen"]] * 2
    assert out["pad_between_seqs"].tolist() == [g["derived"]["pad_between_seqs"]] * 2


def test_split_ragged_chunks_are_filled_with_the_sentinel():
    # Hand case: chunk 0 holds 3 sequences, chunk 1 one, so chunk 1's arrays
    # are filled with the sentinel up to chunk 0's length 4.  Chunk 0 is
    # tight up to its last sequence (absorbs: [0,2,5,8]); chunk 1's single
    # sequence absorbs too ([0,1] -> [0,4]).
    out = oracle.split_thd([[2, 3, 1], [1, V, V]], [[2, 3, 1], [1, V, V]], S=8,
                           num_chunks=2)
    assert out["status"] == 0
    assert out["cu_seqlens_padded"].tolist() == [[0, 2, 5, 8], [0, 8, V, V]]
    assert out["cu_seqlens"].tolist() == [[0, 2, 5, 8], [0, 8, V, V]]
    assert out["num_seqs"].tolist() == [3, 1]
    assert out["max_seqlen"].tolist() == [3, 8]
    assert out["pad_between_seqs"].tolist() == [0, 0]
    assert np.flatnonzero(out["padding_mask"][0]).tolist() == [6, 7]
    assert np.flatnonzero(out["padding_mask"][1]).tolist() == list(range(1, 8))


def test_split_is_per_row_local():
    # Rows are independent once each row's tail pad is folded into it, so
    # the chunks' physical boundaries are the whole batch's, rebased, and
    # the stacked mask is the whole batch's mask.  Absorption is per chunk:
    # the real boundaries agree with the whole batch's except at a chunk end.
    w = synth.thd_tables(B=16)
    L, Lp, S = w["seq_lens"], w["seq_lens_padded"], w["S"]
    whole = oracle.thd_tables(L, Lp, S)
    for chunks in (1, 2, 4, 16):
        out = oracle.split_thd(L, Lp, S, chunks)
        assert out["status"] == 0
        rows = L.shape[0] // chunks
        assert np.array_equal(out["padding_mask"].reshape(-1), whole["padding_mask"])
        first = 0
        for c in range(chunks):
            k = int(out["num_seqs"][c])
            cp_whole = whole["cu_seqlens_padded"][first:first + k + 1].astype(np.int64)
            assert np.array_equal(out["cu_seqlens_padded"][c, :k + 1], cp_whole - c * rows * S)
            cu_whole = whole["cu_seqlens"][first:first + k].astype(np.int64)
            assert np.array_equal(out["cu_seqlens"][c, :k], cu_whole - cu_whole[0])
            assert np.all(out["cu_seqlens"][c, k + 1:] == V)
            first += k
        assert first == whole["num_seqs"]


def test_split_rejects_uneven_chunks():
    with pytest.raises(ValueError):
        oracle.split_thd([[1], [1], [1]], None, S=2, num_chunks=2)


def test_split_status_is_the_or_over_chunks():
    # Each chunk is its own process_input_for_thd call, and the split fails
    # when any of them does: an empty row in the first chunk only, then a
    # row overflow in the last chunk as well.
    L = [[V, V], [2, 3], [1, V], [4, V]]
    out = oracle.split_thd(L, None, S=6, num_chunks=2)
    assert out["status"] == oracle.EMPTY_ROW
    L2 = [[V, V], [2, 3], [1, V], [7, V]]
    out = oracle.split_thd(L2, None, S=6, num_chunks=2)
    assert out["status"] == oracle.EMPTY_ROW | oracle.ROW_OVERFLOW


def test_row_fold_with_tail_pad_in_every_row():
    out = oracle.thd_tables([[3, 2], [6, V]], [[4, 2], [6, V]], S=8)
    assert out["cu_seqlens"].tolist() == [0, 3, 5, 11]
    assert out["cu_seqlens_padded"].tolist() == [0, 4, 8, 16]
    assert out["max_seqlen"] == 6
    assert out["pad_between_seqs"] == 1
    assert np.flatnonzero(out["padding_mask"]).tolist() == [3, 6, 7, 14, 15]


def test_absorption_fires_and_max_follows_it():
    out = oracle.thd_tables([[3, 2]], [[3, 2]], S=8)
    assert out["cu_seqlens_padded"].tolist() == [0, 3, 8]
    assert out["cu_seqlens"].tolist() == [0, 3, 8]
    assert out["pad_between_seqs"] == 0
    assert out["max_seqlen"] == 5
    assert np.flatnonzero(out["padding_mask"]).tolist() == [5, 6, 7]


def test_second_row_starts_at_its_row():
    # A literal cumsum would start row 1's sequence at slot 3.
    out = oracle.thd_tables([[3], [4]], [[3], [4]], S=4)
    assert out["cu_seqlens_padded"].tolist() == [0, 4, 8]
    assert out["cu_seqlens"].tolist() == [0, 3, 7]
    assert out["pad_between_seqs"] == 1
    assert out["max_seqlen"] == 4
    assert np.flatnonzero(out["padding_mask"]).tolist() == [3]


def test_without_padded_table():
    out = oracle.thd_tables([[3, 2], [6, V]], None, S=6)
    assert out["status"] == 0
    assert out["cu_seqlens_padded"].tolist() == [0, 3, 6, 12]
    assert out["cu_seqlens"].tolist() == [0, 3, 5, 11]
    assert out["pad_between_seqs"] == 1
    assert np.flatnonzero(out["padding_mask"]).tolist() == [5]


@pytest.mark.parametrize("L,Lp,S,bits", [
    ([[3, V]], [[3, 2]], 8, oracle.TABLE_MISMATCH),
    ([[3, 2]], [[3, V]], 8, oracle.TABLE_MISMATCH | oracle.BAD_LENGTH),
    ([[5]], [[4]], 8, oracle.BAD_LENGTH),
    ([[-1]], [[2]], 8, oracle.BAD_LENGTH),
    ([[V, V], [2, V]], [[V, V], [2, V]], 8, oracle.EMPTY_ROW),
    ([[4, 4]], [[5, 4]], 8, oracle.ROW_OVERFLOW),
    ([[4]], [[2**62]], 8, oracle.ROW_OVERFLOW),
    ([[5], [V]], [[4], [V]], 8, oracle.BAD_LENGTH | oracle.EMPTY_ROW),
])
def test_data_errors(L, Lp, S, bits):
    assert oracle.thd_tables(L, Lp, S)["status"] == bits


def test_zero_length_sequences_are_legal():
    out = oracle.thd_tables([[0, 3]], [[0, 4]], S=4)
    assert out["status"] == 0
    assert out["cu_seqlens"].tolist() == [0, 0, 4]   # absorbed
    assert out["cu_seqlens_padded"].tolist() == [0, 0, 4]


def test_brute_force_small_tables():
    """Every table with B <= 2, P <= 2, real <= padded <= 3, S in {3, 4, 6}."""
    pairs = [(V, V)] + [(r, p) for p in range(0, 4) for r in range(0, p + 1)]
    checked = 0
    for B in (1, 2):
        for P in (1, 2):
            for S in (3, 4, 6):
                for combo in itertools.product(pairs, repeat=B * P):
                    L = np.array([c[0] for c in combo]).reshape(B, P)
                    Lp = np.array([c[1] for c in combo]).reshape(B, P)
                    rows_ok = all((L[r] != V).any() and Lp[r][L[r] != V].sum() <= S
                                  for r in range(B))
                    out = oracle.thd_tables(L, Lp, S)
                    if not rows_ok:
                        assert out["status"] != 0
                        continue
                    assert out["status"] == 0, (L, Lp, S)
                    ref = grid_formulation(L, Lp, S)
                    for key in ("cu_seqlens", "cu_seqlens_padded", "padding_mask"):
                        assert np.asarray(out[key]).tolist() == ref[key], (key, L, Lp, S)
                    assert out["max_seqlen"] == ref["max_seqlen"]
                    assert out["pad_between_seqs"] == ref["pad_between_seqs"]
                    checked += 1
    assert checked > 1000


def test_workload_tables():
    w = synth.thd_tables()
    S = w["S"]
    L, Lp = w["seq_lens"], w["seq_lens_padded"]
    out = oracle.thd_tables(L, Lp, S)
    assert out["status"] == 0
    cu, cp = out["cu_seqlens"].astype(np.int64), out["cu_seqlens_padded"].astype(np.int64)
    B = L.shape[0]
    valid = L != V
    n = int(valid.sum())
    assert out["num_seqs"] == n and len(cu) == n + 1
    assert cp[-1] == B * S
    # every row's physical boundaries end at the row end
    ends = np.cumsum(valid.sum(axis=1))
    assert cp[ends].tolist() == [(r + 1) * S for r in range(B)]
    # physical steps are at least the real lengths
    assert np.all(np.diff(cp) >= L[valid])
    # the mask keeps exactly the real tokens
    assert int((out["padding_mask"] == 0).sum()) == int(L[valid].sum())
    # pad_between iff the arrays differ; max is the widest real step
    assert out["pad_between_seqs"] == int(not np.array_equal(cu, cp))
    assert out["max_seqlen"] == int(np.diff(cu).max())
    ref = grid_formulation(L, Lp, S)
    assert cu.tolist() == ref["cu_seqlens"] and cp.tolist() == ref["cu_seqlens_padded"]
    assert out["padding_mask"].tolist() == ref["padding_mask"]


@pytest.mark.parametrize("seed", range(8))
def test_random_tables_against_grid(seed):
    # medium random tables (holes, zero lengths, tight and padded rows)
    rng = np.random.default_rng(200 + seed)
    B, P, S = int(rng.integers(1, 6)), int(rng.integers(1, 9)), int(rng.integers(4, 120))
    L = np.full((B, P), V, dtype=np.int64)
    Lp = np.full((B, P), V, dtype=np.int64)
    for r in range(B):
        used = 0
        slots = sorted(rng.choice(P, size=int(rng.integers(1, P + 1)), replace=False))
        for j in slots:
            real = int(rng.integers(0, S // 3 + 1))
            padded = real + (0 if seed % 3 == 0 else int(rng.integers(0, 4)))
            if used + padded > S:
                break
            L[r, j], Lp[r, j] = real, padded
            used += padded
        if not (L[r] != V).any():
            L[r, slots[0]], Lp[r, slots[0]] = 0, 0
    out = oracle.thd_tables(L, Lp, S)
    assert out["status"] == 0
    ref = grid_formulation(L, Lp, S)
    assert out["cu_seqlens"].tolist() == ref["cu_seqlens"]
    assert out["cu_seqlens_padded"].tolist() == ref["cu_seqlens_padded"]
    assert out["max_seqlen"] == ref["max_seqlen"]
    assert out["pad_between_seqs"] == ref["pad_between_seqs"]
    assert out["padding_mask"].tolist() == ref["padding_mask"]
