"""Pins for the oracle's document-map segmentation (CPU only).

The oracle follows the NeMo AutoModel API page
``nemo_automodel.components.datasets.packed_seq`` (module text and
``packed_seq_params_from_doc_ids``).  It is pinned here to things other than
itself: the page's example map, hand cases of the segment rule, brute force
over every tiny map against an independent ``itertools.groupby``
formulation, a numpy reduction, and invariants on the seeded workloads.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth
from conftest import load_golden


def groupby_segments(doc):
    """Independent formulation: per row, the lengths of runs of equal values."""
    doc = np.asarray(doc)
    lens = []
    for r in range(doc.shape[0]):
        for _, grp in itertools.groupby(doc[r].tolist()):
            lens.append(len(list(grp)))
    cu = [0] + list(itertools.accumulate(lens))
    return cu, (max(lens) if lens else 0)


def numpy_segments(doc):
    """Library reduction: run starts from np.diff per row plus the row offsets."""
    doc = np.asarray(doc)
    B, S = doc.shape
    starts = []
    for r in range(B):
        starts.append(np.array([r * S]))
        starts.append(r * S + np.flatnonzero(np.diff(doc[r])) + 1)
    st = np.concatenate(starts) if B * S else np.zeros(0, dtype=np.int64)
    return np.concatenate([st, [B * S]]).astype(np.int64)


def test_page_example_map():
    g = load_golden("doc_map_example.json")
    out = oracle.doc_segments(np.array(g["input"]["doc_ids"]))
    d = g["derived"]
    assert out["cu_seqlens"].tolist() == d["cu_seqlens"]
    assert out["num_segments"] == d["num_segments"]
    assert out["max_seqlen"] == d["max_seqlen"]
    assert out["padding_mask"].tolist() == d["padding_mask"]


def test_forced_row_start_boundary():
    # A row-filling document must not merge with the next row's document 1.
    out = oracle.doc_segments(np.array([[1, 1, 1], [1, 1, 0]]))
    assert out["cu_seqlens"].tolist() == [0, 3, 5, 6]
    assert out["max_seqlen"] == 3


def test_padding_run_is_a_segment_and_counts_for_max():
    out = oracle.doc_segments(np.array([[1, 0, 0, 0]]))
    assert out["cu_seqlens"].tolist() == [0, 1, 4]
    assert out["max_seqlen"] == 3


def test_repeated_index_is_runs_not_identity():
    out = oracle.doc_segments(np.array([[1, 2, 1]]))
    assert out["cu_seqlens"].tolist() == [0, 1, 2, 3]
    assert out["max_seqlen"] == 1


def test_empty_and_degenerate_shapes():
    for shape in [(0, 5), (3, 0), (0, 0)]:
        out = oracle.doc_segments(np.zeros(shape, dtype=np.int32))
        assert out["cu_seqlens"].tolist() == [0]
        assert out["num_segments"] == 0 and out["max_seqlen"] == 0
    out = oracle.doc_segments(np.array([[7]]))
    assert out["cu_seqlens"].tolist() == [0, 1] and out["max_seqlen"] == 1
    # S = 1: every token is its own segment
    out = oracle.doc_segments(np.array([[3], [3], [0]]))
    assert out["cu_seqlens"].tolist() == [0, 1, 2, 3]


def test_values_are_only_compared():
    # Negative and large indices are legal: only equality matters.
    a = oracle.doc_segments(np.array([[-5, -5, 2**40, 2**40, 0]]))
    b = oracle.doc_segments(np.array([[1, 1, 2, 2, 0]]))
    assert a["cu_seqlens"].tolist() == b["cu_seqlens"].tolist()


def test_brute_force_tiny_maps():
    """Every map over {0,1,2} with B*S <= 8, every B x S factorisation."""
    checked = 0
    for T in range(1, 9):
        shapes = [(B, T // B) for B in range(1, T + 1) if T % B == 0]
        for vals in itertools.product((0, 1, 2), repeat=T):
            flat = np.array(vals, dtype=np.int64)
            for B, S in shapes:
                doc = flat.reshape(B, S)
                out = oracle.doc_segments(doc)
                cu, mx = groupby_segments(doc)
                assert out["cu_seqlens"].tolist() == cu, (doc, out)
                assert out["max_seqlen"] == mx
                assert out["padding_mask"].tolist() == (flat == 0).astype(int).tolist()
                checked += 1
    assert checked > 20000


def _check_invariants(doc, out):
    B, S = doc.shape
    cu = out["cu_seqlens"].astype(np.int64)
    assert cu[0] == 0 and cu[-1] == B * S
    assert np.all(np.diff(cu) > 0)
    assert set(range(0, B * S, S)).issubset(set(cu.tolist()))
    flat = doc.reshape(-1)
    for k in range(len(cu) - 1):
        seg = flat[cu[k]:cu[k + 1]]
        assert np.all(seg == seg[0])
    assert out["max_seqlen"] == int(np.diff(cu).max()) <= S


@pytest.mark.parametrize("gen", [synth.doc_map_small, synth.doc_map_medium])
def test_workload_maps(gen):
    doc = gen()
    out = oracle.doc_segments(doc)
    _check_invariants(doc, out)
    assert out["cu_seqlens"].tolist() == numpy_segments(doc).tolist()
    assert out["padding_mask"].tolist() == (doc.reshape(-1) == 0).astype(int).tolist()


def test_stage_embedding_map_numpy_reduction():
    doc = synth.stage_embedding()["doc_ids"]
    out = oracle.doc_segments(doc)
    ref = numpy_segments(doc)
    assert np.array_equal(out["cu_seqlens"].astype(np.int64), ref)
    assert out["max_seqlen"] == int(np.diff(ref).max())


def test_copy_rows_is_identity():
    rng = np.random.default_rng(0)
    a = rng.integers(0, 2**63 - 1, size=(5, 7), dtype=np.int64)
    got = oracle.copy_rows(a, rows=5, row_bytes=7 * 8, src_row_stride_bytes=7 * 8)
    assert got.tobytes() == a.tobytes()
    # strided rows: the first 3 columns of every row
    got = oracle.copy_rows(a, rows=5, row_bytes=3 * 8, src_row_stride_bytes=7 * 8)
    assert got.tobytes() == np.ascontiguousarray(a[:, :3]).tobytes()


@pytest.mark.parametrize("seed", range(6))
def test_random_maps_against_groupby(seed):
    # medium random maps of every flavour (long runs, short runs, heavy pad)
    rng = np.random.default_rng(100 + seed)
    B, S = int(rng.integers(1, 9)), int(rng.integers(1, 700))
    alphabet = int(rng.integers(1, 6))
    doc = rng.integers(0, alphabet, size=(B, S))
    if seed % 2:                       # long runs: repeat each value a few times
        doc = np.repeat(doc, int(rng.integers(2, 9)), axis=1)[:, :S]
    out = oracle.doc_segments(doc)
    cu, mx = groupby_segments(doc)
    assert out["cu_seqlens"].tolist() == cu
    assert out["max_seqlen"] == mx
    assert out["padding_mask"].tolist() == (doc.reshape(-1) == 0).astype(int).tolist()
