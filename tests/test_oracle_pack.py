"""Pins for the oracle's squeeze into fixed-capacity packs (CPU only).

The oracle follows "Who packs the sequences: the loader, or the trainer?"
(What the data looks like at each hop: Trainer packs, Loader packs).  Pinned
by the printed examples ([0,5,15] / [0,8,20] at width 20, [0,8,36] at
capacity 36, 16 tail pad, 15 real of 36), a numpy reduction (pad multiple 1,
no fold, one pack holding everything is a concatenation), brute force against
an independent list-building formulation, and invariants on the workload.
The trainer-path squeeze straight from the padded rectangle is pinned by the
same printed trainer example (width 20 is the widest bin's padded sum), the
concatenation reduction, and brute force over small rectangles and bin
splits against the list formulation.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth
from conftest import load_golden


def list_formulation(sources, members, q, C, fold, pad):
    """Independent formulation: build the row as a Python list."""
    row, tm, cu, cp = [], [], [0], [0]
    for i in members:
        toks = list(sources[i])
        padded = -(-len(toks) // q) * q
        row += toks + [pad] * (padded - len(toks))
        tm += [1] * len(toks) + [0] * (padded - len(toks))
        cu.append(cu[-1] + len(toks))
        cp.append(len(row))
    row += [pad] * (C - len(row))
    tm += [0] * (C - len(tm))
    if fold:
        cp[-1] = C
    return row, tm, cu, cp


def _flat(sources):
    lens = np.array([len(s) for s in sources], dtype=np.int32)
    off = np.zeros(len(sources), dtype=np.int64)
    if len(sources) > 1:
        off[1:] = np.cumsum(lens[:-1])
    src = np.concatenate([np.asarray(s, dtype=np.int64) for s in sources]) if sources else \
        np.zeros(0, dtype=np.int64)
    return src, off, lens


@pytest.mark.parametrize("name", ["trainer_pack_example.json", "loader_pack_example.json"])
def test_page_examples(name):
    g = load_golden(name)
    inp = g["input"]
    A = list(range(101, 101 + inp["real_len"][0]))
    Bt = list(range(201, 201 + inp["real_len"][1]))
    src, off, lens = _flat([A, Bt])
    out = oracle.pack(src, off, lens, inp["pad_to"], [0, 2], inp["capacity"],
                      fold=inp["fold"], pad_token=0)
    assert out["status"] == 0
    pr = g["printed"]
    assert list(out["packed"].shape) == pr["packed_shape"]
    assert out["cu_seqlens"].tolist() == pr["cu_seqlens"]
    assert out["cu_seqlens_padded"].tolist() == pr["cu_seqlens_padded"]
    row = out["packed"][0].tolist()
    # A, its pad, B, its pad (then the tail)
    assert row[0:5] == A and row[5:8] == [0] * 3 and row[8:18] == Bt
    ones = [list(x) for x in g["derived"]["token_mask_ones"]]
    want = np.zeros(inp["capacity"], dtype=np.uint8)
    for a, b in ones:
        want[a:b] = 1
    assert out["token_mask"][0].tolist() == want.tolist()
    if "tail_pad" in pr:
        assert row[20:] == [0] * pr["tail_pad"]
        assert int(out["token_mask"].sum()) == pr["real_tokens"]


def test_library_reduction_concatenation():
    rng = np.random.default_rng(7)
    sources = [rng.integers(0, 1000, size=int(n)).tolist() for n in rng.integers(0, 9, size=12)]
    src, off, lens = _flat(sources)
    C = int(lens.sum())
    out = oracle.pack(src, off, lens, 1, [0, len(sources)], max(C, 1), fold=False, pad_token=-7)
    assert out["status"] == 0
    assert out["packed"][0][:C].tolist() == np.concatenate([src]).tolist()
    ref_cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    assert out["cu_seqlens"].tolist() == ref_cu
    assert out["cu_seqlens_padded"].tolist() == ref_cu


def test_brute_force_small_packs():
    checked = 0
    for lens in itertools.product(range(0, 5), repeat=3):
        sources = [[10 * (i + 1) + j for j in range(n)] for i, n in enumerate(lens)]
        src, off, rl = _flat(sources)
        for q in (1, 2, 3, 4):
            padded = [-(-n // q) * q for n in lens]
            for split in range(0, 4):         # packs [0,split) and [split,3)
                starts = [0, split, 3] if 0 < split < 3 else [0, 3]
                for fold in (False, True):
                    need = max(sum(padded[a:b]) for a, b in zip(starts[:-1], starts[1:]))
                    for C in (need, need + 3):
                        if C == 0:
                            continue
                        out = oracle.pack(src, off, rl, q, starts, C, fold=fold, pad_token=-1)
                        assert out["status"] == 0
                        cu_l = oracle.pack_csr_slices(out["cu_seqlens"], starts)
                        cp_l = oracle.pack_csr_slices(out["cu_seqlens_padded"], starts)
                        for p in range(len(starts) - 1):
                            members = range(starts[p], starts[p + 1])
                            row, tm, cu, cp = list_formulation(sources, members, q, C, fold, -1)
                            assert out["packed"][p].tolist() == row
                            assert out["token_mask"][p].tolist() == tm
                            assert cu_l[p].tolist() == cu and cp_l[p].tolist() == cp
                        checked += 1
    assert checked > 2000


def test_pack_order_and_errors():
    sources = [[1, 2, 3], [4], [5, 6]]
    src, off, rl = _flat(sources)
    # pack 0 holds sources 2 then 0, pack 1 holds source 1 (q = 2: 2 + 4 and 2 slots)
    out = oracle.pack(src, off, rl, 2, [0, 2, 3], 6, fold=True, pad_token=0, order=[2, 0, 1])
    assert out["status"] == 0
    assert out["packed"][0].tolist() == [5, 6, 1, 2, 3, 0]
    assert out["packed"][1].tolist() == [4, 0, 0, 0, 0, 0]
    assert out["token_mask"][0].tolist() == [1, 1, 1, 1, 1, 0]
    assert out["cu_seqlens"].tolist() == [0, 2, 5, 0, 1]
    assert out["cu_seqlens_padded"].tolist() == [0, 2, 6, 0, 6]


def test_error_bits():
    sources = [[1, 2, 3], [4], [5, 6]]
    src, off, rl = _flat(sources)
    # 3 -> 4 slots plus 1 -> 2 slots exceeds 5
    assert oracle.pack(src, off, rl, 2, [0, 2, 3], 5)["status"] == oracle.PACK_OVERFLOW
    assert oracle.pack(src, off, rl, 2, [0, 0, 3], 8)["status"] == oracle.EMPTY_PACK
    assert oracle.pack(src, off, rl, 2, [0, 4], 8)["status"] == oracle.BAD_INDEX
    assert oracle.pack(src, off, rl, 2, [0, 3], 8, order=[0, 1, 3])["status"] == oracle.BAD_INDEX
    # a pack range reaching past the N member entries is out of range, even
    # where the caller's order buffer happens to hold more (valid) entries
    assert oracle.pack(src, off, rl, 2, [0, 4], 8, order=[0, 1, 2, 0])["status"] == oracle.BAD_INDEX
    bad = rl.copy()
    bad[1] = -2
    assert oracle.pack(src, off, bad, 2, [0, 3], 8)["status"] == oracle.BAD_LENGTH
    # source running past the end of the token buffer
    off2 = off.copy()
    off2[2] = 5
    assert oracle.pack(src, off2, rl, 2, [0, 3], 8)["status"] == oracle.BAD_INDEX


def test_workload_invariants():
    w = synth.pack_sources(N=4096)
    q, C = w["q"], w["capacity"]
    ps = w["pack_start"]
    out = oracle.pack(w["src"], w["src_off"], w["real_len"], q, ps, C, fold=True)
    assert out["status"] == 0
    P = ps.size - 1
    cu_l = oracle.pack_csr_slices(out["cu_seqlens"], ps)
    cp_l = oracle.pack_csr_slices(out["cu_seqlens_padded"], ps)
    rl = w["real_len"].astype(np.int64)
    for p in range(P):
        members = np.arange(ps[p], ps[p + 1])
        real = rl[members]
        assert int(out["token_mask"][p].sum()) == int(real.sum())
        assert cu_l[p][-1] == real.sum() and cp_l[p][-1] == C
        steps = np.diff(cp_l[p].astype(np.int64))
        assert np.all(steps[:-1] % q == 0) and np.all(steps >= real)
        # each source's tokens sit at its padded offset
        for j, i in enumerate(members):
            a = int(cp_l[p][j])
            got = out["packed"][p][a:a + int(rl[i])]
            assert np.array_equal(got, w["src"][w["src_off"][i]:w["src_off"][i] + rl[i]])


def test_trainer_rectangle_printed_example():
    # input_ids [2, 10] holding A (5 tokens) and B (10), bins [[0, 1]], q = 4:
    # packed [1, 20] = A, its pad, B, its pad; [0,5,15] and [0,8,20].
    g = load_golden("trainer_pack_example.json")
    inp = g["input"]
    rows = np.zeros((2, 10), dtype=np.int64)
    rows[0, :5] = np.arange(101, 106)
    rows[1, :10] = np.arange(201, 211)
    out = oracle.pack_rect(rows, inp["real_len"], inp["pad_to"], inp["bins"])
    assert out["status"] == 0
    pr = g["printed"]
    assert out["width"] == inp["capacity"]
    assert list(out["packed"].shape) == pr["packed_shape"]
    assert out["cu_seqlens"].tolist() == pr["cu_seqlens"]
    assert out["cu_seqlens_padded"].tolist() == pr["cu_seqlens_padded"]
    assert out["packed"][0].tolist() == list(range(101, 106)) + [0] * 3 + \
        list(range(201, 211)) + [0] * 2
    # the rectangle had 5 of its 20 slots as padding; the squeeze keeps 15 real
    assert int(out["token_mask"].sum()) == 15


def test_trainer_rectangle_concatenation():
    rng = np.random.default_rng(11)
    N, W = 9, 7
    rows = rng.integers(0, 1000, size=(N, W))
    lens = rng.integers(0, W + 1, size=N).astype(np.int32)
    out = oracle.pack_rect(rows, lens, 1, [list(range(N))])
    assert out["status"] == 0
    want = np.concatenate([rows[i, :lens[i]] for i in range(N)])
    assert out["width"] == want.size
    assert out["packed"][0].tolist() == want.tolist()
    assert out["cu_seqlens"].tolist() == out["cu_seqlens_padded"].tolist() == \
        np.concatenate([[0], np.cumsum(lens)]).tolist()


def test_trainer_rectangle_brute_force():
    checked = 0
    W = 4
    for lens in itertools.product(range(0, W + 1), repeat=3):
        rows = np.array([[10 * (i + 1) + j for j in range(W)] for i in range(3)])
        sources = [rows[i, :lens[i]].tolist() for i in range(3)]
        for q in (1, 3, 4):
            for bins in ([[0, 1, 2]], [[2, 0], [1]], [[1], [2], [0]], [[0, 2, 1]]):
                for fold in (False, True):
                    out = oracle.pack_rect(rows, list(lens), q, bins, fold=fold, pad_token=-5)
                    if out["width"] == 0:
                        continue
                    assert out["status"] == 0
                    C = out["width"]
                    starts = out["pack_start"]
                    cu_l = oracle.pack_csr_slices(out["cu_seqlens"], starts)
                    cp_l = oracle.pack_csr_slices(out["cu_seqlens_padded"], starts)
                    for p, members in enumerate(bins):
                        row, tm, cu, cp = list_formulation(sources, members, q, C, fold, -5)
                        assert out["packed"][p].tolist() == row
                        assert out["token_mask"][p].tolist() == tm
                        assert cu_l[p].tolist() == cu and cp_l[p].tolist() == cp
                    checked += 1
    assert checked > 800


def test_trainer_rectangle_length_beyond_row_is_rejected():
    rows = np.zeros((2, 4), dtype=np.int64)
    assert oracle.pack_rect(rows, [4, 5], 1, [[0, 1]], width=9)["status"] == oracle.BAD_LENGTH
    assert oracle.pack_rect(rows, [4, -1], 1, [[0, 1]], width=9)["status"] == oracle.BAD_LENGTH
    # every condition is reported: a too-long member (not counted toward the
    # pack's fill) together with an empty bin
    st = oracle.pack_rect(rows, [7, 3], 1, [[0, 1], []], width=3)["status"]
    assert st == oracle.BAD_LENGTH | oracle.EMPTY_PACK
