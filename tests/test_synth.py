"""Checks on the seeded input generators (CPU only)."""
import numpy as np

import oracle
import synth


def test_generators_are_seeded():
    assert np.array_equal(synth.doc_map_small(), synth.doc_map_small())
    assert not np.array_equal(synth.doc_map_small(1), synth.doc_map_small(11))
    a, b = synth.thd_tables(), synth.thd_tables()
    assert all(np.array_equal(a[k], b[k]) for k in ("seq_lens", "input_ids", "position_ids"))


def test_doc_map_small_shape_and_pad():
    d = synth.doc_map_small()
    assert d.shape == (4, 64) and d.dtype == np.int32
    for row in d:
        nz = np.flatnonzero(row == 0)
        if nz.size:                      # padding is one trailing run of at most 16
            assert nz[0] >= 64 - 16 and np.all(row[nz[0]:] == 0)
        assert row[0] == 1               # indices restart at 1 every row


def test_doc_map_medium_has_single_doc_row():
    d = synth.doc_map_medium()
    assert d.shape == (8, 4096)
    full = [r for r in range(8) if np.all(d[r] == 1)]
    assert len(full) == 1 and full[0] < 7


def test_thd_tables_fill_rule():
    w = synth.thd_tables()
    L, Lp, S = w["seq_lens"], w["seq_lens_padded"], w["S"]
    valid = L != -1000
    assert np.array_equal(valid, Lp != -1000)
    assert np.all(Lp[valid] % 8 == 0) and np.all(Lp[valid] >= L[valid])
    assert np.all((Lp * valid).sum(axis=1) <= S)
    for r in range(L.shape[0]):      # valid slots are a prefix of the row
        k = int(valid[r].sum())
        assert valid[r, :k].all() and not valid[r, k:].any()
    assert (w["input_ids"] == 0).sum() >= 0 and w["input_ids"].max() <= synth.TOKEN_HIGH


def test_next_fit_closure():
    w = synth.pack_sources(N=3000)
    q, C = w["q"], w["capacity"]
    padded = (w["real_len"].astype(np.int64) + q - 1) // q * q
    ps = w["pack_start"]
    assert ps[0] == 0 and ps[-1] == 3000 and np.all(np.diff(ps) > 0)
    for p in range(ps.size - 1):
        used = int(padded[ps[p]:ps[p + 1]].sum())
        assert used <= C
        if p + 1 < ps.size - 1:        # the next source would not have fitted
            assert used + int(padded[ps[p + 1]]) > C


def test_run_positions():
    d = np.array([[1, 1, 2, 0, 0], [1, 1, 1, 1, 0]])
    assert synth.run_positions(d).tolist() == [[0, 1, 0, 0, 1], [0, 1, 2, 3, 0]]


def test_token_budget_bins():
    padded = np.array([64, 128, 16384, 64, 8192, 8192, 192])
    bins, fill = synth.token_budget_bins(padded, 16384)
    flat = sorted(i for b in bins for i in b)
    assert flat == list(range(padded.size))
    assert all(int(padded[b].sum()) <= 16384 for b in bins)
    assert fill == [int(padded[b].sum()) for b in bins]
    assert bins[0] == [2]                     # the longest source opens the first bin
    w = synth.trainer_rectangle()
    rows, rl = w["rows"], w["real_len"]
    # the packer's width is the fullest bin's padded sum, as the oracle computes it
    assert w["width"] == oracle.trainer_width(rl, w["bins"], w["q"])
    assert rows.shape == (256, int(rl.max()))
    assert sorted(i for b in w["bins"] for i in b) == list(range(256))
    for i in range(0, 256, 17):               # zero past each length
        assert not rows[i, rl[i]:].any()


def test_pad_tail_stream():
    w = synth.pad_tail_stream()
    ids, pad, tail = w["input_ids"], w["pad_id"], w["tail"]
    assert ids.size == 131072 and pad > synth.TOKEN_HIGH
    assert np.all(ids[ids.size - tail:] == pad) and not np.any(ids[:ids.size - tail] == pad)


def _runs(row):
    """(value, length) of each maximal run of a row."""
    edges = np.flatnonzero(np.diff(row)) + 1
    starts = np.concatenate([[0], edges])
    ends = np.concatenate([edges, [row.size]])
    return [(int(row[a]), int(b - a)) for a, b in zip(starts, ends)]


def _check_doc_rows(d, max_doc, max_pad):
    for row in d:
        runs = _runs(row)
        pad = runs[-1][1] if runs[-1][0] == 0 else 0
        assert pad <= max_pad
        docs = runs[:-1] if pad else runs
        # indices restart at 1 and count up by one; only the last document may
        # be cut short by the row end, none is longer than the recipe allows
        assert [v for v, _ in docs] == list(range(1, len(docs) + 1))
        assert all(1 <= n <= max_doc for _, n in docs)


def test_recipes_match_the_configs():
    # config 1 and the stage map: documents of 1..24 tokens, a pad tail of 0..16
    _check_doc_rows(synth.doc_map_small(), 24, 16)
    st = synth.stage_embedding()
    _check_doc_rows(st["doc_ids"], 24, 16)
    assert st["doc_ids"].shape == (32, 32768)
    assert np.array_equal(st["position_ids"], synth.run_positions(st["doc_ids"]))
    # config 2: documents clipped to 1..4096, a pad tail of 0..512
    _check_doc_rows(synth.doc_map_medium(), 4096, 512)
    # config 3: real lengths 1..2048, padded exactly to the next multiple of 8,
    # at most 64 per row, tokens 0..151935
    w = synth.thd_tables()
    L, Lp = w["seq_lens"], w["seq_lens_padded"]
    valid = L != -1000
    assert L[valid].min() >= 1 and L[valid].max() <= 2048
    assert np.array_equal(Lp[valid], -(-L[valid] // 8) * 8)
    assert valid.sum(axis=1).max() <= 64
    assert w["input_ids"].shape == (16, 8192) and w["input_ids"].min() >= 0
    assert w["input_ids"].max() <= synth.TOKEN_HIGH == 151935
    # config 4: 65 536 sources of 1..8192 tokens, stored end to end
    p = synth.pack_sources()
    rl = p["real_len"]
    assert rl.size == 65536 and rl.min() >= 1 and rl.max() <= 8192
    assert np.array_equal(p["src_off"], np.concatenate([[0], np.cumsum(rl)[:-1]]))
    assert p["src"].size == int(rl.sum()) and p["src"].max() <= 151935
    assert p["capacity"] == 16384 and p["q"] == 64
