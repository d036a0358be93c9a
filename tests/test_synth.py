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
