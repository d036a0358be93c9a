"""Seeded random sweeps of every entry point against the oracle.

Each test draws many random cases from one seed: shapes log-uniform over
several orders of magnitude (so the cases cross every kernel path and tile
size of the call), both index dtypes, and the input features each call
distinguishes (padding runs, holes and sentinels in length tables, empty
sources, member orders, pad tails and pad ids inside the content).  Every
case is compared element by element with the oracle through the same checks
as the hand-picked parity tests.  The case printed before each call names
it, so a failure can be rerun alone.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import test_gpu_next as nxt
import test_gpu_parity as par
from varlen_attention_metadata_amd import _lib

pytestmark = pytest.mark.gpu
V = -1000


@pytest.fixture(scope="module")
def dev():
    _lib.load()
    return torch.device("cuda:0")


def log_uniform(rng, lo, hi):
    return int(np.exp(rng.uniform(np.log(lo), np.log(hi + 1))))


def random_map(rng, B, S):
    kind = int(rng.integers(4))
    if kind == 0:                                   # a small alphabet: many boundaries
        return rng.integers(0, 3, size=(B, S))
    if kind == 1:                                   # one document per row
        return np.ones((B, S), dtype=np.int64)
    if kind == 2:                                   # mostly padding
        return np.where(rng.random((B, S)) < 0.8, 0, rng.integers(1, 4, size=(B, S)))
    mean = log_uniform(rng, 1, 5000)                # runs of random mean length
    d = np.empty((B, S), dtype=np.int64)
    for r in range(B):
        lens = rng.geometric(1.0 / mean, size=S // max(mean // 4, 1) + 8)
        ends = np.minimum(np.cumsum(lens), S)
        k = int(np.searchsorted(ends, S)) + 1
        ids = np.arange(1, k + 1)
        ids[rng.random(k) < 0.1] = 0
        d[r] = np.repeat(ids, np.diff(np.concatenate([[0], ends[:k]])))
    return d


def test_sweep_doc_maps(dev):
    rng = np.random.default_rng(101)
    for case in range(80):
        S = log_uniform(rng, 1, 70000)
        B = max(1, min(log_uniform(rng, 1, 64), 2_000_000 // S))
        d = random_map(rng, B, S)
        if rng.random() < 0.5:
            par.check_doc(dev, d.astype(np.int32), torch.int32)
        else:                                       # neighbours differ only in the high half
            par.check_doc(dev, np.where(d == 0, 0, d * (1 << 32) + 5), torch.int64)


def test_sweep_length_tables(dev):
    rng = np.random.default_rng(102)
    for case in range(80):
        P = log_uniform(rng, 1, 128)
        B = max(1, min(log_uniform(rng, 1, 128), 8192 // P))
        S = log_uniform(rng, 1, 20000)
        q = int(rng.choice([1, 4, 8, 64]))
        L, Lp = par.rand_tables(rng, B, P, S, q, tight=rng.random() < 0.3,
                                holes=rng.random() < 0.3,
                                maxlen=max(1, S // max(1, P // 4)) if rng.random() < 0.5 else None)
        dtype = torch.int32 if rng.random() < 0.5 else torch.int64
        par.check_thd(dev, L, None if rng.random() < 0.2 else Lp, S, dtype)


def test_sweep_row_groups(dev):
    rng = np.random.default_rng(103)
    for case in range(50):
        G = log_uniform(rng, 1, 80)
        Bc = log_uniform(rng, 1, 16)
        B = G * Bc
        P = max(1, min(log_uniform(rng, 1, 96), 8192 // B))
        S = log_uniform(rng, 1, 12000)
        q = int(rng.choice([1, 4, 8]))
        L, Lp = nxt.rand_tables(rng, B, P, S, q)
        dtype = torch.int32 if rng.random() < 0.5 else torch.int64
        nxt.check_split(dev, L, None if rng.random() < 0.2 else Lp, S, G, dtype)


def test_sweep_squeeze(dev):
    rng = np.random.default_rng(104)
    for case in range(50):
        q = int(rng.choice([1, 2, 8, 64]))
        hi = log_uniform(rng, 1, 6000)
        C = -(-hi // q) * q + log_uniform(rng, 1, 20000)
        N = min(log_uniform(rng, 1, 900), max(1, 4_000_000 // C))   # at most 4 M slots
        rl = rng.integers(0, hi + 1, size=N).astype(np.int32)
        rl[rng.random(N) < 0.05] = 0                 # empty sources
        off = np.concatenate([[0], np.cumsum(rl)[:-1]]).astype(np.int64)
        src = rng.integers(0, 151936, size=int(rl.sum()) + 1)
        padded = -(-rl.astype(np.int64) // q) * q
        order = None
        if rng.random() < 0.4:                       # members in a shuffled order
            order = rng.permutation(N).astype(np.int32)
            padded = padded[order]
        ps = synth.next_fit(padded, C)
        fold = bool(rng.random() < 0.5)
        pad_token = int(rng.choice([0, -1, 151935]))
        par.check_pack(dev, src, off, rl, q, ps, C, fold, pad_token, order,
                       what=f"sweep case {case}")


def test_sweep_pad_ids(dev):
    rng = np.random.default_rng(105)
    for case in range(60):
        T = log_uniform(rng, 1, 600000) - 1
        pad = int(rng.choice([0, 7, 151329]))
        ids = rng.integers(0, 151936, size=T)
        ids[ids == pad] = pad + 1
        tail = int(rng.integers(0, T + 1)) if rng.random() < 0.8 else 0
        ids[T - tail:] = pad
        if T > tail and rng.random() < 0.3:           # the pad id inside the content
            ids[int(rng.integers(0, T - tail))] = pad
        dtype = torch.int32 if rng.random() < 0.5 else torch.int64
        nxt.check_padids(dev, ids, pad, dtype, offset=int(rng.integers(0, 3)))


def test_sweep_trainer_rectangles(dev):
    rng = np.random.default_rng(106)
    for case in range(40):
        N = log_uniform(rng, 1, 64)
        W = log_uniform(rng, 1, 4000)
        q = int(rng.choice([1, 4, 64]))
        rl = rng.integers(0, W + 1, size=N).astype(np.int32)
        rows = rng.integers(0, 151936, size=(N, W))
        members = rng.permutation(N)[: int(rng.integers(1, N + 1))]
        n_bins = int(rng.integers(1, len(members) + 1))
        cuts = np.sort(rng.choice(np.arange(1, len(members)), size=n_bins - 1, replace=False)) \
            if n_bins > 1 else np.array([], dtype=np.int64)
        bins = [b.tolist() for b in np.split(members, cuts)]
        C = max(1, oracle.trainer_width(rl, bins, q))   # a row of at least one slot
        nxt.check_rect(dev, rows, rl, q, bins, C=C, fold=bool(rng.random() < 0.3))
