"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every output is an integer or a byte copy, so every comparison is exact.
Cases cover the five workloads at full size, seeded fuzz across tile and
chunk boundaries, the degenerate shapes, the data-error bits, repeat-run
determinism (the cross-workgroup look-back), and the workspace contract.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import varlen_attention_metadata_amd as psq
from varlen_attention_metadata_amd import _lib

pytestmark = pytest.mark.gpu
V = -1000


def say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def dev():
    _lib.load()                       # fails loudly if the library is missing
    return torch.device("cuda:0")


# ---------------------------------------------------------------------------
# document maps
# ---------------------------------------------------------------------------

def run_doc(dev, doc_np, dtype=torch.int32, want_mask=True):
    """Raw C-ABI call: returns (cu[:n+1], n, max, mask, status)."""
    d = torch.from_numpy(np.ascontiguousarray(doc_np)).to(dev, dtype)
    B, S = doc_np.shape
    cu = torch.full((B * S + 1,), -7, dtype=torch.int32, device=dev)
    scal = torch.full((4,), -7, dtype=torch.int32, device=dev)
    mask = torch.full((max(B * S, 1),), 7, dtype=torch.uint8, device=dev)
    ws = psq.workspace_for(dev, _lib.psq_params_from_doc_ids_workspace(B, S))
    sp = scal.data_ptr()
    _lib.psq_params_from_doc_ids(d.data_ptr(), _lib.I32 if dtype == torch.int32 else _lib.I64,
                                 B, S, cu.data_ptr(), sp, sp + 4,
                                 mask.data_ptr() if want_mask else None, sp + 8,
                                 ws.data_ptr(), ws.numel(), torch.cuda.current_stream(dev).cuda_stream)
    n, mx, st, _ = scal.cpu().tolist()
    return cu[: n + 1].cpu().numpy(), n, mx, mask[: B * S].cpu().numpy(), st


def check_doc(dev, doc_np, dtype=torch.int32):
    say(f"doc map {doc_np.shape} {dtype}")
    cu, n, mx, mask, st = run_doc(dev, doc_np, dtype)
    ref = oracle.doc_segments(doc_np)
    assert st == 0
    assert n == ref["num_segments"]
    assert np.array_equal(cu, ref["cu_seqlens"]), "cu_seqlens differ"
    assert mx == ref["max_seqlen"]
    assert np.array_equal(mask, ref["padding_mask"])


@pytest.mark.parametrize("gen", [synth.doc_map_small, synth.doc_map_medium])
def test_doc_workloads(dev, gen):
    check_doc(dev, gen())


def test_doc_stage_embedding_map(dev):
    check_doc(dev, synth.stage_embedding()["doc_ids"])


def test_doc_page_examples(dev):
    for m in ([[1, 1, 2, 2, 2, 0]], [[1, 1, 1], [1, 1, 0]], [[1, 0, 0, 0]], [[1, 2, 1]]):
        check_doc(dev, np.array(m, dtype=np.int32))


@pytest.mark.parametrize("B,S", [(0, 5), (3, 0), (1, 1), (5, 1), (1, 2), (2, 3), (3, 4),
                                 (1, 5), (2, 63), (3, 64), (2, 65), (1, 255), (4, 256),
                                 (3, 1000), (2, 4095), (1, 4096), (2, 4097), (3, 8191),
                                 (1, 12289), (2, 50000), (7, 3333), (4097, 1), (16384, 2),
                                 (1, 32767), (1, 32768), (1, 32769), (8, 4096)])
@pytest.mark.parametrize("kind", ["alphabet3", "runs", "const", "pad_heavy"])
def test_doc_fuzz(dev, B, S, kind):
    rng = np.random.default_rng(hash((B, S, kind)) % 2**32)
    if kind == "alphabet3":
        d = rng.integers(0, 3, size=(B, S))
    elif kind == "const":
        d = np.ones((B, S), dtype=np.int64)          # only row starts are boundaries
    elif kind == "pad_heavy":
        d = np.where(rng.random((B, S)) < 0.8, 0, rng.integers(1, 4, size=(B, S)))
    else:
        d = np.zeros((B, S), dtype=np.int64)
        for r in range(B):
            t, idx = 0, 1
            while t < S:
                n = int(rng.geometric(1 / 300))
                d[r, t:t + n] = idx if rng.random() > 0.1 else 0
                t += n
                idx += 1
    check_doc(dev, d.astype(np.int32), torch.int32)
    if B * S <= 20000:
        # values that differ only in their upper 32 bits
        check_doc(dev, d.astype(np.int64) * (1 << 32) + 7, torch.int64)


def _long_runs(rng, B, S, mean):
    """Rows of runs with geometric lengths of the given mean, a tenth of them
    padding; built with vector operations (the maps here hold millions of
    positions)."""
    d = np.empty((B, S), dtype=np.int32)
    for r in range(B):
        lens = rng.geometric(1.0 / mean, size=S // max(int(mean) // 4, 1) + 8)
        ends = np.cumsum(lens)
        k = int(np.searchsorted(ends, S)) + 1
        ids = np.arange(1, k + 1, dtype=np.int32)
        ids[rng.random(k) < 0.1] = 0
        d[r] = np.repeat(ids, np.diff(np.concatenate([[0], np.minimum(ends[:k], S)])))
    return d


@pytest.mark.parametrize("B,S", [(1, 4096 * 1024 + 1), (3, 2100000), (2, 4200000),
                                 (1, 3 * 4096 * 1024 + 7)])
@pytest.mark.parametrize("kind", ["runs", "long_runs", "const", "two_then_one"])
def test_doc_many_chunks_per_workgroup(dev, B, S, kind):
    """Maps of more than 1024 chunks of 4096 positions: each workgroup of the
    two launches walks several chunks, and segments cross workgroups."""
    rng = np.random.default_rng(S * 7 + B)
    if kind == "runs":
        d = _long_runs(rng, B, S, 300)
    elif kind == "long_runs":
        d = _long_runs(rng, B, S, 60000)       # most workgroups hold no boundary
    elif kind == "const":
        d = np.ones((B, S), dtype=np.int32)     # one segment per row
    else:
        d = np.full((B, S), 2, dtype=np.int32)  # every boundary in the first chunk of a row
        d[:, 0] = 1
    check_doc(dev, d)


@pytest.mark.parametrize("B,S", [(3, 300001), (2, 1000000), (1, 4194304), (1, 4194305),
                                 (3, 2100000)],
                         ids=["one_launch_4", "one_launch_8", "one_launch_16", "two_launch",
                              "two_launch_rows"])
def test_doc_int64_maps_on_every_path(dev, B, S):
    """int64 maps large enough for the one-launch kernel at 4096, 8192 and
    16384 positions per tile and for the two launches; neighbouring ids
    differ only in their upper 32 bits, and padding (0) stays 0."""
    rng = np.random.default_rng(B * 1000003 + S)
    d = _long_runs(rng, B, S, 300).astype(np.int64)
    d = np.where(d == 0, 0, d * (1 << 32) + 7)
    check_doc(dev, d, torch.int64)


def test_doc_one_launch_sequence(dev):
    """Maps of up to 256 chunks of 16384 positions take one launch, over the
    smallest tiles (1024 to 16384 positions) that need at most 256 of them,
    whose workgroups publish tagged records; the tags of a call must never
    be taken for those of a later one.  The sequence changes the tile
    count and size up and down on one workspace (256 tiles, then 32, then 256
    again reuses tiles 32..255 with the first call's parity; 64, 65, 128 and
    129 tiles put the last record at either side of a wave's slice), with
    two-launch maps and one-chunk maps in between."""
    shapes = [(32, 32768), (8, 4096), (32, 32768), (2, 4097), (1, 64 * 4096 - 1),
              (7, 9000), (1, 65 * 4096), (129, 4096), (4, 64), (64, 4096), (3, 4096),
              (128, 4096), (1, 257 * 4096 - 3), (1, 256 * 4096), (16, 16384), (1, 8193),
              (255, 4096), (16, 4096), (1, 65537), (32, 4096), (1, 131073), (1, 262145),
              (1, 524289), (1, 2000), (1, (1 << 22) + 1), (2, 1 << 20), (32, 32768)]
    for i, (B, S) in enumerate(shapes):
        rng = np.random.default_rng(100 + i)
        d = _long_runs(rng, B, S, [3, 300, 5000][i % 3]) if B * S > 64 else \
            rng.integers(0, 3, size=(B, S)).astype(np.int32)
        check_doc(dev, d)


@pytest.mark.parametrize("total", [1024, 1025, 2048, 2049, 4096, 4097, 65536, 65537, 131072,
                                   131073, 262144, 262145, 524288, 524289, 1048576, 1048577,
                                   2097152, 2097153, 4194304, 4194305])
def test_doc_tile_size_boundaries(dev, total):
    """Each side of every change of tile size and path: one chunk of 1024,
    2048 or 4096 positions, one launch over up to 256 tiles of 1024, 2048,
    4096, 8192 or 16384 positions, then two launches.  Each total runs as
    one row and as several rows (its smallest divisor above 1, when it has
    one), so row starts fall inside tiles."""
    rows = [1] + [r for r in range(2, 64) if total % r == 0][:1]
    for B in rows:
        S = total // B
        rng = np.random.default_rng(total * 3 + B)
        check_doc(dev, _long_runs(rng, B, S, 40))
        check_doc(dev, rng.integers(0, 3, size=(B, S)).astype(np.int32))


@pytest.mark.parametrize("B,S", [(3, 1000), (8, 4096), (3, 300001), (1, 4194304), (3, 2100000)],
                         ids=["one_workgroup", "one_launch_1", "one_launch_4", "one_launch_16",
                              "two_launch"])
@pytest.mark.parametrize("dtype", [torch.int32, torch.int64])
def test_doc_unaligned_input(dev, B, S, dtype):
    """A map view one element into its storage (not 16-byte aligned: the
    scalar-load path) and a mask one byte in (not 4-byte aligned: byte
    stores), on every kernel path."""
    rng = np.random.default_rng(B * 7 + S)
    d = _long_runs(rng, B, S, 300) if B * S > 100000 else synth.doc_map_medium(2, B, S)
    np_dt = np.int32 if dtype == torch.int32 else np.int64
    base = torch.from_numpy(np.concatenate([[9], d.reshape(-1)]).astype(np_dt)).to(dev)
    view = base[1:].view(d.shape)
    assert view.data_ptr() % 16 != 0
    cu = torch.empty(B * S + 1, dtype=torch.int32, device=dev)
    scal = torch.empty(4, dtype=torch.int32, device=dev)
    mask = torch.empty(B * S + 1, dtype=torch.uint8, device=dev)[1:]   # unaligned mask too
    ws = psq.workspace_for(dev, _lib.psq_params_from_doc_ids_workspace(B, S))
    sp = scal.data_ptr()
    say(f"doc map unaligned {B}x{S} {dtype}")
    _lib.psq_params_from_doc_ids(view.data_ptr(), _lib.I32 if dtype == torch.int32 else _lib.I64,
                                 B, S, cu.data_ptr(), sp, sp + 4, mask.data_ptr(), sp + 8,
                                 ws.data_ptr(), ws.numel(),
                                 torch.cuda.current_stream(dev).cuda_stream)
    n, mx, st, _ = scal.cpu().tolist()
    ref = oracle.doc_segments(d)
    assert st == 0 and n == ref["num_segments"] and mx == ref["max_seqlen"]
    assert np.array_equal(cu[: n + 1].cpu().numpy(), ref["cu_seqlens"])
    assert np.array_equal(mask.cpu().numpy(), ref["padding_mask"])


def test_doc_repeat_determinism(dev):
    d = synth.stage_embedding()["doc_ids"]
    first = run_doc(dev, d)
    for i in range(20):
        again = run_doc(dev, d)
        assert np.array_equal(first[0], again[0]) and first[1:3] == again[1:3], i


def test_doc_python_api(dev):
    d = synth.doc_map_medium()
    t = torch.from_numpy(d).to(dev)
    p = psq.packed_seq_params_from_doc_ids(t)
    ref = oracle.doc_segments(d)
    assert p.doc_ids is t
    assert p.cu_seqlens.dtype == torch.int32
    assert np.array_equal(p.cu_seqlens.cpu().numpy(), ref["cu_seqlens"])
    assert p.max_seqlen == ref["max_seqlen"]
    kw = psq.to_flash_attention_kwargs(p)
    assert kw["cu_seq_lens_q"] is kw["cu_seq_lens_k"] is p.cu_seqlens
    assert kw["max_length_q"] == kw["max_length_k"] == p.max_seqlen


DOC_RECORDS = (256, 49664)     # the document-map region: records and one-launch state


def _nonzero_outside(ws, lo, hi):
    torch.cuda.synchronize()
    w = ws.clone()
    w[lo:hi] = 0
    return int(w.count_nonzero())


def test_workspace_left_zeroed(dev):
    """The parts of the shared workspace that calls rely on finding zero stay
    zero; the document-map calls write only into their record region (which
    still holds the records of earlier, larger maps of this process)."""
    d = synth.doc_map_medium()
    run_doc(dev, d)
    ws = psq.workspace_for(dev, 0)
    assert _nonzero_outside(ws, *DOC_RECORDS) == 0
    L = torch.tensor([[3, 2], [6, V]], device=dev)
    psq.process_input_for_thd({"input_ids": torch.zeros((2, 6), dtype=torch.int64, device=dev),
                               "position_ids": torch.zeros((2, 6), dtype=torch.int64, device=dev),
                               "seq_lens": L})
    assert _nonzero_outside(psq.workspace_for(dev, 0), *DOC_RECORDS) == 0


def test_doc_records_do_not_disturb_tables(dev):
    """A multi-workgroup table call (look-back descriptors after the record
    region) on the workspace a large document map has just used."""
    run_doc(dev, synth.stage_embedding()["doc_ids"])
    rng = np.random.default_rng(11)
    B, P, S = 1100, 4, 64
    L = rng.integers(0, 9, size=(B, P)).astype(np.int64)
    Lp = L + 8 - L % 8
    Lp[:, 3] = V
    L[:, 3] = V
    say("tables 1100x4 after a document map")
    got = run_thd_raw(dev, L, Lp, S)
    ref = oracle.thd_tables(L, Lp, S)
    assert got["status"] == 0
    for k in ("cu_seqlens", "cu_seqlens_padded", "padding_mask"):
        assert np.array_equal(got[k], ref[k]), k
    assert got["max_seqlen"] == ref["max_seqlen"]
    assert _nonzero_outside(psq.workspace_for(dev, 0), *DOC_RECORDS) == 0


# ---------------------------------------------------------------------------
# length tables (THD)
# ---------------------------------------------------------------------------

def run_thd_raw(dev, L, Lp, S, dtype=torch.int64, copies=()):
    """Raw C-ABI call on tables; returns a dict like the oracle's."""
    B, P = L.shape
    tL = torch.from_numpy(np.ascontiguousarray(L)).to(dev, dtype)
    tLp = torch.from_numpy(np.ascontiguousarray(Lp)).to(dev, dtype) if Lp is not None else None
    cap = B * P + 1
    cu = torch.full((cap,), -7, dtype=torch.int32, device=dev)
    cp = torch.full((cap,), -7, dtype=torch.int32, device=dev)
    mask = torch.full((max(B * S, 1),), 7, dtype=torch.uint8, device=dev)
    scal = torch.full((4,), -7, dtype=torch.int32, device=dev)
    lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, tL.data_ptr(),
                           tLp.data_ptr() if tLp is not None else None,
                           _lib.I64 if dtype == torch.int64 else _lib.I32, P, V)
    ws = psq.workspace_for(dev, _lib.psq_process_thd_workspace(lay, B, S))
    arr, n_c = _lib.make_copies(list(copies))
    sp = scal.data_ptr()
    _lib.psq_process_thd(lay, B, S, cu.data_ptr(), cp.data_ptr(), sp, sp + 4, sp + 8,
                         mask.data_ptr(), arr, n_c, sp + 12, ws.data_ptr(), ws.numel(),
                         torch.cuda.current_stream(dev).cuda_stream)
    n, mx, pb, st = scal.cpu().tolist()
    if st != 0:
        return {"status": st}
    return {"status": 0, "cu_seqlens": cu[: n + 1].cpu().numpy(),
            "cu_seqlens_padded": cp[: n + 1].cpu().numpy(), "num_seqs": n, "max_seqlen": mx,
            "pad_between_seqs": pb, "padding_mask": mask[: B * S].cpu().numpy()}


def check_thd(dev, L, Lp, S, dtype=torch.int64):
    say(f"thd tables {L.shape} S={S} padded={Lp is not None} {dtype}")
    got = run_thd_raw(dev, L, Lp, S, dtype)
    ref = oracle.thd_tables(L, Lp, S)
    assert got["status"] == ref["status"]
    if ref["status"] != 0:
        return
    for key in ("cu_seqlens", "cu_seqlens_padded", "padding_mask"):
        assert np.array_equal(got[key], ref[key]), key
    for key in ("num_seqs", "max_seqlen", "pad_between_seqs"):
        assert got[key] == ref[key], key


def test_thd_page_example(dev):
    check_thd(dev, np.array([[3, 2], [6, V]]), np.array([[4, 2], [6, V]]), 6)


@pytest.mark.parametrize("L,Lp,S", [
    ([[3, 2], [6, V]], [[4, 2], [6, V]], 8),
    ([[3, 2]], [[3, 2]], 8),
    ([[3], [4]], [[3], [4]], 4),
    ([[0, 3]], [[0, 4]], 4),
    ([[3, 2], [6, V]], None, 6),
    ([[2, V, 3]], [[2, V, 3]], 9),            # a hole in the middle of a row
])
def test_thd_hand_cases(dev, L, Lp, S):
    check_thd(dev, np.array(L), None if Lp is None else np.array(Lp), S)


# Empty tables and rows of no length (they take the multi-workgroup kernel):
# no rows at all; rows without a slot (EMPTY_ROW); rows of length 0 holding
# empty sequences; a token in a row of length 0 (ROW_OVERFLOW).
@pytest.mark.parametrize("L,S", [
    (np.zeros((0, 3), np.int64), 8),
    (np.zeros((0, 100), np.int64), 8),
    (np.zeros((2, 0), np.int64), 8),
    (np.zeros((100, 0), np.int64), 8),
    (np.array([[0]]), 0),
    (np.array([[0, V], [0, 0]]), 0),
    (np.array([[1]]), 0),
], ids=["no_rows", "no_rows_wide", "no_slots", "no_slots_many_rows", "zero_length_row",
        "zero_length_rows", "token_in_zero_length_row"])
@pytest.mark.parametrize("dtype", [torch.int64, torch.int32])
def test_thd_degenerate_shapes(dev, L, S, dtype):
    check_thd(dev, L, None, S, dtype)
    check_thd(dev, L, L.copy(), S, dtype)


@pytest.mark.parametrize("S", [(1 << 25) - 1, 1 << 25, (1 << 25) + 7])
@pytest.mark.parametrize("dtype", [torch.int64, torch.int32])
def test_thd_rows_long_rows(dev, S, dtype):
    """Small tables (one wave per row) with rows on either side of 2^25
    positions: below it the row scans are plain sums, from it on they
    saturate; both must give the oracle's outputs and status bits."""
    rng = np.random.default_rng(S)
    lens = rng.integers(1, 1 << 19, size=60)
    L = np.full((3, 64), V, dtype=np.int64)
    Lp = np.full((3, 64), V, dtype=np.int64)
    L[0, :60] = lens
    Lp[0, :60] = lens + rng.integers(0, 5, size=60)
    L[1, :2], Lp[1, :2] = [S - 100, 40], [S - 100, 60]       # padded sum S - 40
    L[2, 0], Lp[2, 0] = S, S                                 # one full row
    check_thd(dev, L, Lp, S, dtype)
    # a padded sum of S + 1, and a length beyond the row: ROW_OVERFLOW
    check_thd(dev, np.array([[S, 1]]), np.array([[S, 1]]), S, dtype)
    check_thd(dev, np.array([[S + 5, V]]), np.array([[S + 5, V]]), S, dtype)


@pytest.mark.parametrize("L,Lp,S", [
    ([[3, V]], [[3, 2]], 8),
    ([[3, 2]], [[3, V]], 8),
    ([[5]], [[4]], 8),
    ([[-1]], [[2]], 8),
    ([[V, V], [2, V]], [[V, V], [2, V]], 8),
    ([[4, 4]], [[5, 4]], 8),
    ([[4]], [[2**62]], 8),
    ([[5], [V]], [[4], [V]], 8),
])
@pytest.mark.parametrize("wide", [False, True])
def test_thd_error_bits(dev, L, Lp, S, wide):
    L, Lp = np.array(L), np.array(Lp)
    if wide:
        # sentinel columns change nothing but take the table past the
        # single-workgroup size, so the multi-workgroup kernel decides
        extra = np.full((L.shape[0], 4200), V)
        L, Lp = np.hstack([L, extra]), np.hstack([Lp, extra])
    check_thd(dev, L, Lp, S)


# tables on either side of the single-workgroup limit (4096 entries)
@pytest.mark.parametrize("B,P,S", [(64, 64, 300), (65, 64, 300), (1, 4096, 5000), (1, 4097, 5000),
                                   (512, 1, 7), (1024, 4, 40), (1025, 4, 40)])
def test_thd_single_workgroup_limits(dev, B, P, S):
    rng = np.random.default_rng(B * 10007 + P)
    L, Lp = rand_tables(rng, B, P, S, 4, maxlen=max(1, S // max(1, P // 4)))
    check_thd(dev, L, Lp, S)
    check_thd(dev, L, None, S)


def rand_tables(rng, B, P, S, q, tight=False, holes=False, zero_frac=0.1, maxlen=None):
    L = np.full((B, P), V, dtype=np.int64)
    Lp = np.full((B, P), V, dtype=np.int64)
    maxlen = maxlen or max(1, S // 3)
    for r in range(B):
        used, j = 0, 0
        slots = rng.permutation(P) if holes else np.arange(P)
        order = sorted(slots[: rng.integers(1, P + 1)])
        for j in order:
            real = 0 if rng.random() < zero_frac else int(rng.integers(1, maxlen + 1))
            padded = real if tight else -(-real // q) * q + int(rng.integers(0, 2)) * q
            if used + padded > S:
                break
            L[r, j], Lp[r, j] = real, padded
            used += padded
        if not (L[r] != V).any():
            L[r, order[0]], Lp[r, order[0]] = 0, 0
    return L, Lp


@pytest.mark.parametrize("B,P,S", [(1, 1, 1), (1, 4, 7), (3, 5, 16), (2, 8, 4096),
                                   (3, 16, 4097), (2, 64, 8192), (4, 7, 12345),
                                   (1, 2000, 30000), (1, 3000, 9000), (2, 3000, 9000)])
@pytest.mark.parametrize("mode", ["plain", "tight", "holes", "nopad", "int32"])
def test_thd_fuzz(dev, B, P, S, mode):
    rng = np.random.default_rng(hash((B, P, S, mode)) % 2**32)
    q = int(rng.choice([1, 4, 8]))
    L, Lp = rand_tables(rng, B, P, S, q, tight=(mode == "tight"), holes=(mode == "holes"),
                        maxlen=(8 if P > 1000 else None))
    if mode == "nopad":
        check_thd(dev, L, None, S)
    else:
        check_thd(dev, L, Lp, S, torch.int32 if mode == "int32" else torch.int64)


def corrupt_tables(rng, L, Lp, S, n_bad):
    """Plant n_bad random faults in copies of valid tables: a sentinel in one
    table only, a negative length, real > padded, a row overflow, an emptied
    row, or a length far above S."""
    L, Lp = L.copy(), Lp.copy()
    B, P = L.shape
    for _ in range(n_bad):
        r, j = int(rng.integers(B)), int(rng.integers(P))
        kind = int(rng.integers(6))
        if kind == 0:
            (L if rng.random() < 0.5 else Lp)[r, j] = V
        elif kind == 1:
            L[r, j], Lp[r, j] = -int(rng.integers(1, 5)), max(int(Lp[r, j]), 0)
        elif kind == 2:
            L[r, j] = max(int(Lp[r, j]), 0) + int(rng.integers(1, 5))
            Lp[r, j] = max(int(Lp[r, j]), 0)
        elif kind == 3:
            L[r, j], Lp[r, j] = 1, S
        elif kind == 4:
            L[r, :], Lp[r, :] = V, V
        else:
            L[r, j], Lp[r, j] = 1, 2**40
    return L, Lp


# every fault, alone or combined, must give the oracle's status word exactly,
# on the single-workgroup kernel and (with sentinel columns) the multi-workgroup one
@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("wide", [False, True])
def test_thd_fault_fuzz(dev, seed, wide):
    rng = np.random.default_rng(1000 + seed)
    B, P, S = int(rng.integers(1, 9)), int(rng.integers(1, 9)), int(rng.integers(4, 64))
    L, Lp = rand_tables(rng, B, P, S, 4)
    L, Lp = corrupt_tables(rng, L, Lp, S, int(rng.integers(1, 4)))
    if wide:
        extra = np.full((B, 4200), V)
        L, Lp = np.hstack([L, extra]), np.hstack([Lp, extra])
    check_thd(dev, L, Lp, S)
    check_thd(dev, L, Lp, S, torch.int32 if np.abs(np.concatenate([L, Lp])).max() < 2**31 else torch.int64)


def test_thd_full_rows_absorb(dev):
    # every row fully tight except the very last sequence: absorption fires
    L = np.array([[100, 28], [64, 50]])
    Lp = np.array([[100, 28], [64, 64]])
    check_thd(dev, L, Lp, 128)


def test_thd_workload_with_copies(dev):
    w = synth.thd_tables()
    S = w["S"]
    B = w["seq_lens"].shape[0]
    say("thd workload 3 via process_input_for_thd")
    batch = {k: torch.from_numpy(w[k]).to(dev) for k in
             ("input_ids", "labels", "position_ids", "seq_lens", "seq_lens_padded")}
    batch["qkv_format"] = "thd"
    out = psq.process_input_for_thd(batch)
    ref = oracle.thd_tables(w["seq_lens"], w["seq_lens_padded"], S)
    assert ref["status"] == 0
    assert np.array_equal(out["cu_seqlens"].cpu().numpy(), ref["cu_seqlens"])
    assert np.array_equal(out["cu_seqlens_padded"].cpu().numpy(), ref["cu_seqlens_padded"])
    assert int(out["max_seqlen"]) == ref["max_seqlen"]
    assert out["max_seqlen"].dtype == torch.int32 and out["max_seqlen"].dim() == 0
    assert out["pad_between_seqs"] == bool(ref["pad_between_seqs"])
    assert np.array_equal(out["padding_mask"].cpu().numpy().astype(np.uint8), ref["padding_mask"])
    assert out["qkv_format"] == "thd"
    for key in ("input_ids", "labels", "position_ids"):
        want = oracle.copy_rows(w[key], 1, w[key].nbytes, w[key].nbytes)
        got = out[key].cpu().numpy()
        assert got.shape == (B * S,)
        assert got.tobytes() == want.tobytes(), key


def test_thd_embeddings_mrope_and_strided(dev):
    rng = np.random.default_rng(11)
    B, S, H, n_rope = 3, 40, 24, 3
    emb = torch.randn((B, S, H), dtype=torch.bfloat16, device=dev)
    pos = torch.from_numpy(rng.integers(0, 50, size=(n_rope, B, S))).to(dev)
    wide = torch.from_numpy(rng.integers(0, 9, size=(B, S + 5))).to(dev)
    labels = wide[:, :S]                                  # row-strided view
    L = torch.tensor([[10, 20], [40, V], [5, V]], device=dev)
    say("thd embeddings + mRoPE + strided labels")
    out = psq.process_input_for_thd({"input_ids": emb, "labels": labels, "position_ids": pos,
                                     "seq_lens": L})
    assert out["input_ids"].shape == (B * S, H)
    assert torch.equal(out["input_ids"].view(torch.int16), emb.reshape(B * S, H).view(torch.int16))
    assert out["position_ids"].shape == (n_rope, 1, B * S)
    assert torch.equal(out["position_ids"], pos.reshape(n_rope, 1, B * S))
    got = out["labels"].cpu().numpy()
    want = oracle.copy_rows(wide.cpu().numpy(), B, S * 8, (S + 5) * 8)
    assert got.tobytes() == want.tobytes()
    assert "cu_seqlens_padded" not in out
    ref = oracle.thd_tables(L.cpu().numpy(), None, S)
    assert np.array_equal(out["cu_seqlens"].cpu().numpy(), ref["cu_seqlens"])


# One copy of each kind the planner tells apart: unit size 16/8/4/1 bytes,
# dense or strided rows (a strided destination too), ragged unit counts.
# (byte offset from 16-byte alignment, rows, row_bytes, src stride, dst stride)
COPY_SPECS = [(0, 1, 16 * 1000, 16 * 1000, 0), (0, 37, 48, 80, 0),
              (8, 1, 8 * 777, 8 * 777, 0), (8, 5, 24, 40, 0),
              (4, 1, 4 * 999, 4 * 999, 0), (4, 9, 12, 20, 16),
              (1, 1, 1001, 1001, 0), (1, 13, 7, 11, 9)]


@pytest.mark.parametrize("path", ["small_tables", "large_tables", "doc_map", "split"])
def test_copy_kinds_on_every_path(dev, path):
    """Every copy kind in one call, on each launch that carries copies: the
    16-byte dense copy fused into the single-workgroup table kernel, into
    the multi-workgroup table kernel, or launched alone after a document
    map, and the split.  The whole destination buffer is compared, so a
    write outside a copy's rows would show."""
    rng = np.random.default_rng(17)
    placed, s_cur, d_cur = [], 0, 0
    for off, rows, rb, ss, ds in COPY_SPECS:
        s0 = -(-s_cur // 16) * 16 + off
        d0 = -(-d_cur // 16) * 16 + off
        dstep = ds if ds else rb
        placed.append((s0, d0, rows, rb, ss, ds))
        s_cur = s0 + (rows - 1) * ss + rb + 32
        d_cur = d0 + (rows - 1) * dstep + rb + 32
    src_np = rng.integers(0, 256, size=s_cur, dtype=np.uint8)
    src = torch.from_numpy(src_np).to(dev)
    dst = torch.full((d_cur,), 0xA5, dtype=torch.uint8, device=dev)
    want = np.full(d_cur, 0xA5, dtype=np.uint8)
    descs = []
    for s0, d0, rows, rb, ss, ds in placed:
        descs.append((src.data_ptr() + s0, dst.data_ptr() + d0, rows, rb, ss, ds))
        dense = oracle.copy_rows(src_np[s0:], rows, rb, ss).reshape(rows, rb)
        step = ds if ds else rb
        for r in range(rows):
            want[d0 + r * step: d0 + r * step + rb] = dense[r]
    arr, n_c = _lib.make_copies(descs)
    assert n_c == _lib.MAX_COPIES
    say(f"copy kinds on the {path} path")
    scal = torch.full((8,), -7, dtype=torch.int32, device=dev)
    sp = scal.data_ptr()
    stream = torch.cuda.current_stream(dev).cuda_stream
    if path == "doc_map":
        doc = torch.ones((2, 64), dtype=torch.int32, device=dev)
        lay = _lib.make_layout(_lib.LAYOUT_DOC_IDS, doc_ids=doc.data_ptr())
        B, S, P = 2, 64, 0
    else:
        B, P = (2, 1) if path != "large_tables" else (1, 5000)
        S = 64
        L = np.full((B, P), V, dtype=np.int64)
        L[:, 0] = S
        tL = torch.from_numpy(L).to(dev)
        lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, tL.data_ptr(), None, _lib.I64, P, V)
    cu = torch.empty(max(B * max(P, S), 1) + 4, dtype=torch.int32, device=dev)
    mask = torch.empty(B * S, dtype=torch.uint8, device=dev)
    if path == "split":
        G = 2
        per = torch.empty((3, G), dtype=torch.int32, device=dev)
        pp = per.data_ptr()
        ws = psq.workspace_for(dev, _lib.psq_split_thd_workspace(lay, B, S, G))
        _lib.psq_split_thd(lay, B, S, G, cu.data_ptr(), None, sp, pp, pp + 4 * G, pp + 8 * G,
                           mask.data_ptr(), arr, n_c, sp + 4, ws.data_ptr(), ws.numel(), stream)
        status = int(scal[1].item())
    else:
        ws = psq.workspace_for(dev, _lib.psq_process_thd_workspace(lay, B, S))
        _lib.psq_process_thd(lay, B, S, cu.data_ptr(), None, sp, sp + 4, sp + 8,
                             mask.data_ptr(), arr, n_c, sp + 12, ws.data_ptr(), ws.numel(),
                             stream)
        status = int(scal[3].item())
    assert status == 0
    assert np.array_equal(dst.cpu().numpy(), want)


def test_stage_embedding_full(dev):
    """Workload 5 at full size: doc-map layout, bf16 hidden [32,32768,4096]."""
    w = synth.stage_embedding()
    B, S, H = 32, 32768, 4096
    say("workload 5 full size")
    hidden = synth.stage_hidden(5, B, S, H, dev)
    doc = torch.from_numpy(w["doc_ids"]).to(dev)
    pos = torch.from_numpy(w["position_ids"]).to(dev)
    out = psq.process_input_for_thd({"input_ids": hidden, "position_ids": pos, "doc_ids": doc})
    ref = oracle.doc_segments(w["doc_ids"])
    assert np.array_equal(out["cu_seqlens"].cpu().numpy(), ref["cu_seqlens"])
    assert int(out["max_seqlen"]) == ref["max_seqlen"]
    assert out["pad_between_seqs"] is False
    assert np.array_equal(out["padding_mask"].cpu().numpy().astype(np.uint8), ref["padding_mask"])
    flat = out["input_ids"]
    assert flat.shape == (B * S, H)
    # identity at full size, checked on the device ...
    assert torch.equal(flat.view(torch.int16), hidden.reshape(B * S, H).view(torch.int16))
    assert torch.equal(out["position_ids"], pos.reshape(-1))
    # ... and sampled token rows through the oracle's copy
    rng = np.random.default_rng(5)
    for t in rng.integers(0, B * S, size=16).tolist() + [0, B * S - 1]:
        src = hidden.reshape(B * S, H)[t].view(torch.int16).cpu().numpy()
        want = oracle.copy_rows(src, 1, H * 2, H * 2)
        assert flat[t].view(torch.int16).cpu().numpy().tobytes() == want.tobytes()
    del hidden, flat, out
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# the squeeze into packs
# ---------------------------------------------------------------------------

def run_pack_raw(dev, src, off, rl, q, ps, C, fold, pad_token=0, order=None):
    N = len(rl)
    P = len(ps) - 1
    t_src = torch.from_numpy(np.ascontiguousarray(src, dtype=np.int64)).to(dev) if len(src) else \
        torch.zeros(1, dtype=torch.int64, device=dev)
    t_off = torch.from_numpy(np.ascontiguousarray(off, dtype=np.int64)).to(dev)
    t_rl = torch.from_numpy(np.ascontiguousarray(rl, dtype=np.int32)).to(dev)
    t_ps = torch.from_numpy(np.ascontiguousarray(ps, dtype=np.int64)).to(dev)
    t_od = torch.from_numpy(np.ascontiguousarray(order, dtype=np.int32)).to(dev) if order is not None else None
    packed = torch.full((max(P, 1), C), -5, dtype=torch.int64, device=dev)
    tm = torch.full((max(P, 1), C), 9, dtype=torch.uint8, device=dev)
    csr = max(N + P, 1)
    cu = torch.full((csr,), -7, dtype=torch.int32, device=dev)
    cp = torch.full((csr,), -7, dtype=torch.int32, device=dev)
    st = torch.full((1,), -7, dtype=torch.int32, device=dev)
    ws = psq.workspace_for(dev, _lib.psq_pack_rows_workspace(N, P, C))
    _lib.psq_pack_rows(t_src.data_ptr(), len(src), t_off.data_ptr(), t_rl.data_ptr(), N, q,
                       t_od.data_ptr() if t_od is not None else None, t_ps.data_ptr(), P, C,
                       int(fold), pad_token, packed.data_ptr(), tm.data_ptr(), cu.data_ptr(),
                       cp.data_ptr(), st.data_ptr(), ws.data_ptr(), ws.numel(),
                       torch.cuda.current_stream(dev).cuda_stream)
    status = int(st.item())
    if status != 0:
        return {"status": status}
    used = (int(ps[-1]) + P) if P else 0
    return {"status": 0, "packed": packed[:P].cpu().numpy(), "token_mask": tm[:P].cpu().numpy(),
            "cu_seqlens": cu[:used].cpu().numpy(), "cu_seqlens_padded": cp[:used].cpu().numpy()}


def check_pack(dev, src, off, rl, q, ps, C, fold, pad_token=0, order=None, what=""):
    say(f"pack {what} N={len(rl)} P={len(ps) - 1} q={q} C={C} fold={fold}")
    got = run_pack_raw(dev, src, off, rl, q, ps, C, fold, pad_token, order)
    ref = oracle.pack(src, off, rl, q, ps, C, fold=fold, pad_token=pad_token, order=order)
    assert got["status"] == ref["status"]
    if ref["status"] != 0:
        return
    for key in ("packed", "token_mask", "cu_seqlens", "cu_seqlens_padded"):
        assert np.array_equal(got[key], ref[key]), key


@pytest.mark.parametrize("C,fold", [(20, False), (36, True)])
def test_pack_page_examples(dev, C, fold):
    src = np.arange(100, 115)
    check_pack(dev, src, [0, 5], [5, 10], 4, [0, 2], C, fold, what="page")


def test_pack_workload_full(dev):
    w = synth.pack_sources()
    check_pack(dev, w["src"], w["src_off"], w["real_len"], w["q"], w["pack_start"],
               w["capacity"], True, what="workload 4")


@pytest.mark.parametrize("q,C,fold", [(1, 64, True), (3, 100, False), (8, 4096, True),
                                      (64, 16384, True), (2, 9001, True), (5, 8191, False),
                                      (64, 20000, True)])
@pytest.mark.parametrize("ordered", [False, True])
def test_pack_fuzz(dev, q, C, fold, ordered):
    rng = np.random.default_rng(hash((q, C, fold, ordered)) % 2**32)
    N = int(rng.integers(1, 700))
    hi = max(1, C // 3)
    rl = np.where(rng.random(N) < 0.05, 0, rng.integers(1, hi + 1, size=N)).astype(np.int32)
    off = np.zeros(N, dtype=np.int64)
    off[1:] = np.cumsum(rl[:-1])
    src = rng.integers(0, 151936, size=int(rl.sum()) + 3)
    order = rng.permutation(N).astype(np.int32) if ordered else None
    members = order if ordered else np.arange(N)
    padded = -(-rl[members].astype(np.int64) // q) * q
    ps = synth.next_fit(padded, C)
    check_pack(dev, src, off, rl, q, ps, C, fold, pad_token=int(rng.integers(-5, 5)),
               order=order, what="fuzz")


def test_pack_many_members_per_pack(dev):
    # more than one LDS batch of members in a pack (q = 1, tiny sources)
    rng = np.random.default_rng(3)
    N = 3000
    rl = rng.integers(0, 4, size=N).astype(np.int32)
    off = np.zeros(N, dtype=np.int64)
    off[1:] = np.cumsum(rl[:-1])
    src = rng.integers(0, 1000, size=int(rl.sum()))
    C = int(rl.sum()) + 17
    check_pack(dev, src, off, rl, 1, [0, 1000, N], C, True, what="many members")


@pytest.mark.parametrize("case", ["overflow", "empty", "pack_range", "pack_range_long_order",
                                  "order_range", "src_range", "neg_len", "neg_len_bad_off", "neg_len_neg_off",
                                  "neg_len_and_other_src_range", "neg_off"])
def test_pack_error_bits(dev, case):
    """Each status word is compared exactly with the oracle's, also when one
    member has several faults: a member whose length is bad is not checked
    further (its offset is not looked at), another member's faults still
    count."""
    src = np.arange(1, 7)
    off = np.array([0, 3, 4])
    rl = np.array([3, 1, 2])
    q, ps, C, order = 2, [0, 2, 3], 8, None
    if case == "overflow":
        C = 5
    elif case == "empty":
        ps = [0, 0, 3]
    elif case == "pack_range":
        ps = [0, 4]
    elif case == "pack_range_long_order":
        # the range passes the N member entries; the order buffer holds one
        # more (valid) entry, which must not be taken as a member
        ps, order = [0, 4], [0, 1, 2, 0]
    elif case == "order_range":
        ps, order = [0, 3], [0, 1, 3]
    elif case == "src_range":
        off = np.array([0, 3, 5])
    elif case == "neg_len":
        rl = np.array([3, -2, 2])
    elif case == "neg_len_bad_off":
        rl, off = np.array([3, -2, 2]), np.array([0, 100, 4])
    elif case == "neg_len_neg_off":
        rl, off = np.array([3, -2, 2]), np.array([0, -5, 4])
    elif case == "neg_len_and_other_src_range":
        rl, off = np.array([3, -2, 2]), np.array([0, 3, 5])
    elif case == "neg_off":
        off = np.array([0, -1, 4])
    check_pack(dev, src, off, rl, q, ps, C, True, order=order, what=case)


def test_pack_no_packs(dev):
    check_pack(dev, np.arange(3), [0], [3], 1, [0], 8, True, what="P=0")


def test_pack_no_sources(dev):
    """Packs but no sources: every pack is empty (EMPTY_PACK)."""
    empty = np.zeros(0, np.int64)
    check_pack(dev, empty, empty, np.zeros(0, np.int32), 2, [0, 0, 0], 8, True, what="N=0")


def test_pack_workspace_header_left_zeroed(dev):
    # the squeeze's counters (finish word, fallback list) are cleared by the
    # call itself; descriptors are rewritten by every call
    rng = np.random.default_rng(5)
    rl = rng.integers(0, 4, size=600).astype(np.int32)          # q = 1: many runs,
    off = np.zeros(600, dtype=np.int64)                          # fallback chunks
    off[1:] = np.cumsum(rl[:-1])
    src = rng.integers(0, 1000, size=int(rl.sum()))
    C = int(rl.sum()) + 5
    for _ in range(2):
        check_pack(dev, src, off, rl, 1, [0, 300, 600], C, True, what="fallback twice")
    torch.cuda.synchronize()
    ws = psq.workspace_for(dev, 0)
    assert int(ws[:256].count_nonzero()) == 0


def test_pack_python_api(dev):
    src = torch.arange(100, 115, dtype=torch.int64, device=dev)
    out = psq.pack_rows(src, torch.tensor([0, 5], device=dev),
                        torch.tensor([5, 10], dtype=torch.int32, device=dev), [0, 2],
                        capacity=36, pad_to=4)
    assert out["cu_seqlens"][0].cpu().tolist() == [0, 5, 15]
    assert out["cu_seqlens_padded"][0].cpu().tolist() == [0, 8, 36]
    assert int(out["token_mask"].sum()) == 15
    with pytest.raises(ValueError, match="capacity"):
        psq.pack_rows(src, torch.tensor([0, 5], device=dev),
                      torch.tensor([5, 10], dtype=torch.int32, device=dev), [0, 2],
                      capacity=16, pad_to=4)
