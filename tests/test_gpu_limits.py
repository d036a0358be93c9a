"""GPU checks at the size limits of the C ABI, through the C ABI.

Boundary arrays are int32, so a document map or a THD batch may hold up to
2^31 - 1 tokens and a pack up to 2^30 slots.  At those sizes the CPU oracle
would need tens of GB, so the outputs are checked against properties that
hold at any size and that the inputs fix in closed form: every row start is
a boundary, a row of one document and one trailing pad run has exactly two
segments, the padding mask counts exactly the pad slots, and a squeezed
source sits at its padded offset.  The same closed forms are checked against
the oracle at small sizes first, so they are pinned to it.
"""
import numpy as np
import pytest
import torch

import oracle
import varlen_attention_metadata_amd as psq
from varlen_attention_metadata_amd import _lib

pytestmark = pytest.mark.gpu
V = -1000


def say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def dev():
    _lib.load()
    return torch.device("cuda:0")


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def two_run_rows(B, S, pad):
    """Closed form of a map whose rows are one document then `pad` zeros."""
    starts = []
    for r in range(B):
        starts.append(r * S)
        if 0 < pad < S:
            starts.append(r * S + S - pad)
    return np.array(starts + [B * S], dtype=np.int64)


def squeeze_closed_form(lens, order, q):
    """Closed form of one pack holding sources `order` (lengths `lens`) end
    to end, each padded to a multiple of q, fold off: the real and padded
    boundaries and each member's first slot."""
    cu, cp, at = [0], [0], []
    for i in order:
        at.append(cp[-1])
        cu.append(cu[-1] + lens[i])
        cp.append(cp[-1] + -(-lens[i] // q) * q)
    return cu, cp, at


def test_closed_form_matches_oracle_small():
    B, S, pad = 5, 12, 3
    doc = np.ones((B, S), dtype=np.int64)
    doc[:, S - pad:] = 0
    ref = oracle.doc_segments(doc)
    assert np.array_equal(ref["cu_seqlens"], two_run_rows(B, S, pad))
    assert ref["max_seqlen"] == S - pad
    ref = oracle.thd_tables(np.array([[S - pad, V]] * B), np.array([[S - pad, V]] * B), S)
    assert ref["cu_seqlens_padded"].tolist() == [r * S for r in range(B + 1)]
    assert ref["cu_seqlens"].tolist() == [r * (S - pad) for r in range(B + 1)]
    assert ref["pad_between_seqs"] == 1 and ref["max_seqlen"] == S - pad
    # the same rows split into row groups: every group has the same closed form
    ref = oracle.split_thd(np.array([[S - pad, V]] * 6), np.array([[S - pad, V]] * 6), S, 2)
    assert ref["cu_seqlens_padded"].tolist() == [[r * S for r in range(4)]] * 2
    assert ref["cu_seqlens"].tolist() == [[r * (S - pad) for r in range(4)]] * 2
    assert ref["num_seqs"].tolist() == [3, 3] and ref["max_seqlen"].tolist() == [S - pad] * 2
    assert ref["pad_between_seqs"].tolist() == [1, 1]
    # a padded rectangle squeezed into one bin, members out of row order
    lens, order, q, W = [5, 1000, 7000], [2, 0, 1], 64, 7003
    rng = np.random.default_rng(4)
    rows = rng.integers(0, 1 << 40, size=(3, W))
    ref = oracle.pack_rect(rows, lens, q, [order], width=9000)
    cu, cp, at = squeeze_closed_form(lens, order, q)
    assert ref["status"] == 0
    assert ref["cu_seqlens"].tolist() == cu and ref["cu_seqlens_padded"].tolist() == cp
    for i, a in zip(order, at):
        assert np.array_equal(ref["packed"][0, a:a + lens[i]], rows[i, :lens[i]])
    # loader sources end to end in one folded pack, a source ending exactly at
    # the token buffer's end; one token less in the buffer is BAD_INDEX
    src, offs = np.arange(100, 100 + 8005), [1000, 0, 1005]
    ref = oracle.pack(src, offs, lens, q, [0, 3], 9000, fold=True)
    cu, cp, at = squeeze_closed_form(lens, range(3), q)
    assert ref["status"] == 0
    assert ref["cu_seqlens"].tolist() == cu and ref["cu_seqlens_padded"].tolist() == cp[:-1] + [9000]
    assert oracle.pack(src[:-1], offs, lens, q, [0, 3], 9000)["status"] == oracle.BAD_INDEX
    # a content prefix then a pad tail; and the same with the pad id planted at 7
    T, tail = 50, 9
    ids = np.ones(T, dtype=np.int64)
    ids[T - tail:] = 0
    ref = oracle.pad_mask_from_ids(ids, 0)
    assert ref["status"] == 0 and ref["num_content"] == T - tail
    assert int(ref["padding_mask"].sum()) == tail and ref["padding_mask"][T - tail] == 1
    ids[7] = 0
    ref = oracle.pad_mask_from_ids(ids, 0)
    assert ref["status"] == oracle.PAD_IS_CONTENT and ref["num_content"] == 7


def test_doc_map_at_int32_limit(dev):
    B, S, pad = 2047, 1 << 20, 4099
    T = B * S
    assert T < 2 ** 31
    say(f"doc map at the int32 limit: B={B} S={S} (T={T})")
    doc = torch.ones((B, S), dtype=torch.int32, device=dev)
    doc[:, S - pad:] = 0
    want = two_run_rows(B, S, pad)
    cu_full = torch.empty(T + 1, dtype=torch.int32, device=dev)
    scal = torch.full((4,), -7, dtype=torch.int32, device=dev)
    mask = torch.empty(T, dtype=torch.uint8, device=dev)
    ws = psq.workspace_for(dev, _lib.psq_params_from_doc_ids_workspace(B, S))
    sp = scal.data_ptr()
    _lib.psq_params_from_doc_ids(doc.data_ptr(), _lib.I32, B, S, cu_full.data_ptr(), sp, sp + 4,
                                 mask.data_ptr(), sp + 8, ws.data_ptr(), ws.numel(),
                                 _stream(dev))
    n, mx, st, _ = scal.cpu().tolist()
    assert st == 0
    assert n == want.size - 1
    assert np.array_equal(cu_full[: n + 1].cpu().numpy(), want)
    assert mx == S - pad
    assert int(mask.sum(dtype=torch.int64).item()) == B * pad
    del doc, mask, cu_full


def test_thd_tables_at_int32_limit(dev):
    B, S, real = 2047, 1 << 20, (1 << 20) - 4099
    T = B * S
    say(f"thd tables at the int32 limit: B={B} S={S}")
    L = torch.tensor([[real, V]] * B, dtype=torch.int64, device=dev)
    cap = B * 2 + 1
    cu = torch.empty(cap, dtype=torch.int32, device=dev)
    cp = torch.empty(cap, dtype=torch.int32, device=dev)
    mask = torch.empty(T, dtype=torch.uint8, device=dev)
    scal = torch.full((4,), -7, dtype=torch.int32, device=dev)
    lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, L.data_ptr(), L.data_ptr(), _lib.I64, 2, V)
    ws = psq.workspace_for(dev, _lib.psq_process_thd_workspace(lay, B, S))
    arr, n_c = _lib.make_copies([])
    sp = scal.data_ptr()
    _lib.psq_process_thd(lay, B, S, cu.data_ptr(), cp.data_ptr(), sp, sp + 4, sp + 8,
                         mask.data_ptr(), arr, n_c, sp + 12, ws.data_ptr(), ws.numel(),
                         _stream(dev))
    n, mx, pb, st = scal.cpu().tolist()
    assert st == 0 and n == B
    assert cp[: n + 1].cpu().tolist() == [r * S for r in range(B + 1)]
    # every row folds its tail pad: no interior boundary agrees, no absorption
    assert cu[: n + 1].cpu().tolist() == [r * real for r in range(B + 1)]
    assert pb == 1 and mx == real
    assert int(mask.sum(dtype=torch.int64).item()) == B * (S - real)
    del mask


def test_split_at_int32_limit(dev):
    """The table batch near 2^31 tokens split into 2 row groups: each group
    holds 1023 rows (over 2^30 tokens) and is stacked into a [2, 1024] array."""
    B, S, real, G = 2046, 1 << 20, (1 << 20) - 4099, 2
    T, Bc = B * S, B // G
    say(f"split at the int32 limit: B={B} S={S} G={G}")
    L = torch.tensor([[real, V]] * B, dtype=torch.int64, device=dev)
    cap = G * (Bc * 2 + 1)
    cu = torch.empty(cap, dtype=torch.int32, device=dev)
    cp = torch.empty(cap, dtype=torch.int32, device=dev)
    mask = torch.empty(T, dtype=torch.uint8, device=dev)
    per = torch.full((3, G), -7, dtype=torch.int32, device=dev)
    scal = torch.full((2,), -7, dtype=torch.int32, device=dev)
    lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, L.data_ptr(), L.data_ptr(), _lib.I64, 2, V)
    ws = psq.workspace_for(dev, _lib.psq_split_thd_workspace(lay, B, S, G))
    arr, n_c = _lib.make_copies([])
    pp, sp = per.data_ptr(), scal.data_ptr()
    _lib.psq_split_thd(lay, B, S, G, cu.data_ptr(), cp.data_ptr(), sp, pp, pp + 4 * G,
                       pp + 8 * G, mask.data_ptr(), arr, n_c, sp + 4, ws.data_ptr(), ws.numel(),
                       _stream(dev))
    width, st = scal.cpu().tolist()
    assert st == 0 and width == Bc + 1
    want_cp = [r * S for r in range(Bc + 1)]
    want_cu = [r * real for r in range(Bc + 1)]
    assert cp[: G * width].view(G, width).cpu().tolist() == [want_cp] * G
    assert cu[: G * width].view(G, width).cpu().tolist() == [want_cu] * G
    assert per.cpu().tolist() == [[Bc] * G, [real] * G, [1] * G]
    assert int(mask.sum(dtype=torch.int64).item()) == B * (S - real)
    del mask


def test_pack_at_capacity_limit(dev):
    C = 1 << 30
    q = 64
    lens = [5, 1000, 70000]
    N = len(lens)
    say(f"squeeze into one pack of {C} slots")
    rng = np.random.default_rng(3)
    toks = [rng.integers(0, 1 << 40, size=n) for n in lens]
    src = torch.from_numpy(np.concatenate(toks)).to(dev)
    off = torch.tensor(np.concatenate([[0], np.cumsum(lens)[:-1]]), dtype=torch.int64, device=dev)
    rl = torch.tensor(lens, dtype=torch.int32, device=dev)
    ps = torch.tensor([0, N], dtype=torch.int64, device=dev)
    packed = torch.empty((1, C), dtype=torch.int64, device=dev)
    tm = torch.empty((1, C), dtype=torch.uint8, device=dev)
    cu = torch.empty(N + 1, dtype=torch.int32, device=dev)
    cp = torch.empty(N + 1, dtype=torch.int32, device=dev)
    st = torch.full((1,), -7, dtype=torch.int32, device=dev)
    ws = psq.workspace_for(dev, _lib.psq_pack_rows_workspace(N, 1, C))
    _lib.psq_pack_rows(src.data_ptr(), src.numel(), off.data_ptr(), rl.data_ptr(), N, q, None,
                       ps.data_ptr(), 1, C, 1, -1, packed.data_ptr(), tm.data_ptr(),
                       cu.data_ptr(), cp.data_ptr(), st.data_ptr(), ws.data_ptr(), ws.numel(),
                       _stream(dev))
    assert int(st.item()) == 0
    padded = [-(-n // q) * q for n in lens]
    assert cu.cpu().tolist() == [0, 5, 1005, 71005]
    assert cp.cpu().tolist() == [0, padded[0], padded[0] + padded[1], C]
    at = 0
    for n, p, t in zip(lens, padded, toks):
        assert np.array_equal(packed[0, at:at + n].cpu().numpy(), t)
        assert bool((packed[0, at + n:at + p] == -1).all())
        at += p
    assert int(tm.sum(dtype=torch.int64).item()) == sum(lens)
    assert bool((packed[0, at:] == -1).all())
    del packed, tm


@pytest.mark.parametrize("dtype", [torch.int64, torch.int32])
def test_pad_ids_at_int32_limit(dev, dtype):
    """2^31 - 1 ids: the first pad slot and one past the last content slot
    fill their 31-bit record fields, and each workgroup strides over 512
    tiles or more."""
    T, tail = (1 << 31) - 1, 12345
    say(f"pad ids at the int32 limit: T={T} {dtype}")
    ids = torch.ones(T, dtype=dtype, device=dev)
    ids[T - tail:] = 0
    mask = torch.empty(T, dtype=torch.uint8, device=dev)
    scal = torch.full((2,), -7, dtype=torch.int32, device=dev)
    ws = psq.workspace_for(dev, _lib.psq_padding_mask_from_token_ids_workspace(T))
    sp = scal.data_ptr()
    kind = _lib.I64 if dtype == torch.int64 else _lib.I32
    for planted in (None, 7):
        if planted is not None:
            ids[planted] = 0
        _lib.psq_padding_mask_from_token_ids(ids.data_ptr(), kind, T, 0, mask.data_ptr(), sp,
                                             sp + 4, ws.data_ptr(), ws.numel(), _stream(dev))
        nc, st = scal.cpu().tolist()
        if planted is None:
            assert st == 0 and nc == T - tail
            assert int(mask.sum(dtype=torch.int64).item()) == tail
            assert int(mask[T - tail - 1].item()) == 0 and int(mask[T - tail].item()) == 1
        else:
            assert st == _lib.DATA_PAD_IS_CONTENT and nc == planted
            assert int(mask.sum(dtype=torch.int64).item()) == tail + 1
    del ids, mask


def test_trainer_rows_beyond_int32_elements(dev):
    """A padded rectangle whose rows start past 2^31 elements (row 2 begins
    at byte 16 GiB): the trainer squeeze's row offsets are 64-bit."""
    W, q, C = (1 << 30) + 3, 64, 1 << 20
    lens, order = [5, 1000, 70000], [2, 0, 1]
    N = len(lens)
    say(f"trainer squeeze from a [{N}, {W}] rectangle")
    rng = np.random.default_rng(5)
    rows = torch.empty((N, W), dtype=torch.int64, device=dev)
    toks = []
    for i, n in enumerate(lens):
        t = rng.integers(0, 1 << 40, size=n)
        rows[i, :n] = torch.from_numpy(t).to(dev)
        toks.append(t)
    rl = torch.tensor(lens, dtype=torch.int32, device=dev)
    od = torch.tensor(order, dtype=torch.int32, device=dev)
    ps = torch.tensor([0, N], dtype=torch.int64, device=dev)
    packed = torch.empty((1, C), dtype=torch.int64, device=dev)
    tm = torch.empty((1, C), dtype=torch.uint8, device=dev)
    cu_d = torch.empty(N + 1, dtype=torch.int32, device=dev)
    cp_d = torch.empty(N + 1, dtype=torch.int32, device=dev)
    st = torch.full((1,), -7, dtype=torch.int32, device=dev)
    ws = psq.workspace_for(dev, _lib.psq_pack_rows_workspace(N, 1, C))
    _lib.psq_pack_padded_rows(rows.data_ptr(), W, rl.data_ptr(), N, q, od.data_ptr(),
                              ps.data_ptr(), 1, C, 0, -1, packed.data_ptr(), tm.data_ptr(),
                              cu_d.data_ptr(), cp_d.data_ptr(), st.data_ptr(), ws.data_ptr(),
                              ws.numel(), _stream(dev))
    assert int(st.item()) == 0
    cu, cp, at = squeeze_closed_form(lens, order, q)
    assert cu_d.cpu().tolist() == cu and cp_d.cpu().tolist() == cp
    for i, a in zip(order, at):
        assert np.array_equal(packed[0, a:a + lens[i]].cpu().numpy(), toks[i])
        assert bool((packed[0, a + lens[i]:a + -(-lens[i] // q) * q] == -1).all())
    assert bool((packed[0, cp[-1]:] == -1).all())
    assert int(tm.sum(dtype=torch.int64).item()) == sum(lens)
    del rows, packed, tm


def test_loader_sources_beyond_int32_elements(dev):
    """Loader sources at offsets past 2^31 elements of a 16 GiB token buffer,
    the last one ending exactly at the buffer's end (the inclusive bound)."""
    q, C = 64, 1 << 20
    lens = [5, 1000, 70000]
    base = 1 << 31
    offs = [base + 7, 3, base + 10000]
    src_len = offs[2] + lens[2]
    say(f"loader squeeze from a {src_len}-token buffer")
    rng = np.random.default_rng(6)
    src = torch.empty(src_len, dtype=torch.int64, device=dev)
    toks = []
    for o, n in zip(offs, lens):
        t = rng.integers(0, 1 << 40, size=n)
        src[o:o + n] = torch.from_numpy(t).to(dev)
        toks.append(t)
    N = len(lens)
    off = torch.tensor(offs, dtype=torch.int64, device=dev)
    rl = torch.tensor(lens, dtype=torch.int32, device=dev)
    ps = torch.tensor([0, N], dtype=torch.int64, device=dev)
    packed = torch.empty((1, C), dtype=torch.int64, device=dev)
    tm = torch.empty((1, C), dtype=torch.uint8, device=dev)
    cu_d = torch.empty(N + 1, dtype=torch.int32, device=dev)
    cp_d = torch.empty(N + 1, dtype=torch.int32, device=dev)
    st = torch.full((1,), -7, dtype=torch.int32, device=dev)
    ws = psq.workspace_for(dev, _lib.psq_pack_rows_workspace(N, 1, C))
    _lib.psq_pack_rows(src.data_ptr(), src_len, off.data_ptr(), rl.data_ptr(), N, q, None,
                       ps.data_ptr(), 1, C, 1, -1, packed.data_ptr(), tm.data_ptr(),
                       cu_d.data_ptr(), cp_d.data_ptr(), st.data_ptr(), ws.data_ptr(),
                       ws.numel(), _stream(dev))
    assert int(st.item()) == 0
    cu, cp, at = squeeze_closed_form(lens, range(N), q)
    assert cu_d.cpu().tolist() == cu and cp_d.cpu().tolist() == cp[:-1] + [C]
    for i, a in enumerate(at):
        assert np.array_equal(packed[0, a:a + lens[i]].cpu().numpy(), toks[i])
    assert int(tm.sum(dtype=torch.int64).item()) == sum(lens)
    # one token more and the last source runs past the buffer: BAD_INDEX
    _lib.psq_pack_rows(src.data_ptr(), src_len - 1, off.data_ptr(), rl.data_ptr(), N, q, None,
                       ps.data_ptr(), 1, C, 1, -1, packed.data_ptr(), tm.data_ptr(),
                       cu_d.data_ptr(), cp_d.data_ptr(), st.data_ptr(), ws.data_ptr(),
                       ws.numel(), _stream(dev))
    assert int(st.item()) == _lib.DATA_BAD_INDEX
    del src, packed, tm
