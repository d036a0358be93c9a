"""GPU parity for the steps around the five workloads, through the C ABI:

* ``psq_split_thd`` (``split_batch_into_thd_chunks``): row groups converted
  in one launch, stacked, boundary arrays filled with the sentinel;
* ``psq_padding_mask_from_token_ids`` (``thd_padding_mask_from_token_ids``):
  the value-compare mask and its right-padded-tail check;
* ``psq_pack_padded_rows`` (the trainer's squeeze from the padded rectangle).

Each is compared element by element with the CPU oracle on the same seeded
inputs; every output is an integer, a mask byte or a byte copy, so every
comparison is exact.
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
    _lib.load()
    return torch.device("cuda:0")


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


# ---------------------------------------------------------------------------
# split_batch_into_thd_chunks
# ---------------------------------------------------------------------------

def run_split_raw(dev, L, Lp, S, G, dtype=torch.int64):
    B, P = L.shape
    tL = torch.from_numpy(np.ascontiguousarray(L)).to(dev, dtype)
    tLp = torch.from_numpy(np.ascontiguousarray(Lp)).to(dev, dtype) if Lp is not None else None
    Bc = B // G
    cap = G * (Bc * P + 1)
    cu = torch.full((cap,), -7, dtype=torch.int32, device=dev)
    cp = torch.full((cap,), -7, dtype=torch.int32, device=dev)
    mask = torch.full((max(B * S, 1),), 7, dtype=torch.uint8, device=dev)
    per = torch.full((3, G), -7, dtype=torch.int32, device=dev)
    scal = torch.full((2,), -7, dtype=torch.int32, device=dev)
    lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, tL.data_ptr(),
                           tLp.data_ptr() if tLp is not None else None,
                           _lib.I64 if dtype == torch.int64 else _lib.I32, P, V)
    ws = psq.workspace_for(dev, _lib.psq_split_thd_workspace(lay, B, S, G))
    arr, n_c = _lib.make_copies([])
    pp, sp = per.data_ptr(), scal.data_ptr()
    _lib.psq_split_thd(lay, B, S, G, cu.data_ptr(), cp.data_ptr(), sp, pp, pp + 4 * G,
                       pp + 8 * G, mask.data_ptr(), arr, n_c, sp + 4, ws.data_ptr(), ws.numel(),
                       _stream(dev))
    width, st = scal.cpu().tolist()
    if st != 0:
        return {"status": st, "width": width}
    return {"status": 0, "width": width,
            "cu_seqlens": cu[: G * width].view(G, width).cpu().numpy(),
            "cu_seqlens_padded": cp[: G * width].view(G, width).cpu().numpy(),
            "num_seqs": per[0].cpu().numpy(), "max_seqlen": per[1].cpu().numpy(),
            "pad_between_seqs": per[2].cpu().numpy(),
            "padding_mask": mask[: B * S].view(G, Bc * S).cpu().numpy()}


def check_split(dev, L, Lp, S, G, dtype=torch.int64):
    say(f"split {L.shape} S={S} G={G} padded={Lp is not None} {dtype}")
    got = run_split_raw(dev, L, Lp, S, G, dtype)
    ref = oracle.split_thd(L, Lp, S, G)
    assert got["status"] == ref["status"]
    if ref["status"] != 0:
        assert got["width"] == 0
        return
    assert got["width"] == ref["cu_seqlens"].shape[1]
    for key in ("cu_seqlens", "cu_seqlens_padded", "padding_mask", "num_seqs", "max_seqlen",
                "pad_between_seqs"):
        assert np.array_equal(got[key], ref[key]), key


def rand_tables(rng, B, P, S, q, tight_frac=0.3):
    L = np.full((B, P), V, dtype=np.int64)
    Lp = np.full((B, P), V, dtype=np.int64)
    for r in range(B):
        used = 0
        k = int(rng.integers(1, P + 1))
        tight = rng.random() < tight_frac
        for j in range(k):
            real = int(rng.integers(0, max(2, S // 3)))
            padded = real if tight else -(-real // q) * q
            if used + padded > S:
                break
            L[r, j], Lp[r, j] = real, padded
            used += padded
        if L[r, 0] == V:
            L[r, 0], Lp[r, 0] = 0, 0
    return L, Lp


def test_split_page_example(dev):
    g = oracle_golden = __import__("conftest").load_golden("thd_chunks_example.json")
    inp = g["input"]
    say("split page example via split_batch_into_thd_chunks")
    batch = {k: torch.tensor(inp[k], device=dev) for k in
             ("input_ids", "labels", "position_ids", "seq_lens", "seq_lens_padded")}
    out = psq.split_batch_into_thd_chunks(batch, num_chunks=inp["num_chunks"])
    pr = oracle_golden["printed"]
    assert list(out["input_ids"].shape) == pr["input_ids_shape"]
    assert list(out["cu_seqlens"].shape) == pr["cu_seqlens_shape"]
    assert out["cu_seqlens"].cpu().tolist() == pr["cu_seqlens_per_chunk"]
    assert out["cu_seqlens"].dtype == torch.int32
    flat = np.array(inp["input_ids"]).reshape(2, 12)
    assert np.array_equal(out["input_ids"].cpu().numpy(), flat)
    # num_chunks <= 1 is process_input_for_thd itself
    one = psq.split_batch_into_thd_chunks(batch, num_chunks=1)
    assert one["cu_seqlens"].cpu().tolist() == [0, 6, 12, 18, 24]


@pytest.mark.parametrize("B,P,S,G", [(2, 3, 8, 2), (4, 1, 6, 4), (4, 5, 16, 2), (6, 8, 100, 3),
                                     (8, 64, 8192, 8), (3, 2000, 30000, 3), (600, 2, 8, 600),
                                     (600, 2, 8, 300), (512, 3, 20, 2), (5, 4, 4097, 5)])
@pytest.mark.parametrize("mode", ["padded", "nopad", "int32"])
def test_split_fuzz(dev, B, P, S, G, mode):
    rng = np.random.default_rng(hash((B, P, S, G, mode)) % 2**32)
    q = int(rng.choice([1, 4, 8]))
    L, Lp = rand_tables(rng, B, P, S, q)
    if mode == "nopad":
        check_split(dev, L, None, S, G)
    else:
        check_split(dev, L, Lp, S, G, torch.int32 if mode == "int32" else torch.int64)


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("wide", [False, True])
def test_split_fault_fuzz(dev, seed, wide):
    # the faults of the table fuzz, on row groups: status words and (when
    # clean) the stacked outputs must match the oracle on both kernels
    from test_gpu_parity import corrupt_tables
    rng = np.random.default_rng(2000 + seed)
    G = int(rng.integers(1, 5))
    B, P, S = G * int(rng.integers(1, 4)), int(rng.integers(1, 7)), int(rng.integers(4, 48))
    L, Lp = rand_tables(rng, B, P, S, 4)
    if seed % 2:
        L, Lp = corrupt_tables(rng, L, Lp, S, int(rng.integers(1, 3)))
    if wide:
        extra = np.full((B, 4200), V)
        L, Lp = np.hstack([L, extra]), np.hstack([Lp, extra])
    check_split(dev, L, Lp, S, G)


def test_split_hand_ragged(dev):
    check_split(dev, np.array([[2, 3, 1], [1, V, V]]), np.array([[2, 3, 1], [1, V, V]]), 8, 2)


# no rows (each chunk is an empty batch: cu_seqlens [0]); rows of length 0
# holding empty sequences; rows without a slot (EMPTY_ROW)
@pytest.mark.parametrize("L,S,G", [(np.zeros((0, 3), np.int64), 8, 2),
                                   (np.array([[0], [0]]), 0, 2),
                                   (np.zeros((4, 0), np.int64), 8, 2)],
                         ids=["no_rows", "zero_length_rows", "no_slots"])
def test_split_degenerate_shapes(dev, L, S, G):
    check_split(dev, L, None, S, G)


@pytest.mark.parametrize("L,Lp,S,G", [
    ([[3, 2], [5, V]], [[4, 2], [4, V]], 8, 2),     # real > padded in chunk 1
    ([[3, 2], [V, V]], [[4, 2], [V, V]], 8, 2),     # empty row in chunk 1
    ([[9], [2]], [[9], [2]], 8, 2),                 # row overflow in chunk 0
])
@pytest.mark.parametrize("wide", [False, True])
def test_split_error_bits(dev, L, Lp, S, G, wide):
    L, Lp = np.array(L), np.array(Lp)
    if wide:
        # sentinel columns: the same tables, past the single-workgroup size
        extra = np.full((L.shape[0], 4200), V)
        L, Lp = np.hstack([L, extra]), np.hstack([Lp, extra])
    check_split(dev, L, Lp, S, G)


# on either side of the single-workgroup limits (4096 entries, 64 groups)
@pytest.mark.parametrize("B,P,S,G", [(128, 2, 16, 64), (130, 2, 16, 65), (64, 64, 100, 64),
                                     (64, 65, 100, 16)])
def test_split_single_workgroup_limits(dev, B, P, S, G):
    rng = np.random.default_rng(B * 7919 + P * 31 + G)
    L, Lp = rand_tables(rng, B, P, S, 4)
    check_split(dev, L, Lp, S, G)


def test_split_matches_process_thd_at_one_chunk(dev):
    w = synth.thd_tables()
    L, Lp, S = w["seq_lens"], w["seq_lens_padded"], w["S"]
    check_split(dev, L, Lp, S, 1)


@pytest.mark.parametrize("G", [2, 4, 16])
def test_split_workload_with_copies(dev, G):
    w = synth.thd_tables()
    S = w["S"]
    B = w["seq_lens"].shape[0]
    say(f"workload 3 split into {G} chunks via split_batch_into_thd_chunks")
    batch = {k: torch.from_numpy(w[k]).to(dev) for k in
             ("input_ids", "labels", "position_ids", "seq_lens", "seq_lens_padded")}
    batch["qkv_format"] = "thd"
    out = psq.split_batch_into_thd_chunks(batch, G)
    ref = oracle.split_thd(w["seq_lens"], w["seq_lens_padded"], S, G)
    assert ref["status"] == 0
    assert np.array_equal(out["cu_seqlens"].cpu().numpy(), ref["cu_seqlens"])
    assert np.array_equal(out["cu_seqlens_padded"].cpu().numpy(), ref["cu_seqlens_padded"])
    assert np.array_equal(out["max_seqlen"].cpu().numpy(), ref["max_seqlen"])
    assert np.array_equal(out["pad_between_seqs"].cpu().numpy(),
                          ref["pad_between_seqs"].astype(bool))
    assert np.array_equal(out["padding_mask"].cpu().numpy().astype(np.uint8),
                          ref["padding_mask"])
    assert out["qkv_format"] == "thd"
    Bc = B // G
    for key in ("input_ids", "labels", "position_ids"):
        got = out[key].cpu().numpy()
        assert got.shape == (G, Bc * S)
        for c in range(G):
            part = np.ascontiguousarray(w[key][c * Bc:(c + 1) * Bc])
            want = oracle.copy_rows(part, 1, part.nbytes, part.nbytes)
            assert got[c].tobytes() == want.tobytes(), (key, c)


def test_split_embeddings_and_mrope(dev):
    rng = np.random.default_rng(12)
    B, S, H, n_rope, G = 4, 24, 16, 3, 2
    emb = torch.randn((B, S, H), dtype=torch.bfloat16, device=dev)
    pos_np = rng.integers(0, 50, size=(n_rope, B, S))
    pos = torch.from_numpy(pos_np).to(dev)
    L = torch.tensor([[10, 9], [24, V], [5, V], [1, 2]], device=dev)
    say("split embeddings + mRoPE")
    out = psq.split_batch_into_thd_chunks({"input_ids": emb, "position_ids": pos, "seq_lens": L},
                                          G)
    Bc = B // G
    assert out["input_ids"].shape == (G, Bc * S, H)
    assert torch.equal(out["input_ids"].view(torch.int16),
                       emb.reshape(G, Bc * S, H).view(torch.int16))
    assert out["position_ids"].shape == (G, n_rope, 1, Bc * S)
    got = out["position_ids"].cpu().numpy()
    for c in range(G):
        part = np.ascontiguousarray(pos_np[:, c * Bc:(c + 1) * Bc, :])
        want = oracle.copy_rows(part, 1, part.nbytes, part.nbytes)
        assert got[c].tobytes() == want.tobytes(), c
    ref = oracle.split_thd(L.cpu().numpy(), None, S, G)
    assert np.array_equal(out["cu_seqlens"].cpu().numpy(), ref["cu_seqlens"])
    assert "cu_seqlens_padded" not in out


def test_split_workspace_left_zeroed_and_repeatable(dev):
    rng = np.random.default_rng(5)
    L, Lp = rand_tables(rng, 64, 16, 512, 8)
    first = run_split_raw(dev, L, Lp, 512, 8)
    for _ in range(5):
        again = run_split_raw(dev, L, Lp, 512, 8)
        for key in ("cu_seqlens", "cu_seqlens_padded", "padding_mask", "max_seqlen"):
            assert np.array_equal(first[key], again[key])
    B, P = L.shape
    lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, 1, None, _lib.I64, P, V)
    need = _lib.psq_split_thd_workspace(lay, B, 512, 8)
    ws = psq.workspace_for(dev, need)
    torch.cuda.synchronize(dev)
    # header, descriptors, group records and the staged boundaries are all
    # zero again, after a good call and after a call with a data error
    assert int(ws[:need].to(torch.int32).abs().sum()) == 0
    bad = L.copy()
    bad[3, 0] = -5
    assert run_split_raw(dev, bad, Lp, 512, 8)["status"] != 0
    torch.cuda.synchronize(dev)
    assert int(ws[:need].to(torch.int32).abs().sum()) == 0


def test_split_python_api_errors(dev):
    batch = {"input_ids": torch.zeros((3, 4), dtype=torch.int64, device=dev),
             "position_ids": torch.zeros((3, 4), dtype=torch.int64, device=dev),
             "seq_lens": torch.tensor([[4], [4], [4]], device=dev)}
    with pytest.raises(ValueError, match="divide"):
        psq.split_batch_into_thd_chunks(batch, 2)
    bad = dict(batch, seq_lens=torch.tensor([[5], [4], [4]], device=dev))
    with pytest.raises(ValueError, match="row length"):
        psq.split_batch_into_thd_chunks(bad, 3)


# ---------------------------------------------------------------------------
# thd_padding_mask_from_token_ids
# ---------------------------------------------------------------------------

def run_padids_raw(dev, ids_np, pad, dtype=torch.int64, offset=0):
    T = ids_np.size
    base = torch.zeros(T + offset, dtype=dtype, device=dev)
    base[offset:] = torch.from_numpy(np.ascontiguousarray(ids_np)).to(dev, dtype)
    ids = base[offset:]
    mask = torch.full((T + 1,), 7, dtype=torch.uint8, device=dev)
    scal = torch.full((2,), -7, dtype=torch.int32, device=dev)
    ws = psq.workspace_for(dev, _lib.psq_padding_mask_from_token_ids_workspace(T))
    sp = scal.data_ptr()
    _lib.psq_padding_mask_from_token_ids(ids.data_ptr(), _lib.I64 if dtype == torch.int64
                                         else _lib.I32, T, pad, mask.data_ptr(), sp, sp + 4,
                                         ws.data_ptr(), ws.numel(), _stream(dev))
    nc, st = scal.cpu().tolist()
    m = mask.cpu().numpy()
    assert m[T] == 7, "wrote past the mask"
    return m[:T], nc, st


def check_padids(dev, ids_np, pad, dtype=torch.int64, offset=0):
    say(f"pad ids T={ids_np.size} pad={pad} {dtype} offset={offset}")
    mask, nc, st = run_padids_raw(dev, ids_np, pad, dtype, offset)
    ref = oracle.pad_mask_from_ids(ids_np, pad)
    assert st == ref["status"]
    assert np.array_equal(mask, ref["padding_mask"])
    assert nc == ref["num_content"]


@pytest.mark.parametrize("ids,pad", [([5, 6, 7, 0, 0], 0), ([5, 6, 7], 0), ([9, 9, 9], 9),
                                     ([], 0), ([0, 5, 6], 0), ([5, 0, 6, 0], 0),
                                     ([17, 18, 151329, 40, 151329, 151329], 151329)])
@pytest.mark.parametrize("dtype", [torch.int64, torch.int32])
def test_padids_hand_cases(dev, ids, pad, dtype):
    check_padids(dev, np.array(ids, dtype=np.int64), pad, dtype)


# 4194305 int64 ids need 2049 tiles and 9000001 int32 ids 2198: more than the
# 2048 workgroups of a launch, so workgroups take several tiles
@pytest.mark.parametrize("T", [1, 2, 3, 4095, 4096, 4097, 8191, 8193, 65537, 131072, 1048579,
                               4194305, 9000001])
@pytest.mark.parametrize("kind", ["tail", "collide_early", "collide_late", "none", "all"])
@pytest.mark.parametrize("dtype", [torch.int64, torch.int32])
def test_padids_fuzz(dev, T, kind, dtype):
    rng = np.random.default_rng(hash((T, kind, str(dtype))) % 2**32)
    pad = 7
    ids = rng.integers(8, 1000, size=T).astype(np.int64)
    tail = int(rng.integers(0, T + 1))
    if kind in ("tail", "collide_early", "collide_late"):
        ids[T - tail:] = pad
    if kind == "collide_early" and T - tail > 0:
        ids[int(rng.integers(0, T - tail))] = pad
    if kind == "collide_late" and T - tail > 1:
        ids[T - tail - 2] = pad             # a pad two slots before the tail
    if kind == "all":
        ids[:] = pad
    check_padids(dev, ids, pad, dtype)


@pytest.mark.parametrize("offset", [1, 3])
def test_padids_unaligned(dev, offset):
    ids = np.arange(10, 10 + 5000, dtype=np.int64)
    ids[4000:] = 2
    check_padids(dev, ids, 2, torch.int64, offset)
    check_padids(dev, ids, 2, torch.int32, offset)


def test_padids_high_bits(dev):
    pad = 1 << 40
    ids = np.array([pad + 1, pad - 1, pad ^ (1 << 62), pad, pad], dtype=np.int64)
    check_padids(dev, ids, pad)
    # with int32 ids, a pad id beyond int32 matches nothing
    mask, nc, st = run_padids_raw(dev, np.array([1, 2, 0], dtype=np.int64), 1 << 33,
                                  torch.int32)
    assert st == 0 and mask.tolist() == [0, 0, 0] and nc == 3


def test_padids_workload(dev):
    w = synth.pad_tail_stream()
    check_padids(dev, w["input_ids"], w["pad_id"])
    # the same stream with pad id 0, which also occurs as content: rejected
    check_padids(dev, w["input_ids"], 0)


def test_padids_python_api(dev):
    ids = torch.tensor([4, 5, 6, 0, 0], device=dev)
    m = psq.thd_padding_mask_from_token_ids(ids, 0)
    assert m.dtype == torch.bool and m.cpu().tolist() == [False, False, False, True, True]
    with pytest.raises(ValueError, match="content"):
        psq.thd_padding_mask_from_token_ids(torch.tensor([4, 0, 6, 0], device=dev), 0)
    # the workspace header is clean after a rejected call
    m = psq.thd_padding_mask_from_token_ids(torch.tensor([1, 2, 3], device=dev), 0)
    assert m.cpu().tolist() == [False, False, False]


# ---------------------------------------------------------------------------
# the trainer's squeeze from the padded rectangle
# ---------------------------------------------------------------------------

def run_rect_raw(dev, rows, rl, q, bins, C, fold, pad_token=0):
    N, W = rows.shape
    order, start = oracle.bins_to_csr(bins)
    order_full = np.zeros(max(N, 1), dtype=np.int32)
    order_full[:order.size] = order
    P = len(bins)
    t_rows = torch.from_numpy(np.ascontiguousarray(rows)).to(dev)
    t_rl = torch.from_numpy(np.asarray(rl, dtype=np.int32)).to(dev)
    t_order = torch.from_numpy(order_full).to(dev)
    t_ps = torch.from_numpy(start).to(dev)
    packed = torch.full((P, C), -9, dtype=torch.int64, device=dev)
    tm = torch.full((P, C), 9, dtype=torch.uint8, device=dev)
    csr = max(N + P, 1)
    cu = torch.full((csr,), -7, dtype=torch.int32, device=dev)
    cp = torch.full((csr,), -7, dtype=torch.int32, device=dev)
    st = torch.full((1,), -7, dtype=torch.int32, device=dev)
    ws = psq.workspace_for(dev, _lib.psq_pack_rows_workspace(N, P, C))
    _lib.psq_pack_padded_rows(t_rows.data_ptr(), W, t_rl.data_ptr(), N, q, t_order.data_ptr(),
                              t_ps.data_ptr(), P, C, int(fold), pad_token, packed.data_ptr(),
                              tm.data_ptr(), cu.data_ptr(), cp.data_ptr(), st.data_ptr(),
                              ws.data_ptr(), ws.numel(), _stream(dev))
    status = int(st.item())
    used = order.size + P
    return {"status": status, "packed": packed.cpu().numpy(), "token_mask": tm.cpu().numpy(),
            "cu_seqlens": cu[:used].cpu().numpy(), "cu_seqlens_padded": cp[:used].cpu().numpy()}


def check_rect(dev, rows, rl, q, bins, C=None, fold=False, pad_token=0):
    C = oracle.trainer_width(rl, bins, q) if C is None else C
    say(f"rect squeeze N={rows.shape[0]} W={rows.shape[1]} bins={len(bins)} q={q} C={C} "
        f"fold={fold}")
    got = run_rect_raw(dev, rows, rl, q, bins, C, fold, pad_token)
    ref = oracle.pack_rect(rows, rl, q, bins, width=C, fold=fold, pad_token=pad_token)
    assert got["status"] == ref["status"]
    if ref["status"] != 0:
        return
    for key in ("packed", "token_mask", "cu_seqlens", "cu_seqlens_padded"):
        assert np.array_equal(got[key], ref[key]), key


def test_rect_page_example(dev):
    rows = np.zeros((2, 10), dtype=np.int64)
    rows[0, :5] = np.arange(101, 106)
    rows[1, :10] = np.arange(201, 211)
    check_rect(dev, rows, [5, 10], 4, [[0, 1]])
    say("rect page example via pack_padded_rows")
    out = psq.pack_padded_rows(torch.from_numpy(rows).to(dev), [5, 10], [[0, 1]], 4, width=20)
    assert out["width"] == 20 and tuple(out["input_ids"].shape) == (1, 20)
    assert out["cu_seqlens"][0].cpu().tolist() == [0, 5, 15]
    assert out["cu_seqlens_padded"][0].cpu().tolist() == [0, 8, 20]


@pytest.mark.parametrize("N,W,q", [(1, 1, 1), (3, 7, 4), (17, 100, 8), (64, 4097, 64),
                                   (300, 33, 3)])
@pytest.mark.parametrize("fold", [False, True])
def test_rect_fuzz(dev, N, W, q, fold):
    rng = np.random.default_rng(hash((N, W, q, fold)) % 2**32)
    rows = rng.integers(0, 1 << 40, size=(N, W))
    rl = rng.integers(0, W + 1, size=N).astype(np.int32)
    perm = rng.permutation(N)[: max(1, int(rng.integers(1, N + 1)))]
    cuts = sorted(set(rng.integers(1, max(perm.size, 2), size=3).tolist()))
    bins = [b.tolist() for b in np.split(perm, [c for c in cuts if c < perm.size]) if b.size]
    width = oracle.trainer_width(rl, bins, q)
    check_rect(dev, rows, rl, q, bins, C=max(width, 1) + int(rng.integers(0, 9)), fold=fold,
               pad_token=-3)


def test_rect_errors(dev):
    rows = np.zeros((2, 4), dtype=np.int64)
    check_rect(dev, rows, [7, 3], 1, [[0, 1], []], C=3)      # BAD_LENGTH | EMPTY_PACK
    check_rect(dev, rows, [4, 4], 1, [[0, 1]], C=7)          # PACK_OVERFLOW


def test_rect_trainer_workload(dev):
    w = synth.trainer_rectangle()
    check_rect(dev, w["rows"], w["real_len"], w["q"], w["bins"])
    say("trainer workload via pack_padded_rows")
    out = psq.pack_padded_rows(torch.from_numpy(w["rows"]).to(dev), w["real_len"], w["bins"],
                               w["q"], width=w["width"])
    ref = oracle.pack_rect(w["rows"], w["real_len"], w["q"], w["bins"])
    assert ref["status"] == 0 and out["width"] == ref["width"] == w["width"]
    assert np.array_equal(out["input_ids"].cpu().numpy(), ref["packed"])
    assert np.array_equal(out["token_mask"].cpu().numpy(), ref["token_mask"])
    assert np.array_equal(out["cu_seqlens_flat"].cpu().numpy(), ref["cu_seqlens"])
    assert np.array_equal(out["cu_seqlens_padded_flat"].cpu().numpy(), ref["cu_seqlens_padded"])
    # the per-bin views are the CSR slices, each starting at 0
    k = 0
    for b, (c, cp) in enumerate(zip(out["cu_seqlens"], out["cu_seqlens_padded"])):
        n = len(w["bins"][b]) + 1
        assert c.cpu().tolist() == ref["cu_seqlens"][k:k + n].tolist()
        assert cp.cpu().tolist() == ref["cu_seqlens_padded"][k:k + n].tolist()
        k += n


def test_pack_padded_rows_rejects_bad_widths_and_lengths(dev):
    rows = torch.zeros((2, 10), dtype=torch.int64, device=dev)
    say("pack_padded_rows: width too small, length beyond int32")
    with pytest.raises(ValueError, match="capacity"):
        psq.pack_padded_rows(rows, [5, 10], [[0, 1]], 4, width=19)
    with pytest.raises(ValueError, match="int32"):
        psq.pack_padded_rows(rows, [5, 1 << 31], [[0, 1]], 4, width=20)


@pytest.mark.parametrize("seed", range(24))
def test_rows_path_fuzz(dev, seed):
    """Tables of at most 64 rows of at most 64 entries take the rows-in-wave
    path of the single-workgroup kernel; the same tables widened past 64
    entries per row with unused slots (identical outputs) take its general
    path.  Random shapes at and around those limits, any row-group count,
    half of them with planted faults, both paths against the oracle."""
    from test_gpu_parity import corrupt_tables, rand_tables as rand_tables_holes
    rng = np.random.default_rng(3000 + seed)
    B = int(rng.choice([1, 2, 3, 16, 33, 63, 64, int(rng.integers(1, 65))]))
    P = int(rng.choice([1, 2, 5, 31, 32, 33, 63, 64, int(rng.integers(1, 65))]))
    divisors = [g for g in range(1, B + 1) if B % g == 0]
    G = int(rng.choice(divisors))
    S = int(rng.choice([1, 4, 37, 512, 8192, int(rng.integers(1, 3000))]))
    q = int(rng.choice([1, 4, 8]))
    L, Lp = rand_tables_holes(rng, B, P, S, q, holes=bool(seed % 3 == 0))
    if seed % 2:
        L, Lp = corrupt_tables(rng, L, Lp, S, int(rng.integers(1, 3)))
    extra = np.full((B, 65), V)
    for lt, lpt in ((L, Lp), (np.hstack([L, extra]), np.hstack([Lp, extra]))):
        check_split(dev, lt, lpt, S, G)
        check_split(dev, lt, None, S, G)
        if G == 1:
            from test_gpu_parity import check_thd
            fits = np.abs(np.concatenate([lt, lpt])).max() < 2**31
            check_thd(dev, lt, lpt, S, torch.int32 if fits else torch.int64)
