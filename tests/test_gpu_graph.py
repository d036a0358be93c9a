"""The C-ABI calls inside HIP graphs and on concurrent streams.

Every call enqueues only kernels (the workspace is cleared by the kernels
themselves and by a fill kernel, never by a memset node), so a captured call
can be replayed.  Each graph here is replayed several times with eager work
and synchronizations between replays, and every replay is compared with the
CPU oracle.  Calls on two streams with their own workspaces must not
interfere.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from varlen_attention_metadata_amd import _lib

pytestmark = pytest.mark.gpu
V = -1000


def say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def dev():
    _lib.load()
    return torch.device("cuda:0")


def zeroed_workspace(dev, nbytes):
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _lib.psq_workspace_init(ws.data_ptr(), ws.numel(), torch.cuda.current_stream(dev).cuda_stream)
    return ws


def replay_and_check(dev, call, outputs, check, replays=4):
    """Capture `call(stream)` in a graph, then replay it `replays` times with
    the outputs overwritten eagerly before each replay."""
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream(dev).cuda_stream)
    for rep in range(replays):
        for t in outputs:
            t.fill_(7 + rep)                     # eager work between replays
        torch.cuda.synchronize(dev)
        g.replay()
        torch.cuda.synchronize(dev)
        check(rep)


# workload 3's 16 x 64 tables (the single-workgroup kernel), and 64 x 128 tables
# (the multi-workgroup kernel with its ticket, look-back and clean-up, the
# 16-byte collapses fused into its launch)
@pytest.mark.parametrize("B,S,P", [(16, 8192, 64), (64, 4096, 128)],
                         ids=["single_workgroup", "multi_workgroup"])
def test_graph_thd_tables_with_copies(dev, B, S, P):
    w = synth.thd_tables(3, B=B, S=S, P=P)
    assert w["seq_lens"].shape == (B, P)
    T = B * S
    say(f"graph: thd tables {B}x{P} S={S} + 3 collapses")
    t = {k: torch.from_numpy(w[k]).to(dev) for k in
         ("input_ids", "labels", "position_ids", "seq_lens", "seq_lens_padded")}
    outs = {k: torch.empty(T, dtype=torch.int64, device=dev) for k in ("input_ids", "labels", "position_ids")}
    cu = torch.empty(B * P + 1, dtype=torch.int32, device=dev)
    cp = torch.empty_like(cu)
    mask = torch.empty(T, dtype=torch.uint8, device=dev)
    scal = torch.empty(4, dtype=torch.int32, device=dev)
    lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, t["seq_lens"].data_ptr(),
                           t["seq_lens_padded"].data_ptr(), _lib.I64, P, V)
    ws = zeroed_workspace(dev, _lib.psq_process_thd_workspace(lay, B, S))
    arr, n_c = _lib.make_copies([(t[k].data_ptr(), outs[k].data_ptr(), 1, T * 8, T * 8)
                                 for k in ("input_ids", "labels", "position_ids")])
    sp = scal.data_ptr()
    ref = oracle.thd_tables(w["seq_lens"], w["seq_lens_padded"], S)

    def call(stream):
        _lib.psq_process_thd(lay, B, S, cu.data_ptr(), cp.data_ptr(), sp, sp + 4, sp + 8,
                             mask.data_ptr(), arr, n_c, sp + 12, ws.data_ptr(), ws.numel(),
                             stream)

    def check(rep):
        n, mx, pb, st = scal.cpu().tolist()
        assert st == 0 and n == ref["num_seqs"], rep
        assert (mx, pb) == (ref["max_seqlen"], ref["pad_between_seqs"]), rep
        assert np.array_equal(cu[: n + 1].cpu().numpy(), ref["cu_seqlens"]), rep
        assert np.array_equal(cp[: n + 1].cpu().numpy(), ref["cu_seqlens_padded"]), rep
        assert np.array_equal(mask.cpu().numpy(), ref["padding_mask"]), rep
        for k in outs:
            assert np.array_equal(outs[k].cpu().numpy(), w[k].reshape(-1)), (rep, k)

    replay_and_check(dev, call, [cu, cp, mask, scal] + list(outs.values()), check)


# every document-map path: one workgroup; one launch of 32 tiles of 1024
# positions, of 220 tiles of 4096, of 256 tiles of 16384; and two launches
@pytest.mark.parametrize("B,S", [(4, 64), (8, 4096), (3, 300001), (1, 4194304), (3, 2100000)],
                         ids=["one_workgroup", "one_launch_1", "one_launch_4", "one_launch_16",
                              "two_launch"])
def test_graph_doc_map_with_copy(dev, B, S):
    d = synth.doc_map_medium(2, B, S)
    T = B * S
    H = 64 if T <= 100000 else 8
    say(f"graph: doc map {B}x{S} + bf16 collapse of {H} columns")
    doc = torch.from_numpy(d).to(dev)
    hidden = torch.randn((B, S, H), dtype=torch.bfloat16, device=dev)
    out_h = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    cu = torch.empty(T + 1, dtype=torch.int32, device=dev)
    mask = torch.empty(T, dtype=torch.uint8, device=dev)
    scal = torch.empty(4, dtype=torch.int32, device=dev)
    lay = _lib.make_layout(_lib.LAYOUT_DOC_IDS, doc_ids=doc.data_ptr(), doc_dtype=_lib.I32)
    ws = zeroed_workspace(dev, _lib.psq_process_thd_workspace(lay, B, S))
    arr, n_c = _lib.make_copies([(hidden.data_ptr(), out_h.data_ptr(), 1, hidden.numel() * 2,
                                  hidden.numel() * 2)])
    sp = scal.data_ptr()
    ref = oracle.doc_segments(d)

    def call(stream):
        _lib.psq_process_thd(lay, B, S, cu.data_ptr(), None, sp, sp + 4, sp + 8, mask.data_ptr(),
                             arr, n_c, sp + 12, ws.data_ptr(), ws.numel(), stream)

    def check(rep):
        n, mx, pb, st = scal.cpu().tolist()
        assert (n, mx, pb, st) == (ref["num_segments"], ref["max_seqlen"], 0, 0), rep
        assert np.array_equal(cu[: n + 1].cpu().numpy(), ref["cu_seqlens"]), rep
        assert np.array_equal(mask.cpu().numpy(), ref["padding_mask"]), rep
        assert torch.equal(out_h.view(torch.int16), hidden.reshape(T, H).view(torch.int16)), rep

    replay_and_check(dev, call, [cu, mask, scal, out_h], check)


def test_graph_pack_split_and_padids(dev):
    w = synth.pack_sources(N=2048)
    C, q = w["capacity"], w["q"]
    N = w["real_len"].size
    P = w["pack_start"].size - 1
    say(f"graph: squeeze of {N} sources into {P} packs, a 4-group split, a pad-id mask")
    src = torch.from_numpy(w["src"]).to(dev)
    off = torch.from_numpy(w["src_off"]).to(dev)
    rl = torch.from_numpy(w["real_len"]).to(dev)
    ps = torch.from_numpy(w["pack_start"]).to(dev)
    packed = torch.empty((P, C), dtype=torch.int64, device=dev)
    tm = torch.empty((P, C), dtype=torch.uint8, device=dev)
    pcu = torch.empty(N + P, dtype=torch.int32, device=dev)
    pcp = torch.empty(N + P, dtype=torch.int32, device=dev)
    pst = torch.empty(1, dtype=torch.int32, device=dev)
    ws_pack = zeroed_workspace(dev, _lib.psq_pack_rows_workspace(N, P, C))
    ref_pack = oracle.pack(w["src"], w["src_off"], w["real_len"], q, w["pack_start"], C)

    t3 = synth.thd_tables()
    S3 = t3["S"]
    B3, P3 = t3["seq_lens"].shape
    G = 4
    L = torch.from_numpy(t3["seq_lens"]).to(dev)
    Lp = torch.from_numpy(t3["seq_lens_padded"]).to(dev)
    cap = G * (B3 // G * P3 + 1)
    scu = torch.empty(cap, dtype=torch.int32, device=dev)
    scp = torch.empty(cap, dtype=torch.int32, device=dev)
    smask = torch.empty(B3 * S3, dtype=torch.uint8, device=dev)
    per = torch.empty((3, G), dtype=torch.int32, device=dev)
    sscal = torch.empty(2, dtype=torch.int32, device=dev)
    lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, L.data_ptr(), Lp.data_ptr(), _lib.I64, P3, V)
    ws_split = zeroed_workspace(dev, _lib.psq_split_thd_workspace(lay, B3, S3, G))
    noc, _ = _lib.make_copies([])
    ref_split = oracle.split_thd(t3["seq_lens"], t3["seq_lens_padded"], S3, G)

    pt = synth.pad_tail_stream()
    ids = torch.from_numpy(pt["input_ids"]).to(dev)
    Ti = ids.numel()
    imask = torch.empty(Ti, dtype=torch.uint8, device=dev)
    iscal = torch.empty(2, dtype=torch.int32, device=dev)
    ws_ids = zeroed_workspace(dev, _lib.psq_padding_mask_from_token_ids_workspace(Ti))
    ref_ids = oracle.pad_mask_from_ids(pt["input_ids"], pt["pad_id"])

    def call(stream):
        _lib.psq_pack_rows(src.data_ptr(), src.numel(), off.data_ptr(), rl.data_ptr(), N, q,
                           None, ps.data_ptr(), P, C, 1, 0, packed.data_ptr(), tm.data_ptr(),
                           pcu.data_ptr(), pcp.data_ptr(), pst.data_ptr(), ws_pack.data_ptr(),
                           ws_pack.numel(), stream)
        pp, sp = per.data_ptr(), sscal.data_ptr()
        _lib.psq_split_thd(lay, B3, S3, G, scu.data_ptr(), scp.data_ptr(), sp, pp, pp + 4 * G,
                           pp + 8 * G, smask.data_ptr(), noc, 0, sp + 4, ws_split.data_ptr(),
                           ws_split.numel(), stream)
        ip = iscal.data_ptr()
        _lib.psq_padding_mask_from_token_ids(ids.data_ptr(), _lib.I64, Ti, pt["pad_id"],
                                             imask.data_ptr(), ip, ip + 4, ws_ids.data_ptr(),
                                             ws_ids.numel(), stream)

    def check(rep):
        used = ref_pack["cu_seqlens"].size
        assert int(pst.item()) == 0, rep
        assert np.array_equal(packed.cpu().numpy(), ref_pack["packed"]), rep
        assert np.array_equal(tm.cpu().numpy(), ref_pack["token_mask"]), rep
        assert np.array_equal(pcu[:used].cpu().numpy(), ref_pack["cu_seqlens"]), rep
        assert np.array_equal(pcp[:used].cpu().numpy(), ref_pack["cu_seqlens_padded"]), rep
        width, st = sscal.cpu().tolist()
        assert st == 0 and width == ref_split["cu_seqlens"].shape[1], rep
        assert np.array_equal(scu[: G * width].view(G, width).cpu().numpy(), ref_split["cu_seqlens"]), rep
        assert np.array_equal(scp[: G * width].view(G, width).cpu().numpy(),
                              ref_split["cu_seqlens_padded"]), rep
        assert np.array_equal(per[1].cpu().numpy(), ref_split["max_seqlen"]), rep
        assert np.array_equal(smask.cpu().numpy().reshape(G, -1), ref_split["padding_mask"]), rep
        nc, ist = iscal.cpu().tolist()
        assert (nc, ist) == (ref_ids["num_content"], ref_ids["status"]), rep
        assert np.array_equal(imask.cpu().numpy(), ref_ids["padding_mask"]), rep

    replay_and_check(dev, call, [packed, tm, pcu, pcp, pst, scu, scp, smask, per, sscal, imask,
                                 iscal], check)


def test_graph_split_on_the_multi_workgroup_kernel(dev):
    """The split of 64 x 128 tables into 4 row groups: the multi-workgroup
    kernel stages each group's boundaries in the workspace and the last
    workgroup stacks them and clears the staging, on every replay."""
    w = synth.thd_tables(3, B=64, S=4096, P=128)
    B, P, S, G = 64, 128, 4096, 4
    say(f"graph: split of {B}x{P} tables into {G} row groups")
    L = torch.from_numpy(w["seq_lens"]).to(dev)
    Lp = torch.from_numpy(w["seq_lens_padded"]).to(dev)
    cap = G * (B // G * P + 1)
    cu = torch.empty(cap, dtype=torch.int32, device=dev)
    cp = torch.empty(cap, dtype=torch.int32, device=dev)
    mask = torch.empty(B * S, dtype=torch.uint8, device=dev)
    per = torch.empty((3, G), dtype=torch.int32, device=dev)
    scal = torch.empty(2, dtype=torch.int32, device=dev)
    lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, L.data_ptr(), Lp.data_ptr(), _lib.I64, P, V)
    ws = zeroed_workspace(dev, _lib.psq_split_thd_workspace(lay, B, S, G))
    noc, _ = _lib.make_copies([])
    ref = oracle.split_thd(w["seq_lens"], w["seq_lens_padded"], S, G)
    assert ref["status"] == 0
    pp, sp = per.data_ptr(), scal.data_ptr()

    def call(stream):
        _lib.psq_split_thd(lay, B, S, G, cu.data_ptr(), cp.data_ptr(), sp, pp, pp + 4 * G,
                           pp + 8 * G, mask.data_ptr(), noc, 0, sp + 4, ws.data_ptr(), ws.numel(),
                           stream)

    def check(rep):
        width, st = scal.cpu().tolist()
        assert st == 0 and width == ref["cu_seqlens"].shape[1], rep
        assert np.array_equal(cu[: G * width].view(G, width).cpu().numpy(), ref["cu_seqlens"]), rep
        assert np.array_equal(cp[: G * width].view(G, width).cpu().numpy(),
                              ref["cu_seqlens_padded"]), rep
        for i, key in enumerate(("num_seqs", "max_seqlen", "pad_between_seqs")):
            assert np.array_equal(per[i].cpu().numpy(), ref[key]), (rep, key)
        assert np.array_equal(mask.cpu().numpy().reshape(G, B // G * S), ref["padding_mask"]), rep

    replay_and_check(dev, call, [cu, cp, mask, per, scal], check)
    assert int(ws.count_nonzero().item()) == 0, "workspace left dirty"


def test_graph_trainer_squeeze(dev):
    """The trainer's squeeze of a 256-row rectangle into 15 bins: few enough
    chunks that the 256-slot kernel runs; its completion word is cleared by
    the last pack leader on every replay."""
    w = synth.trainer_rectangle()
    rows_np, rl_np, bins, q, C = w["rows"], w["real_len"], w["bins"], w["q"], w["width"]
    N, W = rows_np.shape
    order, start = oracle.bins_to_csr(bins)
    P = len(bins)
    ref = oracle.pack_rect(rows_np, rl_np, q, bins, width=C)
    assert ref["status"] == 0
    say(f"graph: trainer squeeze {N}x{W} into {P} bins of {C}")
    rows = torch.from_numpy(rows_np).to(dev)
    rl = torch.from_numpy(np.asarray(rl_np, dtype=np.int32)).to(dev)
    order_full = np.zeros(N, dtype=np.int32)
    order_full[:order.size] = order
    od = torch.from_numpy(order_full).to(dev)
    ps = torch.from_numpy(start).to(dev)
    packed = torch.empty((P, C), dtype=torch.int64, device=dev)
    tm = torch.empty((P, C), dtype=torch.uint8, device=dev)
    cu = torch.empty(N + P, dtype=torch.int32, device=dev)
    cp = torch.empty(N + P, dtype=torch.int32, device=dev)
    st = torch.empty(1, dtype=torch.int32, device=dev)
    ws = zeroed_workspace(dev, _lib.psq_pack_rows_workspace(N, P, C))
    used = order.size + P

    def call(stream):
        _lib.psq_pack_padded_rows(rows.data_ptr(), W, rl.data_ptr(), N, q, od.data_ptr(),
                                  ps.data_ptr(), P, C, 0, 0, packed.data_ptr(), tm.data_ptr(),
                                  cu.data_ptr(), cp.data_ptr(), st.data_ptr(), ws.data_ptr(),
                                  ws.numel(), stream)

    def check(rep):
        assert int(st.item()) == 0, rep
        assert np.array_equal(packed.cpu().numpy(), ref["packed"]), rep
        assert np.array_equal(tm.cpu().numpy(), ref["token_mask"]), rep
        assert np.array_equal(cu[:used].cpu().numpy(), ref["cu_seqlens"]), rep
        assert np.array_equal(cp[:used].cpu().numpy(), ref["cu_seqlens_padded"]), rep

    replay_and_check(dev, call, [packed, tm, cu, cp, st], check)
    assert int(ws.count_nonzero().item()) == 0, "workspace left dirty"


@pytest.mark.parametrize("dtype", [torch.int64, torch.int32])
def test_graph_pad_ids_grid_stride(dev, dtype):
    """The pad-id mask over 5 M ids: 2048 workgroups striding over more tiles
    than that (int64: 2442 tiles), its tagged words read and zeroed by the
    last workgroup on every replay; a planted pad id in the content."""
    T = 5_000_000
    w = synth.pad_tail_stream(9, T=T, tail_hi=T // 3)
    ids_np = w["input_ids"].copy()
    ids_np[12345] = w["pad_id"]
    ref = oracle.pad_mask_from_ids(ids_np, w["pad_id"])
    say(f"graph: pad ids T={T} {dtype}")
    ids = torch.from_numpy(ids_np).to(dev, dtype)
    mask = torch.empty(T, dtype=torch.uint8, device=dev)
    scal = torch.empty(2, dtype=torch.int32, device=dev)
    ws = zeroed_workspace(dev, _lib.psq_padding_mask_from_token_ids_workspace(T))
    kind = _lib.I64 if dtype == torch.int64 else _lib.I32
    sp = scal.data_ptr()

    def call(stream):
        _lib.psq_padding_mask_from_token_ids(ids.data_ptr(), kind, T, w["pad_id"],
                                             mask.data_ptr(), sp, sp + 4, ws.data_ptr(),
                                             ws.numel(), stream)

    def check(rep):
        nc, st = scal.cpu().tolist()
        assert st == ref["status"] and nc == ref["num_content"], rep
        assert np.array_equal(mask.cpu().numpy(), ref["padding_mask"]), rep

    replay_and_check(dev, call, [mask, scal], check)
    assert int(ws.count_nonzero().item()) == 0, "workspace left dirty"


def test_two_streams_with_own_workspaces(dev):
    """Two different tables on two streams at once, each with its workspace."""
    rng = np.random.default_rng(21)
    cases = []
    for k in range(2):
        B, P, S = 12 + 4 * k, 40, 3000
        L = np.full((B, P), V, dtype=np.int64)
        for r in range(B):
            m = int(rng.integers(1, P))
            L[r, :m] = rng.integers(0, S // (2 * m) + 1, size=m)
        cases.append((L, S))
    say("two streams, two workspaces")
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    bufs = []
    for (L, S), s in zip(cases, streams):
        B, P = L.shape
        tL = torch.from_numpy(L).to(dev)
        cu = torch.empty(B * P + 1, dtype=torch.int32, device=dev)
        mask = torch.empty(B * S, dtype=torch.uint8, device=dev)
        scal = torch.empty(4, dtype=torch.int32, device=dev)
        lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, tL.data_ptr(), None, _lib.I64, P, V)
        ws = zeroed_workspace(dev, _lib.psq_process_thd_workspace(lay, B, S))
        bufs.append((tL, cu, mask, scal, lay, ws, B, S, P))
    torch.cuda.synchronize(dev)
    arr, _ = _lib.make_copies([])
    for it in range(10):
        for (tL, cu, mask, scal, lay, ws, B, S, P), s in zip(bufs, streams):
            sp = scal.data_ptr()
            _lib.psq_process_thd(lay, B, S, cu.data_ptr(), None, sp, sp + 4, sp + 8,
                                 mask.data_ptr(), arr, 0, sp + 12, ws.data_ptr(), ws.numel(),
                                 s.cuda_stream)
    torch.cuda.synchronize(dev)
    for (L, S), (tL, cu, mask, scal, lay, ws, B, _, P) in zip(cases, bufs):
        ref = oracle.thd_tables(L, None, S)
        n, mx, pb, st = scal.cpu().tolist()
        assert st == 0 and n == ref["num_seqs"] and mx == ref["max_seqlen"]
        assert np.array_equal(cu[: n + 1].cpu().numpy(), ref["cu_seqlens"])
        assert np.array_equal(mask.cpu().numpy(), ref["padding_mask"])


def _big_tables(seed, B, P, S):
    rng = np.random.default_rng(seed)
    L = np.full((B, P), V, dtype=np.int64)
    for r in range(B):
        m = int(rng.integers(1, P))
        L[r, :m] = rng.integers(0, S // (2 * m) + 1, size=m)
    return L


def test_two_streams_protocol_kernels(dev):
    """The kernels that exchange records through the workspace on two
    streams at once: the one-launch document map (tile counts alternating
    between 256 and 147, int32 and int64 maps), the pad-id mask (one grid
    of 1465 workgroups, one of 2048 striding over 2442 tiles; clean and
    colliding streams) and the multi-workgroup table kernel (64 x 100
    entries).  Each stream has one workspace that all its calls share, as
    the Python binding does; every call writes its own outputs and each is
    compared with the oracle.  A 4 GiB fill heads each stream, so both
    streams' calls are queued before either starts and their kernels can
    run side by side (the streams sit on separate hardware queues)."""
    rounds = 4
    doc_shapes = [(16, 16384), (3, 100001)]
    pad_T = [3000001, 5000000]
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    plans = []
    for k in range(2):
        dtype = torch.int32 if k == 0 else torch.int64
        docs = [synth.doc_map_medium(40 + 2 * k + i, B, S) for i, (B, S) in enumerate(doc_shapes)]
        pw = synth.pad_tail_stream(7 + k, T=pad_T[k])
        ids_clean = pw["input_ids"].copy()
        ids_coll = ids_clean.copy()
        ids_coll[1000 + k] = pw["pad_id"]
        L = _big_tables(50 + k, 64, 100, 4096)
        lay_dummy = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, 1, None, _lib.I64, 100, V)
        need = max([_lib.load().psq_params_from_doc_ids_workspace(B, S) for B, S in doc_shapes]
                   + [_lib.load().psq_padding_mask_from_token_ids_workspace(pad_T[k]),
                      _lib.psq_process_thd_workspace(lay_dummy, 64, 4096)])
        plans.append(dict(
            dtype=dtype, docs=[torch.from_numpy(d).to(dev, dtype) for d in docs],
            doc_refs=[oracle.doc_segments(d) for d in docs],
            ids=[torch.from_numpy(x).to(dev) for x in (ids_clean, ids_coll)],
            pad_refs=[oracle.pad_mask_from_ids(x, pw["pad_id"]) for x in (ids_clean, ids_coll)],
            pad_id=pw["pad_id"], tL=torch.from_numpy(L).to(dev),
            thd_ref=oracle.thd_tables(L, None, 4096), ws=zeroed_workspace(dev, need)))
    outs = []
    for r in range(rounds):
        for k in range(2):
            B, S = doc_shapes[r % 2]
            T = pad_T[k]
            outs.append(dict(
                cu=torch.full((B * S + 1,), -7, dtype=torch.int32, device=dev),
                dmask=torch.full((B * S,), 7, dtype=torch.uint8, device=dev),
                pmask=torch.full((T,), 7, dtype=torch.uint8, device=dev),
                tcu=torch.full((64 * 100 + 1,), -7, dtype=torch.int32, device=dev),
                tmask=torch.full((64 * 4096,), 7, dtype=torch.uint8, device=dev),
                scal=torch.full((12,), -7, dtype=torch.int32, device=dev)))
    heads = [torch.empty(1 << 32, dtype=torch.uint8, device=dev) for _ in range(2)]
    torch.cuda.synchronize(dev)
    say("two streams: document maps, pad-id masks and tables, one workspace per stream")
    for k, s in enumerate(streams):
        with torch.cuda.stream(s):
            heads[k].fill_(k + 1)
    for r in range(rounds):
        for k, s in enumerate(streams):
            p, o = plans[k], outs[2 * r + k]
            B, S = doc_shapes[r % 2]
            dt = _lib.I32 if p["dtype"] == torch.int32 else _lib.I64
            ws, sp = p["ws"], o["scal"].data_ptr()
            st = s.cuda_stream
            assert _lib.load().psq_params_from_doc_ids(
                p["docs"][r % 2].data_ptr(), dt, B, S, o["cu"].data_ptr(), sp, sp + 4,
                o["dmask"].data_ptr(), sp + 8, ws.data_ptr(), ws.numel(), st) == 0
            assert _lib.load().psq_padding_mask_from_token_ids(
                p["ids"][r % 2].data_ptr(), _lib.I64, pad_T[k], p["pad_id"],
                o["pmask"].data_ptr(), sp + 12, sp + 16, ws.data_ptr(), ws.numel(), st) == 0
            lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, p["tL"].data_ptr(), None, _lib.I64,
                                   100, V)
            arr, _ = _lib.make_copies([])
            _lib.psq_process_thd(lay, 64, 4096, o["tcu"].data_ptr(), None, sp + 20, sp + 24,
                                 sp + 28, o["tmask"].data_ptr(), arr, 0, sp + 32, ws.data_ptr(),
                                 ws.numel(), st)
    torch.cuda.synchronize(dev)
    for r in range(rounds):
        for k in range(2):
            p, o = plans[k], outs[2 * r + k]
            say(f"two streams: check round {r} stream {k}")
            n, mx, dst, nc, pst, tn, tmx, tpb, tst = o["scal"].cpu().tolist()[:9]
            dref = p["doc_refs"][r % 2]
            assert dst == 0 and n == dref["num_segments"] and mx == dref["max_seqlen"]
            assert np.array_equal(o["cu"][: n + 1].cpu().numpy(), dref["cu_seqlens"])
            assert np.array_equal(o["dmask"].cpu().numpy(), dref["padding_mask"])
            pref = p["pad_refs"][r % 2]
            assert pst == pref["status"] and nc == pref["num_content"]
            assert np.array_equal(o["pmask"].cpu().numpy(), pref["padding_mask"])
            tref = p["thd_ref"]
            assert tst == 0 and tn == tref["num_seqs"] and tmx == tref["max_seqlen"]
            assert tpb == tref["pad_between_seqs"]
            assert np.array_equal(o["tcu"][: tn + 1].cpu().numpy(), tref["cu_seqlens"])
            assert np.array_equal(o["tmask"].cpu().numpy(), tref["padding_mask"])
    for p in plans:
        w = p["ws"].cpu().numpy()
        assert not w[:256].any() and not w[49664:].any(), "workspace left dirty"
