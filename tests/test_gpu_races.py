"""Race tests: the kernels with cross-workgroup protocols, run on the
race-test build of the library (``libpsq_jitter.so``, built with PSQ_JITTER).

In that build every wave sleeps a pseudo-random time, drawn afresh on each
call, before each protocol step: claiming a tile ticket, publishing a
look-back descriptor, looking back, and counting itself finished.  The
orders in which workgroups reach those steps are therefore shuffled from
call to call.  Each case runs repeatedly on the same inputs and every run
must equal the CPU oracle exactly and leave the workspace zero-filled.

A last case interleaves random calls of the three kernels that exchange
records through the workspace (maps, pad-id streams, split tables), all
through one shared workspace.

The kernels covered: the one-launch document map of up to 256 tiles of
1024 to 16384 positions (tagged records, waits on the earlier tiles, the
last tile's reset of the state),
the multi-workgroup length-table kernel with and without row groups (ticket,
look-back over rows, completion count), the squeeze (completion word) and
the pad-id mask (tagged words, read and zeroed by the last workgroup).  Larger document maps take two
launches with no cross-workgroup step (the second reads the first one's
records); they run here too, as a repeat check.  The single-workgroup table
kernel has no cross-workgroup step.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from varlen_attention_metadata_amd import _build, _lib

pytestmark = pytest.mark.gpu
V = -1000
# runs per case; PSQ_RACE_REPEATS raises it for a longer stress run
REPEATS = int(os.environ.get("PSQ_RACE_REPEATS", "6"))


def say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def jl():
    return _lib.open_library(_build.JITTER_LIB)


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _workspace(dev, nbytes):
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=dev)


def _assert_zero(ws, scratch=None):
    """Every byte a call relies on finding zero is zero again; ``scratch`` is a
    (start, end) byte range the call may leave holding data (the document-map
    region: records and the one-launch state)."""
    torch.cuda.synchronize()
    kept = ws.clone()
    if scratch is not None:
        kept[scratch[0]:scratch[1]] = 0
    assert int(kept.count_nonzero()) == 0, "workspace not left zero-filled"


# tiles of 1024 positions: (8, 4096) 32, (16, 16384) 256, (7, 9000) 62, (2, 4097) 9;
# of 2048: (3, 100003) 147; of 4096: (32, 32768) 256; of 8192: (1, 257 * 4096) 129;
# of 16384: (16, 131072) 128; (2, 2100000) takes two launches
@pytest.mark.parametrize("shape", [(8, 4096), (32, 32768), (3, 100003), (16, 16384), (7, 9000),
                                   (2, 4097), (1, 257 * 4096), (16, 131072), (2, 2100000)])
def test_doc_map_tiles_under_jitter(jl, dev, shape):
    B, S = shape
    doc_np = synth.stage_embedding(5, B, S)["doc_ids"] if S == 32768 else \
        synth.doc_map_medium(2, B, S)
    ref = oracle.doc_segments(doc_np)
    d = torch.from_numpy(doc_np).to(dev)
    ws = _workspace(dev, jl.psq_params_from_doc_ids_workspace(B, S))
    for rep in range(REPEATS):
        say(f"jitter doc map {shape} run {rep}")
        cu = torch.full((B * S + 1,), -7, dtype=torch.int32, device=dev)
        mask = torch.full((B * S,), 7, dtype=torch.uint8, device=dev)
        scal = torch.full((3,), -7, dtype=torch.int32, device=dev)
        sp = scal.data_ptr()
        assert jl.psq_params_from_doc_ids(d.data_ptr(), _lib.I32, B, S, cu.data_ptr(), sp,
                                          sp + 4, mask.data_ptr(), sp + 8, ws.data_ptr(),
                                          ws.numel(), _stream(dev)) == 0
        n, mx, st = scal.cpu().tolist()
        assert st == 0
        assert n == ref["num_segments"] and mx == ref["max_seqlen"]
        assert np.array_equal(cu[: n + 1].cpu().numpy(), ref["cu_seqlens"])
        assert np.array_equal(mask.cpu().numpy(), ref["padding_mask"])
        _assert_zero(ws, scratch=(256, 49664))


def test_doc_map_one_launch_sequence_under_jitter(jl, dev):
    """One workspace, tile counts and sizes going up and down (256 of 4096
    positions, 32 of 1024, 256 of 4096, 12 of 1024, 129 of 4096, 129 of 8192,
    a two-launch map, 256 of 4096): every call's tagged records must be told
    apart from the previous calls' under shuffled progress."""
    shapes = [(32, 32768), (8, 4096), (32, 32768), (3, 4096), (129, 4096), (1, 257 * 4096),
              (2, 2100000), (32, 32768)]
    maps = [synth.doc_map_medium(20 + i, B, S) for i, (B, S) in enumerate(shapes)]
    refs = [oracle.doc_segments(m) for m in maps]
    ws = _workspace(dev, max(jl.psq_params_from_doc_ids_workspace(B, S) for B, S in shapes))
    for rep in range(REPEATS):
        for (B, S), doc_np, ref in zip(shapes, maps, refs):
            say(f"jitter doc map sequence {B}x{S} run {rep}")
            d = torch.from_numpy(doc_np).to(dev)
            cu = torch.full((B * S + 1,), -7, dtype=torch.int32, device=dev)
            scal = torch.full((3,), -7, dtype=torch.int32, device=dev)
            sp = scal.data_ptr()
            assert jl.psq_params_from_doc_ids(d.data_ptr(), _lib.I32, B, S, cu.data_ptr(), sp,
                                              sp + 4, None, sp + 8, ws.data_ptr(), ws.numel(),
                                              _stream(dev)) == 0
            n, mx, st = scal.cpu().tolist()
            assert st == 0 and n == ref["num_segments"] and mx == ref["max_seqlen"]
            assert np.array_equal(cu[: n + 1].cpu().numpy(), ref["cu_seqlens"])
    _assert_zero(ws, scratch=(256, 49664))


def _tables(seed, B, P, S):
    rng = np.random.default_rng(seed)
    L = np.full((B, P), V, dtype=np.int64)
    Lp = np.full((B, P), V, dtype=np.int64)
    for r in range(B):
        used = 0
        for j in range(int(rng.integers(1, P + 1))):
            real = int(rng.integers(0, 12))
            padded = -(-real // 4) * 4 + 4 * int(rng.integers(0, 2))
            if used + padded > S:
                break
            L[r, j], Lp[r, j] = real, padded
            used += padded
        if not (L[r] != V).any():
            L[r, 0], Lp[r, 0] = 0, 0
    return L, Lp


# all above the single-workgroup table size, so the multi-workgroup kernel runs
@pytest.mark.parametrize("B,P,S,G", [(1100, 4, 64, 1), (80, 64, 5000, 1), (600, 4, 64, 300),
                                     (160, 32, 300, 8)])
def test_tables_under_jitter(jl, dev, B, P, S, G):
    L, Lp = _tables(B * 31 + P, B, P, S)
    ref = oracle.split_thd(L, Lp, S, G) if G > 1 else oracle.thd_tables(L, Lp, S)
    assert ref["status"] == 0
    tL, tLp = torch.from_numpy(L).to(dev), torch.from_numpy(Lp).to(dev)
    lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, tL.data_ptr(), tLp.data_ptr(), _lib.I64, P, V)
    Bc = B // G
    cap = G * (Bc * P + 1)
    ws = _workspace(dev, jl.psq_split_thd_workspace(ctypes.byref(lay), B, S, G))
    arr, n_c = _lib.make_copies([])
    for rep in range(REPEATS):
        say(f"jitter tables B={B} P={P} S={S} G={G} run {rep}")
        cu = torch.full((cap,), -7, dtype=torch.int32, device=dev)
        cp = torch.full((cap,), -7, dtype=torch.int32, device=dev)
        mask = torch.full((B * S,), 7, dtype=torch.uint8, device=dev)
        per = torch.full((3, G), -7, dtype=torch.int32, device=dev)
        scal = torch.full((2,), -7, dtype=torch.int32, device=dev)
        pp, sp = per.data_ptr(), scal.data_ptr()
        assert jl.psq_split_thd(ctypes.byref(lay), B, S, G, cu.data_ptr(), cp.data_ptr(), sp,
                                pp, pp + 4 * G, pp + 8 * G, mask.data_ptr(), arr, n_c, sp + 4,
                                ws.data_ptr(), ws.numel(), _stream(dev)) == 0
        width, st = scal.cpu().tolist()
        assert st == 0
        got_mask = mask.cpu().numpy()
        if G == 1:
            n = int(per[0, 0].item())
            assert n == ref["num_seqs"]
            assert np.array_equal(cu[: n + 1].cpu().numpy(), ref["cu_seqlens"])
            assert np.array_equal(cp[: n + 1].cpu().numpy(), ref["cu_seqlens_padded"])
            assert int(per[1, 0].item()) == ref["max_seqlen"]
            assert int(per[2, 0].item()) == ref["pad_between_seqs"]
            assert np.array_equal(got_mask, ref["padding_mask"])
        else:
            assert width == ref["cu_seqlens"].shape[1]
            assert np.array_equal(cu[: G * width].view(G, width).cpu().numpy(), ref["cu_seqlens"])
            assert np.array_equal(cp[: G * width].view(G, width).cpu().numpy(),
                                  ref["cu_seqlens_padded"])
            for i, key in enumerate(("num_seqs", "max_seqlen", "pad_between_seqs")):
                assert np.array_equal(per[i].cpu().numpy(), ref[key]), key
            assert np.array_equal(got_mask.reshape(G, Bc * S), ref["padding_mask"])
        _assert_zero(ws)


def test_pack_under_jitter(jl, dev):
    w = synth.pack_sources(4, N=4096)
    C, q = w["capacity"], w["q"]
    src, off, rl, ps = w["src"], w["src_off"], w["real_len"], w["pack_start"]
    N, P = rl.size, ps.size - 1
    ref = oracle.pack(src, off, rl, q, ps, C, fold=True)
    assert ref["status"] == 0
    t = [torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (src, off, rl, ps)]
    ws = _workspace(dev, jl.psq_pack_rows_workspace(N, P, C))
    for rep in range(REPEATS):
        say(f"jitter pack N={N} P={P} run {rep}")
        packed = torch.full((P, C), -5, dtype=torch.int64, device=dev)
        tm = torch.full((P, C), 9, dtype=torch.uint8, device=dev)
        cu = torch.full((N + P,), -7, dtype=torch.int32, device=dev)
        cp = torch.full((N + P,), -7, dtype=torch.int32, device=dev)
        st = torch.full((1,), -7, dtype=torch.int32, device=dev)
        assert jl.psq_pack_rows(t[0].data_ptr(), src.size, t[1].data_ptr(), t[2].data_ptr(), N,
                                q, None, t[3].data_ptr(), P, C, 1, 0, packed.data_ptr(),
                                tm.data_ptr(), cu.data_ptr(), cp.data_ptr(), st.data_ptr(),
                                ws.data_ptr(), ws.numel(), _stream(dev)) == 0
        assert int(st.item()) == 0
        assert np.array_equal(packed.cpu().numpy(), ref["packed"])
        assert np.array_equal(tm.cpu().numpy(), ref["token_mask"])
        assert np.array_equal(cu.cpu().numpy(), ref["cu_seqlens"])
        assert np.array_equal(cp.cpu().numpy(), ref["cu_seqlens_padded"])
        _assert_zero(ws)


@pytest.mark.parametrize("T", [1 << 20, 5_000_000])
@pytest.mark.parametrize("kind", ["tail", "collide"])
def test_pad_ids_under_jitter(jl, dev, kind, T):
    w = synth.pad_tail_stream(7, T=T)
    ids = w["input_ids"].copy()
    pad = w["pad_id"]
    if kind == "collide":
        ids[1000] = pad
    ref = oracle.pad_mask_from_ids(ids, pad)
    t = torch.from_numpy(ids).to(dev)
    ws = _workspace(dev, jl.psq_padding_mask_from_token_ids_workspace(T))
    for rep in range(REPEATS):
        say(f"jitter pad ids {kind} T={T} run {rep}")
        mask = torch.full((T,), 7, dtype=torch.uint8, device=dev)
        scal = torch.full((2,), -7, dtype=torch.int32, device=dev)
        sp = scal.data_ptr()
        assert jl.psq_padding_mask_from_token_ids(t.data_ptr(), _lib.I64, T, pad,
                                                  mask.data_ptr(), sp, sp + 4, ws.data_ptr(),
                                                  ws.numel(), _stream(dev)) == 0
        nc, st = scal.cpu().tolist()
        assert st == ref["status"]
        assert np.array_equal(mask.cpu().numpy(), ref["padding_mask"])
        assert nc == ref["num_content"]
        _assert_zero(ws)


def test_random_calls_share_one_workspace_under_jitter(jl, dev):
    """Random calls of the three kernels that exchange records through the
    workspace, interleaved through one workspace as the Python binding shares
    it on a stream: document maps of 4097 to 6 M positions (the one-launch
    path at every chunk size, and two launches), pad-id streams of up to 5 M
    ids with and without a planted pad id, and length tables above the
    single-workgroup size split into random row groups.  Each call's outputs
    equal the oracle's; the workspace is clean at the end."""
    rng = np.random.default_rng(2024)

    def lu(lo, hi):
        return int(np.exp(rng.uniform(np.log(lo), np.log(hi + 1))))

    cases = []
    for i in range(60):
        kind = i % 3
        if kind == 0:
            total = lu(4097, 6_000_000)
            B = max(1, min(lu(1, 64), total // 64))
            S = max(1, total // B)
            cases.append(("doc", B, S, synth.doc_map_medium(300 + i, B, min(S, 4096))
                          if S <= 4096 else None))
        elif kind == 1:
            cases.append(("pad", lu(1, 5_000_000)))
        else:
            B = lu(1, 1200)
            P = max(-(-4097 // B), lu(1, 16))
            G = int(rng.choice([g for g in range(1, min(B, 300) + 1) if B % g == 0]))
            cases.append(("tables", B, P, lu(64, 5000), G))
    need = 256
    for c in cases:
        if c[0] == "doc":
            need = max(need, jl.psq_params_from_doc_ids_workspace(c[1], c[2]))
        elif c[0] == "pad":
            need = max(need, jl.psq_padding_mask_from_token_ids_workspace(c[1]))
        else:
            lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, 1, 1, _lib.I64, c[2], V)
            need = max(need, jl.psq_split_thd_workspace(ctypes.byref(lay), c[1], c[3], c[4]))
    ws = _workspace(dev, need)
    arr, n_c = _lib.make_copies([])
    for i, c in enumerate(cases):
        if c[0] == "doc":
            B, S = c[1], c[2]
            d = c[3] if c[3] is not None else np.repeat(
                rng.integers(0, 4, size=(B, S // 97 + 1)), 97, axis=1)[:, :S].astype(np.int32)
            say(f"jitter random call {i}: doc map {B}x{S}")
            ref = oracle.doc_segments(d)
            t = torch.from_numpy(np.ascontiguousarray(d)).to(dev)
            cu = torch.full((B * S + 1,), -7, dtype=torch.int32, device=dev)
            mask = torch.full((B * S,), 7, dtype=torch.uint8, device=dev)
            scal = torch.full((3,), -7, dtype=torch.int32, device=dev)
            sp = scal.data_ptr()
            assert jl.psq_params_from_doc_ids(t.data_ptr(), _lib.I32, B, S, cu.data_ptr(), sp,
                                              sp + 4, mask.data_ptr(), sp + 8, ws.data_ptr(),
                                              ws.numel(), _stream(dev)) == 0
            n, mx, st = scal.cpu().tolist()
            assert st == 0 and n == ref["num_segments"] and mx == ref["max_seqlen"]
            assert np.array_equal(cu[: n + 1].cpu().numpy(), ref["cu_seqlens"])
            assert np.array_equal(mask.cpu().numpy(), ref["padding_mask"])
        elif c[0] == "pad":
            T = c[1]
            w = synth.pad_tail_stream(400 + i, T=T, tail_hi=max(1, T // 2))
            ids = w["input_ids"].copy()
            if rng.random() < 0.3:
                ids[int(rng.integers(0, T))] = w["pad_id"]
            say(f"jitter random call {i}: pad ids T={T}")
            ref = oracle.pad_mask_from_ids(ids, w["pad_id"])
            t = torch.from_numpy(ids).to(dev)
            mask = torch.full((T,), 7, dtype=torch.uint8, device=dev)
            scal = torch.full((2,), -7, dtype=torch.int32, device=dev)
            sp = scal.data_ptr()
            assert jl.psq_padding_mask_from_token_ids(t.data_ptr(), _lib.I64, T, w["pad_id"],
                                                      mask.data_ptr(), sp, sp + 4, ws.data_ptr(),
                                                      ws.numel(), _stream(dev)) == 0
            nc, st = scal.cpu().tolist()
            assert st == ref["status"] and nc == ref["num_content"]
            assert np.array_equal(mask.cpu().numpy(), ref["padding_mask"])
        else:
            B, P, S, G = c[1], c[2], c[3], c[4]
            L, Lp = _tables(500 + i, B, P, S)
            say(f"jitter random call {i}: tables B={B} P={P} S={S} G={G}")
            ref = oracle.split_thd(L, Lp, S, G)
            assert ref["status"] == 0
            tL, tLp = torch.from_numpy(L).to(dev), torch.from_numpy(Lp).to(dev)
            lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, tL.data_ptr(), tLp.data_ptr(), _lib.I64,
                                   P, V)
            cap = G * (B // G * P + 1)
            cu = torch.full((cap,), -7, dtype=torch.int32, device=dev)
            cp = torch.full((cap,), -7, dtype=torch.int32, device=dev)
            mask = torch.full((B * S,), 7, dtype=torch.uint8, device=dev)
            per = torch.full((3, G), -7, dtype=torch.int32, device=dev)
            scal = torch.full((2,), -7, dtype=torch.int32, device=dev)
            pp, sp = per.data_ptr(), scal.data_ptr()
            assert jl.psq_split_thd(ctypes.byref(lay), B, S, G, cu.data_ptr(), cp.data_ptr(), sp,
                                    pp, pp + 4 * G, pp + 8 * G, mask.data_ptr(), arr, n_c,
                                    sp + 4, ws.data_ptr(), ws.numel(), _stream(dev)) == 0
            width, st = scal.cpu().tolist()
            assert st == 0 and width == ref["cu_seqlens"].shape[1]
            assert np.array_equal(cu[: G * width].view(G, width).cpu().numpy(), ref["cu_seqlens"])
            assert np.array_equal(cp[: G * width].view(G, width).cpu().numpy(),
                                  ref["cu_seqlens_padded"])
            for j, key in enumerate(("num_seqs", "max_seqlen", "pad_between_seqs")):
                assert np.array_equal(per[j].cpu().numpy(), ref[key]), key
            assert np.array_equal(mask.cpu().numpy().reshape(G, B // G * S), ref["padding_mask"])
    _assert_zero(ws, scratch=(256, 49664))
