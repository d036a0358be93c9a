"""psq_params_from_doc_ids_noalloc against psq_params_from_doc_ids.

The no-allocation entry point runs the same kernels with the library's own
per-GPU scratch in place of a caller's workspace.  Each case calls it through
the C ABI and compares every output bit for bit with the workspace call on
the same map (and both with the oracle).  The calls come in a row, from the
largest map down, so every call after the first finds the records an earlier
and larger call left in the shared scratch.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import varlen_attention_metadata_amd as psq
from varlen_attention_metadata_amd import _lib

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def dev():
    _lib.load()
    return torch.device("cuda:0")


def _outputs(dev, B, S):
    cu = torch.full((B * S + 1,), -7, dtype=torch.int32, device=dev)
    scal = torch.full((3,), -7, dtype=torch.int32, device=dev)
    mask = torch.full((max(B * S, 1),), 7, dtype=torch.uint8, device=dev)
    return cu, scal, mask


def _collect(cu, scal, mask, B, S):
    torch.cuda.synchronize()
    n, mx, st = scal.cpu().tolist()
    return cu[: n + 1].cpu().numpy(), n, mx, st, mask[: B * S].cpu().numpy()


def _noalloc(dev, d, dt, B, S):
    cu, scal, mask = _outputs(dev, B, S)
    sp = scal.data_ptr()
    _lib.psq_params_from_doc_ids_noalloc(d.data_ptr(), dt, B, S, cu.data_ptr(), sp, sp + 4,
                                         mask.data_ptr(), sp + 8,
                                         torch.cuda.current_stream(dev).cuda_stream)
    return _collect(cu, scal, mask, B, S)


def _with_workspace(dev, d, dt, B, S):
    cu, scal, mask = _outputs(dev, B, S)
    sp = scal.data_ptr()
    ws = psq.workspace_for(dev, _lib.psq_params_from_doc_ids_workspace(B, S))
    _lib.psq_params_from_doc_ids(d.data_ptr(), dt, B, S, cu.data_ptr(), sp, sp + 4,
                                 mask.data_ptr(), sp + 8, ws.data_ptr(), ws.numel(),
                                 torch.cuda.current_stream(dev).cuda_stream)
    return _collect(cu, scal, mask, B, S)


def _same(a, b):
    assert a[1:4] == b[1:4], (a[1:4], b[1:4])
    assert np.array_equal(a[0], b[0]), "cu_seqlens differ"
    assert np.array_equal(a[4], b[4]), "padding_mask differs"


def _maps():
    """Largest first: 256 workgroups (chunks of 4096 positions), 32 (chunks of
    1024) and 1, then an int64 map of 147 chunks of 2048, and a 4.2 M-position
    map whose two-launch workgroups walk two chunks each."""
    long_row = np.ones((1, 4096 * 1024 + 9), dtype=np.int32)
    long_row[0, 5000:9000] = 0
    long_row[0, 2_000_000:] = 3
    yield "stage map [32,32768]", synth.stage_embedding()["doc_ids"], torch.int32
    yield "doc_map_medium [8,4096]", synth.doc_map_medium(), torch.int32
    yield "doc_map_small [4,64]", synth.doc_map_small(), torch.int32
    yield "[3,100003] int64", synth.doc_map_medium(2, 3, 100003).astype(np.int64), torch.int64
    yield "[1,4194313] two chunks per workgroup", long_row, torch.int32
    yield "[2,3333] after the large one", synth.doc_map_medium(9, 2, 3333), torch.int32


def test_noalloc_calls_in_a_row_match_the_workspace_call(dev):
    for name, doc_np, tdt in _maps():
        say(f"noalloc {name}")
        B, S = doc_np.shape
        d = torch.from_numpy(np.ascontiguousarray(doc_np)).to(dev, tdt)
        dt = _lib.I32 if tdt == torch.int32 else _lib.I64
        got = _noalloc(dev, d, dt, B, S)
        want = _with_workspace(dev, d, dt, B, S)
        _same(got, want)
        ref = oracle.doc_segments(doc_np)
        assert got[3] == 0
        assert got[1] == ref["num_segments"] and got[2] == ref["max_seqlen"]
        assert np.array_equal(got[0], ref["cu_seqlens"])
        assert np.array_equal(got[4], ref["padding_mask"])


def test_noalloc_second_call_smaller(dev):
    """Exactly two calls: a map of 256 workgroups, then one of 32."""
    big = synth.stage_embedding()["doc_ids"]
    small = synth.doc_map_medium()
    for doc_np in (big, small):
        say(f"noalloc pair {doc_np.shape}")
        B, S = doc_np.shape
        d = torch.from_numpy(doc_np).to(dev)
        _same(_noalloc(dev, d, _lib.I32, B, S), _with_workspace(dev, d, _lib.I32, B, S))


def test_noalloc_empty_and_degenerate(dev):
    for B, S in ((0, 5), (3, 0), (1, 1), (4097, 1)):
        say(f"noalloc degenerate {B}x{S}")
        doc_np = np.arange(B * S, dtype=np.int32).reshape(B, S) % 3
        d = torch.from_numpy(doc_np).to(dev)
        _same(_noalloc(dev, d, _lib.I32, B, S), _with_workspace(dev, d, _lib.I32, B, S))


def test_noalloc_host_errors(dev):
    d = torch.zeros((2, 2), dtype=torch.int32, device=dev)
    x = d.data_ptr()
    rc = _lib.psq_params_from_doc_ids_noalloc(x, _lib.I32, 1 << 16, 1 << 15, x, x, x, None,
                                              None, None, check=False)
    assert rc == _lib.ERR_OVERFLOW
    rc = _lib.psq_params_from_doc_ids_noalloc(x, 9, 2, 2, x, x, x, None, None, None, check=False)
    assert rc == _lib.ERR_ARG
    rc = _lib.psq_params_from_doc_ids_noalloc(x, _lib.I32, 2, 2, None, x, x, None, None, None,
                                              check=False)
    assert rc == _lib.ERR_ARG


def test_noalloc_graph_replays(dev):
    """Captured in a HIP graph (no allocation under capture) and replayed with
    eager work between the replays; every replay equals the eager call."""
    doc_np = synth.stage_embedding()["doc_ids"]
    B, S = doc_np.shape
    d = torch.from_numpy(doc_np).to(dev)
    want = _with_workspace(dev, d, _lib.I32, B, S)
    cu, scal, mask = _outputs(dev, B, S)
    sp = scal.data_ptr()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _lib.psq_params_from_doc_ids_noalloc(d.data_ptr(), _lib.I32, B, S, cu.data_ptr(), sp,
                                             sp + 4, mask.data_ptr(), sp + 8,
                                             torch.cuda.current_stream().cuda_stream)
    other = synth.doc_map_medium()
    od = torch.from_numpy(other).to(dev)
    for rep in range(4):
        say(f"noalloc graph replay {rep}")
        cu.fill_(-7)
        mask.fill_(7)
        g.replay()
        got = _collect(cu, scal, mask, B, S)
        _same(got, want)
        # eager work between the replays, through the same scratch
        _noalloc(dev, od, _lib.I32, *other.shape)
    del g
