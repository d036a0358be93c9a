"""The C-ABI library on the host (CPU only): it loads, exports every
function ``include/psq.h`` declares, and rejects bad arguments before any
HIP call.  No case here reaches a kernel launch."""
import ctypes
import subprocess

import pytest

from varlen_attention_metadata_amd import _lib

FAKE = 0x10000          # never dereferenced: every case fails validation first


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_function(lib):
    names = _lib.header_functions()
    assert {"psq_params_from_doc_ids", "psq_process_thd", "psq_pack_rows",
            "psq_split_thd", "psq_padding_mask_from_token_ids", "psq_pack_padded_rows",
            "psq_status_string", "psq_workspace_init"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    assert _lib.status_string(0, False) == "ok"
    assert "workspace" in _lib.status_string(_lib.ERR_WORKSPACE, False)
    assert "capacity" in _lib.status_string(_lib.DATA_PACK_OVERFLOW, True)
    assert "no sequence" in _lib.status_string(_lib.DATA_EMPTY_ROW, True)
    assert _lib.status_string(999, False) == "unknown error code"
    assert "content" in _lib.status_string(_lib.DATA_PAD_IS_CONTENT, True)


def test_workspace_sizes(lib):
    assert lib.psq_params_from_doc_ids_workspace(0, 0) >= 256
    a = lib.psq_params_from_doc_ids_workspace(4, 64)
    b = lib.psq_params_from_doc_ids_workspace(32, 32768)
    assert a >= 256 and b > a and b % 256 == 0
    lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, FAKE, None, _lib.I64, 64)
    assert _lib.psq_process_thd_workspace(lay, 16, 8192) >= 256 + 8 * 16
    assert lib.psq_pack_rows_workspace(65536, 3555, 16384) >= 256
    assert lib.psq_padding_mask_from_token_ids_workspace(131072) >= 256
    # the split stages both boundary arrays of every group: 2 * 4 * G * (Bc*P+1)
    one = _lib.psq_split_thd_workspace(lay, 16, 8192, 1)
    four = _lib.psq_split_thd_workspace(lay, 16, 8192, 4)
    assert one == _lib.psq_process_thd_workspace(lay, 16, 8192)
    assert four >= one + 2 * 4 * 4 * (4 * 64 + 1)
    assert _lib.psq_split_thd_workspace(lay, 16, 8192, 3) == 0     # 3 does not divide 16
    assert _lib.psq_split_thd_workspace(lay, 16, 8192, 0) == 0
    # sizes the calls reject as overflowing: the queries return 0 and form no product
    assert lib.psq_params_from_doc_ids_workspace(1 << 40, 1 << 40) == 0
    assert lib.psq_params_from_doc_ids_workspace(1 << 16, 1 << 15) == 0   # B*S = 2^31
    assert lib.psq_params_from_doc_ids_workspace((1 << 16) - 1, 1 << 15) > 0
    assert _lib.psq_process_thd_workspace(lay, 1 << 40, 1 << 40) == 0
    huge = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, FAKE, None, _lib.I64, 1 << 40)
    assert _lib.psq_process_thd_workspace(huge, 1 << 40, 0) == 0
    assert _lib.psq_split_thd_workspace(huge, 1 << 40, 0, 1) == 0
    assert _lib.psq_split_thd_workspace(lay, 1 << 32, 0, 1 << 32) == 0
    assert _lib.psq_process_thd_workspace(_lib.make_layout(7), 4, 4) == 0
    doc = _lib.make_layout(_lib.LAYOUT_DOC_IDS, doc_ids=FAKE)
    assert _lib.psq_process_thd_workspace(doc, 4, 64) == a


def _doc(lib, **kw):
    a = dict(doc=FAKE, dt=_lib.I32, B=4, S=64, cu=FAKE, n=FAKE, mx=FAKE, mask=None,
             st=None, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.psq_params_from_doc_ids(a["doc"], a["dt"], a["B"], a["S"], a["cu"], a["n"],
                                       a["mx"], a["mask"], a["st"], a["ws"], a["wsb"], a["stream"])


def test_doc_ids_validation(lib):
    assert _doc(lib, B=-1) == _lib.ERR_ARG
    assert _doc(lib, S=-3) == _lib.ERR_ARG
    assert _doc(lib, dt=7) == _lib.ERR_ARG
    assert _doc(lib, B=1 << 16, S=1 << 15) == _lib.ERR_OVERFLOW
    assert _doc(lib, B=1, S=1 << 31) == _lib.ERR_OVERFLOW
    assert _doc(lib, cu=None) == _lib.ERR_ARG
    assert _doc(lib, doc=None) == _lib.ERR_ARG
    assert _doc(lib, ws=None) == _lib.ERR_WORKSPACE
    assert _doc(lib, ws=FAKE, wsb=8) == _lib.ERR_WORKSPACE


def _noalloc(lib, **kw):
    a = dict(doc=FAKE, dt=_lib.I32, B=4, S=64, cu=FAKE, n=FAKE, mx=FAKE, mask=None,
             st=None, stream=None)
    a.update(kw)
    return lib.psq_params_from_doc_ids_noalloc(a["doc"], a["dt"], a["B"], a["S"], a["cu"],
                                               a["n"], a["mx"], a["mask"], a["st"], a["stream"])


def test_doc_ids_noalloc_validation(lib):
    """The no-allocation entry point rejects what psq_params_from_doc_ids
    rejects, on the host, before it looks up its scratch."""
    assert _noalloc(lib, B=-1) == _lib.ERR_ARG
    assert _noalloc(lib, S=-3) == _lib.ERR_ARG
    assert _noalloc(lib, dt=7) == _lib.ERR_ARG
    assert _noalloc(lib, B=1 << 16, S=1 << 15) == _lib.ERR_OVERFLOW
    assert _noalloc(lib, B=1, S=1 << 31) == _lib.ERR_OVERFLOW
    assert _noalloc(lib, cu=None) == _lib.ERR_ARG
    assert _noalloc(lib, n=None) == _lib.ERR_ARG
    assert _noalloc(lib, mx=None) == _lib.ERR_ARG
    assert _noalloc(lib, doc=None) == _lib.ERR_ARG


def test_workspace_alignment(lib):
    """A workspace that is not 16-byte aligned is refused by every call before
    anything is enqueued (records are read as 16-byte vectors)."""
    for off in (4, 8, 12):
        assert _doc(lib, ws=FAKE + off, wsb=1 << 20) == _lib.ERR_WORKSPACE
        assert _padids(lib, ws=FAKE + off) == _lib.ERR_WORKSPACE
        assert _pack(lib, ws=FAKE + off) == _lib.ERR_WORKSPACE
        assert _rect(lib, ws=FAKE + off) == _lib.ERR_WORKSPACE
        lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, FAKE, FAKE, _lib.I64, 2)
        assert _thd(lib, lay, ws=FAKE + off, wsb=1 << 20) == _lib.ERR_WORKSPACE
        doc = _lib.make_layout(_lib.LAYOUT_DOC_IDS, doc_ids=FAKE)
        assert _thd(lib, doc, ws=FAKE + off, wsb=1 << 20) == _lib.ERR_WORKSPACE
        assert _split(lib, lay, ws=FAKE + off, wsb=1 << 20) == _lib.ERR_WORKSPACE


def _thd(lib, layout, copies=None, n_copies=0, **kw):
    a = dict(B=2, S=6, cu=FAKE, cp=None, n=FAKE, mx=FAKE, pb=FAKE, mask=None, st=FAKE,
             ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    if copies is None:
        copies, _ = _lib.make_copies([])
    lay = ctypes.byref(layout) if layout is not None else None
    return lib.psq_process_thd(lay, a["B"], a["S"], a["cu"], a["cp"], a["n"], a["mx"], a["pb"],
                               a["mask"], copies, n_copies, a["st"], a["ws"], a["wsb"],
                               a["stream"])


def test_process_thd_validation(lib):
    lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, FAKE, FAKE, _lib.I64, 2)
    assert _thd(lib, None) == _lib.ERR_ARG
    assert _thd(lib, lay, B=-1) == _lib.ERR_ARG
    assert _thd(lib, lay, st=None) == _lib.ERR_ARG
    assert _thd(lib, lay, cu=None) == _lib.ERR_ARG
    assert _thd(lib, _lib.make_layout(5)) == _lib.ERR_ARG
    assert _thd(lib, _lib.make_layout(_lib.LAYOUT_SEQ_LENS, FAKE, None, 9, 2)) == _lib.ERR_ARG
    assert _thd(lib, _lib.make_layout(_lib.LAYOUT_SEQ_LENS, FAKE, None, _lib.I64, -1)) == _lib.ERR_ARG
    assert _thd(lib, _lib.make_layout(_lib.LAYOUT_SEQ_LENS, None, None, _lib.I64, 2)) == _lib.ERR_ARG
    assert _thd(lib, _lib.make_layout(_lib.LAYOUT_DOC_IDS, doc_ids=FAKE, doc_dtype=3)) == _lib.ERR_ARG
    assert _thd(lib, _lib.make_layout(_lib.LAYOUT_DOC_IDS, doc_ids=None)) == _lib.ERR_ARG
    big = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, FAKE, None, _lib.I64, 1 << 20)
    assert _thd(lib, big, B=1 << 11, S=4) == _lib.ERR_OVERFLOW
    assert _thd(lib, lay, B=1 << 20, S=1 << 12) == _lib.ERR_OVERFLOW
    # S = 0 leaves B free of the row-length bound; B*P must still be bounded first
    huge = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, FAKE, None, _lib.I64, 1 << 40)
    assert _thd(lib, huge, B=1 << 40, S=0) == _lib.ERR_OVERFLOW
    assert _thd(lib, lay) == _lib.ERR_WORKSPACE           # wsb = 0
    assert _thd(lib, lay, ws=None, wsb=1 << 20) == _lib.ERR_WORKSPACE
    # copies: too many, null pointers, overlap, bad stride
    arr, _ = _lib.make_copies([(FAKE, FAKE + 4096, 1, 64, 64)] * 9)
    assert _thd(lib, lay, copies=arr, n_copies=9, wsb=1 << 20) == _lib.ERR_ARG
    arr, n = _lib.make_copies([(None, FAKE, 1, 64, 64)])
    assert _thd(lib, lay, copies=arr, n_copies=n, wsb=1 << 20) == _lib.ERR_ARG
    arr, n = _lib.make_copies([(FAKE, FAKE + 32, 1, 64, 64)])
    assert _thd(lib, lay, copies=arr, n_copies=n, wsb=1 << 20) == _lib.ERR_ARG
    arr, n = _lib.make_copies([(FAKE, FAKE + 65536, 4, 64, 32)])
    assert _thd(lib, lay, copies=arr, n_copies=n, wsb=1 << 20) == _lib.ERR_ARG
    arr, n = _lib.make_copies([(FAKE, FAKE + 65536, -1, 64, 64)])
    assert _thd(lib, lay, copies=arr, n_copies=n, wsb=1 << 20) == _lib.ERR_ARG
    # a destination stride below the row length, or negative
    arr, n = _lib.make_copies([(FAKE, FAKE + 65536, 4, 64, 64, 32)])
    assert _thd(lib, lay, copies=arr, n_copies=n, wsb=1 << 20) == _lib.ERR_ARG
    arr, n = _lib.make_copies([(FAKE, FAKE + 65536, 1, 64, 64, -8)])
    assert _thd(lib, lay, copies=arr, n_copies=n, wsb=1 << 20) == _lib.ERR_ARG
    # more units than one launch grid holds: 2^31 + 1 single-byte units
    arr, n = _lib.make_copies([(FAKE + 1, FAKE + (1 << 40), 1, (1 << 31) + 1, (1 << 31) + 1)])
    assert _thd(lib, lay, copies=arr, n_copies=n, wsb=1 << 20) == _lib.ERR_OVERFLOW
    arr, n = _lib.make_copies([(FAKE, FAKE + (1 << 40), 1 << 40, 1 << 30, 1 << 30)])
    assert _thd(lib, lay, copies=arr, n_copies=n, wsb=1 << 20) == _lib.ERR_OVERFLOW  # 2^70 B
    # one 256-thread workgroup per row chunk of 4096 slots: 2^24 rows need 2^32 threads
    assert _thd(lib, lay, B=1 << 24, S=64) == _lib.ERR_OVERFLOW
    assert _thd(lib, lay, B=(1 << 24) - 1, S=64) == _lib.ERR_WORKSPACE
    # ... and the fused 16-byte copy units (one thread each) count toward the same grid
    arr, n = _lib.make_copies([(FAKE, FAKE + (1 << 40), 1, 1 << 34, 1 << 34)])
    assert _thd(lib, lay, B=3 << 22, S=64, copies=arr, n_copies=n) == _lib.ERR_OVERFLOW
    assert _thd(lib, lay, B=(3 << 22) - 1, S=64, copies=arr, n_copies=n) == _lib.ERR_WORKSPACE
    # destination rows at a stride reaching back into the source
    arr, n = _lib.make_copies([(FAKE + 4096, FAKE, 4, 64, 64, 2048)])
    assert _thd(lib, lay, copies=arr, n_copies=n, wsb=1 << 20) == _lib.ERR_ARG


def _split(lib, layout, **kw):
    a = dict(B=4, S=6, G=2, cu=FAKE, cp=None, w=FAKE, n=FAKE, mx=FAKE, pb=FAKE, mask=None,
             st=FAKE, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    copies, _ = _lib.make_copies([])
    lay = ctypes.byref(layout) if layout is not None else None
    return lib.psq_split_thd(lay, a["B"], a["S"], a["G"], a["cu"], a["cp"], a["w"], a["n"],
                             a["mx"], a["pb"], a["mask"], copies, 0, a["st"], a["ws"], a["wsb"],
                             a["stream"])


def test_split_thd_validation(lib):
    lay = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, FAKE, FAKE, _lib.I64, 1)
    assert _split(lib, None) == _lib.ERR_ARG
    assert _split(lib, lay, G=0) == _lib.ERR_ARG
    assert _split(lib, lay, G=3) == _lib.ERR_ARG                   # does not divide B
    assert _split(lib, _lib.make_layout(_lib.LAYOUT_DOC_IDS, doc_ids=FAKE)) == _lib.ERR_ARG
    assert _split(lib, lay, w=None) == _lib.ERR_ARG
    wide = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, FAKE, FAKE, _lib.I64, 1, -(1 << 40))
    assert _split(lib, wide) == _lib.ERR_ARG                       # sentinel beyond int32
    assert _split(lib, lay, n=None) == _lib.ERR_ARG
    assert _split(lib, lay, st=None) == _lib.ERR_ARG
    assert _split(lib, lay, B=1 << 20, S=1 << 12, G=1 << 10) == _lib.ERR_OVERFLOW
    huge = _lib.make_layout(_lib.LAYOUT_SEQ_LENS, FAKE, FAKE, _lib.I64, 1 << 40)
    assert _split(lib, huge, B=1 << 40, S=0, G=1) == _lib.ERR_OVERFLOW
    assert _split(lib, lay, B=1 << 40, S=0, G=1 << 40) == _lib.ERR_OVERFLOW
    assert _split(lib, lay, B=1 << 32, S=0, G=1 << 32) == _lib.ERR_OVERFLOW
    assert _split(lib, lay, B=1 << 24, S=64, G=1 << 10) == _lib.ERR_OVERFLOW
    assert _split(lib, lay, B=(1 << 24) - 1024, S=64, G=1 << 10, ws=None) == _lib.ERR_WORKSPACE
    assert _split(lib, lay, ws=None) == _lib.ERR_WORKSPACE
    assert _split(lib, lay, wsb=256) == _lib.ERR_WORKSPACE


def _padids(lib, **kw):
    a = dict(ids=FAKE, dt=_lib.I64, T=64, pad=0, mask=FAKE, nc=None, st=FAKE, ws=FAKE,
             wsb=256, stream=None)
    a.update(kw)
    return lib.psq_padding_mask_from_token_ids(a["ids"], a["dt"], a["T"], a["pad"], a["mask"],
                                               a["nc"], a["st"], a["ws"], a["wsb"], a["stream"])


def test_padding_mask_from_token_ids_validation(lib):
    assert _padids(lib, T=-1) == _lib.ERR_ARG
    assert _padids(lib, dt=2) == _lib.ERR_ARG
    assert _padids(lib, T=1 << 31) == _lib.ERR_OVERFLOW
    assert _padids(lib, ids=None) == _lib.ERR_ARG
    assert _padids(lib, mask=None) == _lib.ERR_ARG
    assert _padids(lib, st=None) == _lib.ERR_ARG
    assert _padids(lib, ws=None) == _lib.ERR_WORKSPACE
    assert _padids(lib, wsb=8) == _lib.ERR_WORKSPACE


def _rect(lib, **kw):
    a = dict(rows=FAKE, W=10, rl=FAKE, N=2, q=4, order=None, ps=FAKE, P=1, C=20, fold=0,
             pad=0, packed=FAKE, tm=FAKE, cu=FAKE, cp=FAKE, st=FAKE, ws=FAKE, wsb=256,
             stream=None)
    a.update(kw)
    return lib.psq_pack_padded_rows(a["rows"], a["W"], a["rl"], a["N"], a["q"], a["order"],
                                    a["ps"], a["P"], a["C"], a["fold"], a["pad"], a["packed"],
                                    a["tm"], a["cu"], a["cp"], a["st"], a["ws"], a["wsb"],
                                    a["stream"])


def test_pack_padded_rows_validation(lib):
    assert _rect(lib, W=-1) == _lib.ERR_ARG
    assert _rect(lib, q=0) == _lib.ERR_ARG
    assert _rect(lib, C=0) == _lib.ERR_ARG
    assert _rect(lib, N=1 << 30, W=1 << 33) == _lib.ERR_OVERFLOW
    assert _rect(lib, rows=None) == _lib.ERR_ARG
    assert _rect(lib, rl=None) == _lib.ERR_ARG
    assert _rect(lib, ps=None) == _lib.ERR_ARG
    assert _rect(lib, cu=None) == _lib.ERR_ARG
    assert _rect(lib, ws=None) == _lib.ERR_WORKSPACE


def _pack(lib, **kw):
    a = dict(src=FAKE, src_len=100, off=FAKE, rl=FAKE, N=4, q=4, order=None, ps=FAKE, P=2,
             C=36, fold=1, pad=0, packed=FAKE, tm=FAKE, cu=FAKE, cp=FAKE, st=FAKE, ws=FAKE,
             wsb=256, stream=None)
    a.update(kw)
    return lib.psq_pack_rows(a["src"], a["src_len"], a["off"], a["rl"], a["N"], a["q"],
                             a["order"], a["ps"], a["P"], a["C"], a["fold"], a["pad"],
                             a["packed"], a["tm"], a["cu"], a["cp"], a["st"], a["ws"], a["wsb"],
                             a["stream"])


def test_pack_rows_validation(lib):
    assert _pack(lib, q=0) == _lib.ERR_ARG
    assert _pack(lib, C=0) == _lib.ERR_ARG
    assert _pack(lib, C=(1 << 30) + 1) == _lib.ERR_ARG
    assert _pack(lib, N=-1) == _lib.ERR_ARG
    assert _pack(lib, P=-1) == _lib.ERR_ARG
    assert _pack(lib, N=(1 << 31) - 5, P=10) == _lib.ERR_OVERFLOW
    assert _pack(lib, ps=None) == _lib.ERR_ARG
    assert _pack(lib, st=None) == _lib.ERR_ARG
    assert _pack(lib, packed=None) == _lib.ERR_ARG
    assert _pack(lib, rl=None) == _lib.ERR_ARG
    assert _pack(lib, src=None) == _lib.ERR_ARG
    assert _pack(lib, ws=None) == _lib.ERR_WORKSPACE
    assert _pack(lib, wsb=16) == _lib.ERR_WORKSPACE
    # one workgroup of 64 threads per chunk of a pack: 2^26 of them would need 2^32 threads
    assert _pack(lib, P=1 << 26, C=64, ws=None) == _lib.ERR_OVERFLOW
    assert _pack(lib, P=(1 << 26) - 1, C=64, ws=None) == _lib.ERR_WORKSPACE
    assert _pack(lib, P=1 << 22, C=16384, ws=None) == _lib.ERR_OVERFLOW     # 19 chunks each
    assert _pack(lib, P=1 << 21, C=16384, ws=None) == _lib.ERR_WORKSPACE
    assert _rect(lib, P=1 << 26, C=64, ws=None) == _lib.ERR_OVERFLOW
    assert _rect(lib, P=(1 << 26) - 1, C=64, ws=None) == _lib.ERR_WORKSPACE


def test_python_api_refuses_cpu_tensors():
    import torch
    import varlen_attention_metadata_amd as psq
    with pytest.raises(ValueError, match="GPU"):
        psq.packed_seq_params_from_doc_ids(torch.zeros((2, 3), dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        psq.process_input_for_thd({"input_ids": torch.zeros((1, 4), dtype=torch.int64),
                                   "position_ids": torch.zeros((1, 4), dtype=torch.int64),
                                   "seq_lens": torch.tensor([[4]])})
    with pytest.raises(ValueError, match="GPU"):
        psq.split_batch_into_thd_chunks({"input_ids": torch.zeros((2, 4), dtype=torch.int64),
                                         "position_ids": torch.zeros((2, 4), dtype=torch.int64),
                                         "seq_lens": torch.tensor([[4], [4]])}, 2)
    with pytest.raises(ValueError, match="GPU"):
        psq.thd_padding_mask_from_token_ids(torch.zeros(4, dtype=torch.int64), 0)
    with pytest.raises(ValueError, match="GPU"):
        psq.pack_padded_rows(torch.zeros((2, 4), dtype=torch.int64), [1, 2], [[0, 1]], 4, 8)


def test_workspace_status_drops_the_cached_workspace(monkeypatch):
    """A status word with the workspace bit raises and discards the stream's
    cached workspace (it may hold records left by a wait that gave up); any
    other bit raises and keeps it."""
    import torch
    import varlen_attention_metadata_amd as psq
    monkeypatch.setattr(psq, "_stream", lambda device: 77)
    dev = torch.device("cuda", 0)
    cache = psq._WORKSPACES
    saved = dict(cache)
    try:
        cache.clear()
        cache[(0, 77)] = "kept"
        cache[(0, 78)] = "other stream"
        with pytest.raises(ValueError, match="0x81"):
            psq._raise_status(_lib.DATA_BAD_LENGTH | _lib.DATA_WORKSPACE, "call", dev)
        assert (0, 77) not in cache and cache[(0, 78)] == "other stream"
        cache[(0, 77)] = "kept"
        with pytest.raises(ValueError, match="negative length"):
            psq._raise_status(_lib.DATA_BAD_LENGTH, "call", dev)
        assert cache[(0, 77)] == "kept"
        psq._raise_status(0, "call", dev)
    finally:
        cache.clear()
        cache.update(saved)


def test_readme_c_example_compiles(tmp_path):
    """The C example in README.md compiles as C99 against include/psq.h and
    the HIP runtime headers, with no warnings."""
    import os
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    text = open(os.path.join(root, "README.md")).read()
    blocks = re.findall(r"```c\n(.*?)```", text, flags=re.S)
    assert len(blocks) == 1
    src = tmp_path / "example.c"
    src.write_text(blocks[0])
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                        "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(root, "include"),
                        "-I", "/opt/rocm/include", str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_header_is_c_and_matches_the_binding(tmp_path):
    """``include/psq.h`` compiles as C99 and as C++, every function it declares
    links against ``libpsq.so``, and its structs and constants have the
    layout and values the ctypes binding assumes."""
    import os
    names = _lib.header_functions()
    src = tmp_path / "abi.c"
    src.write_text(
        "#include <stddef.h>\n#include <stdio.h>\n#include \"psq.h\"\n"
        "int main(void) {\n"
        "    const void *fns[] = {" + ", ".join(f"(const void *)&{n}" for n in names) + "};\n"
        "    size_t i, n = 0;\n"
        "    for (i = 0; i < sizeof fns / sizeof fns[0]; ++i) n += fns[i] != NULL;\n"
        "    printf(\"%zu\\n\", n);\n"
        "    printf(\"%zu %zu %zu %zu %zu %zu %zu\\n\", sizeof(psq_copy),\n"
        "           offsetof(psq_copy, src), offsetof(psq_copy, dst), offsetof(psq_copy, rows),\n"
        "           offsetof(psq_copy, row_bytes), offsetof(psq_copy, src_row_stride_bytes),\n"
        "           offsetof(psq_copy, dst_row_stride_bytes));\n"
        "    printf(\"%zu %zu %zu %zu %zu %zu %zu %zu %zu\\n\", sizeof(psq_thd_layout),\n"
        "           offsetof(psq_thd_layout, kind), offsetof(psq_thd_layout, seq_lens),\n"
        "           offsetof(psq_thd_layout, seq_lens_padded), offsetof(psq_thd_layout, lens_dtype),\n"
        "           offsetof(psq_thd_layout, P), offsetof(psq_thd_layout, pad_value),\n"
        "           offsetof(psq_thd_layout, doc_ids), offsetof(psq_thd_layout, doc_dtype));\n"
        "    printf(\"%d %d %d %d %d %d %d %d %d %d\\n\", PSQ_I32, PSQ_I64, PSQ_OK, PSQ_ERR_ARG,\n"
        "           PSQ_ERR_OVERFLOW, PSQ_ERR_WORKSPACE, PSQ_ERR_HIP, PSQ_LAYOUT_SEQ_LENS,\n"
        "           PSQ_LAYOUT_DOC_IDS, PSQ_MAX_COPIES);\n"
        "    printf(\"%d %d %d %d %d %d %d %d %d\\n\", PSQ_DATA_BAD_LENGTH,\n"
        "           PSQ_DATA_TABLE_MISMATCH, PSQ_DATA_ROW_OVERFLOW, PSQ_DATA_EMPTY_ROW,\n"
        "           PSQ_DATA_PACK_OVERFLOW, PSQ_DATA_EMPTY_PACK, PSQ_DATA_BAD_INDEX,\n"
        "           PSQ_DATA_WORKSPACE, PSQ_DATA_PAD_IS_CONTENT);\n"
        "    printf(\"%s\\n\", psq_status_string(PSQ_DATA_PACK_OVERFLOW, 1));\n"
        "    return 0;\n}\n")
    inc = os.path.dirname(_lib.HEADER)
    libdir = os.path.dirname(_lib.LIB_PATH)
    exe = tmp_path / "abi"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", inc, str(src),
                    "-L", libdir, "-l:libpsq.so", f"-Wl,-rpath,{libdir}",
                    "-Wl,--allow-shlib-undefined", "-o", str(exe)], check=True)
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Werror", "-fsyntax-only", "-x", "c++",
                    "-I", inc, str(src)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    assert int(out[0]) == len(names)
    C, L = _lib.PsqCopy, _lib.PsqThdLayout
    assert [int(x) for x in out[1].split()] == [ctypes.sizeof(C)] + [
        getattr(C, f).offset for f in ("src", "dst", "rows", "row_bytes",
                                       "src_row_stride_bytes", "dst_row_stride_bytes")]
    assert [int(x) for x in out[2].split()] == [ctypes.sizeof(L)] + [
        getattr(L, f).offset for f in ("kind", "seq_lens", "seq_lens_padded", "lens_dtype", "P",
                                       "pad_value", "doc_ids", "doc_dtype")]
    assert [int(x) for x in out[3].split()] == [
        _lib.I32, _lib.I64, _lib.OK, _lib.ERR_ARG, _lib.ERR_OVERFLOW, _lib.ERR_WORKSPACE,
        _lib.ERR_HIP, _lib.LAYOUT_SEQ_LENS, _lib.LAYOUT_DOC_IDS, _lib.MAX_COPIES]
    assert [int(x) for x in out[4].split()] == [
        _lib.DATA_BAD_LENGTH, _lib.DATA_TABLE_MISMATCH, _lib.DATA_ROW_OVERFLOW,
        _lib.DATA_EMPTY_ROW, _lib.DATA_PACK_OVERFLOW, _lib.DATA_EMPTY_PACK, _lib.DATA_BAD_INDEX,
        _lib.DATA_WORKSPACE, _lib.DATA_PAD_IS_CONTENT]
    assert out[5] == _lib.status_string(_lib.DATA_PACK_OVERFLOW, True)


def test_missing_library_fails_loudly(tmp_path):
    """Without the built HIP library there is no path at all: loading raises,
    and so does the first call of the torch-facing API in a fresh process
    whose library path points at nothing."""
    with pytest.raises(RuntimeError, match="build the HIP library"):
        _lib.open_library(str(tmp_path / "libpsq.so"))
    import os
    import sys
    code = ("import torch, varlen_attention_metadata_amd as psq\n"
            "from varlen_attention_metadata_amd import _lib\n"
            f"_lib.LIB_PATH = {str(tmp_path / 'libpsq.so')!r}\n"
            "try:\n"
            "    _lib.psq_params_from_doc_ids_workspace(1, 1)\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                         check=True).stdout
    assert out.startswith("raised:") and "is missing" in out
