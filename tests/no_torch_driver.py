"""Drive the C ABI with ctypes and the HIP runtime alone, without PyTorch.

It loads the ctypes binding module by file path (the package's __init__
would import torch), allocates device memory with hipMalloc, and runs the
pages' three worked examples (the document map, process_input_for_thd's
Example, the loader's pack).  Run on its own (python tests/no_torch_driver.py)
it prints the outputs and whether torch was loaded as one JSON line;
tests/test_gpu_no_torch.py calls run_examples() in the test process and
compares the outputs with the examples' values.
"""
import ctypes
import importlib.util
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP = None      # the HIP runtime libpsq.so is linked against (see run_examples)
H2D, D2H = 1, 2


def hip_ok(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what}: hipError {rc}")


def load_binding():
    spec = importlib.util.spec_from_file_location(
        "psq_lib", os.path.join(ROOT, "varlen_attention_metadata_amd", "_lib.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


class Dev:
    """Device buffers, freed together."""

    def __init__(self):
        self.ptrs = []

    def alloc(self, nbytes):
        p = ctypes.c_void_p()
        hip_ok(HIP.hipMalloc(ctypes.byref(p), ctypes.c_size_t(max(nbytes, 1))), "hipMalloc")
        self.ptrs.append(p)
        return p.value

    def put(self, ctype, values):
        arr = (ctype * len(values))(*values)
        p = self.alloc(ctypes.sizeof(arr))
        hip_ok(HIP.hipMemcpy(ctypes.c_void_p(p), arr, ctypes.c_size_t(ctypes.sizeof(arr)), H2D),
               "hipMemcpy to device")
        return p

    def get(self, ctype, p, n):
        arr = (ctype * n)()
        hip_ok(HIP.hipDeviceSynchronize(), "hipDeviceSynchronize")
        hip_ok(HIP.hipMemcpy(arr, ctypes.c_void_p(p), ctypes.c_size_t(ctypes.sizeof(arr)), D2H),
               "hipMemcpy to host")
        return list(arr)

    def workspace(self, lib, nbytes):
        p = self.alloc(nbytes)
        lib.psq_workspace_init(p, max(nbytes, 1), None)
        return p, max(nbytes, 1)

    def free(self):
        for p in self.ptrs:
            HIP.hipFree(p)


def doc_map(lib, dev):
    doc = [1, 1, 2, 2, 2, 0]
    d = dev.put(ctypes.c_int32, doc)
    cu, scal, mask = dev.alloc(4 * 7), dev.alloc(4 * 3), dev.alloc(6)
    ws, wsb = dev.workspace(lib, lib.psq_params_from_doc_ids_workspace(1, 6))
    lib.psq_params_from_doc_ids(d, lib.I32, 1, 6, cu, scal, scal + 4, mask, scal + 8, ws, wsb,
                                None)
    n, mx, st = dev.get(ctypes.c_int32, scal, 3)
    return {"status": st, "num_segments": n, "max_seqlen": mx,
            "cu_seqlens": dev.get(ctypes.c_int32, cu, n + 1),
            "padding_mask": dev.get(ctypes.c_uint8, mask, 6)}


def thd_example(lib, dev, g):
    inp = g["input"]
    S = inp["S"]
    B, P = len(inp["seq_lens"]), len(inp["seq_lens"][0])
    L = dev.put(ctypes.c_int64, sum(inp["seq_lens"], []))
    Lp = dev.put(ctypes.c_int64, sum(inp["seq_lens_padded"], []))
    ids = sum(inp["input_ids"], [])
    src = dev.put(ctypes.c_int64, ids)
    dst = dev.alloc(8 * len(ids))
    cu, cp = dev.alloc(4 * (B * P + 1)), dev.alloc(4 * (B * P + 1))
    scal, mask = dev.alloc(4 * 4), dev.alloc(B * S)
    lay = lib.make_layout(lib.LAYOUT_SEQ_LENS, L, Lp, lib.I64, P, -1000)
    arr, n_c = lib.make_copies([(src, dst, 1, 8 * len(ids), 8 * len(ids))])
    ws, wsb = dev.workspace(lib, lib.psq_process_thd_workspace(lay, B, S))
    lib.psq_process_thd(lay, B, S, cu, cp, scal, scal + 4, scal + 8, mask, arr, n_c, scal + 12,
                        ws, wsb, None)
    n, mx, pb, st = dev.get(ctypes.c_int32, scal, 4)
    return {"status": st, "max_seqlen": mx, "pad_between_seqs": pb,
            "cu_seqlens": dev.get(ctypes.c_int32, cu, n + 1),
            "cu_seqlens_padded": dev.get(ctypes.c_int32, cp, n + 1),
            "padding_mask": dev.get(ctypes.c_uint8, mask, B * S),
            "flat_input_ids": dev.get(ctypes.c_int64, dst, len(ids))}


def loader_pack(lib, dev, g):
    inp = g["input"]
    rl = inp["real_len"]
    C, q = inp["capacity"], inp["pad_to"]
    # the sources' tokens, stored end to end: source i holds 100 (i + 1) + k
    tokens = [100 * (i + 1) + k for i, r in enumerate(rl) for k in range(r)]
    offs = [sum(rl[:i]) for i in range(len(rl))]
    members = inp["bins"][0]
    N, P = len(rl), 1
    src = dev.put(ctypes.c_int64, tokens)
    so = dev.put(ctypes.c_int64, offs)
    rlen = dev.put(ctypes.c_int32, rl)
    order = dev.put(ctypes.c_int32, members)
    ps = dev.put(ctypes.c_int64, [0, len(members)])
    packed, tmask = dev.alloc(8 * C), dev.alloc(C)
    cu, cp, st = dev.alloc(4 * (N + P)), dev.alloc(4 * (N + P)), dev.alloc(4)
    ws, wsb = dev.workspace(lib, lib.psq_pack_rows_workspace(N, P, C))
    lib.psq_pack_rows(src, len(tokens), so, rlen, N, q, order, ps, P, C, int(inp["fold"]), 0,
                      packed, tmask, cu, cp, st, ws, wsb, None)
    return {"status": dev.get(ctypes.c_int32, st, 1)[0], "tokens": tokens,
            "packed": dev.get(ctypes.c_int64, packed, C),
            "token_mask": dev.get(ctypes.c_uint8, tmask, C),
            "cu_seqlens": dev.get(ctypes.c_int32, cu, N + P),
            "cu_seqlens_padded": dev.get(ctypes.c_int32, cp, N + P)}


def run_examples():
    golden = os.path.join(ROOT, "tests", "golden")
    with open(os.path.join(golden, "thd_example.json")) as f:
        thd_g = json.load(f)
    with open(os.path.join(golden, "loader_pack_example.json")) as f:
        pack_g = json.load(f)
    global HIP
    lib = load_binding()
    lib.load()
    # by its soname: the runtime libpsq.so already loaded (a process may hold
    # only one, and one that uses PyTorch holds PyTorch's copy)
    HIP = ctypes.CDLL("libamdhip64.so.7")
    dev = Dev()
    try:
        print("[case] no-torch document map", file=sys.stderr, flush=True)
        out = {"doc_map": doc_map(lib, dev)}
        print("[case] no-torch process_input_for_thd example", file=sys.stderr, flush=True)
        out["thd"] = thd_example(lib, dev, thd_g)
        print("[case] no-torch loader pack example", file=sys.stderr, flush=True)
        out["pack"] = loader_pack(lib, dev, pack_g)
    finally:
        dev.free()
    return out


def main():
    out = run_examples()
    out["torch_loaded"] = "torch" in sys.modules
    print(json.dumps(out))


if __name__ == "__main__":
    main()
