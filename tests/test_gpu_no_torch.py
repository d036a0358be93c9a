"""The C ABI driven with ctypes and the HIP runtime alone: device memory
from hipMalloc, the null stream, no PyTorch object anywhere in the calls
(tests/no_torch_driver.py), on the pages' worked examples; the outputs are
compared here with the examples' values (tests/golden).  The driver runs in
this process (the GPU suite's process has started the GPU, so it starts no
other program); run on its own, it also reports that torch was never
loaded.  A CPU test checks that neither it nor the binding imports torch."""
import ast
import importlib.util
import json
import os

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _golden(name):
    with open(os.path.join(HERE, "golden", name)) as f:
        return json.load(f)


def _imports(path):
    tree = ast.parse(open(path).read())
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module:
            names.add(node.module.split(".")[0])
    return names


def test_driver_and_binding_import_no_torch():
    for path in (os.path.join(HERE, "no_torch_driver.py"),
                 os.path.join(ROOT, "varlen_attention_metadata_amd", "_lib.py")):
        assert "torch" not in _imports(path), path


@pytest.mark.gpu
def test_c_abi_without_torch():
    print("[case] C ABI with hipMalloc memory and the null stream", flush=True)
    spec = importlib.util.spec_from_file_location("no_torch_driver",
                                                  os.path.join(HERE, "no_torch_driver.py"))
    drv = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(drv)
    out = drv.run_examples()

    g = _golden("doc_map_example.json")["derived"]
    d = out["doc_map"]
    assert d["status"] == 0
    assert d["cu_seqlens"] == g["cu_seqlens"] and d["num_segments"] == g["num_segments"]
    assert d["max_seqlen"] == g["max_seqlen"] and d["padding_mask"] == g["padding_mask"]

    g = _golden("thd_example.json")
    t = out["thd"]
    assert t["status"] == 0
    assert t["cu_seqlens"] == g["printed"]["cu_seqlens"]
    assert t["cu_seqlens_padded"] == g["printed"]["cu_seqlens_padded"]
    assert t["max_seqlen"] == g["printed"]["max_seqlen"]
    assert len(t["flat_input_ids"]) == g["printed"]["flat_length"]
    assert t["flat_input_ids"] == sum(g["input"]["input_ids"], [])
    assert t["padding_mask"] == g["derived"]["padding_mask"]
    assert t["pad_between_seqs"] == g["derived"]["pad_between_seqs"]

    g = _golden("loader_pack_example.json")
    p = out["pack"]
    assert p["status"] == 0
    assert p["cu_seqlens"] == g["printed"]["cu_seqlens"]
    assert p["cu_seqlens_padded"] == g["printed"]["cu_seqlens_padded"]
    C = g["input"]["capacity"]
    assert len(p["packed"]) == C == g["printed"]["packed_shape"][1]
    ones = [i for i, m in enumerate(p["token_mask"]) if m]
    want = [i for a, b in g["derived"]["token_mask_ones"] for i in range(a, b)]
    assert ones == want and len(ones) == g["printed"]["real_tokens"]
    # the tokens sit where the mask is 1, in source order, and every other
    # slot holds the pad token 0; the slots past the last source's own pad
    # (its unfolded padded boundary) are the tail
    assert [p["packed"][i] for i in ones] == p["tokens"]
    assert all(p["packed"][i] == 0 for i in range(C) if i not in set(ones))
    last_source_end = g["derived"]["token_mask_ones"][-1][0] + p["cu_seqlens"][-1] - \
        p["cu_seqlens"][-2]
    q = g["input"]["pad_to"]
    tail_start = -(-last_source_end // q) * q
    assert C - tail_start == g["printed"]["tail_pad"]
