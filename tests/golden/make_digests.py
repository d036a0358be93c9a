"""Write ``workload_digests.json``: SHA-256 digests of the oracle's outputs on
every benchmark workload.

``bench.py`` compares the GPU outputs of its timed calls with these digests, so
the benchmark checks parity in the same run without calling the oracle itself.
This script calls only ``oracle/`` (and ``synth/`` for the seeded inputs);
no value here comes from the GPU path.  Run it again whenever the oracle or a
generator changes:

    python tests/golden/make_digests.py
"""
from __future__ import annotations

import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(HERE, "workload_digests.json")


def digest(a, dtype) -> str:
    return hashlib.sha256(np.ascontiguousarray(np.asarray(a), dtype=dtype).tobytes()).hexdigest()


def compute() -> dict:
    d = {}
    for name, gen in (("doc_map_small", synth.doc_map_small), ("doc_map_medium", synth.doc_map_medium)):
        r = oracle.doc_segments(gen(), want_mask=False)
        d[name] = {"num_segments": r["num_segments"], "max_seqlen": r["max_seqlen"],
                   "cu_seqlens": digest(r["cu_seqlens"], np.int32)}

    w = synth.thd_tables()
    r = oracle.thd_tables(w["seq_lens"], w["seq_lens_padded"], w["S"])
    d["thd_tables"] = {"status": r["status"], "num_seqs": r["num_seqs"],
                       "max_seqlen": r["max_seqlen"], "pad_between_seqs": r["pad_between_seqs"],
                       "cu_seqlens": digest(r["cu_seqlens"], np.int32),
                       "cu_seqlens_padded": digest(r["cu_seqlens_padded"], np.int32),
                       "padding_mask": digest(r["padding_mask"], np.uint8)}
    for k in ("input_ids", "labels", "position_ids"):
        src = w[k]
        d["thd_tables"][k] = digest(oracle.copy_rows(src, 1, src.nbytes, src.nbytes), np.uint8)

    r = oracle.split_thd(w["seq_lens"], w["seq_lens_padded"], w["S"], 4)
    d["thd_split_4"] = {"status": r["status"], "cu_width": int(r["cu_seqlens"].shape[1]),
                        "cu_seqlens": digest(r["cu_seqlens"], np.int32),
                        "cu_seqlens_padded": digest(r["cu_seqlens_padded"], np.int32),
                        "per_chunk": digest(np.stack([r["num_seqs"], r["max_seqlen"],
                                                      r["pad_between_seqs"]]), np.int32),
                        "padding_mask": digest(r["padding_mask"], np.uint8)}

    w = synth.pack_sources()
    r = oracle.pack(w["src"], w["src_off"], w["real_len"], w["q"], w["pack_start"],
                    w["capacity"], fold=True)
    d["pack_sources"] = {"status": r["status"], "csr_entries": int(r["cu_seqlens"].size),
                         "packed": digest(r["packed"], np.int64),
                         "token_mask": digest(r["token_mask"], np.uint8),
                         "cu_seqlens": digest(r["cu_seqlens"], np.int32),
                         "cu_seqlens_padded": digest(r["cu_seqlens_padded"], np.int32)}

    w = synth.pad_tail_stream()
    r = oracle.pad_mask_from_ids(w["input_ids"], w["pad_id"])
    d["pad_tail_stream"] = {"status": r["status"], "num_content": r["num_content"],
                            "padding_mask": digest(r["padding_mask"], np.uint8)}

    w = synth.trainer_rectangle()
    r = oracle.pack_rect(w["rows"], w["real_len"], w["q"], w["bins"])
    d["trainer_rectangle"] = {"status": r["status"], "width": r["width"],
                              "csr_entries": int(r["cu_seqlens"].size),
                              "packed": digest(r["packed"], np.int64),
                              "token_mask": digest(r["token_mask"], np.uint8),
                              "cu_seqlens": digest(r["cu_seqlens"], np.int32),
                              "cu_seqlens_padded": digest(r["cu_seqlens_padded"], np.int32)}

    w = synth.stage_embedding()
    r = oracle.doc_segments(w["doc_ids"])
    pos = w["position_ids"]
    d["stage_embedding"] = {"num_segments": r["num_segments"], "max_seqlen": r["max_seqlen"],
                            "cu_seqlens": digest(r["cu_seqlens"], np.int32),
                            "padding_mask": digest(r["padding_mask"], np.uint8),
                            "position_ids": digest(oracle.copy_rows(pos, 1, pos.nbytes, pos.nbytes),
                                                   np.uint8)}
    d["_note"] = ("SHA-256 of the oracle's outputs on the seeded workloads "
                  "(tests/golden/make_digests.py); bench.py compares its GPU outputs with them")
    return d


def main() -> None:
    d = compute()
    with open(OUT, "w") as f:
        json.dump(d, f, indent=1, sort_keys=True)
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
