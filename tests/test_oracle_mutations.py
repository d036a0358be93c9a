"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a scratch copy of the oracle: a
dropped step, a wrong bound or index, an inverted comparison, a missed
argument.  It rebuilds the copy and runs the pin tests that should catch the
mistake there; the case passes only if one of them fails.  A mutation whose
anchor text no longer occurs exactly once in the oracle also fails, so the
list has to follow the oracle's text when it changes.  A control run of the
unmodified copy must pass the same pin tests, so a caught mutation is never a
broken harness.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DOC = ["test_oracle_doc.py"]
THD = ["test_oracle_thd.py"]
PACK = ["test_oracle_pack.py"]
PADIDS = ["test_oracle_padids.py"]

C_SRC = "psq_oracle.c"
PY_SRC = "__init__.py"

# (name, file under oracle/, text, replacement, pin test files)
MUTATIONS = [
    # packed_seq_params_from_doc_ids
    ("doc_no_row_start", C_SRC, "int starts_row = (t % S) == 0;", "int starts_row = (t == 0);", DOC),
    ("doc_ordered_compare", C_SRC, "(doc[t] != doc[t - 1])", "(doc[t] > doc[t - 1])", DOC),
    ("doc_no_close", C_SRC, "cu[nseg] = (int32_t)T;", "cu[nseg] = (int32_t)(T - 1);", DOC),
    ("doc_max_off_by_one", C_SRC, "int32_t len = cu[k + 1] - cu[k];",
     "int32_t len = cu[k + 1] - cu[k] - 1;", DOC),
    ("doc_max_skips_last", C_SRC, "for (k = 0; k < nseg; k++) {", "for (k = 0; k + 1 < nseg; k++) {",
     DOC),
    ("doc_mask_inverted", C_SRC, "mask[t] = (uint8_t)(doc[t] == 0);",
     "mask[t] = (uint8_t)(doc[t] != 0);", DOC),
    # the collapse of a [B, S, ...] tensor (pinned in the document-map pins)
    ("copy_ignores_source_stride", C_SRC, "src[r * src_row_stride_bytes + b]",
     "src[r * row_bytes + b]", DOC),
    ("copy_drops_last_byte", C_SRC, "for (b = 0; b < row_bytes; b++)",
     "for (b = 0; b + 1 < row_bytes; b++)", DOC),
    ("doc_second_position_skipped", C_SRC, "int new_doc = (t > 0) && (doc[t] != doc[t - 1]);",
     "int new_doc = (t > 1) && (doc[t] != doc[t - 1]);", DOC),
    # process_input_for_thd on length tables
    ("thd_no_mismatch_check", C_SRC, "status |= ORC_TABLE_MISMATCH;", "status |= 0;", THD),
    ("thd_padded_below_real_allowed", C_SRC, "if (l < 0 || lp < l)", "if (l < 0)", THD),
    ("thd_row_overflow_at_equal", C_SRC, "if (padded_sum > S)", "if (padded_sum >= S)", THD),
    ("thd_no_empty_row", C_SRC, "status |= ORC_EMPTY_ROW;", "status |= 0;", THD),
    ("thd_no_row_fold", C_SRC, "phys[last] += S - row_used;", "phys[last] += 0;", THD),
    ("thd_mask_over_padded", C_SRC, "for (t = cp[i]; t < cp[i] + real[i]; t++)",
     "for (t = cp[i]; t < cp[i + 1]; t++)", THD),
    ("thd_no_absorption", C_SRC, "cu[n] = (int32_t)T;", "cu[n] = cu[n];", THD),
    ("thd_absorption_ungated", C_SRC, "if (interior_agree && cu[n] < T)", "if (cu[n] < T)", THD),
    ("thd_absorption_gate_skips_last", C_SRC,
     "for (i = 1; i < n; i++) {\n            if (cu[i] != cp[i])\n                interior_agree = 0;",
     "for (i = 1; i + 1 < n; i++) {\n            if (cu[i] != cp[i])\n                interior_agree = 0;",
     THD),
    ("thd_max_before_absorption", C_SRC, "int32_t step = cu[i + 1] - cu[i];",
     "int32_t step = (int32_t)real[i];", THD),
    # (skipping the last entry here would be an equivalent mutant: after the
    # fold and the absorption the two arrays always agree there)
    ("thd_pad_between_wrong_sign", C_SRC, "if (cu[i] != cp[i])\n            *pad_between = 1;",
     "if (cu[i] > cp[i])\n            *pad_between = 1;", THD),
    ("thd_no_padded_table_pads_one", C_SRC, "phys[n] = (Lp != NULL) ? Lp[r * P + j] : l;",
     "phys[n] = (Lp != NULL) ? Lp[r * P + j] : l + (l & 1);", THD),
    ("thd_real_boundaries_physical", C_SRC, "cu[i + 1] = cu[i] + (int32_t)real[i];",
     "cu[i + 1] = cu[i] + (int32_t)phys[i];", THD),
    ("thd_physical_boundaries_real", C_SRC, "cp[i + 1] = cp[i] + (int32_t)phys[i];",
     "cp[i + 1] = cp[i] + (int32_t)real[i];", THD),
    ("thd_overflow_clamp_at_row", C_SRC, "padded_sum += (lp > S) ? S + 1 : lp;",
     "padded_sum += (lp > S) ? S : lp;", THD),
    ("thd_mask_starts_as_tokens", C_SRC, "for (t = 0; t < T; t++)\n        mask[t] = 1;",
     "for (t = 0; t < T; t++)\n        mask[t] = 0;", THD),
    ("thd_negative_length_allowed", C_SRC, "if (l < 0 || lp < l)", "if (lp < l)", THD),
    ("thd_mismatch_one_sided", C_SRC, "if (Lp != NULL && ((lp != v) != valid))",
     "if (Lp != NULL && lp == v && valid)", THD),
    # the squeeze
    ("pack_no_fold", C_SRC, "pcp[k] = C;", "pcp[k] = pcp[k];", PACK),
    ("pack_padding_rounds_down", C_SRC, "int64_t padded = (real + q - 1) / q * q;",
     "int64_t padded = real / q * q;", PACK),
    ("pack_mask_on_pad", C_SRC, "mrow[off + s] = 0;", "mrow[off + s] = 1;", PACK),
    ("pack_csr_without_pack_offset", C_SRC, "int32_t *pcu = cu + a + p;", "int32_t *pcu = cu + a;",
     PACK),
    ("pack_overflow_at_equal", C_SRC, "if (used > C)", "if (used >= C)", PACK),
    ("pack_tail_ignores_pad_token", C_SRC, "row[s] = pad_token;\n            mrow[s] = 0;",
     "row[s] = 0;\n            mrow[s] = 0;", PACK),
    ("pack_source_reversed", C_SRC, "row[off + s] = src[src_off[i] + s];",
     "row[off + s] = src[src_off[i] + real - 1 - s];", PACK),
    ("pack_padded_boundary_is_real", C_SRC, "pcp[j + 1] = (int32_t)off;",
     "pcp[j + 1] = pcu[j] + (int32_t)real;", PACK),
    ("pack_order_ignored", C_SRC, "int64_t i = (order != NULL) ? (int64_t)order[a + j] : a + j;",
     "int64_t i = a + j;", PACK),
    ("rect_stride_off_by_one", C_SRC, "off[i] = i * W;", "off[i] = i * W - i;", PACK),
    ("pack_range_upper_unchecked", C_SRC, "if (a < 0 || b > N || b < a) {",
     "if (a < 0 || b < a) {", PACK),
    ("pack_empty_unflagged", C_SRC, "status |= ORC_EMPTY_PACK;", "status |= 0;", PACK),
    ("pack_source_end_exclusive", C_SRC, "src_off[i] > src_len - real",
     "src_off[i] >= src_len - real", PACK),
    ("pack_real_boundary_padded", C_SRC, "pcu[j + 1] = pcu[j] + (int32_t)real;",
     "pcu[j + 1] = pcu[j] + (int32_t)padded;", PACK),
    ("pack_first_token_unmasked", C_SRC, "row[off + s] = src[src_off[i] + s];\n                mrow[off + s] = 1;",
     "row[off + s] = src[src_off[i] + s];\n                mrow[off + s] = (uint8_t)(s > 0);", PACK),
    ("pack_tail_skips_first_slot", C_SRC, "for (s = off; s < C; s++) {",
     "for (s = off + 1; s < C; s++) {", PACK),
    ("rect_length_at_width_rejected", C_SRC, "real > row_width", "real >= row_width", PACK),
    ("trainer_width_of_narrowest_bin", PY_SRC, "return max(widths) if widths else 0",
     "return min(widths) if widths else 0", PACK),
    ("bins_to_csr_starts_shifted", PY_SRC, "start[1:] = np.cumsum([len(b) for b in bins])",
     "start[1:] = np.cumsum([len(b) for b in bins]) - (len(bins) > 1)", PACK),
    ("pack_slices_without_pack_offset", PY_SRC, "out.append(np.asarray(cu_csr)[a + p: b + p + 1])",
     "out.append(np.asarray(cu_csr)[a: b + 1])", PACK),
    ("trainer_width_from_real", PY_SRC,
     "widths = [sum(-(-int(rl[i]) // q) * q for i in b) for b in bins]",
     "widths = [sum(int(rl[i]) for i in b) for b in bins]", PACK),
    # thd_padding_mask_from_token_ids
    ("padids_no_tail_check", C_SRC, "status |= ORC_PAD_IS_CONTENT;", "status |= 0;", PADIDS),
    ("padids_last_pad_found", C_SRC, "first_pad = t;\n            break;", "first_pad = t;", PADIDS),
    ("padids_mask_inverted", C_SRC, "mask[t] = (uint8_t)(ids[t] == pad);",
     "mask[t] = (uint8_t)(ids[t] != pad);", PADIDS),
    ("padids_content_count_short", C_SRC, "*num_content = first_pad;",
     "*num_content = first_pad - (first_pad > 0);", PADIDS),
    ("padids_no_pad_means_empty", C_SRC, "int64_t t, first_pad = T;",
     "int64_t t, first_pad = 0;", PADIDS),
    # split_batch_into_thd_chunks (the Python stacking over the table oracle)
    ("split_fill_zero", PY_SRC, "out = np.full((num_chunks, width), pad_value, dtype=np.int32)",
     "out = np.zeros((num_chunks, width), dtype=np.int32)", THD),
    ("split_uneven_rows", PY_SRC, "rows = B // num_chunks",
     "rows = max(1, B // num_chunks - 1) if B > 2 else B // num_chunks", THD),
    ("split_status_of_last_chunk", PY_SRC, 'status |= part["status"]',
     'status = part["status"]', THD),
]

ALL_PINS = sorted({f for m in MUTATIONS for f in m[4]})


def _scratch(base: str) -> str:
    """A copy of what the pin tests need: oracle sources, synth, tests, ini."""
    os.makedirs(base)
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(base, "oracle"),
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "synth"), os.path.join(base, "synth"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(base, "tests"))
    shutil.copy(os.path.join(ROOT, "tests", "conftest.py"), os.path.join(base, "tests"))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(base, "tests", "golden"))
    for f in ALL_PINS:
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(base, "tests"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), base)
    return base


def _build_oracle(base: str) -> None:
    src = os.path.join(base, "oracle", C_SRC)
    lib = os.path.join(base, "oracle", "liboracle.so")
    r = subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", lib, src],
                       capture_output=True, text=True)
    assert r.returncode == 0, f"mutated oracle does not compile:\n{r.stderr}"


def _run_pins(base: str, files) -> subprocess.CompletedProcess:
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"]
    cmd += [os.path.join("tests", f) for f in files]
    return subprocess.run(cmd, cwd=base, env=env, capture_output=True, text=True, timeout=600)


def _mutate_and_run(base: str, mutation) -> tuple:
    name, fname, text, repl, files = mutation
    _scratch(base)
    path = os.path.join(base, "oracle", fname)
    with open(path) as f:
        source = f.read()
    count = source.count(text)
    if count != 1:
        return name, "anchor", f"anchor occurs {count} times in oracle/{fname}"
    with open(path, "w") as f:
        f.write(source.replace(text, repl))
    _build_oracle(base)
    r = _run_pins(base, files)
    tail = (r.stdout.strip().splitlines() or [""])[-1]
    return name, r.returncode, tail


@pytest.fixture(scope="module")
def results(tmp_path_factory):
    root = str(tmp_path_factory.mktemp("mutants"))
    control = _scratch(os.path.join(root, "control"))
    _build_oracle(control)
    r = _run_pins(control, ALL_PINS)
    assert r.returncode == 0, "the unmodified oracle fails its pins:\n" + r.stdout[-2000:]
    workers = max(1, min(6, (os.cpu_count() or 2) - 1))
    with concurrent.futures.ThreadPoolExecutor(workers) as pool:
        futs = [pool.submit(_mutate_and_run, os.path.join(root, m[0]), m) for m in MUTATIONS]
        return {name: (rc, tail) for name, rc, tail in (f.result() for f in futs)}


@pytest.mark.parametrize("name", [m[0] for m in MUTATIONS])
def test_pins_catch_mutation(results, name):
    rc, tail = results[name]
    assert rc != "anchor", tail
    # caught: pytest exit code 1 (a pin failed), or the pins' process died of
    # the mistake itself (a signal: the mutated oracle wrote out of bounds,
    # e.g. folding into the last sequence of a row that has none)
    caught = (rc == 1 and "failed" in tail) or rc < 0
    assert caught, f"{name} was not caught by its pins (exit {rc}): {tail!r}"
