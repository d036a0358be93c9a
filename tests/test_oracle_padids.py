"""Pins for the oracle's metadata-free padding mask (CPU only).

The oracle follows the NeMo AutoModel 0.5 API page
``nemo_automodel.components.distributed.thd_utils``,
``thd_padding_mask_from_token_ids``: padding is marked by comparing ids with
the pad id.  By the page, that comparison is only valid when the pad slots
form one run at the end of the stream; anything else is rejected (the
page's example is a model whose pad id is also its end-of-text id).

Pinned by hand cases, the pad == end-of-text collision, the degenerate
streams (empty, no pad, all pad), and brute force over every stream in
{0,1,2}^T (T <= 7) against an independent formulation: the stream is valid
exactly when its 0/1 pad indicator is sorted, and the content length is then
the number of zeros.
"""
import itertools

import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("ids,pad,mask,n", [
    ([5, 6, 7, 0, 0], 0, [0, 0, 0, 1, 1], 3),
    ([5, 6, 7], 0, [0, 0, 0], 3),           # no pad at all
    ([9, 9, 9], 9, [1, 1, 1], 0),           # nothing but pad
    ([], 0, [], 0),                         # empty stream
    ([4, 3, 2, 1], 1, [0, 0, 0, 1], 3),     # a one-slot tail
])
def test_right_padded_streams(ids, pad, mask, n):
    out = oracle.pad_mask_from_ids(ids, pad)
    assert out["status"] == 0
    assert out["padding_mask"].tolist() == mask
    assert out["num_content"] == n


def test_pad_id_that_is_also_end_of_text_is_rejected():
    # Two documents, each closed by the end-of-text id, then a tail of the
    # same id used as pad: the first end-of-text is content, so the value
    # comparison would mask it out.  The call must fail.
    EOT = 151329
    ids = [17, 18, EOT, 40, 41, 42, EOT, EOT, EOT]
    out = oracle.pad_mask_from_ids(ids, EOT)
    assert out["status"] == oracle.PAD_IS_CONTENT
    # the same stream with a distinct pad id is fine
    ids2 = [17, 18, EOT, 40, 41, 42, EOT, 0, 0]
    out2 = oracle.pad_mask_from_ids(ids2, 0)
    assert out2["status"] == 0 and out2["num_content"] == 7


def test_pad_in_the_middle_or_at_the_start_is_rejected():
    assert oracle.pad_mask_from_ids([0, 5, 6], 0)["status"] == oracle.PAD_IS_CONTENT
    assert oracle.pad_mask_from_ids([5, 0, 6, 0], 0)["status"] == oracle.PAD_IS_CONTENT


def test_brute_force_against_sorted_indicator():
    checked = 0
    for T in range(0, 8):
        for ids in itertools.product((0, 1, 2), repeat=T):
            for pad in (0, 1):
                ind = [int(x == pad) for x in ids]
                valid = ind == sorted(ind)
                out = oracle.pad_mask_from_ids(list(ids), pad)
                assert out["padding_mask"].tolist() == ind
                assert (out["status"] == 0) == valid
                if valid:
                    assert out["num_content"] == ind.count(0)
                checked += 1
    assert checked > 6000


def test_large_values_compare_exactly():
    # ids differing from the pad id only in high bits are content
    pad = 1 << 40
    ids = np.array([pad + 1, pad - 1, pad ^ (1 << 62), pad, pad], dtype=np.int64)
    out = oracle.pad_mask_from_ids(ids, pad)
    assert out["status"] == 0 and out["padding_mask"].tolist() == [0, 0, 0, 1, 1]
