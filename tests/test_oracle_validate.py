"""Pins for the oracle's index validation (IndexShare host `validate_indices`).

The rules, in the page's check order for each column scanned left to right:
-1 sets padding; below -1 is an invalid sentinel; any other value after
padding is an error; a value >= the batch's cache length is out of range; a
value equal to the previous valid one is a duplicate; a smaller one breaks
strict increase. A row with no valid entry is all -1. The first failing row in
(batch, head, query) order and its first failing column are reported.

The brute-force test enumerates every row of width <= 4 over {-3..3} with a
cache length of 3 and classifies each row with a rule table written here from
scratch in a different form (a grammar: a strictly increasing prefix of
in-range values followed only by -1s).
"""
import itertools

import numpy as np
import pytest

import oracle

SENT, AFTER, RANGE, DUP, ORDER, ALLPAD = 1, 2, 3, 4, 5, 6


def classify_by_grammar(row, bound):
    """Independent statement: find the longest valid prefix, then name why the
    next column breaks it."""
    valid_prefix_len = 0
    seen_pad = False
    last = None
    for v in row:
        if v == -1:
            seen_pad = True
            valid_prefix_len += 1
            continue
        ok = (v >= 0) and (not seen_pad) and (v < bound) and (last is None or v > last)
        if not ok:
            break
        last = v
        valid_prefix_len += 1
    if valid_prefix_len == len(row):
        return (ALLPAD, len(row)) if last is None else (0, -1)
    c = valid_prefix_len
    v = row[c]
    # reasons in priority order
    if v < -1:
        return SENT, c
    if seen_pad:
        return AFTER, c
    if v >= bound:
        return RANGE, c
    return (DUP if v == last else ORDER), c


def test_brute_force_all_small_rows():
    values = range(-3, 4)
    bound = 3
    for width in range(1, 5):
        rows = list(itertools.product(values, repeat=width))
        idx = np.array(rows, np.int32).reshape(1, 1, len(rows), width)
        word, cls, first, _ = oracle.validate_indices(idx, [bound])
        for r, row in enumerate(rows):
            want, col = classify_by_grammar(list(row), bound)
            assert cls[r] == want, (row, cls[r], want)
        bad = [r for r, row in enumerate(rows) if classify_by_grammar(list(row), bound)[0] != 0]
        expect_word = 0
        for r in bad:
            expect_word |= 1 << (classify_by_grammar(list(rows[r]), bound)[0] - 1)
        if bad:
            expect_word |= 512
            assert first[0] == bad[0] and first[1] == classify_by_grammar(list(rows[bad[0]]), bound)[1]
        else:
            assert first is None
        assert word == expect_word


@pytest.mark.parametrize("row,cls,col,msg", [
    ([0, 1, -2, -1], SENT, 2, "column=2]: invalid sentinel -2"),
    ([0, -1, 2, -1], AFTER, 2, "column=2]: index 2 follows trailing -1 padding"),
    ([0, 1, 9, -1], RANGE, 2, "column=2]: index 9 is out of range for cache length 5"),
    ([0, 3, 3, -1], DUP, 2, "column=2]: duplicate index 3"),
    ([0, 3, 2, -1], ORDER, 2, "column=2]: indices are not strictly increasing: 3 then 2"),
    ([-1, -1, -1, -1], ALLPAD, 4, "row [batch=0, head=1, query=0] is all -1"),
    ([0, 1, 2, 4], 0, -1, ""),
])
def test_each_class_and_message(row, cls, col, msg):
    idx = np.zeros((1, 2, 1, 4), np.int64)
    idx[0, 0, 0] = [0, 1, -1, -1]
    idx[0, 1, 0] = row
    word, classes, first, text = oracle.validate_indices(idx, [5])
    assert classes[0] == 0 and classes[1] == cls
    if cls:
        assert first == (1, col, cls)
        assert word == (1 << (cls - 1)) | 512
        assert text.startswith("selected_indices")
        assert text.endswith(msg)
        with pytest.raises(oracle.IndexError_):
            oracle.validate_indices(idx, [5], raise_first=True)
    else:
        assert word == 0 and first is None


def test_per_batch_bound_and_first_error_order():
    idx = np.full((3, 1, 2, 3), -1, np.int32)
    idx[0, 0, 0] = [0, 5, -1]        # ok for bound 6
    idx[0, 0, 1] = [1, 2, 3]
    idx[1, 0, 0] = [0, 5, -1]        # range for bound 5
    idx[1, 0, 1] = [0, 0, -1]        # duplicate
    idx[2, 0, 0] = [-5, -1, -1]      # sentinel
    idx[2, 0, 1] = [-1, -1, -1]      # all padding
    word, cls, first, text = oracle.validate_indices(idx, [6, 5, 9])
    assert list(cls) == [0, 0, RANGE, DUP, SENT, ALLPAD]
    assert first == (2, 1, RANGE)
    assert "batch=1, head=0, query=0, column=1" in text
    assert word == 512 | (1 << (RANGE - 1)) | (1 << (DUP - 1)) | (1 << (SENT - 1)) | (1 << (ALLPAD - 1))
