"""CPU tests: plant plausible mistakes in a copy of the oracle and make sure a pin fails.

Each mutant is a small variation of one oracle step (a dropped bit flip, a
wrong sign, an off-by-one, a transposed operand).  None of them touches the
oracle module itself; they are local functions handed to the pins.
"""
import numpy as np
import pytest

import pins
from oracle import topk_oracle as T


def _keymap_no_negative_flip(values):
    bits = np.ascontiguousarray(values, dtype=np.float32).view(np.uint32)
    return (bits | np.uint32(0x80000000)).astype(np.uint32)


def _keymap_sign_xor_only(values):
    bits = np.ascontiguousarray(values, dtype=np.float32).view(np.uint32)
    return (bits ^ np.uint32(0x80000000)).astype(np.uint32)


def _keymap_signed_compare(values):
    # order as signed int32 reinterpretation (negatives in reverse)
    bits = np.ascontiguousarray(values, dtype=np.float32).view(np.int32).astype(np.int64)
    return (bits + 2**31).astype(np.uint32)


@pytest.mark.parametrize("mutant", [_keymap_no_negative_flip, _keymap_sign_xor_only, _keymap_signed_compare])
def test_keymap_mutants_fail(mutant):
    with pytest.raises(AssertionError):
        pins.pin_keymap_exhaustive(mutant, stride=4099, chunk=1 << 22, procs=1)
    with pytest.raises(AssertionError):
        pins.pin_keymap_specials(mutant)


def _row_fn(select=None, transform=None, n_fn=None, clamp=True, keymap=None):
    """Builds a variant of topk_transform_row with one step replaced."""
    keymap = keymap or T.order_key
    select = select or T.select_row
    transform = transform or T.transform_positions

    def row(scores_row, seq_len, table_row, k, page_size):
        W = scores_row.shape[0]
        L = T.row_length(seq_len, W) if clamp else max(int(seq_len), 0)
        L_eff = min(L, W)
        sel = select(scores_row, L_eff, k)
        if n_fn is not None:
            sel = sel[:n_fn(k, L_eff)]
        n = sel.size
        raw = np.full(k, -1, np.int32)
        out = np.full(k, -1, np.int32)
        if n == 0:
            return out, raw, T.RowInfo(L, 0, None, 0, 0)
        raw[:n] = sel
        out[:n] = transform(sel, table_row, page_size)
        keys = keymap(scores_row[:L_eff])
        thr = int(keys[sel[-1]])
        return out, raw, T.RowInfo(L, n, thr, int(np.count_nonzero(keys > thr)),
                                   int(np.count_nonzero(keys == thr)))
    return row


def _select_ascending(scores_row, L, k):
    n = min(k, L)
    keys = T.order_key(scores_row[:L])
    return np.lexsort((np.arange(L), keys))[:n]


def _select_float_argsort(scores_row, L, k):
    # plain float argsort: loses the -0.0 < +0.0 distinction and -inf handling is fine
    n = min(k, L)
    return np.argsort(-scores_row[:L].astype(np.float64), kind="stable")[:n]


def _select_with_keymap(keymap):
    def sel(scores_row, L, k):
        n = min(k, L)
        keys = keymap(scores_row[:L])
        return np.lexsort((np.arange(L), ~keys))[:n]
    return sel


def _transform_swapped(positions, table_row, ps):
    positions = np.asarray(positions, np.int64)
    return table_row.astype(np.int64)[positions % ps] * ps + positions // ps


def _transform_no_offset(positions, table_row, ps):
    positions = np.asarray(positions, np.int64)
    return table_row.astype(np.int64)[positions // ps] * ps


def _transform_wrong_sign(positions, table_row, ps):
    positions = np.asarray(positions, np.int64)
    return table_row.astype(np.int64)[positions // ps] * ps - positions % ps


MUTANTS = {
    "select_ascending": _row_fn(select=_select_ascending),
    "select_float_order": _row_fn(select=_select_float_argsort),
    "select_sign_xor_keymap": _row_fn(select=_select_with_keymap(_keymap_sign_xor_only)),
    "n_off_by_one_low": _row_fn(n_fn=lambda k, L: max(min(k, L) - 1, 0)),
    "transform_swapped": _row_fn(transform=_transform_swapped),
    "transform_no_offset": _row_fn(transform=_transform_no_offset),
    "transform_wrong_sign": _row_fn(transform=_transform_wrong_sign),
    "no_clamp": _row_fn(clamp=False),
}


def _run_all_pins(row_fn, transform_fn):
    pins.pin_select_bruteforce(row_fn)
    pins.pin_closed_forms(row_fn)
    pins.pin_transform(row_fn, transform_fn)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_row_mutants_fail(name):
    row_fn = MUTANTS[name]
    transform_fn = {"transform_swapped": _transform_swapped, "transform_no_offset": _transform_no_offset,
                    "transform_wrong_sign": _transform_wrong_sign}.get(name, T.transform_positions)
    # a pin fails by assertion, or by the mutant indexing outside the table
    with pytest.raises((AssertionError, IndexError)):
        _run_all_pins(row_fn, transform_fn)


def test_unmutated_passes_same_pins():
    _run_all_pins(_row_fn(), T.transform_positions)
