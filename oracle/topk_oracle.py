"""CPU oracle for the fused per-row top-k + page-table transform.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module: it
may be imported, called or executed only by the test suite, by the smoke check
and by the benchmark's CPU-baseline leg.  It shares no code, header, table or
constant with the HIP library (the two never import each other); the only thing
both sides consume is the seeded input generator in ``workloads``.

It is the plain definition, written out with numpy, one row at a time:

  1. L = clamp(seq_len[b], 0, W) and n = min(k, L).
     (Rows carry their own length -- SGLang PR #26788 "DeepSeek-V4 DSA indexer:
     faster top-k + page-table transform", Feature section: ragged per-batch
     sequence lengths, runtime k up to 2048.  A length above the width is read
     as the width; a negative one as empty -- the follow-up "Harden top-k
     kernels against negative padded seq_lens" mentioned on the same page shows
     negative padded lengths reach the kernel in practice.)
  2. Every valid score is mapped to an order key (``order_key``): an unsigned
     32-bit integer whose unsigned order is the order of the scores
     (flash-float-jit-kernels README, second method bullet: a bin map with
     bin(x) >= bin(y) implying x >= y, taken on the fp32 bit pattern).
  3. The n positions with the greatest keys are the selected set: sort the
     (key descending, position ascending) pairs and take the first n.  The set
     is what is defined; within it the order is unspecified (LiteTopk PR #32094
     "Add LiteTopk fused indexer top-k prefill path for SM100", Notes: exact
     top-k set, unspecified order, ties broken by arrival order).  Taking the
     lowest position first among equal keys is only this oracle's canonical
     pick for display; the checker accepts any distinct equal-key fill.
  4. raw[b, j] = j-th selected position for j < n, else -1 (PR #26788, commit
     note adding the raw-index side output: pre-transform position per slot, or
     -1 for padding; LiteTopk PR, "sglang deviations": -1 padding is the dense
     ragged transform contract).
  5. out[b, j] = page_table[b, raw // page_size] * page_size + raw % page_size
     for j < n, else -1.  This is the paged-KV reading of "maps the selected
     indices through a page table" (PR #26788, Motivation) with an arbitrary
     power-of-two page size (Feature section): position i sits at offset
     i % page_size of logical page i / page_size, and the table names that
     logical page's physical page.  Computed in int64 and required to fit int32.

Value order, stated once: the key order equals IEEE-754 order on every non-NaN
value except that -0.0 sorts strictly below +0.0 (IEEE calls them equal, so the
key order picks one of the answers IEEE order allows).  -inf is an ordinary
value that can be selected.  NaN is outside the contract.

Parity status: every function here is pinned by the CPU tests (exhaustive key
monotonicity over all 2^32 bit patterns, brute force over all subsets on tiny
rows, torch.topk on distinct-valued rows, closed forms for ascending /
descending / constant / short rows, and the transform's identity / permutation
inverses).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np


def order_key(values: np.ndarray) -> np.ndarray:
    """fp32 values -> uint32 keys whose unsigned order is the value order.

    Non-negative floats (sign bit clear) already order like their bit patterns;
    setting the top bit lifts them above every negative.  Negative floats order
    in reverse of their bit patterns; complementing all bits reverses that and
    clears the top bit, leaving them below every non-negative.
    """
    bits = np.ascontiguousarray(values, dtype=np.float32).view(np.uint32)
    negative = (bits >> np.uint32(31)) == np.uint32(1)
    return np.where(negative, ~bits, bits | np.uint32(0x80000000)).astype(np.uint32)


def row_length(seq_len: int, width: int) -> int:
    """Valid length of a row: seq_len clamped to [0, width]."""
    return min(max(int(seq_len), 0), int(width))


def select_row(scores_row: np.ndarray, L: int, k: int) -> np.ndarray:
    """Positions of the n = min(k, L) greatest keys in scores_row[:L].

    Order: key descending, then position ascending (the canonical pick among
    equal keys).  Returns an int64 array of length n.
    """
    n = min(int(k), int(L))
    if n <= 0:
        return np.zeros(0, dtype=np.int64)
    keys = order_key(scores_row[:L])
    positions = np.arange(L, dtype=np.int64)
    # np.lexsort sorts by the last key first, ascending: ~keys ascending is keys
    # descending; positions ascending break ties.
    order = np.lexsort((positions, ~keys))
    return order[:n].astype(np.int64)


def transform_positions(positions: np.ndarray, table_row: np.ndarray, page_size: int) -> np.ndarray:
    """Physical index of each logical position through one row of the page table."""
    positions = np.asarray(positions, dtype=np.int64)
    pages = table_row.astype(np.int64)[positions // page_size]
    phys = pages * page_size + positions % page_size
    if phys.size and (phys.max() >= 2**31 or phys.min() < -(2**31)):
        raise OverflowError("transformed index does not fit in int32")
    return phys


@dataclasses.dataclass
class RowInfo:
    """What is unique about one row's answer.

    n: number of valid slots; threshold: key of the n-th greatest element (the
    smallest selected key) or None when n == 0; n_greater: how many positions in
    [0, L) have a key strictly above the threshold (all of them must be
    selected); n_equal: how many positions carry exactly the threshold key.
    """
    L: int
    n: int
    threshold: Optional[int]
    n_greater: int
    n_equal: int


def topk_transform_row(scores_row: np.ndarray, seq_len: int, table_row: np.ndarray, k: int,
                       page_size: int) -> Tuple[np.ndarray, np.ndarray, RowInfo]:
    """One row of the oracle: (out[k], raw[k], RowInfo)."""
    W = scores_row.shape[0]
    L = row_length(seq_len, W)
    sel = select_row(scores_row, L, k)
    n = sel.size
    raw = np.full(k, -1, dtype=np.int32)
    out = np.full(k, -1, dtype=np.int32)
    if n == 0:
        return out, raw, RowInfo(L, 0, None, 0, 0)
    raw[:n] = sel
    out[:n] = transform_positions(sel, table_row, page_size)
    keys = order_key(scores_row[:L])
    thr = int(keys[sel[-1]])
    info = RowInfo(L, n, thr, int(np.count_nonzero(keys > np.uint32(thr))),
                   int(np.count_nonzero(keys == np.uint32(thr))))
    return out, raw, info


def topk_transform(scores: np.ndarray, seq_lens: np.ndarray, page_table: np.ndarray, k: int,
                   page_size: int, rows: Optional[List[int]] = None
                   ) -> Tuple[np.ndarray, np.ndarray, List[RowInfo]]:
    """Whole-batch oracle.  Returns out (B', k), raw (B', k) int32 and per-row info.

    ``rows`` restricts the computation to a subset of rows (B' = len(rows)).
    """
    if k < 1:
        raise ValueError("k must be >= 1")
    if page_size < 1 or (page_size & (page_size - 1)) != 0:
        raise ValueError("page_size must be a power of two")
    B = scores.shape[0]
    rows = list(range(B)) if rows is None else list(rows)
    out = np.full((len(rows), k), -1, dtype=np.int32)
    raw = np.full((len(rows), k), -1, dtype=np.int32)
    infos: List[RowInfo] = []
    for r, b in enumerate(rows):
        o, w, info = topk_transform_row(scores[b], int(seq_lens[b]), page_table[b], k, page_size)
        out[r] = o
        raw[r] = w
        infos.append(info)
    return out, raw, infos
