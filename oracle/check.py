"""Checker: compares a candidate (out, raw) against the oracle.  TEST INFRASTRUCTURE ONLY.

Where several answers are correct -- which of the tied elements fill the last
slots, and the order of the slots -- it compares what is unique and checks that
the rest is valid (LiteTopk PR #32094, Notes: exact top-k set with unspecified
order and arrival-order tie breaking; SGLang PR #26788, raw-index commit note:
out[j] must equal the page transform of raw[j], with aligned -1 padding):

  (i)   slots [n, k) hold -1 in out (and in raw when present);
  (ii)  slots [0, n) hold distinct positions in [0, L);
  (iii) every position whose key is strictly above the oracle's threshold key
        is present (bit-exact integer compare on the keys);
  (iv)  every other selected position carries exactly the threshold key;
  (v)   out[j] == transform(raw[j]) slot by slot.

When raw is absent, out is mapped back through the inverse of the row's page
table (which must then be injective on the pages in use) and (ii)-(iv) are
applied to the recovered positions.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from .topk_oracle import RowInfo, order_key, row_length, topk_transform_row, transform_positions


def _inverse_positions(out_valid: np.ndarray, table_row: np.ndarray, L: int, page_size: int
                       ) -> Optional[np.ndarray]:
    used = -(-L // page_size)
    pages = table_row[:used].astype(np.int64)
    if np.unique(pages).size != pages.size:
        return None
    inv: Dict[int, int] = {int(p): lp for lp, p in enumerate(pages.tolist())}
    phys = out_valid.astype(np.int64)
    page = phys // page_size
    off = phys % page_size
    logical = np.array([inv.get(int(p), -1) for p in page.tolist()], dtype=np.int64)
    pos = np.where(logical >= 0, logical * page_size + off, -1)
    return pos


def check_row(scores_row: np.ndarray, seq_len: int, table_row: np.ndarray, k: int, page_size: int,
              out_row: np.ndarray, raw_row: Optional[np.ndarray], info: Optional[RowInfo] = None
              ) -> List[str]:
    """Errors (empty when the candidate row is a correct answer)."""
    errs: List[str] = []
    W = scores_row.shape[0]
    if info is None:
        _, _, info = topk_transform_row(scores_row, seq_len, table_row, k, page_size)
    L, n = info.L, info.n
    assert L == row_length(seq_len, W)
    out_row = np.asarray(out_row, dtype=np.int64)
    if np.any(out_row[n:] != -1):
        errs.append(f"out tail [n={n}, k={k}) not all -1: {out_row[n:][out_row[n:] != -1][:8].tolist()}")
    if raw_row is not None:
        raw_row = np.asarray(raw_row, dtype=np.int64)
        if np.any(raw_row[n:] != -1):
            errs.append(f"raw tail [n={n}, k={k}) not all -1")
        pos = raw_row[:n]
    else:
        pos = _inverse_positions(out_row[:n], table_row, L, page_size)
        if pos is None:
            return ["page table row not injective on its used pages: cannot check out alone"]
    if n == 0:
        return errs
    if np.any((pos < 0) | (pos >= L)):
        bad = pos[(pos < 0) | (pos >= L)]
        errs.append(f"{bad.size} selected positions outside [0, L={L}): {bad[:8].tolist()}")
        return errs
    if np.unique(pos).size != n:
        errs.append(f"selected positions are not distinct ({n - np.unique(pos).size} duplicates)")
        return errs
    keys = order_key(scores_row[:L])
    sel_keys = keys[pos]
    thr = np.uint32(info.threshold)
    if np.any(sel_keys < thr):
        errs.append(f"{int(np.count_nonzero(sel_keys < thr))} selected keys below the threshold key")
    n_gt = int(np.count_nonzero(sel_keys > thr))
    if n_gt != info.n_greater:
        errs.append(f"strictly-greater elements: selected {n_gt}, expected all {info.n_greater}")
    if raw_row is not None:
        exp = transform_positions(pos, table_row, page_size)
        if np.any(exp != out_row[:n]):
            j = int(np.nonzero(exp != out_row[:n])[0][0])
            errs.append(f"out[{j}]={int(out_row[j])} != transform(raw[{j}]={int(pos[j])})={int(exp[j])}")
    return errs


def check_batch(scores: np.ndarray, seq_lens: np.ndarray, page_table: np.ndarray, k: int,
                page_size: int, out: np.ndarray, raw: Optional[np.ndarray],
                rows: Optional[List[int]] = None, max_report: int = 5) -> List[str]:
    """Check the listed rows (all by default); returns error strings prefixed with the row."""
    B = scores.shape[0]
    rows = list(range(B)) if rows is None else list(rows)
    errors: List[str] = []
    for b in rows:
        e = check_row(scores[b], int(seq_lens[b]), page_table[b], k, page_size, out[b],
                      None if raw is None else raw[b])
        errors.extend(f"row {b}: {m}" for m in e)
        if len(errors) >= max_report:
            break
    return errors
