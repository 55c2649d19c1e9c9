"""CPU oracle for the fused indexer scoring + top-k (the step before the top-k).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module: it
may be imported, called or executed only by the test suite, by the smoke check
and by the benchmark's CPU-baseline leg.  It shares no code, header, table or
constant with the HIP library.

What is computed (LiteTopk PR #32094 "Add LiteTopk fused indexer top-k prefill
path for SM100": Summary, the Background list, and the Validation section's
reference formula):

  score[r, j] = s[j] * sum_h w[r, h] * relu( sum_d q[r, h, d] * kv[j, d] )

for every position j of row r's key range [ks[r], ke[r]), with q and kv held as
fp8 codes, w the per-row head weights, and s the per-position dequantisation
scale of the fp8 key cache.  The row's output is the exact top-k *set* of its
scores, as absolute key positions, with -1 in the slots beyond
min(k, ke - ks) (Notes: exact top-k set with unspecified order; "sglang
deviations": -1 padding, output coordinates are absolute positions in the
gathered key buffer).  The GLM indexer shape is fixed: H = 32 heads of
D = 128 (Notes).

Readings where the page is silent:
  * fp8 format: the OCP E4M3 encoding (bias 7, no infinities, S.1111.111 is
    NaN, largest finite 448), the one the page's fp8 key cache and the gfx950
    matrix cores both use.  ``fp8_e4m3_decode`` writes it out from the
    definition; NaN codes are outside the contract.
  * Ranges: ks and ke are clamped to [0, N] (N = number of key positions); an
    empty or inverted range is an empty row (all -1).
  * Ties: any distinct fill of the equal-score slots is correct; this oracle's
    own pick is the lowest position, for display only.
  * Precision: the oracle computes in float64.  A GPU computes the same sum in
    fp32, so its scores differ by rounding; the page checks its kernel with a
    tie-tolerant test around the k-th score (Validation section).  The checker
    here uses the same test with a tolerance derived from the fp32 arithmetic
    (``fp32_error_bound``), which is tighter than the page's 1e-3 relative one.

Parity status: pinned by the CPU tests -- the decoder against torch's
float8_e4m3fn conversion of all 256 codes and the format's closed forms; the
scores against a plain matrix product in the single-head, non-negative case,
one-hot closed forms for the relu, head weights and scale, and brute force
over all subsets for the selection on tiny rows.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

HEADS = 32
HEAD_DIM = 128


def fp8_e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 OCP E4M3 codes -> float64 values.

    Fields: sign (bit 7), exponent e (bits 6..3, bias 7), mantissa m (bits
    2..0).  e > 0: (-1)^s * 2^(e-7) * (1 + m/8).  e == 0: (-1)^s * 2^-6 * m/8
    (subnormals and the two zeros).  e == 15 and m == 7: NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = sign * np.ldexp(m / 8.0, -6)
    out = np.where(e > 0, normal, sub)
    return np.where((e == 15) & ((c & 0x7) == 7), np.nan, out)


def key_range(ks: int, ke: int, num_kv: int) -> range:
    """Positions row r scores: [clamp(ks), clamp(ke)), empty when inverted."""
    lo = min(max(int(ks), 0), num_kv)
    hi = min(max(int(ke), 0), num_kv)
    return range(lo, max(lo, hi))


def indexer_scores_row(q_row: np.ndarray, w_row: np.ndarray, kv: np.ndarray, kv_scale: np.ndarray,
                       positions: range) -> np.ndarray:
    """Scores of one query row over ``positions`` (float64, in position order).

    q_row (H, D) uint8 codes, w_row (H,) float32, kv (N, D) uint8 codes,
    kv_scale (N,) float32.  Steps in the order of the formula: the per-head dot
    product of the query with each key, relu, the head-weighted sum, then the
    position's scale.
    """
    if len(positions) == 0:
        return np.zeros(0, np.float64)
    q = fp8_e4m3_decode(q_row)                                    # (H, D)
    keys = fp8_e4m3_decode(kv[positions.start:positions.stop])    # (n, D)
    dots = keys @ q.T                                             # (n, H): q[h] . kv[j]
    per_head = np.maximum(dots, 0.0)
    weighted = per_head @ np.asarray(w_row, np.float64)           # sum_h w[h] * relu(.)
    return weighted * np.asarray(kv_scale[positions.start:positions.stop], np.float64)


def fp32_error_bound(q_row: np.ndarray, w_row: np.ndarray, kv: np.ndarray, kv_scale: np.ndarray,
                     positions: range) -> np.ndarray:
    """Largest difference between a score summed in fp32 (any order) and the
    exact one, per position.

    Each fp8 x fp8 product is exact in fp32 (4-bit significands, exponents far
    inside fp32's range).  Summing D products, multiplying by w, summing H
    heads and multiplying by s makes at most D + H + 2 roundings along any
    path, so the standard bound gives
        |fp32 - exact| <= gamma_(D+H+2) * |s| * sum_h |w_h| * sum_d |q_hd kv_d|
    with gamma_n = n u / (1 - n u), u = 2^-24 (relu is 1-Lipschitz and exact).
    """
    if len(positions) == 0:
        return np.zeros(0, np.float64)
    q = np.abs(fp8_e4m3_decode(q_row))
    keys = np.abs(fp8_e4m3_decode(kv[positions.start:positions.stop]))
    mag = (keys @ q.T) @ np.abs(np.asarray(w_row, np.float64))
    mag *= np.abs(np.asarray(kv_scale[positions.start:positions.stop], np.float64))
    n = q.shape[1] + q.shape[0] + 2
    u = 2.0 ** -24
    return mag * (n * u / (1.0 - n * u))


@dataclasses.dataclass
class IndexerRow:
    lo: int                 # first position of the row's range
    length: int             # ke - ks after clamping
    n: int                  # min(k, length)
    v_k: float              # the n-th best score (nan when n == 0)
    selected: np.ndarray    # canonical selection (absolute positions), length n


def indexer_topk_row(q_row, w_row, kv, kv_scale, ks: int, ke: int, k: int) -> IndexerRow:
    """Exact top-min(k, L) positions of one row by score, ties to the lowest position."""
    pos = key_range(ks, ke, kv.shape[0])
    scores = indexer_scores_row(q_row, w_row, kv, kv_scale, pos)
    n = min(k, len(pos))
    order = np.lexsort((np.arange(len(pos)), -scores))[:n]
    sel = np.asarray(order, np.int64) + pos.start
    v_k = float(scores[order[-1]]) if n else float("nan")
    return IndexerRow(pos.start, len(pos), n, v_k, sel)


def indexer_topk(q, w, kv, kv_scale, ks, ke, k: int, rows: Optional[List[int]] = None):
    """(num_q, k) int32 absolute positions, -1 padded, plus per-row info.

    q (num_q, H, D) uint8, w (num_q, H) float32, kv (N, D) uint8,
    kv_scale (N,) float32, ks / ke (num_q,) int32.
    """
    num_q = q.shape[0]
    rows = range(num_q) if rows is None else rows
    out = np.full((num_q, k), -1, np.int32)
    infos = {}
    for r in rows:
        info = indexer_topk_row(q[r], w[r], kv, kv_scale, int(ks[r]), int(ke[r]), k)
        out[r, :info.n] = info.selected
        infos[r] = info
    return out, infos


def check_indexer_row(scores: np.ndarray, lo: int, k: int, got: np.ndarray, eps: float) -> List[str]:
    """Tie-tolerant exactness of one output row (LiteTopk PR #32094,
    Validation: selected scores >= v_k - eps, every score > v_k + eps
    selected, plus count, -1 padding, uniqueness and range).

    scores: exact scores of the row's positions [lo, lo + len(scores)).
    """
    errs: List[str] = []
    L = len(scores)
    n = min(k, L)
    got = np.asarray(got, np.int64)
    if np.any(got[n:] != -1):
        errs.append(f"padding slots [{n}, {k}) not all -1")
    head = got[:n]
    if np.any((head < lo) | (head >= lo + L)):
        errs.append("selected position outside the row's key range")
        return errs
    if len(np.unique(head)) != n:
        errs.append("duplicate positions")
        return errs
    if n == 0:
        return errs
    v_k = np.sort(scores)[::-1][n - 1]
    picked = scores[head - lo]
    if np.any(picked < v_k - eps):
        errs.append(f"selected score {picked.min()!r} below v_k - eps ({v_k!r} - {eps!r})")
    must = np.nonzero(scores > v_k + eps)[0] + lo
    missing = np.setdiff1d(must, head)
    if len(missing):
        errs.append(f"{len(missing)} positions scoring above v_k + eps missing (first {missing[0]})")
    return errs
