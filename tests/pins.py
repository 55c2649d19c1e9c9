"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin takes the function(s) under test as arguments, so the mutation tests
can hand it a deliberately broken oracle and confirm the pin fails.

  * the key map against the hardware's own float comparison, over every
    non-NaN fp32 bit pattern (or a strided sample of them);
  * the selection against brute force over all subsets of tiny rows, with the
    order written independently of the key map (Python float compare, -0.0
    below +0.0);
  * the checker against that same brute force: it must accept exactly the
    valid subsets;
  * the selection against torch.topk on rows whose values are distinct (the
    answer is unique there);
  * closed forms: ascending / descending rows, constant rows, short rows
    (seq_len <= k), seq_len <= 0, seq_len > width;
  * the transform: hand-computed values, identity table (out == raw),
    permutation table (the inverse permutation recovers raw), page_size 1.
"""
from __future__ import annotations

import itertools
import math
import multiprocessing as mp
from typing import Callable, List

import numpy as np

# ----------------------------------------------------------------------------
# Key map
# ----------------------------------------------------------------------------

NONNEG_MAX = 0x7F800000      # +inf
NEG_MIN = 0x80000000         # -0.0
NEG_MAX = 0xFF800000         # -inf
N_NON_NAN = 2**32 - 2**24 + 2


def _ascending_segments(chunk: int):
    """Non-NaN fp32 bit patterns in increasing value order, split in segments.

    Negatives run from -inf (0xFF800000) down the bit patterns to -0.0
    (0x80000000); non-negatives from +0.0 (0) up to +inf (0x7F800000).  Each
    segment repeats the previous segment's last element, so the pairs across a
    segment boundary are checked too.
    """
    segs = []
    start = NEG_MAX
    while start >= NEG_MIN:
        end = max(NEG_MIN, start - chunk + 1)
        segs.append(("neg", start, end))
        start = end - 1
    start = 0
    while start <= NONNEG_MAX:
        end = min(NONNEG_MAX, start + chunk - 1)
        segs.append(("pos", start, end))
        start = end + 1
    return segs


def _segment_bits(seg, stride: int) -> np.ndarray:
    kind, a, b = seg
    if kind == "neg":
        bits = np.arange(a, b - 1, -stride, dtype=np.int64)
    else:
        bits = np.arange(a, b + 1, stride, dtype=np.int64)
    return bits.astype(np.uint32)


def _check_segment(args):
    order_key, seg, prev_bits, stride = args
    bits = _segment_bits(seg, stride)
    if prev_bits is not None:
        bits = np.concatenate([np.array([prev_bits], dtype=np.uint32), bits])
    vals = bits.view(np.float32)
    keys = np.asarray(order_key(vals), dtype=np.uint32)
    a, b = vals[:-1], vals[1:]
    # hardware float order: strictly increasing, except -0.0 -> +0.0 (equal).
    zero_pair = (a == 0) & (b == 0)
    float_ok = bool(np.all((b > a) | zero_pair))
    key_ok = bool(np.all(keys[1:] > keys[:-1]))
    return int(bits.size - (0 if prev_bits is None else 1)), float_ok, key_ok


def pin_keymap_exhaustive(order_key: Callable, stride: int = 1, chunk: int = 1 << 24,
                          procs: int = 8) -> None:
    """Keys strictly increase along the float order of all non-NaN patterns."""
    segs = _ascending_segments(chunk)
    jobs = []
    prev = None
    for seg in segs:
        jobs.append((order_key, seg, prev, stride))
        last = _segment_bits(seg, stride)[-1]
        prev = int(last)
    if procs > 1:
        ctx = mp.get_context("fork")
        with ctx.Pool(procs) as pool:
            results = pool.map(_check_segment, jobs, chunksize=1)
    else:
        results = [_check_segment(j) for j in jobs]
    count = sum(r[0] for r in results)
    assert all(r[1] for r in results), "enumeration is not in increasing float order"
    if stride == 1:
        assert count == N_NON_NAN, (count, N_NON_NAN)
    assert all(r[2] for r in results), "order key is not strictly increasing along the float order"


SPECIALS = np.array([-np.inf, -3.0e38, -1.0, -1.0e-38, -1.0e-45, -0.0, 0.0, 1.0e-45, 1.0e-38, 1.0, 3.0e38,
                     np.inf], dtype=np.float32)


def pin_keymap_specials(order_key: Callable) -> None:
    keys = np.asarray(order_key(SPECIALS), dtype=np.int64)
    assert np.all(np.diff(keys) > 0), "specials are not in increasing key order"
    neg0, pos0 = keys[5], keys[6]
    assert pos0 == neg0 + 1, "-0.0 and +0.0 are not adjacent keys"


# ----------------------------------------------------------------------------
# Selection: brute force with an order written independently of the key map.
# ----------------------------------------------------------------------------

def total_order(v: float):
    """Python-side total order: float compare, -0.0 placed just below +0.0."""
    v = float(v)
    return (v, 1 if (v == 0.0 and math.copysign(1.0, v) > 0) else 0)


def valid_subsets(values: List[float], n: int):
    """All n-subsets S of range(len(values)) with min(S) >= max(rest) in total_order."""
    L = len(values)
    tv = [total_order(x) for x in values]
    out = []
    for S in itertools.combinations(range(L), n):
        rest = [i for i in range(L) if i not in S]
        if not S or not rest or min(tv[i] for i in S) >= max(tv[i] for i in rest):
            out.append(frozenset(S))
    return out


TINY_ALPHABET = np.array([-np.inf, -1.0, -0.0, 0.0, 1.0, 2.0], dtype=np.float32)


def tiny_rows(seed: int = 7, count: int = 300):
    rng = np.random.Generator(np.random.PCG64(seed))
    for _ in range(count):
        L = int(rng.integers(0, 9))
        if rng.random() < 0.7:
            vals = TINY_ALPHABET[rng.integers(0, TINY_ALPHABET.size, size=L)]
        else:
            vals = rng.standard_normal(L).astype(np.float32)
        k = int(rng.integers(1, 11))
        yield vals.astype(np.float32), k


def pin_select_bruteforce(topk_transform_row: Callable) -> None:
    """The oracle's set is one of the valid subsets, and its size is min(k, L)."""
    for vals, k in tiny_rows():
        L = vals.size
        W = L + 2
        row = np.full(W, np.inf, dtype=np.float32)   # poison beyond L
        row[:L] = vals
        table = np.arange(W, dtype=np.int32)
        out, raw, info = topk_transform_row(row, L, table, k, 1)
        n = min(k, L)
        assert info.n == n, (vals, k, info)
        got = [int(x) for x in raw[:n]]
        assert len(set(got)) == n
        assert frozenset(got) in valid_subsets(list(vals), n), (vals.tolist(), k, got)
        assert np.all(raw[n:] == -1) and np.all(out[n:] == -1)


def pin_checker_bruteforce(check_row: Callable, topk_transform_row: Callable) -> None:
    """The checker accepts exactly the valid subsets (every n-subset is tried)."""
    for vals, k in itertools.islice(tiny_rows(seed=11, count=200), 200):
        L = vals.size
        n = min(k, L)
        W = L + 1
        row = np.full(W, np.inf, dtype=np.float32)
        row[:L] = vals
        table = np.arange(W, dtype=np.int32)[::-1].copy()   # injective, not identity
        _, _, info = topk_transform_row(row, L, table, k, 1)
        valid = set(valid_subsets(list(vals), n))
        for S in itertools.combinations(range(L), n):
            raw = np.full(k, -1, dtype=np.int64)
            raw[:n] = S
            out = np.full(k, -1, dtype=np.int64)
            out[:n] = table[np.array(S, dtype=np.int64)] if n else []
            ok_raw = not check_row(row, L, table, k, 1, out, raw, info)
            ok_out = not check_row(row, L, table, k, 1, out, None, info)
            expect = frozenset(S) in valid
            assert ok_raw == expect, (vals.tolist(), k, S)
            assert ok_out == expect, (vals.tolist(), k, S)


def pin_select_vs_torch(topk_transform_row: Callable, seed: int = 3) -> None:
    """On distinct values the answer is unique: it must equal torch.topk's set."""
    import torch
    rng = np.random.Generator(np.random.PCG64(seed))
    for trial in range(40):
        L = int(rng.integers(1, 5000))
        k = int(rng.integers(1, 2049))
        vals = rng.permutation(L).astype(np.float32) * np.float32(0.37) - np.float32(L / 5)
        vals = np.where(vals == 0, np.float32(0.5), vals).astype(np.float32)  # no signed-zero pairs
        assert np.unique(vals).size == L
        table = np.arange(L, dtype=np.int32)
        _, raw, info = topk_transform_row(vals, L, table, k, 1)
        n = min(k, L)
        ref = torch.topk(torch.from_numpy(vals), n).indices.numpy()
        assert set(raw[:n].tolist()) == set(ref.tolist())


def pin_closed_forms(topk_transform_row: Callable) -> None:
    W = 100
    table = np.arange(W, dtype=np.int32)
    asc = np.arange(W, dtype=np.float32) - 50
    desc = -asc
    for L in (0, 1, 7, 50, 100):
        for k in (1, 5, 50, 99, 100, 128):
            n = min(k, L)
            _, raw, info = topk_transform_row(asc, L, table, k, 1)
            assert set(raw[:n].tolist()) == set(range(L - n, L)), (L, k)
            _, raw, _ = topk_transform_row(desc, L, table, k, 1)
            assert set(raw[:n].tolist()) == set(range(n)), (L, k)
            assert np.all(raw[n:] == -1)
    # short rows: everything selected
    vals = np.random.Generator(np.random.PCG64(5)).standard_normal(W).astype(np.float32)
    _, raw, _ = topk_transform_row(vals, 30, table, 64, 1)
    assert sorted(raw[:30].tolist()) == list(range(30)) and np.all(raw[30:] == -1)
    # seq_len <= 0: nothing
    for L in (0, -1, -(2**31)):
        out, raw, info = topk_transform_row(vals, L, table, 8, 1)
        assert info.n == 0 and np.all(raw == -1) and np.all(out == -1)
    # seq_len > width: clamped to the width
    _, raw, info = topk_transform_row(desc, 10**6, table, 10, 1)
    assert info.L == W and set(raw[:10].tolist()) == set(range(10))
    _, raw, info = topk_transform_row(desc, W + 1, table, 200, 1)
    assert info.n == W and sorted(raw[:W].tolist()) == list(range(W))
    # constant row: n distinct positions, all equal
    const = np.full(W, 1.5, dtype=np.float32)
    _, raw, info = topk_transform_row(const, W, table, 17, 1)
    assert np.unique(raw[:17]).size == 17 and info.n_greater == 0 and info.n_equal == W
    # -0.0 is below +0.0
    z = np.array([-0.0, 0.0, -0.0, 0.0], dtype=np.float32)
    _, raw, _ = topk_transform_row(z, 4, table[:4], 2, 1)
    assert set(raw[:2].tolist()) == {1, 3}
    # -inf is an ordinary value below every finite one
    mi = np.array([-np.inf, -1e30, -np.inf, 3.0], dtype=np.float32)
    _, raw, _ = topk_transform_row(mi, 4, table[:4], 3, 1)
    assert set(raw[:3].tolist()) == {1, 3, 0} or set(raw[:3].tolist()) == {1, 3, 2}


def pin_transform(topk_transform_row: Callable, transform_positions: Callable) -> None:
    # Hand-computed: table row [7, 3, 5], page_size 4.
    #   position 0  -> page 0 -> 7*4 + 0 = 28
    #   position 5  -> page 1 -> 3*4 + 1 = 13
    #   position 11 -> page 2 -> 5*4 + 3 = 23
    t = np.array([7, 3, 5], dtype=np.int32)
    got = transform_positions(np.array([0, 5, 11]), t, 4)
    assert got.tolist() == [28, 13, 23], got
    # same through the full row function: descending row selects positions 0..2
    row = np.array([9, 8, 7, 1, 1, 1, 1, 1, 1, 1, 1, 1], dtype=np.float32)
    out, raw, _ = topk_transform_row(row, 12, t, 3, 4)
    assert sorted(zip(raw[:3].tolist(), out[:3].tolist())) == [(0, 28), (1, 29), (2, 30)]
    row2 = np.zeros(12, dtype=np.float32)
    row2[5], row2[11] = 4.0, 3.0
    out, raw, _ = topk_transform_row(row2, 12, t, 2, 4)
    assert dict(zip(raw[:2].tolist(), out[:2].tolist())) == {5: 13, 11: 23}
    rng = np.random.Generator(np.random.PCG64(9))
    for ps in (1, 2, 16, 64, 256):
        W = ps * 37 + (ps // 2)
        P = -(-W // ps)
        vals = rng.standard_normal(W).astype(np.float32)
        ident = np.arange(P, dtype=np.int32)
        out, raw, info = topk_transform_row(vals, W, ident, 40, ps)
        assert np.array_equal(out, raw), ps                        # identity table: out == raw
        perm = rng.permutation(P).astype(np.int32)
        out, raw, info = topk_transform_row(vals, W, perm, 40, ps)
        inv = np.argsort(perm)
        n = info.n
        back = inv[out[:n] // ps] * ps + out[:n] % ps
        assert np.array_equal(back, raw[:n]), ps                   # inverse permutation recovers raw
        if ps == 1:
            assert np.array_equal(out[:n], perm[raw[:n]])          # page_size 1: out = table[raw]
