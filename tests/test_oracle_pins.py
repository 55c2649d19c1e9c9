"""CPU tests: the oracle against its pins (no GPU)."""
import numpy as np
import pytest

import pins
from oracle import check_row, order_key, topk_transform, topk_transform_row, transform_positions


def test_keymap_exhaustive_all_patterns():
    pins.pin_keymap_exhaustive(order_key, stride=1, procs=8)


def test_keymap_specials():
    pins.pin_keymap_specials(order_key)
    assert int(order_key(np.array([np.inf], np.float32))[0]) == 0xFF800000
    assert int(order_key(np.array([-np.inf], np.float32))[0]) == 0x007FFFFF


def test_select_bruteforce():
    pins.pin_select_bruteforce(topk_transform_row)


def test_checker_accepts_exactly_valid_subsets():
    pins.pin_checker_bruteforce(check_row, topk_transform_row)


def test_select_vs_torch_topk_distinct():
    pins.pin_select_vs_torch(topk_transform_row)


def test_closed_forms():
    pins.pin_closed_forms(topk_transform_row)


def test_transform():
    pins.pin_transform(topk_transform_row, transform_positions)


def test_torch_answer_passes_checker_on_ties():
    """On tie-heavy rows (no signed zeros) torch.topk's choice is one valid answer."""
    import torch
    rng = np.random.Generator(np.random.PCG64(21))
    for trial in range(30):
        L = int(rng.integers(1, 3000))
        k = int(rng.integers(1, 600))
        vals = rng.integers(-4, 5, size=L).astype(np.float32) + np.float32(0.5)
        table = rng.permutation(L).astype(np.int32)
        n = min(k, L)
        idx = torch.topk(torch.from_numpy(vals), n).indices.numpy()
        raw = np.full(k, -1, np.int64)
        raw[:n] = idx
        out = np.full(k, -1, np.int64)
        out[:n] = table[idx]
        assert check_row(vals, L, table, k, 1, out, raw) == []
        assert check_row(vals, L, table, k, 1, out, None) == []


def test_checker_rejects_corruptions():
    rng = np.random.Generator(np.random.PCG64(4))
    W, k, ps = 4096, 256, 16
    vals = rng.standard_normal(W).astype(np.float32)
    table = rng.permutation(W // ps).astype(np.int32)
    out, raw, info = topk_transform_row(vals, 3000, table, k, ps)
    assert check_row(vals, 3000, table, k, ps, out, raw, info) == []
    # a wrong element
    bad = raw.copy(); bad[3] = int(np.argmin(vals[:3000]))
    assert check_row(vals, 3000, table, k, ps, out, bad, info)
    # a duplicate
    bad = raw.copy(); bad[4] = bad[5]
    assert check_row(vals, 3000, table, k, ps, out, bad, info)
    # out of range (poisoned position beyond seq_len)
    bad = raw.copy(); bad[0] = 3500
    assert check_row(vals, 3000, table, k, ps, out, bad, info)
    # transform mismatch in one slot
    bo = out.copy(); bo[7] += 1
    assert check_row(vals, 3000, table, k, ps, bo, raw, info)
    # a missing -1 in the tail
    short_out, short_raw, sinfo = topk_transform_row(vals, 100, table, k, ps)
    bo = short_out.copy(); bo[150] = 0
    assert check_row(vals, 100, table, k, ps, bo, short_raw, sinfo)
    # out alone: swapped slot values are fine, a changed value is not
    bo = out.copy(); bo[[1, 2]] = bo[[2, 1]]
    assert check_row(vals, 3000, table, k, ps, bo, None, info) == []
    bo = out.copy(); bo[9] = out[9] ^ 1
    assert check_row(vals, 3000, table, k, ps, bo, None, info)


def test_batch_oracle_shapes_and_rows():
    rng = np.random.Generator(np.random.PCG64(8))
    B, W, k, ps = 5, 300, 64, 4
    scores = rng.standard_normal((B, W)).astype(np.float32)
    seq = np.array([0, 10, 64, 65, 1000], dtype=np.int32)
    table = np.tile(np.arange(W // ps, dtype=np.int32), (B, 1))
    out, raw, infos = topk_transform(scores, seq, table, k, ps)
    assert out.shape == (B, k) and raw.shape == (B, k)
    assert [i.n for i in infos] == [0, 10, 64, 64, 64]
    out2, raw2, _ = topk_transform(scores, seq, table, k, ps, rows=[3, 1])
    assert np.array_equal(out2[0], out[3]) and np.array_equal(raw2[1], raw[1])
    with pytest.raises(ValueError):
        topk_transform(scores, seq, table, k, 3)
    with pytest.raises(ValueError):
        topk_transform(scores, seq, table, 0, 4)
