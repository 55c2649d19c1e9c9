"""Pins of the indexer oracle (fp8 decode, scores, selection, checker) to
things other than itself: torch's fp8 conversion, the E4M3 format's closed
forms, one-hot closed forms of the score formula, the heads-folded identity of
the non-negative case, brute force over all subsets, and the checker's
rejection of planted mistakes.  CPU only."""
import itertools

import numpy as np
import pytest
import torch

from oracle import indexer_oracle as ix
from workloads import indexer as wl

ONE = 0x38        # 1.0 in E4M3
HALF = 0x30       # 0.5
TWO = 0x40        # 2.0
NEG_ONE = 0xB8    # -1.0


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = ix.fp8_e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2                         # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0), (0x3C, 1.5), (0x40, 2.0), (0x30, 0.5), (0xB8, -1.0),
    (0x7E, 448.0), (0xFE, -448.0), (0x08, 2.0 ** -6), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
    (0x00, 0.0),
])
def test_decode_closed_forms(code, value):
    assert ix.fp8_e4m3_decode(np.array([code], np.uint8))[0] == value
    assert np.signbit(ix.fp8_e4m3_decode(np.array([0x80], np.uint8))[0])


def _one_hot_inputs(values, heads=3, dim=8, axis=5, head=1, weight=1.0):
    """Query head `head` is e_axis; key j is values[j] * e_axis (as fp8 codes);
    only head `head` carries weight, so score_j = s_j * weight * relu(values[j])."""
    q = np.zeros((heads, dim), np.uint8)
    q[head, axis] = ONE
    kv = np.zeros((len(values), dim), np.uint8)
    kv[:, axis] = wl.to_fp8_codes(np.array(values, np.float32))
    w = np.zeros(heads, np.float32)
    w[head] = weight
    return q, w, kv


def test_scores_one_hot_closed_form():
    values = [1.0, -2.0, 0.5, 3.0, -0.25, 0.0]
    s = np.array([1.0, 2.0, 4.0, 0.5, 3.0, 1.0], np.float32)
    q, w, kv = _one_hot_inputs(values, weight=-1.5)
    got = ix.indexer_scores_row(q, w, kv, s, range(0, len(values)))
    expect = np.array([s[j] * -1.5 * max(values[j], 0.0) for j in range(len(values))])
    assert np.array_equal(got, expect)
    # a sub-range scores only its own positions, in position order
    assert np.array_equal(ix.indexer_scores_row(q, w, kv, s, range(2, 4)), expect[2:4])
    assert len(ix.indexer_scores_row(q, w, kv, s, range(3, 3))) == 0


def test_scores_heads_folded_identity_nonnegative():
    """With non-negative queries and keys the relu is inactive, so
    score_j = s_j * (sum_h w_h q_h) . kv_j: the heads fold into one query."""
    rng = np.random.default_rng(3)
    H, D, n = 32, 128, 40
    q = wl.to_fp8_codes(np.abs(rng.standard_normal((H, D))))
    kv = wl.to_fp8_codes(np.abs(rng.standard_normal((n, D))))
    w = rng.standard_normal(H).astype(np.float32)
    s = rng.uniform(0.5, 2.0, n).astype(np.float32)
    qf = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64)
    kf = torch.from_numpy(kv).view(torch.float8_e4m3fn).to(torch.float64)
    folded = torch.from_numpy(w.astype(np.float64)) @ qf                      # (D,)
    expect = (kf @ folded) * torch.from_numpy(s.astype(np.float64))
    got = ix.indexer_scores_row(q, w, kv, s, range(0, n))
    assert np.allclose(got, expect.numpy(), rtol=1e-12, atol=0)


def test_scores_relu_is_per_head():
    """Head 0 sees +1 and head 1 sees -1 on the same key: relu applies per head
    before the weighted sum (a relu after the sum would give 0 here)."""
    q = np.zeros((2, 4), np.uint8)
    q[0, 0] = ONE
    q[1, 0] = NEG_ONE
    kv = np.zeros((1, 4), np.uint8)
    kv[0, 0] = TWO
    w = np.array([1.0, 1.0], np.float32)
    got = ix.indexer_scores_row(q, w, kv, np.ones(1, np.float32), range(0, 1))
    assert got[0] == 2.0


def test_key_range_clamps():
    assert ix.key_range(-5, 3, 10) == range(0, 3)
    assert ix.key_range(4, 50, 10) == range(4, 10)
    assert len(ix.key_range(6, 2, 10)) == 0
    assert len(ix.key_range(12, 20, 10)) == 0


def _tiny_row(values):
    """Inputs whose scores are exactly `values` (non-negative, fp8-exact)."""
    q, w, kv = _one_hot_inputs(values, heads=2, dim=4, axis=2, head=0)
    return q, w, kv, np.ones(len(values), np.float32)


@pytest.mark.parametrize("values", [
    [0.0, 1.0, 1.0, 2.0, 0.5, 1.0, 2.0],
    [1.0] * 6,
    [3.0, 2.0, 1.0, 0.5, 0.25],
    [0.5, 0.5, 4.0, 0.0, 0.0, 4.0, 1.0, 0.5],
])
def test_selection_brute_force_all_subsets(values):
    q, w, kv, s = _tiny_row(values)
    L = len(values)
    scores = np.array(values, np.float64)
    for k in range(1, L + 3):
        info = ix.indexer_topk_row(q, w, kv, s, 0, L, k)
        n = min(k, L)
        assert info.n == n and len(info.selected) == n
        valid = set()
        for sub in itertools.combinations(range(L), n):
            rest = [i for i in range(L) if i not in sub]
            if not rest or min(scores[list(sub)]) >= max(scores[rest]):
                valid.add(frozenset(sub))
        assert frozenset(info.selected.tolist()) in valid
        for sub in itertools.combinations(range(L), n):
            row = np.full(k, -1, np.int64)
            row[:n] = sub
            ok = not ix.check_indexer_row(scores, 0, k, row, eps=0.0)
            assert ok == (frozenset(sub) in valid), (values, k, sub)


def test_selection_offsets_and_padding():
    values = [1.0, 3.0, 2.0, 0.5]
    q, w, kv, s = _tiny_row(values)
    qs = np.stack([q, q, q])
    ws = np.stack([w, w, w])
    out, infos = ix.indexer_topk(qs, ws, kv, s, np.array([1, 0, 3], np.int32),
                                 np.array([4, 2, 3], np.int32), k=3)
    assert sorted(out[0].tolist()) == [1, 2, 3]          # positions 1..3: all three
    assert out[1].tolist()[:2] == [1, 0] and out[1, 2] == -1
    assert out[2].tolist() == [-1, -1, -1]               # empty range
    assert infos[0].v_k == 0.5 and infos[1].v_k == 1.0


def test_checker_rejects_planted_mistakes():
    rng = np.random.default_rng(5)
    scores = rng.standard_normal(200)
    k = 16
    good = np.argsort(-scores)[:k] + 100
    assert not ix.check_indexer_row(scores, 100, k, good, eps=0.0)
    bad = good.copy()
    bad[3] = np.argsort(-scores)[k] + 100                 # swap in the (k+1)-th
    assert ix.check_indexer_row(scores, 100, k, bad, eps=0.0)
    dup = good.copy()
    dup[1] = dup[0]
    assert ix.check_indexer_row(scores, 100, k, dup, eps=0.0)
    out_of_range = good.copy()
    out_of_range[0] = 99
    assert ix.check_indexer_row(scores, 100, k, out_of_range, eps=0.0)
    short = np.full(k + 4, -1, np.int64)
    short[:k] = good
    assert ix.check_indexer_row(scores, 100, k + 4, short, eps=0.0)    # k + 4 slots must be filled
    padded = np.full(300, -1, np.int64)
    padded[:200] = np.arange(100, 300)
    assert not ix.check_indexer_row(scores, 100, 300, padded, eps=0.0)
    padded[250] = 5
    assert ix.check_indexer_row(scores, 100, 300, padded, eps=0.0)


def test_error_bound_covers_fp32_sums():
    """Scores summed in fp32 in two different orders stay within the bound."""
    w_ = wl.make([(4, 600)], k=64, seed=11)
    for r in range(w_.num_q):
        pos = ix.key_range(int(w_.ks[r]), int(w_.ke[r]), w_.num_kv)
        exact = ix.indexer_scores_row(w_.q[r], w_.weights[r], w_.kv, w_.kv_scale, pos)
        bound = ix.fp32_error_bound(w_.q[r], w_.weights[r], w_.kv, w_.kv_scale, pos)
        qf = torch.from_numpy(w_.q[r]).view(torch.float8_e4m3fn).float()
        kf = torch.from_numpy(w_.kv[pos.start:pos.stop]).view(torch.float8_e4m3fn).float()
        s = torch.from_numpy(w_.kv_scale[pos.start:pos.stop])
        wt = torch.from_numpy(w_.weights[r])
        a = (torch.relu(kf @ qf.T) * wt).sum(1) * s
        b = torch.relu(kf.flip(1) @ qf.flip(1).T).flip(1) @ wt.flip(0) * s
        for got in (a, b):
            err = np.abs(got.double().numpy() - exact)
            assert np.all(err <= bound), (err / np.maximum(bound, 1e-30)).max()
        assert bound.max() < 1e-3 * max(1.0, np.abs(exact).max())


def test_workload_ranges_are_causal():
    ks, ke, n = wl.ranges([(3, 10), (2, 5)])
    assert n == 15
    assert ks.tolist() == [0, 0, 0, 10, 10]
    assert ke.tolist() == [8, 9, 10, 14, 15]
    w_ = wl.make_config("odd_widths_k512")
    assert w_.q.shape == (14, 32, 128) and w_.kv.shape == (5122, 128)
    assert w_.q.dtype == np.uint8 and w_.weights.dtype == np.float32
    assert np.all((w_.q & 0x7F) != 0x7F) and np.all((w_.kv & 0x7F) != 0x7F)
