"""CPU tests: the seeded generators (shapes, poisoning, determinism) and the golden fixture."""
import json
import os

import numpy as np

import workloads
from oracle import topk_transform

HERE = os.path.dirname(os.path.abspath(__file__))


def test_c1_golden_fixture_reproduces():
    with open(os.path.join(HERE, "golden", "c1_expected.json")) as f:
        g = json.load(f)
    w = workloads.c1()
    out, raw, infos = topk_transform(w.scores, w.seq_lens, w.page_table, w.k, w.page_size)
    assert infos[0].threshold == g["threshold_key"]
    assert infos[0].n_greater == g["n_greater"] and infos[0].n_equal == g["n_equal"]
    assert sorted(raw[0][: g["n"]].tolist()) == g["selected_positions_sorted"]
    assert sorted(out[0][: g["n"]].tolist()) == g["transformed_sorted"]


def test_generators_deterministic_and_poisoned():
    a, b = workloads.c2(), workloads.c2()
    assert np.array_equal(a.scores, b.scores) and np.array_equal(a.page_table, b.page_table)
    assert a.scores.dtype == np.float32 and a.seq_lens.dtype == np.int32 and a.page_table.dtype == np.int32
    assert a.scores.shape == (64, 65536) and a.page_table.shape == (64, 1024)
    for r in range(a.batch):
        L = int(a.seq_lens[r])
        assert 4096 <= L <= 65536
        assert np.all(np.isinf(a.scores[r, L:])) and np.all(a.scores[r, L:] > 0)
        used = -(-L // a.page_size)
        assert np.all(a.page_table[r, used:] == workloads.INT32_MIN)
        assert np.unique(a.page_table[r, :used]).size == used
    # exact +0.0 appears (all eight relu terms zero) at roughly 2^-8
    valid = a.scores[0, : a.seq_lens[0]]
    frac = np.count_nonzero(valid == 0) / valid.size
    assert 0.001 < frac < 0.01


def test_c5_structure():
    w = workloads.c5()
    assert w.k == 1024 and w.page_size == 16 and w.scores.shape == (128, 131072)
    assert int(w.seq_lens[7]) == 0 and int(w.seq_lens[15]) == w.k - 1
    for b in range(128):
        if b % 8 == 7:
            assert 0 <= w.seq_lens[b] < w.k
        else:
            assert w.seq_lens[b] == 131072
    finite = w.scores[0][np.isfinite(w.scores[0])]
    assert np.unique(finite).size == 256
    frac_neginf = np.count_nonzero(w.scores[0] == -np.inf) / w.scores.shape[1]
    assert 0.04 < frac_neginf < 0.06
    # bf16-representable: low 16 bits clear
    assert np.all((finite.view(np.uint32) & 0xFFFF) == 0)


def test_custom_kinds():
    for kind in ("normal", "ties", "const", "neginf", "zeros", "asc", "desc", "int", "wide", "crowded"):
        w = workloads.custom(1, 3, 1000, 64, 16, seq_lens=[0, 500, 1000], kind=kind)
        assert w.scores.shape == (3, 1000) and w.page_table.shape == (3, 63)
        assert np.all(np.isposinf(w.scores[1, 500:]))


def test_mixed_structure():
    w = workloads.mixed()
    assert w.k == 2048 and w.page_size == 64 and w.scores.shape == (32, 1 << 20)
    assert w.seq_lens.tolist() == [1 << 20] * 4 + [16384] * 28
    assert np.all(np.isposinf(w.scores[4:, 16384:]))
    assert np.all(w.page_table[4:, 256:] == workloads.INT32_MIN)
    assert np.unique(w.page_table[0]).size == w.page_table.shape[1]
