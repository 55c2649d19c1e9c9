"""GPU parity of the indexer scoring (indexer_logits) and the fused scoring +
exact top-k (indexer_topk) against the CPU oracle, through the C ABI.

Scores: every written logit is compared with the oracle's float64 score within
the oracle's derived fp32 error bound for that position (fp8 products exact,
D + H + 2 roundings).  Selections: the page's tie-tolerant exactness test
(LiteTopk PR #32094, Validation) with the tolerance set to twice the largest
bound of the row, plus count, -1 padding, uniqueness and range.  The fused
path is also checked, without the oracle, to be an exact top-k of the GPU's
own logits (same fp32 values, both kernels share one scoring routine).
"""
import numpy as np
import pytest

from gpu_util import note
from oracle import indexer_oracle as ix
from workloads import indexer as wl

pytestmark = pytest.mark.gpu

SMALL = ["odd_widths_k512", "short_8x1k_k2048", "flat_8x16k_k2048", "ragged_3req_k2048", "single_32x32k_k512"]


class _select_mode:
    """Forces indexer_topk's select mode for a block: 0 the fused scan, 1 dense
    scores + select, -1 automatic (the default, restored on exit)."""

    def __init__(self, lib, mode):
        self.lib, self.mode = lib, mode

    def __enter__(self):
        self.lib.indexer_set_select_mode(self.mode)

    def __exit__(self, *exc):
        self.lib.indexer_set_select_mode(-1)
        return False


def _upload(w):
    import torch
    dev = torch.device("cuda", 0)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return t(w.q), t(w.weights), t(w.kv), t(w.kv_scale), t(w.ks), t(w.ke)


def _lengths(w):
    lo = np.clip(w.ks.astype(np.int64), 0, w.num_kv)
    hi = np.clip(w.ke.astype(np.int64), 0, w.num_kv)
    return lo, np.maximum(hi - lo, 0)


def _logits(lib, w, tensors=None):
    import torch
    tensors = tensors or _upload(w)
    lo, L = _lengths(w)
    width = int(max(1, L.max()))
    out = torch.full((w.num_q, width), float("nan"), dtype=torch.float32, device="cuda")
    lib.indexer_logits(*tensors, width, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _row_eps(w, r):
    pos = ix.key_range(int(w.ks[r]), int(w.ke[r]), w.num_kv)
    b = ix.fp32_error_bound(w.q[r], w.weights[r], w.kv, w.kv_scale, pos)
    return 2.0 * float(b.max()) if len(b) else 0.0


def _check_logits(w, got, rows):
    lo, L = _lengths(w)
    for r in rows:
        pos = ix.key_range(int(w.ks[r]), int(w.ke[r]), w.num_kv)
        exact = ix.indexer_scores_row(w.q[r], w.weights[r], w.kv, w.kv_scale, pos)
        bound = ix.fp32_error_bound(w.q[r], w.weights[r], w.kv, w.kv_scale, pos)
        g = got[r, :L[r]].astype(np.float64)
        assert np.all(np.isfinite(g)), f"{w.name} row {r}: unwritten or non-finite logits"
        err = np.abs(g - exact)
        bad = np.nonzero(err > bound)[0]
        assert len(bad) == 0, (f"{w.name} row {r}: {len(bad)} logits outside the bound, first at {bad[0]}: "
                               f"{g[bad[0]]!r} vs {exact[bad[0]]!r} (bound {bound[bad[0]]!r})")
        assert np.all(np.isnan(got[r, L[r]:])), f"{w.name} row {r}: written past the row's length"


def _check_topk(w, out, rows):
    lo, L = _lengths(w)
    for r in rows:
        pos = ix.key_range(int(w.ks[r]), int(w.ke[r]), w.num_kv)
        exact = ix.indexer_scores_row(w.q[r], w.weights[r], w.kv, w.kv_scale, pos)
        errs = ix.check_indexer_row(exact, pos.start, w.k, out[r], _row_eps(w, r))
        assert not errs, f"{w.name} row {r}: " + "; ".join(errs)


def _check_exact_on_logits(w, out, logits):
    """Without the oracle: the selection is an exact top-n of the GPU's own fp32 logits."""
    lo, L = _lengths(w)
    for r in range(w.num_q):
        n = min(w.k, int(L[r]))
        sel = out[r, :n].astype(np.int64) - lo[r]
        assert np.all(out[r, n:] == -1), f"row {r}: padding"
        assert len(np.unique(sel)) == n and np.all((sel >= 0) & (sel < L[r])), f"row {r}: invalid positions"
        if n == 0 or n == L[r]:
            continue
        row = logits[r, :L[r]]
        mask = np.zeros(L[r], bool)
        mask[sel] = True
        assert row[mask].min() >= row[~mask].max(), f"row {r}: not a top-{n} of the GPU logits"


@pytest.mark.parametrize("name", SMALL)
def test_logits_vs_oracle(lib, name):
    w = wl.make_config(name)
    note(f"indexer_logits {name} num_q={w.num_q} num_kv={w.num_kv}")
    got = _logits(lib, w)
    _check_logits(w, got, range(w.num_q))


def test_logits_every_fp8_code(lib):
    """Key j holds the j-th finite E4M3 code on dimension 5; head 0 sees +1 and
    head 1 sees -1 there, with weights 1 and 2: score = relu(v) + 2 relu(-v),
    exact in fp32 -- the widening of every code, subnormals and zeros included."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    n = len(codes)
    kv = np.zeros((n, 128), np.uint8)
    kv[:, 5] = codes
    q = np.zeros((1, 32, 128), np.uint8)
    q[0, 0, 5] = 0x38
    q[0, 1, 5] = 0xB8
    wts = np.zeros((1, 32), np.float32)
    wts[0, 0], wts[0, 1] = 1.0, 2.0
    w = wl.IndexerWorkload("fp8_codes", q, wts, kv, np.ones(n, np.float32), np.array([0], np.int32),
                           np.array([n], np.int32), k=8, seed=0)
    note("indexer_logits every fp8 code")
    got = _logits(lib, w)[0, :n].astype(np.float64)
    v = ix.fp8_e4m3_decode(codes)
    assert np.array_equal(got, np.maximum(v, 0) + 2 * np.maximum(-v, 0))


def test_logits_narrower_than_rows(lib):
    """An output narrower than some rows: each row's first min(length, width)
    scores are written, within the bound, and nothing past them (a write past
    a row's width would land in the next row's columns)."""
    import torch
    w = wl.make([(5, 3000)], 256, seed=7250)
    w.ks = np.array([0, 100, 2000, -50, 2990], np.int32)
    w.ke = np.array([3000, 2100, 9999, 700, 3000], np.int32)
    _, L = _lengths(w)
    width = 777   # below rows 0..2, above rows 3 and 4; not a multiple of 32
    note(f"indexer_logits narrower output width={width}")
    out = torch.full((w.num_q, width), float("nan"), dtype=torch.float32, device="cuda")
    lib.indexer_logits(*_upload(w), width, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for r in range(w.num_q):
        n = int(min(L[r], width))
        pos = ix.key_range(int(w.ks[r]), int(w.ke[r]), w.num_kv)
        exact = ix.indexer_scores_row(w.q[r], w.weights[r], w.kv, w.kv_scale, pos)[:n]
        bound = ix.fp32_error_bound(w.q[r], w.weights[r], w.kv, w.kv_scale, pos)[:n]
        g = got[r, :n].astype(np.float64)
        assert np.all(np.isfinite(g)), f"row {r}: unwritten logits"
        assert np.all(np.abs(g - exact) <= bound), f"row {r}: logits outside the bound"
        assert np.all(np.isnan(got[r, n:])), f"row {r}: written past min(length, width)"


@pytest.mark.parametrize("mode", [0, 1, -1])
@pytest.mark.parametrize("name", SMALL)
def test_indexer_topk_vs_oracle(lib, name, mode):
    """Each select mode: the fused scan (0), dense scores + select (1) and the
    automatic choice (-1)."""
    import torch
    w = wl.make_config(name)
    note(f"indexer_topk {name} num_q={w.num_q} num_kv={w.num_kv} k={w.k} mode={mode}")
    tensors = _upload(w)
    out = torch.full((w.num_q, w.k), 0x7F7F7F7F, dtype=torch.int32, device="cuda")
    with _select_mode(lib, mode):
        lib.indexer_topk(*tensors, w.k, out=out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    _check_topk(w, o, range(w.num_q))
    _check_exact_on_logits(w, o, _logits(lib, w, tensors))


@pytest.mark.parametrize("requests,k,distinct,window", [
    ([(16, 131072)], 64, None, 0),           # automatic windows
    ([(16, 131072)], 64, None, 1 << 20),     # one window: the lists are trimmed many times
    ([(8, 65536)], 2048, None, 1 << 20),     # trims at the largest k
    ([(8, 65536)], 2048, None, 24576),       # three windows merged by the select
    ([(8, 40000)], 16, 4, 1 << 20),          # four distinct key rows: crowded bins, exact trims
    ([(3, 70000), (5, 9000)], 300, 64, 1 << 20),
    ([(3, 70000), (5, 9000)], 300, 64, 8192),
    ([(8, 40000)], 1, None, 1 << 20),         # k = 1
    ([(8, 40000)], 1, 4, 1 << 20),            # k = 1 among crowded ties
])
def test_indexer_topk_trims(lib, requests, k, distinct, window):
    """Rows much longer than the candidate capacity, so the lists are trimmed
    and the gate raised many times; with few distinct keys the trims take the
    exact (tie-cutting) path."""
    import torch
    lib.indexer_set_window_override(window)
    w = wl.make(requests, k, seed=7100 + k)
    if distinct:
        rng = np.random.default_rng(k)
        rows = w.kv[:distinct].copy()
        w.kv = rows[rng.integers(0, distinct, w.num_kv)]
        w.kv_scale = np.ones(w.num_kv, np.float32)
    note(f"indexer_topk trims requests={requests} k={k} distinct={distinct} window={window}")
    tensors = _upload(w)
    out = torch.full((w.num_q, w.k), 0x7F7F7F7F, dtype=torch.int32, device="cuda")
    try:
        with _select_mode(lib, 0):   # the fused scan, whatever the window
            lib.indexer_topk(*tensors, w.k, out=out)
        torch.cuda.synchronize()
    finally:
        lib.indexer_set_window_override(0)
    o = out.cpu().numpy()
    _check_topk(w, o, range(w.num_q))
    _check_exact_on_logits(w, o, _logits(lib, w, tensors))


@pytest.mark.parametrize("k", [1, 512])
def test_indexer_topk_narrow_scores(lib, k):
    """Every key is the same vector, scaled by a distinct factor in [1, 1.1):
    a row's scores share one or two 11-bit key bins but differ in the next
    digits, so the trims cut at a 22-bit bin edge instead."""
    import torch
    lib.indexer_set_window_override(1 << 20)
    w = wl.make([(8, 65536)], k, seed=7400 + k)
    rng = np.random.default_rng(7400 + k)
    w.kv = np.repeat(w.kv[:1], w.num_kv, axis=0)
    w.kv_scale = rng.uniform(1.0, 1.1, w.num_kv).astype(np.float32)
    note(f"indexer_topk narrow scores k={k}")
    tensors = _upload(w)
    out = torch.full((w.num_q, w.k), 0x7F7F7F7F, dtype=torch.int32, device="cuda")
    try:
        with _select_mode(lib, 0):   # the fused scan, whatever the window
            lib.indexer_topk(*tensors, w.k, out=out)
        torch.cuda.synchronize()
    finally:
        lib.indexer_set_window_override(0)
    o = out.cpu().numpy()
    _check_topk(w, o, range(w.num_q))
    _check_exact_on_logits(w, o, _logits(lib, w, tensors))


@pytest.mark.parametrize("k", [64, 2048])
def test_indexer_topk_calibration_overrated(lib, k):
    """The fused scan starts each long row behind a gate set from a sample of
    its window: the middle stage (64 positions) of each of 32 equal runs of
    the window's stages.  Here exactly those positions have their scale raised
    1000-fold, so the sample overrates every row: the starting gate lies above
    all of the row's other scores, the first pass ends with fewer than k
    entries, and the row is scanned again from gate 0.  The result must still
    be exact."""
    import torch
    lib.indexer_set_window_override(1 << 20)   # one window: the span is [0, 65536), 1024 stages
    w = wl.make([(8, 65536)], k, seed=7500 + k)
    stages = 65536 // 64
    stride = stages // 32
    boosted = np.zeros(w.num_kv, bool)
    for i in range(32):
        st = i * stride + stride // 2
        boosted[st * 64:(st + 1) * 64] = True
    w.kv_scale = np.where(boosted, w.kv_scale * np.float32(1000.0), w.kv_scale).astype(np.float32)
    note(f"indexer_topk calibration overrated k={k}")
    tensors = _upload(w)
    out = torch.full((w.num_q, w.k), 0x7F7F7F7F, dtype=torch.int32, device="cuda")
    try:
        with _select_mode(lib, 0):   # the fused scan, whatever the window
            lib.indexer_topk(*tensors, w.k, out=out)
        torch.cuda.synchronize()
    finally:
        lib.indexer_set_window_override(0)
    o = out.cpu().numpy()
    _check_topk(w, o, range(w.num_q))
    _check_exact_on_logits(w, o, _logits(lib, w, tensors))


@pytest.mark.parametrize("mode", [0, 1])
def test_indexer_edge_ranges(lib, mode):
    """Empty, inverted, clamped and shorter-than-k ranges; rows not a multiple of 8."""
    import torch
    w = wl.make([(5, 3000)], 256, seed=7200)
    w.ks = np.array([0, 100, 2000, -50, 2990], np.int32)
    w.ke = np.array([0, 90, 9999, 40, 3000], np.int32)   # empty, inverted, past the end, before 0, 10 positions
    note(f"indexer_topk edge ranges mode={mode}")
    tensors = _upload(w)
    out = torch.full((w.num_q, w.k), 0x7F7F7F7F, dtype=torch.int32, device="cuda")
    with _select_mode(lib, mode):
        lib.indexer_topk(*tensors, w.k, out=out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[0] == -1) and np.all(o[1] == -1)
    _check_topk(w, o, range(w.num_q))
    _check_logits(w, _logits(lib, w, tensors), range(w.num_q))


@pytest.mark.parametrize("modes", [(0, 0), (1, 1), (1, 0), (0, 1)])
def test_indexer_repeat_calls_and_smaller_input(lib, modes):
    """A second call on a smaller batch reuses the buffers and clears its
    counters, in either select mode after either."""
    import torch
    for reqs, mode in zip(([(24, 20000)], [(6, 5000)]), modes):
        w = wl.make(reqs, 512, seed=7300 + reqs[0][0])
        note(f"indexer_topk repeat {reqs} mode={mode}")
        tensors = _upload(w)
        out = torch.full((w.num_q, w.k), 0x7F7F7F7F, dtype=torch.int32, device="cuda")
        with _select_mode(lib, mode):
            lib.indexer_topk(*tensors, w.k, out=out)
        torch.cuda.synchronize()
        _check_topk(w, out.cpu().numpy(), range(w.num_q))


def test_indexer_prefill_full_size_sampled(lib):
    """The performance shape (8192 query rows over 262144 keys, top-2048):
    sampled rows against the oracle, and every row's size-independent properties."""
    import torch
    w = wl.make_config("prefill_8192x256k_k2048")
    note("indexer_topk prefill 8192 x 262144 k=2048 (sampled)")
    tensors = _upload(w)
    out = torch.full((w.num_q, w.k), 0x7F7F7F7F, dtype=torch.int32, device="cuda")
    lib.indexer_topk(*tensors, w.k, out=out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    lo, L = _lengths(w)
    for r in range(w.num_q):
        n = min(w.k, int(L[r]))
        assert np.all(o[r, n:] == -1)
        head = o[r, :n].astype(np.int64)
        assert len(np.unique(head)) == n and np.all((head >= lo[r]) & (head < lo[r] + L[r]))
    _check_topk(w, o, [0, 1, 2047, 4095, 6000, 8190, 8191])


def test_indexer_short_prefill_sampled(lib):
    """The causal prefill of 1024 query rows over 65536 keys, top-2048: the
    windows are short (16K positions), so the automatic choice scores densely
    and selects; sampled rows against the oracle, every row's properties."""
    import torch
    w = wl.make_config("prefill_1024x64k_k2048")
    note("indexer_topk prefill 1024 x 65536 k=2048 (sampled)")
    tensors = _upload(w)
    out = torch.full((w.num_q, w.k), 0x7F7F7F7F, dtype=torch.int32, device="cuda")
    lib.indexer_topk(*tensors, w.k, out=out)
    torch.cuda.synchronize()
    assert lib.topk_last_launch().startswith("indexer-topk dense"), lib.topk_last_launch()
    o = out.cpu().numpy()
    lo, L = _lengths(w)
    for r in range(w.num_q):
        n = min(w.k, int(L[r]))
        assert np.all(o[r, n:] == -1)
        head = o[r, :n].astype(np.int64)
        assert len(np.unique(head)) == n and np.all((head >= lo[r]) & (head < lo[r] + L[r]))
    _check_topk(w, o, [0, 1, 511, 1022, 1023])
