"""GPU parity of the deterministic entry point (topk_transform_sorted).

Its output is unique -- the plain definition's order: key descending, equal
keys by position ascending, the lowest tied positions taken at the threshold
-- so both outputs are compared with the oracle's slot for slot, bit-exact,
through every kernel shape that can do the selection.
"""
import numpy as np
import pytest

import sparse_attention_indexer_fp32_amd as topk
import workloads
from gpu_util import SENTINEL, note, upload
from oracle import topk_transform as oracle_topk

pytestmark = pytest.mark.gpu


def run_sorted(lib, w, raw=True, tensors=None):
    import torch
    s, sl, pt = tensors if tensors is not None else upload(w)
    out = torch.full((w.batch, w.k), SENTINEL, dtype=torch.int32, device=s.device)
    out_raw = torch.full((w.batch, w.k), SENTINEL, dtype=torch.int32, device=s.device) if raw else None
    lib.topk_transform_sorted(s, sl, pt, w.k, w.page_size, out=out, out_raw=out_raw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (out_raw.cpu().numpy() if raw else None)


def check_exact(w, out, raw, rows=None):
    exp_out, exp_raw, _ = oracle_topk(w.scores, w.seq_lens, w.page_table, w.k, w.page_size, rows=rows)
    got_out = out if rows is None else out[rows]
    bad = np.nonzero((got_out != exp_out).any(axis=1))[0]
    assert bad.size == 0, f"{w.name}: out differs from the oracle in {bad.size} rows (first {bad[:5].tolist()})"
    if raw is not None:
        got_raw = raw if rows is None else raw[rows]
        bad = np.nonzero((got_raw != exp_raw).any(axis=1))[0]
        assert bad.size == 0, f"{w.name}: raw differs from the oracle in {bad.size} rows (first {bad[:5].tolist()})"


@pytest.mark.parametrize("name", ["c1", "c2", "c3_b1", "c3_b4", "c3_b8", "c4b", "c5", "mixed"])
def test_sorted_configs(lib, name):
    note(f"sorted config {name}")
    w = workloads.make(name)
    lib.topk_set_dispatch_override(0, 0)
    t = upload(w)
    out, raw = run_sorted(lib, w, raw=True, tensors=t)
    note(f"sorted config {name}: {lib.topk_last_launch()}")
    check_exact(w, out, raw)
    out2, _ = run_sorted(lib, w, raw=False, tensors=t)
    assert np.array_equal(out2, out)


@pytest.mark.parametrize("finish", [0, 1])
@pytest.mark.parametrize("name", ["c1", "c2", "c3_b1", "c4b"])
def test_sorted_configs_forced_finish(lib, name, finish):
    """Both finishes on configs the automatic choice gives the other one (or
    the same one), against the oracle."""
    note(f"sorted config {name} finish={finish}")
    w = workloads.make(name)
    lib.topk_set_sorted_finish(finish)
    try:
        out, raw = run_sorted(lib, w, raw=True)
        note(f"sorted config {name}: {lib.topk_last_launch()}")
    finally:
        lib.topk_set_sorted_finish(-1)
    check_exact(w, out, raw)


@pytest.mark.parametrize("finish", [-1, 1])
def test_sorted_c4a_sampled(lib, finish):
    note(f"sorted config c4a finish={finish}")
    w = workloads.c4a()
    lib.topk_set_dispatch_override(0, 0)
    lib.topk_set_sorted_finish(finish)
    try:
        out, raw = run_sorted(lib, w, raw=True)
        note(f"sorted config c4a: {lib.topk_last_launch()}")
    finally:
        lib.topk_set_sorted_finish(-1)
    rng = np.random.Generator(np.random.PCG64(78))
    rows = sorted(rng.choice(w.batch, size=192, replace=False).tolist())
    check_exact(w, out, raw, rows=rows)


# every selection path: each streaming shape, split rows, register-resident rows,
# split streaming rows (there wgs is G and shape the split streaming shape)
SORTED_SHAPES = [("stream", 0, 1, 0), ("stream", 0, 1, 1), ("stream", 0, 1, 2), ("split", 4, 3, -1),
                 ("split", 16, 0, -1), ("resident", 16, 1, -1), ("resident", 64, 1, -1), ("sstream", 0, 3, 0),
                 ("sstream", 0, 2, 1)]


@pytest.mark.parametrize("finish", [0, 1])
@pytest.mark.parametrize("path,ept,wgs,shape", SORTED_SHAPES)
@pytest.mark.parametrize("kind", ["normal", "ties", "const", "asc", "desc", "neginf", "int", "zeros", "wide"])
def test_sorted_every_path(lib, path, ept, wgs, shape, kind, finish):
    """Adversarial kinds drive the streaming kernel through its gate raise,
    overflow and low-count fallbacks, and the finish through its memory tie
    select (constant rows have more tied members than its LDS list); "zeros"
    orders -0 before +0, "wide" mixes subnormals and infinities.  `finish`
    forces the one-workgroup-per-row finish (0) or the rank finish (1)."""
    W = {"stream": 50001, "sstream": 90001}.get(path, 3 * 4096 + 123)
    seq = [W, W - 1, W // 3, 2049, 5000, 0, 513, -2]
    for k in (1, 512, 700, 2048):   # 512: the largest k of the small finish shape
        w = workloads.custom(300 + ept + wgs + k, len(seq), W, k, 16, seq_lens=seq, kind=kind, table="perm")
        note(f"sorted path={path} ept={ept} wgs={wgs} shape={shape} kind={kind} k={k} finish={finish}")
        lib.topk_set_sorted_finish(finish)
        if path == "sstream":
            lib.topk_set_split_stream(shape, wgs)
        else:
            lib.topk_set_dispatch_override(ept, wgs)
            lib.topk_set_stream_shape(shape)
        try:
            out, raw = run_sorted(lib, w, raw=True)
        finally:
            lib.topk_set_dispatch_override(0, 0)
            lib.topk_set_stream_shape(-1)
            lib.topk_set_split_stream(-1, 0)
            lib.topk_set_sorted_finish(-1)
        check_exact(w, out, raw)


@pytest.mark.parametrize("finish", [0, 1])
@pytest.mark.parametrize("k", [512, 2048])
def test_sorted_crowded_bucket(lib, k, finish):
    """Short rows (every position selected, so the bin is not cut) holding
    hundreds of equal keys beside a few larger and smaller ones: the rank
    finish's span-fitted buckets put each key's pairs in one bucket, which is
    then split by the positions.  The last row is long: ties at its threshold
    cut the bin."""
    W = 3000
    seq = [k - 7, k // 2, 300, W]
    w = workloads.custom(41 + k, len(seq), W, k, 16, seq_lens=seq, kind="crowded", table="perm")
    note(f"sorted crowded k={k} finish={finish}")
    lib.topk_set_sorted_finish(finish)
    try:
        out, raw = run_sorted(lib, w, raw=True)
        note(f"sorted crowded: {lib.topk_last_launch()}")
    finally:
        lib.topk_set_sorted_finish(-1)
    check_exact(w, out, raw)


@pytest.mark.parametrize("k", [512, 1024])
def test_sorted_rank_crowded_splits(lib, k):
    """The rank finish on rows built so that tied keys crowd its buckets
    (every position of a short row is selected):
      * one far key and one tie group: the group's bucket is split by its
        positions;
      * one far key and two tie groups one ulp apart: both groups share a
        bucket and, split by that bucket's span, one sub-bucket each, so the
        row falls back to its first workgroup's sort;
      * three tie groups of spread keys, and a constant row;
      * a long row beside them (its threshold cut)."""
    W = 4096
    L = k - 24
    one = np.float32(1.0)
    up = np.nextafter(one, np.float32(2.0))
    rng = np.random.Generator(np.random.PCG64(4100 + k))
    rows = []
    r = np.full(W, one, np.float32); r[rng.integers(0, L)] = 100.0; rows.append(r)
    r = np.where(rng.random(W) < 0.5, one, up).astype(np.float32); r[rng.integers(0, L)] = 100.0; rows.append(r)
    r = rng.choice(np.array([-3.0, 0.25, 7.5], np.float32), W).astype(np.float32); rows.append(r)
    rows.append(np.full(W, np.float32(-2.0), np.float32))
    rows.append(rng.choice(np.array([1.0, 2.0, 3.0, 4.0], np.float32), W).astype(np.float32))
    scores = np.stack(rows)
    seq = np.array([L, L, L, L, W], np.int32)
    workloads.poison_scores(scores, seq)
    P = -(-W // 16)
    pt = workloads.identity_table(len(seq), P, seq, 16)
    w = workloads.Workload("sorted_rank_crowded", "tie groups crowding the rank finish's buckets", scores, seq, pt, k,
                           16, True, 4100 + k)
    note(f"sorted rank crowded splits k={k}")
    lib.topk_set_sorted_finish(1)
    try:
        out, raw = run_sorted(lib, w, raw=True)
        assert "rank" in lib.topk_last_launch(), lib.topk_last_launch()
    finally:
        lib.topk_set_sorted_finish(-1)
    check_exact(w, out, raw)


@pytest.mark.parametrize("name", ["c1", "c4b"])
def test_sorted_graph_replay(lib, name):
    """The sorted entry point (selection launch + rank finish) captured in a
    HIP graph: every replay, with eager calls between them, gives the
    oracle's output."""
    import torch
    w = workloads.make(name)
    s, sl, pt = upload(w)
    out = torch.empty((w.batch, w.k), dtype=torch.int32, device=s.device)
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        lib.topk_transform_sorted(s, sl, pt, w.k, w.page_size, out=out)   # buffers allocated outside capture
        stream.synchronize()
        note(f"sorted graph {name}: {lib.topk_last_launch()}")
        check_exact(w, out.cpu().numpy(), None)
        with torch.cuda.graph(g, stream=stream):
            lib.topk_transform_sorted(s, sl, pt, w.k, w.page_size, out=out)
    for rep in range(3):
        out.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        check_exact(w, out.cpu().numpy(), None)
        lib.topk_transform_sorted(s, sl, pt, w.k, w.page_size, out=out)   # an eager call between replays
        torch.cuda.synchronize()


def test_sorted_matches_unsorted_set(lib):
    """Same selected set as topk_transform wherever the threshold is not cut
    (distinct scores: the set is unique), in canonical order."""
    w = workloads.custom(17, 64, 20000, 512, 64, kind="normal")
    t = upload(w)
    import torch
    s, sl, pt = t
    o1, r1 = lib.topk_transform(s, sl, pt, w.k, w.page_size, want_raw=True)
    o2, r2 = lib.topk_transform_sorted(s, sl, pt, w.k, w.page_size, want_raw=True)
    torch.cuda.synchronize()
    r1, r2 = r1.cpu().numpy(), r2.cpu().numpy()
    for b in range(w.batch):
        assert np.array_equal(np.sort(r1[b]), np.sort(r2[b]))
    check_exact(w, o2.cpu().numpy(), r2)
