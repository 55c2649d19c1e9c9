"""GPU parity: the HIP path (through the C-ABI binding) against the CPU oracle.

Integer results, so the bar is bit-exact: the set of strictly-greater positions
is unique and compared exactly; tied slots must hold distinct positions with
exactly the threshold key; the transform is compared slot by slot.
"""
import numpy as np
import pytest

import sparse_attention_indexer_fp32_amd as topk
import workloads
from gpu_util import check, check_properties_all_rows, note, run, upload

pytestmark = pytest.mark.gpu


# ---- the five benchmark workloads at full size ------------------------------

@pytest.mark.parametrize("name", ["c1", "c2", "c3_b1", "c3_b4", "c3_b8", "c4b", "c5", "mixed"])
def test_config_full(lib, name):
    note(f"config {name}")
    w = workloads.make(name)
    lib.topk_set_dispatch_override(0, 0)
    t = upload(w)
    out, raw = run(lib, w, raw=True, tensors=t)
    note(f"config {name}: {lib.topk_last_launch()}")
    check(w, out, raw)
    out2, _ = run(lib, w, raw=False, tensors=t)
    check(w, out2, None)


def test_config_c4a_sampled(lib):
    """batch 2048 x 65536: every row checked by properties, 256 sampled rows by the oracle."""
    note("config c4a")
    w = workloads.c4a()
    lib.topk_set_dispatch_override(0, 0)
    out, raw = run(lib, w, raw=True)
    note(f"config c4a: {lib.topk_last_launch()}")
    check_properties_all_rows(w, out, raw)
    rng = np.random.Generator(np.random.PCG64(77))
    rows = sorted(rng.choice(w.batch, size=256, replace=False).tolist())
    check(w, out, raw, rows=rows)


# ---- every kernel shape, forced, on shapes spanning several tiles + a ragged tail

SHAPES = [
    # (elems_per_thread, wgs_per_row): (0, 1) is the streaming one-workgroup-per-row kernel,
    # (E, 1) the register-resident one, G > 1 the split-row kernel.
    (0, 1), (4, 0), (4, 3), (8, 0), (8, 2), (16, 0), (16, 5), (32, 0), (32, 2), (64, 0), (64, 2), (64, 1),
]


@pytest.mark.parametrize("ept,wgs", SHAPES)
@pytest.mark.parametrize("kind", ["normal", "ties", "int"])
def test_forced_shapes(lib, ept, wgs, kind):
    W = 3 * 4096 + 123          # not a multiple of 4: scalar-load path, ragged tail
    seq = [0, 1, 511, 512, 513, W, W - 1, 2 * 4096 + 7, -3, W + 50]
    for k in (1, 512, 2048):
        w = workloads.custom(100 + ept + wgs, len(seq), W, k, 16, seq_lens=seq, kind=kind)
        note(f"forced ept={ept} wgs={wgs} kind={kind} k={k} W={W}")
        lib.topk_set_dispatch_override(ept, wgs)
        try:
            out, raw = run(lib, w, raw=True)
        finally:
            lib.topk_set_dispatch_override(0, 0)
        check(w, out, raw)


@pytest.mark.parametrize("ept,wgs", [(0, 1), (4, 0), (16, 3), (64, 1), (32, 2)])
def test_forced_shapes_aligned(lib, ept, wgs):
    W = 40960                    # multiple of 4: dwordx4 path, partial last workgroup
    seq = [W, W - 3, 4096, 4097, 0, 2047, 2048, 2049, 30000]
    w = workloads.custom(7, len(seq), W, 2048, 64, seq_lens=seq, kind="normal", table="perm")
    note(f"forced aligned ept={ept} wgs={wgs}")
    lib.topk_set_dispatch_override(ept, wgs)
    try:
        out, raw = run(lib, w, raw=True)
    finally:
        lib.topk_set_dispatch_override(0, 0)
    check(w, out, raw)


# ---- edge cases -------------------------------------------------------------

@pytest.mark.parametrize("kind", ["const", "neginf", "zeros", "asc", "desc", "wide", "ties", "int"])
@pytest.mark.parametrize("W", [5000, 70000])
def test_adversarial_rows(lib, kind, W):
    seq = [W, W // 2, 3, 1025, W - 1]
    w = workloads.custom(11, len(seq), W, 1024, 16, seq_lens=seq, kind=kind)
    note(f"adversarial kind={kind} W={W}")
    lib.topk_set_dispatch_override(0, 0)
    out, raw = run(lib, w, raw=True)
    check(w, out, raw)


@pytest.mark.parametrize("kind", ["const", "neginf", "zeros", "asc", "desc", "wide", "ties", "int", "normal"])
@pytest.mark.parametrize("W", [9000, 50000, 140001])
def test_stream_kernel_adversarial(lib, kind, W):
    """The streaming kernel, including its candidate-overflow re-stream path
    (constant, -inf-only and ascending rows overflow the LDS candidate list)."""
    seq = [W, W - 1, W // 3, 2049, 17000, 0]
    for k in (1, 512, 2048):
        w = workloads.custom(21 + k, len(seq), W, k, 16, seq_lens=seq, kind=kind)
        note(f"stream kind={kind} W={W} k={k}")
        lib.topk_set_dispatch_override(0, 1)
        try:
            out, raw = run(lib, w, raw=True)
        finally:
            lib.topk_set_dispatch_override(0, 0)
        check(w, out, raw)


@pytest.mark.parametrize("k", [1, 7, 512, 1024, 2047, 2048])
@pytest.mark.parametrize("ps", [1, 16, 64, 256])
def test_k_and_page_size(lib, k, ps):
    W = 20000
    seq = [0, 1, k - 1, k, k + 1, W]
    seq = [max(s, 0) for s in seq]
    w = workloads.custom(5 + k + ps, len(seq), W, k, ps, seq_lens=seq, kind="normal", table="perm")
    note(f"k={k} ps={ps}")
    out, raw = run(lib, w, raw=True)
    check(w, out, raw)
    out2, _ = run(lib, w, raw=False)
    assert np.array_equal(out2 == -1, out == -1)
    check(w, out2, None)


def test_batch_zero_and_width_zero(lib):
    import torch
    dev = torch.device("cuda", 0)
    s = torch.zeros((0, 16), dtype=torch.float32, device=dev)
    out, _ = lib.topk_transform(s, torch.zeros(0, dtype=torch.int32, device=dev),
                                torch.zeros((0, 1), dtype=torch.int32, device=dev), 8, 4)
    assert out.shape == (0, 8)
    s = torch.zeros((3, 0), dtype=torch.float32, device=dev)
    out, raw = lib.topk_transform(s, torch.tensor([0, 5, -1], dtype=torch.int32, device=dev),
                                  torch.zeros((3, 1), dtype=torch.int32, device=dev), 8, 4, want_raw=True)
    torch.cuda.synchronize()
    assert (out.cpu() == -1).all() and (raw.cpu() == -1).all()


@pytest.mark.parametrize("ept,wgs", [(0, 1), (32, 0), (8, 0)])   # streaming, resident, split
def test_empty_page_table(lib, ept, wgs):
    """pages_per_row = 0 (the ABI then allows a null page table): every
    transformed slot is -1, while the raw positions are the usual exact set."""
    import ctypes
    import torch
    W = 20000
    seq = [W, 5000, 100, 0]
    w = workloads.custom(808, len(seq), W, 512, 64, seq_lens=seq, kind="normal")
    s, sl, _ = upload(w)
    out = torch.full((w.batch, w.k), -7, dtype=torch.int32, device=s.device)
    raw = torch.full((w.batch, w.k), -7, dtype=torch.int32, device=s.device)
    lib.topk_set_dispatch_override(ept, wgs)
    try:
        st = lib.load().topk_transform(ctypes.c_void_p(s.data_ptr()), ctypes.c_void_p(sl.data_ptr()), None,
                                       w.k, w.page_size, ctypes.c_void_p(out.data_ptr()),
                                       ctypes.c_void_p(raw.data_ptr()),
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), w.batch, W, 0)
        assert st == 0, lib.topk_last_error()
        torch.cuda.synchronize()
    finally:
        lib.topk_set_dispatch_override(0, 0)
    assert (out.cpu().numpy() == -1).all()
    # the raw positions against the oracle, with a table that maps every page to itself
    got_raw = raw.cpu().numpy()
    ident = np.broadcast_to(np.arange(-(-W // w.page_size), dtype=np.int32), (w.batch, -(-W // w.page_size))).copy()
    check(workloads.Workload(w.name, w.description, w.scores, w.seq_lens, ident, w.k, w.page_size, True, w.seed),
          got_raw, got_raw)


def test_repeated_split_rows_stress(lib):
    """The cross-workgroup path, many times with fresh seeds (race check)."""
    for rep in range(40):
        B = 1 + rep % 6
        W = 65536 + 4 * rep
        seq = [W - rep * 37 % 5000 for _ in range(B)]
        kind = ("normal", "ties", "int")[rep % 3]
        w = workloads.custom(1000 + rep, B, W, 512 + rep * 37, 64, seq_lens=seq, kind=kind)
        note(f"stress rep={rep} B={B} kind={kind}")
        out, raw = run(lib, w, raw=rep % 2 == 0)
        check(w, out, raw)
    lib.topk_check_faults()   # raises if a split-row wait gave up


@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_split_rows_cycled_over_slots(lib, kind):
    """More long rows than the split kernel holds resident at once, at a batch
    below half a row per CU: the dispatcher cycles split rows over the resident
    slots (each slot alternates its two workspace regions) rather than
    streaming one row per workgroup.  Long, short, empty and exactly-k rows mix
    within a slot's sequence."""
    import re
    W = 1 << 20
    seq = [W, 16384, W - 3, 0, 5000, W, 2048, 700000, 2049, W - 64] + [W - 17 * i for i in range(14)]
    w = workloads.custom(808 + len(kind), len(seq), W, 2048, 64, seq_lens=seq, kind=kind, table="perm")
    note(f"cycled split rows kind={kind} B={len(seq)} W={W}")
    out, raw = run(lib, w, raw=True)
    launch = lib.topk_last_launch()
    m = re.search(r"slots=(\d+)", launch)
    assert launch.startswith("split-row") and m and int(m.group(1)) < w.batch, launch
    check(w, out, raw)
    lib.topk_check_faults()   # raises if a split-row wait gave up


def test_split_rows_cycled_repeated_and_graph(lib):
    """Split rows cycled over the slots, several rows per slot: long, short and
    trivial (L <= k) rows in any order, so each slot's two workspace regions
    alternate over a mixed sequence; repeated calls with two length patterns,
    and replays of a captured graph with eager calls between them (every
    region and barrier must be back to its initial state after each call)."""
    import re
    import torch
    W = 600000
    rng = np.random.Generator(np.random.PCG64(4242))
    choices = [W, W // 3, 70000, 20000, 3000, 1500, 0]
    seqs = [rng.choice(choices, size=80).tolist() for _ in range(2)]
    ws = [workloads.custom(700 + i, 80, W, 2048, 64, seq_lens=sq, kind="normal", table="perm") for i, sq in
          enumerate(seqs)]
    tens = [upload(w) for w in ws]
    lib.topk_set_dispatch_override(64, 0)
    try:
        outs = []
        for rep in range(3):
            for w, t in zip(ws, tens):
                note(f"cycled split rows rep={rep} seed={w.seed}")
                out, raw = run(lib, w, raw=True, tensors=t)
                launch = lib.topk_last_launch()
                m = re.search(r"slots=(\d+)", launch)
                assert launch.startswith("split-row ept=64") and int(m.group(1)) < w.batch, launch
                check(w, out, raw)
        w, (s, sl, pt) = ws[0], tens[0]
        out = torch.empty((w.batch, w.k), dtype=torch.int32, device=s.device)
        g = torch.cuda.CUDAGraph()
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out)   # the side stream's workspace
            stream.synchronize()
            with torch.cuda.graph(g, stream=stream):
                lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out)
        for rep in range(4):
            note(f"cycled split rows graph replay {rep}")
            out.fill_(-7)
            g.replay()
            torch.cuda.synchronize()
            check(w, out.cpu().numpy(), None)
            w2 = ws[1]
            out2, raw2 = run(lib, w2, raw=True, tensors=tens[1])   # eager queued call between replays
            check(w2, out2, raw2)
    finally:
        lib.topk_set_dispatch_override(0, 0)
    lib.topk_check_faults()   # raises if a split-row wait gave up


@pytest.mark.parametrize("W", [1 << 20, 3 << 19])
def test_split_rows_cycled_device_choice(lib, W):
    """A batch of more long rows than fit resident is cycled over split slots
    in one of two shapes, and the device picks it from the lengths: E = 16
    (four times the workgroups per row) when at most two rounds of its slots'
    worth of rows exceed one E = 16 workgroup, else E = 64.  Both sides,
    eagerly and inside one captured graph whose replays see the lengths
    change (so the choice flips between replays).  At width 1.5M the two
    shapes' grids differ (96 x 2 against 24 x 10 workgroups on 256 CUs), so
    the launch's spare workgroups take the exit path."""
    import dataclasses
    import re
    import torch
    B = 32
    probe = workloads.custom(950, B, W, 2048, 64, seq_lens=[W] * 4 + [16384] * (B - 4), kind="normal", table="perm")
    tens = upload(probe)
    run(lib, probe, raw=False, tensors=tens)
    launch = lib.topk_last_launch()
    note(f"device choice: {launch}")
    m = re.search(r"\| ept=16 wgs_per_row=(\d+) slots=(\d+) when at most (\d+) rows exceed 16384", launch)
    assert launch.startswith("split-row ept=64") and m, launch
    fit = int(m.group(3))   # the most long rows the E = 16 shape takes
    seq_few = [W - 5 * i for i in range(fit)] + [16384, 3000, 0, 2048] * 8
    seq_few = seq_few[:B]
    seq_many = [W - 5 * i for i in range(fit + 1)] + [16384, 3000, 0, 2048] * 8
    seq_many = seq_many[:B]
    variants = {"few": np.array(seq_few, np.int32), "many": np.array(seq_many, np.int32)}
    # scores and table valid up to either pattern's length (both are poisoned past the lengths given)
    seq_max = np.maximum(variants["few"], variants["many"]).tolist()
    w = workloads.custom(951, B, W, 2048, 64, seq_lens=seq_max, kind="normal", table="perm")
    s, sl, pt = upload(w)
    for name, seq in variants.items():
        note(f"device choice eager: {name} long rows")
        sl.copy_(torch.from_numpy(seq))
        out, raw = run(lib, w, raw=True, tensors=(s, sl, pt))
        check(dataclasses.replace(w, seq_lens=seq), out, raw)
    out = torch.empty((B, w.k), dtype=torch.int32, device=s.device)
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out)   # the side stream's workspace
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out)
    for rep, name in enumerate(["few", "many", "few", "many"]):
        note(f"device choice graph replay {rep}: {name} long rows")
        sl.copy_(torch.from_numpy(variants[name]))
        out.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(dataclasses.replace(w, seq_lens=variants[name]), out.cpu().numpy(), None)
    lib.topk_check_faults()   # raises if a split-row wait gave up


def test_graph_replay(lib):
    """Calls captured in a HIP graph and replayed give the eager result every time."""
    import torch
    w = workloads.custom(3, 4, 131072, 2048, 64, kind="normal")
    s, sl, pt = upload(w)
    out = torch.empty((w.batch, w.k), dtype=torch.int32, device=s.device)
    lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out)   # warm-up: workspace allocated outside capture
    torch.cuda.synchronize()
    eager = out.cpu().numpy().copy()
    check(w, eager, None)
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out)  # warm the side stream's workspace
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out)
    for rep in range(5):
        out.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        check(w, got, None)
        s.add_(0.0)  # eager work between replays
        torch.cuda.synchronize()


def test_no_fault_reported(lib):
    lib.topk_check_faults()


# ---- streaming kernel: every compiled shape, and the row queue (batch > grid)

STREAM_SHAPES = topk.STREAM_SHAPES

@pytest.mark.parametrize("shape", range(STREAM_SHAPES))
def test_stream_shapes_row_queue(lib, shape):
    """More rows than workgroups: rows past the first grid come from the
    ticket queue.  Ragged lengths (many rows shorter than k) and an unaligned
    width; the call is repeated to check the queue resets itself."""
    W = 6001
    rng = np.random.Generator(np.random.PCG64(900 + shape))
    B = 2600
    seq = rng.integers(-5, W + 20, size=B)
    short = rng.random(B) < 0.25
    seq[short] = rng.integers(0, 600, size=int(short.sum()))
    w = workloads.custom(40 + shape, B, W, 512, 16, seq_lens=seq.tolist(), kind="normal")
    note(f"stream shape={shape} queue B={B} W={W}")
    lib.topk_set_stream_shape(shape)
    lib.topk_set_dispatch_override(0, 1)
    try:
        t = upload(w)
        out, raw = run(lib, w, raw=True, tensors=t)
        note(f"stream shape={shape}: {lib.topk_last_launch()}")
        check(w, out, raw)
        for _ in range(2):   # slot order may differ between calls; the selection may not
            out2, raw2 = run(lib, w, raw=True, tensors=t)
            check(w, out2, raw2)
    finally:
        lib.topk_set_stream_shape(-1)
        lib.topk_set_dispatch_override(0, 0)


@pytest.mark.parametrize("shape", range(STREAM_SHAPES))
@pytest.mark.parametrize("kind", ["ties", "const", "asc"])
def test_stream_shapes_adversarial(lib, shape, kind):
    """Every shape through its gate-raising and overflow paths."""
    W = 70001
    seq = [W, W - 1, W // 3, 2049, 17000, 0, 513]
    for k in (1, 2048):
        w = workloads.custom(60 + shape + k, len(seq), W, k, 64, seq_lens=seq, kind=kind)
        note(f"stream shape={shape} kind={kind} k={k}")
        lib.topk_set_stream_shape(shape)
        lib.topk_set_dispatch_override(0, 1)
        try:
            out, raw = run(lib, w, raw=True)
        finally:
            lib.topk_set_stream_shape(-1)
            lib.topk_set_dispatch_override(0, 0)
        check(w, out, raw)


def test_graph_replay_row_queue(lib):
    """The row queue inside a replayed HIP graph: it must reset itself on every replay."""
    import torch
    w = workloads.custom(8, 3000, 8192, 256, 16, kind="normal")
    s, sl, pt = upload(w)
    out = torch.empty((w.batch, w.k), dtype=torch.int32, device=s.device)
    lib.topk_set_dispatch_override(0, 1)
    try:
        g = torch.cuda.CUDAGraph()
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out)   # workspace allocated outside capture
            stream.synchronize()
            note(f"graph queue: {lib.topk_last_launch()}")
            eager = out.cpu().numpy().copy()
            check(w, eager, None)
            with torch.cuda.graph(g, stream=stream):
                lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out)
        for rep in range(4):
            out.fill_(-7)
            g.replay()
            torch.cuda.synchronize()
            check(w, out.cpu().numpy(), None)
            lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out)   # eager call between replays
            torch.cuda.synchronize()
    finally:
        lib.topk_set_dispatch_override(0, 0)


@pytest.mark.parametrize("shape", range(STREAM_SHAPES))
def test_stream_rows_within_sample_repeated(lib, shape):
    """Rows no longer than the streaming kernel's sample have no streamed
    chunks; every one of repeated calls must be exact (regression: the list
    count was once read before every wave's appends were in, which only a
    row without chunks exposed, and only on some calls)."""
    for W in (16384, 8192, 3001):   # the sample span of shapes 0 and 2, shape 1's, shorter
        seq = [W, W - 1, 2000, 600]
        w = workloads.custom(70 + shape, len(seq), W, 512, 64, seq_lens=seq, kind="normal")
        note(f"stream shape={shape} within-sample W={W}")
        lib.topk_set_stream_shape(shape)
        lib.topk_set_dispatch_override(0, 1)
        try:
            t = upload(w)
            for rep in range(20):
                out, raw = run(lib, w, raw=rep % 2 == 0, tensors=t)
                check(w, out, raw)
        finally:
            lib.topk_set_stream_shape(-1)
            lib.topk_set_dispatch_override(0, 0)


# ---- split streaming rows: G workgroups per row, the last one out finishes it

SS_FORCED = [(0, 1), (0, 2), (0, 4), (1, 2), (1, 3), (0, 0), (1, 0)]   # G 0: the length-aware form


@pytest.mark.parametrize("shape,G", SS_FORCED)
@pytest.mark.parametrize("kind", ["normal", "ties", "int", "const", "asc", "desc", "neginf", "zeros"])
def test_split_stream_forced(lib, shape, G, kind):
    """Every split streaming shape at several G, on an unaligned width (scalar
    loads, ragged segments) with short, empty, exactly-k and full rows.  The
    adversarial kinds drive it through the per-segment gate raise, lists that
    lose keys, and the finisher's low-count and overflow fallbacks (the row
    finished from memory)."""
    W = 90001
    seq = [W, W - 1, W // 3, 2049, 17000, 0, 513, 2048, -4, W + 9]
    for k in (1, 700, 2048):
        w = workloads.custom(500 + 10 * shape + G + k, len(seq), W, k, 16, seq_lens=seq, kind=kind, table="perm")
        note(f"split stream shape={shape} G={G} kind={kind} k={k}")
        lib.topk_set_split_stream(shape, G)
        try:
            out, raw = run(lib, w, raw=True)
            assert lib.topk_last_launch().startswith("split-row-stream"), lib.topk_last_launch()
        finally:
            lib.topk_set_split_stream(-1, 0)
        check(w, out, raw)


@pytest.mark.parametrize("shape,G", [(0, 4), (1, 2)])
def test_split_stream_aligned_repeated(lib, shape, G):
    """dwordx4 loads (aligned width), a permuted table, no raw output, and
    repeated calls with different lengths: each call leaves the rows' areas
    zeroed for the next."""
    W = 131072
    rng = np.random.Generator(np.random.PCG64(510 + shape))
    for rep in range(4):
        seq = rng.integers(1000, W + 1, size=24).tolist()
        w = workloads.custom(520 + rep, len(seq), W, 1024, 64, seq_lens=seq, kind="normal" if rep % 2 else "ties",
                             table="perm")
        note(f"split stream aligned shape={shape} G={G} rep={rep}")
        lib.topk_set_split_stream(shape, G)
        try:
            out, raw = run(lib, w, raw=rep % 2 == 0)
        finally:
            lib.topk_set_split_stream(-1, 0)
        check(w, out, raw)


def test_split_stream_graph_replay(lib):
    """Split streaming rows in a replayed graph, with eager calls between the
    replays: the row areas reset themselves on every launch."""
    import torch
    w = workloads.custom(530, 16, 200000, 2048, 64, kind="normal", table="perm")
    s, sl, pt = upload(w)
    out = torch.empty((w.batch, w.k), dtype=torch.int32, device=s.device)
    lib.topk_set_split_stream(0, 4)
    try:
        g = torch.cuda.CUDAGraph()
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out)   # workspace allocated outside capture
            stream.synchronize()
            note(f"split stream graph: {lib.topk_last_launch()}")
            check(w, out.cpu().numpy(), None)
            with torch.cuda.graph(g, stream=stream):
                lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out)
        for rep in range(4):
            out.fill_(-7)
            g.replay()
            torch.cuda.synchronize()
            check(w, out.cpu().numpy(), None)
            o2, r2 = lib.topk_transform(s, sl, pt, w.k, w.page_size, want_raw=True)
            torch.cuda.synchronize()
            check(w, o2.cpu().numpy(), r2.cpu().numpy())
    finally:
        lib.topk_set_split_stream(-1, 0)


def test_split_stream_rejects_beyond_residency(lib):
    """A forced G whose grid would not be resident at once is refused (the
    finisher scheme needs no co-residency, but the grid is sized to it)."""
    import torch
    w = workloads.custom(540, 200, 8192, 64, 64, kind="normal")
    s, sl, pt = upload(w)
    lib.topk_set_split_stream(1, 64)
    try:
        with pytest.raises(topk.TopkError) as e:
            lib.topk_transform(s, sl, pt, w.k, w.page_size)
        assert e.value.status == 2
    finally:
        lib.topk_set_split_stream(-1, 0)
    torch.cuda.synchronize()


@pytest.mark.parametrize("shape", [0, 1])
def test_split_stream_length_aware_ragged(lib, shape):
    """The length-aware form on a ragged mid batch whose width is far above
    most lengths: every row gets 1 to 4 workgroups by its length (worked out
    on the device), trivial rows one; repeated calls with other lengths."""
    W = 600000
    rng = np.random.Generator(np.random.PCG64(550 + shape))
    for rep in range(3):
        seq = rng.integers(1000, W + 1, size=100).tolist()
        seq[::17] = [0, 2048, 100, 2049, W, 1][: len(seq[::17])]
        w = workloads.custom(560 + rep, len(seq), W, 512 if rep else 2048, 64, seq_lens=seq, kind="normal",
                             table="perm")
        note(f"split stream length-aware shape={shape} rep={rep}")
        lib.topk_set_split_stream(shape, 0)
        try:
            out, raw = run(lib, w, raw=rep != 1)
            assert "length-aware" in lib.topk_last_launch(), lib.topk_last_launch()
        finally:
            lib.topk_set_split_stream(-1, 0)
        check(w, out, raw)


@pytest.mark.parametrize("B,W,k,lo,expect", [
    (40, 300000, 1024, 2000, "split-row-stream length-aware"),   # mid batch, wide rows: per-row parts
    (48, 100000, 2048, 0, "split-row-stream ept=0 wgs_per_row=4"),   # mid batch, rows up to 256K: G = 4
    (128, 131072, 512, 1000, "split-row-stream ept=0 wgs_per_row=2"),   # one row per two CUs: G = 2
])
def test_split_stream_automatic_choices(lib, B, W, k, lo, expect):
    """The dispatcher's split streaming choices, exact on ragged rows (some
    shorter than k, some empty)."""
    rng = np.random.Generator(np.random.PCG64(B + k))
    seq = rng.integers(lo, W + 1, size=B).tolist() if lo else [W] * B
    if lo:
        for i, v in zip(range(0, B, 9), (0, k, k - 1, 17)):
            seq[i] = v
    w = workloads.custom(570 + B, B, W, k, 64, seq_lens=seq, kind="normal", table="perm")
    note(f"automatic split streaming B={B} W={W} k={k}")
    out, raw = run(lib, w, raw=True)
    assert lib.topk_last_launch().startswith(expect), lib.topk_last_launch()
    check(w, out, raw)
