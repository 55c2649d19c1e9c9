"""GPU tests of the runtime around the kernels: per-(device, stream)
workspaces under concurrent streams, workspace growth and release, and the
deterministic entry point inside a replayed graph."""
import numpy as np
import pytest

import workloads
from gpu_util import check, note, upload
from oracle import topk_transform as oracle_topk

pytestmark = pytest.mark.gpu


def test_two_streams_interleaved(lib):
    """Split rows (workspace regions + barrier) and a queued streaming batch
    launched alternately on two streams with no synchronisation between
    them: each stream has its own workspace, so neither disturbs the other."""
    import torch
    w_split = workloads.custom(31, 4, 300000, 2048, 64, kind="normal")
    w_queue = workloads.custom(32, 1500, 6000, 256, 16, kind="ties")
    ts, tq = upload(w_split), upload(w_queue)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for stream, w, t in ((s1, w_split, ts), (s2, w_queue, tq)):   # allocate workspaces outside the race
        with torch.cuda.stream(stream):
            lib.topk_transform(t[0], t[1], t[2], w.k, w.page_size)
    torch.cuda.synchronize()
    for rep in range(6):
        for stream, w, t in ((s1, w_split, ts), (s2, w_queue, tq)):
            with torch.cuda.stream(stream):
                o, r = lib.topk_transform(t[0], t[1], t[2], w.k, w.page_size, want_raw=True)
                outs.append((w, o, r))
    torch.cuda.synchronize()
    note("two streams: checking")
    for w, o, r in outs:
        check(w, o.cpu().numpy(), r.cpu().numpy())


def test_workspace_growth_and_release(lib):
    """A split batch needing more slots than the workspace holds grows it;
    after topk_release_workspaces the next call allocates again."""
    small = workloads.custom(41, 1, 200000, 512, 64, kind="normal")
    large = workloads.custom(42, 6, 200000, 512, 64, kind="int")
    for w in (small, large, small):
        note(f"growth {w.name}")
        o, r = lib.topk_transform(*upload(w), w.k, w.page_size, want_raw=True)
        import torch
        torch.cuda.synchronize()
        check(w, o.cpu().numpy(), r.cpu().numpy())
    lib.topk_release_workspaces()
    for w in (large, small):
        o, r = lib.topk_transform_sorted(*upload(w), w.k, w.page_size, want_raw=True)
        torch.cuda.synchronize()
        exp_out, exp_raw, _ = oracle_topk(w.scores, w.seq_lens, w.page_table, w.k, w.page_size)
        assert np.array_equal(o.cpu().numpy(), exp_out) and np.array_equal(r.cpu().numpy(), exp_raw)


@pytest.mark.parametrize("name,batch,width,k", [("split", 2, 400000, 2048), ("queue", 1200, 9000, 512)])
def test_sorted_graph_replay(lib, name, batch, width, k):
    """The two launches of the sorted entry point captured in a graph: every
    replay gives the oracle's exact output."""
    import torch
    w = workloads.custom(50 + batch, batch, width, k, 64, kind="ties")
    s, sl, pt = upload(w)
    out = torch.empty((w.batch, w.k), dtype=torch.int32, device=s.device)
    raw = torch.empty((w.batch, w.k), dtype=torch.int32, device=s.device)
    exp_out, exp_raw, _ = oracle_topk(w.scores, w.seq_lens, w.page_table, w.k, w.page_size)
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        lib.topk_transform_sorted(s, sl, pt, w.k, w.page_size, out=out, out_raw=raw)   # buffers allocated here
        stream.synchronize()
        note(f"sorted graph {name}: {lib.topk_last_launch()}")
        with torch.cuda.graph(g, stream=stream):
            lib.topk_transform_sorted(s, sl, pt, w.k, w.page_size, out=out, out_raw=raw)
    for rep in range(3):
        out.fill_(-7)
        raw.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), exp_out), f"replay {rep}"
        assert np.array_equal(raw.cpu().numpy(), exp_raw), f"replay {rep}"


def test_wait_give_up_reported_once_and_not_sticky(lib):
    """A wait limit of one poll makes the split rows' barrier waits give up
    while every kernel still runs to its end (nothing on the device waits
    unbounded).  The faulted call's outputs are invalid, and the library says
    so: the next call on the stream returns TOPK_ERROR_DEVICE_FAULT once and
    queues nothing, or topk_check_faults raises it after a synchronisation.
    The faulted launch put the workspace back in its initial state, so calls
    at the normal limit are exact again, with no fault reported."""
    import torch
    w = workloads.custom(61, 2, 1 << 20, 2048, 64, kind="normal", table="perm")
    s, sl, pt = upload(w)
    out = torch.empty((w.batch, w.k), dtype=torch.int32, device=s.device)
    raw = torch.empty_like(out)
    lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out, out_raw=raw)
    torch.cuda.synchronize()
    note(f"give-up: {lib.topk_last_launch()}")
    assert lib.topk_last_launch().startswith("split-row")
    check(w, out.cpu().numpy(), raw.cpu().numpy())
    lib.topk_check_faults()
    try:
        lib.topk_set_wait_limit(1)
        note("give-up: one-poll waits, reported by topk_check_faults")
        lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out, out_raw=raw)
        with pytest.raises(lib.TopkError) as e:
            lib.topk_check_faults()
        assert e.value.status == lib.TOPK_ERROR_DEVICE_FAULT and "invalid" in str(e.value)
        lib.topk_check_faults()   # reported once
        note("give-up: one-poll waits, reported by the next call")
        lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out, out_raw=raw)
        torch.cuda.synchronize()
        out.fill_(-7)
        with pytest.raises(lib.TopkError) as e:
            lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out, out_raw=raw)
        assert e.value.status == lib.TOPK_ERROR_DEVICE_FAULT
        torch.cuda.synchronize()
        assert bool((out == -7).all()), "the call that reported the fault queued work"
    finally:
        lib.topk_set_wait_limit(0)
    for rep in range(3):
        note(f"give-up: normal limit again, rep {rep}")
        out.fill_(-7)
        raw.fill_(-7)
        lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out, out_raw=raw)
        torch.cuda.synchronize()
        check(w, out.cpu().numpy(), raw.cpu().numpy())
    lib.topk_check_faults()


def test_forced_workspace_allocation_failure(lib, monkeypatch):
    """TOPK_TEST_FAIL_ALLOC makes the next workspace allocation fail: the call
    returns TOPK_ERROR_OUT_OF_MEMORY with a message and queues nothing; once
    the variable is gone, the same call on the same stream runs exactly."""
    import torch
    w = workloads.custom(62, 3, 300000, 1024, 64, kind="normal")
    s, sl, pt = upload(w)
    stream = torch.cuda.Stream()   # a stream with no workspace yet
    out = torch.full((w.batch, w.k), -7, dtype=torch.int32, device=s.device)
    monkeypatch.setenv("TOPK_TEST_FAIL_ALLOC", "1")
    note("forced allocation failure")
    with pytest.raises(lib.TopkError) as e:
        lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out, stream=stream)
    assert e.value.status == 3 and "TOPK_TEST_FAIL_ALLOC" in str(e.value)
    stream.synchronize()
    assert bool((out == -7).all())
    monkeypatch.delenv("TOPK_TEST_FAIL_ALLOC")
    o, r = lib.topk_transform(s, sl, pt, w.k, w.page_size, want_raw=True, stream=stream)
    stream.synchronize()
    check(w, o.cpu().numpy(), r.cpu().numpy())
