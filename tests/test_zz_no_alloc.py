"""GPU test of topk_transform_noalloc, the entry point that allocates nothing
(its workspace is the library's static device scratch), called through the C
ABI and checked against topk_transform on the same inputs.

Inputs are N(0,1) scores, so every row's top-k set is unique: both entry points
must return the same set per row (compared exactly), and both must pass the
oracle's checker (valid slots, -1 tails, out == transform(raw)).  Two calls in
a row, the second on a smaller input, for each workspace user: split rows
(barrier blocks and regions) and a streamed batch larger than the grid (the
row queue in the header)."""
import ctypes

import numpy as np
import pytest

import workloads
from gpu_util import SENTINEL, check, note, upload

pytestmark = pytest.mark.gpu


def _noalloc(lib, w, tensors, raw: bool):
    """topk_transform_noalloc through the C ABI (ctypes, device pointers)."""
    import torch
    s, sl, pt = tensors
    out = torch.full((w.batch, w.k), SENTINEL, dtype=torch.int32, device=s.device)
    out_raw = torch.full((w.batch, w.k), SENTINEL, dtype=torch.int32, device=s.device) if raw else None
    stream = torch.cuda.current_stream()
    st = lib.load().topk_transform_noalloc(s.data_ptr(), sl.data_ptr(), pt.data_ptr(), w.k, w.page_size,
                                           out.data_ptr(), out_raw.data_ptr() if raw else None,
                                           ctypes.c_void_p(stream.cuda_stream), w.batch, w.width, pt.shape[1])
    assert st == 0, lib.topk_last_error()
    torch.cuda.synchronize()
    return out.cpu().numpy(), (out_raw.cpu().numpy() if raw else None)


def _reference(lib, w, tensors):
    import torch
    s, sl, pt = tensors
    out = torch.full((w.batch, w.k), SENTINEL, dtype=torch.int32, device=s.device)
    out_raw = torch.full((w.batch, w.k), SENTINEL, dtype=torch.int32, device=s.device)
    lib.topk_transform(s, sl, pt, w.k, w.page_size, out=out, out_raw=out_raw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), out_raw.cpu().numpy()


def _same_sets(a: np.ndarray, b: np.ndarray) -> None:
    assert np.array_equal(np.sort(a, axis=1), np.sort(b, axis=1))


CASES = {
    # two calls each, the second smaller
    "split": [(71, 6, 500000, 2048, [500000, 499999, 3000, 0, 2048, 400001]), (72, 2, 200000, 512, None)],
    "queue": [(73, 3000, 8192, 512, None), (74, 2600, 4100, 256, None)],
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_noalloc_matches_topk_transform(lib, case):
    for i, (seed, B, W, k, seq) in enumerate(CASES[case]):
        w = workloads.custom(seed, B, W, k, 64, seq_lens=seq, kind="normal", table="perm")
        t = upload(w)
        note(f"noalloc {case} call {i}: B={B} W={W} k={k}")
        out, raw = _noalloc(lib, w, t, raw=True)
        launch = lib.topk_last_launch()
        note(f"noalloc {case} call {i}: {launch}")
        if case == "split":
            assert launch.startswith("split-row"), launch
        else:
            assert launch.startswith("row-per-wg-stream") and int(launch.split("slots=")[1].split()[0]) < B, launch
        check(w, out, raw)
        ref_out, ref_raw = _reference(lib, w, t)
        _same_sets(raw, ref_raw)
        _same_sets(out, ref_out)
        out2, _ = _noalloc(lib, w, t, raw=False)   # no raw output: the same transformed set
        _same_sets(out2, ref_out)
    lib.topk_check_faults()


def test_noalloc_rejects_beyond_scratch(lib):
    """A plan needing more workspace than the scratch holds is refused with
    TOPK_ERROR_UNSUPPORTED and a message, and nothing is queued.  No plan
    needs more than the real scratch (split grids are capped at the resident
    workgroups, at most 128 slots of 2 workgroups), so the scratch the entry
    point may use is lowered to 1M words (4 MiB) for the call: 200 rows forced
    onto 2 split workgroups each need far more."""
    import torch
    w = workloads.custom(75, 200, 8192, 64, 64, kind="normal")
    s, sl, pt = upload(w)
    out = torch.full((w.batch, w.k), -7, dtype=torch.int32, device=s.device)
    lib.topk_set_dispatch_override(4, 2)
    lib.topk_set_scratch_limit(1 << 20)
    try:
        st = lib.load().topk_transform_noalloc(s.data_ptr(), sl.data_ptr(), pt.data_ptr(), w.k, w.page_size,
                                               out.data_ptr(), None,
                                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream),
                                               w.batch, w.width, pt.shape[1])
    finally:
        lib.topk_set_scratch_limit(0)
        lib.topk_set_dispatch_override(0, 0)
    assert st == 2 and "scratch" in lib.topk_last_error(), (st, lib.topk_last_error())
    torch.cuda.synchronize()
    assert bool((out == -7).all())


def test_noalloc_wait_give_up_reported(lib):
    """One-poll waits on the static scratch: the give-up is reported once by
    topk_check_faults, the launch leaves the scratch in its initial state, and
    the next calls are exact again."""
    w = workloads.custom(76, 2, 1 << 20, 2048, 64, kind="normal", table="perm")
    t = upload(w)
    out, raw = _noalloc(lib, w, t, raw=True)
    check(w, out, raw)
    lib.topk_check_faults()
    try:
        lib.topk_set_wait_limit(1)
        note("noalloc give-up: one-poll waits")
        _noalloc(lib, w, t, raw=True)
        with pytest.raises(lib.TopkError) as e:
            lib.topk_check_faults()
        assert e.value.status == lib.TOPK_ERROR_DEVICE_FAULT
        lib.topk_check_faults()
    finally:
        lib.topk_set_wait_limit(0)
    for rep in range(2):
        note(f"noalloc give-up: normal limit again, rep {rep}")
        out, raw = _noalloc(lib, w, t, raw=True)
        check(w, out, raw)
    lib.topk_check_faults()
