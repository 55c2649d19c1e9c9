"""Helpers shared by the GPU parity tests: upload a seeded workload, run the HIP
path through the binding, and check it against the oracle."""
from __future__ import annotations

import sys
from typing import List, Optional

import numpy as np

import workloads
from oracle import check_batch, order_key, row_length

SENTINEL = 0x7F7F7F7F


def note(msg: str) -> None:
    """Names the case about to run on the GPU (flushed, so it survives a crash)."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def upload(w: workloads.Workload):
    import torch
    dev = torch.device("cuda", 0)
    s = torch.from_numpy(w.scores).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    pt = torch.from_numpy(w.page_table).to(dev)
    return s, sl, pt


def run(topk, w: workloads.Workload, raw: bool = True, tensors=None):
    import torch
    s, sl, pt = tensors if tensors is not None else upload(w)
    out = torch.full((w.batch, w.k), SENTINEL, dtype=torch.int32, device=s.device)
    out_raw = torch.full((w.batch, w.k), SENTINEL, dtype=torch.int32, device=s.device) if raw else None
    topk.topk_transform(s, sl, pt, w.k, w.page_size, out=out, out_raw=out_raw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (out_raw.cpu().numpy() if raw else None)


def check(w: workloads.Workload, out: np.ndarray, raw: Optional[np.ndarray],
          rows: Optional[List[int]] = None) -> None:
    errs = check_batch(w.scores, w.seq_lens, w.page_table, w.k, w.page_size, out, raw, rows=rows)
    assert not errs, f"{w.name}: " + "; ".join(errs[:5])


def check_properties_all_rows(w: workloads.Workload, out: np.ndarray, raw: Optional[np.ndarray]) -> None:
    """Size-independent properties on every row (used where the oracle checks a sample):
    -1 tail, no sentinel left, distinct in-range positions, and out == transform(raw)."""
    B, k = out.shape
    assert not np.any(out == SENTINEL), "unwritten out slots"
    for b in range(B):
        L = row_length(int(w.seq_lens[b]), w.width)
        n = min(k, L)
        assert np.all(out[b, n:] == -1)
        if raw is not None:
            r = raw[b, :n].astype(np.int64)
            assert np.all(raw[b, n:] == -1)
            assert np.all((r >= 0) & (r < L)) and np.unique(r).size == n
            phys = w.page_table[b].astype(np.int64)[r // w.page_size] * w.page_size + r % w.page_size
            assert np.array_equal(phys, out[b, :n].astype(np.int64))
            # every selected key >= every unselected key in the row
            keys = order_key(w.scores[b, :L])
            sel = np.zeros(L, dtype=bool)
            sel[r] = True
            if n < L:
                assert keys[sel].min() >= keys[~sel].max()
