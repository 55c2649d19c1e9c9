"""Seeded synthetic inputs for the fused indexer scoring + top-k.

Only *makes inputs*: none of the scoring or selection arithmetic lives here.
Shapes follow LiteTopk PR #32094 ("Add LiteTopk fused indexer top-k prefill
path for SM100"): the GLM indexer shape (H = 32 heads, D = 128), fp8 queries and
keys, prefill batches of requests given as (query rows, key length), the
Validation section's test shapes and the Performance section's Q = 8192,
top-2048 at 256K+ contexts.  The page measures GLM-5.2 tensors, which are not
available; these stand-ins use normal draws quantised to fp8.

A request with Q query rows and key length L occupies L consecutive positions
of the gathered key buffer starting at its offset; its query row i (the i-th of
the last Q tokens) may see positions [offset, offset + L - Q + i + 1) -- the
causal range the page's per-request calibration refers to.

Arrays (host, numpy):
    q         (num_q, 32, 128) uint8  fp8 E4M3 codes
    weights   (num_q, 32)      float32 head weights (mixed signs)
    kv        (N, 128)         uint8  fp8 E4M3 codes
    kv_scale  (N,)             float32 positive per-position scales
    ks, ke    (num_q,)         int32  each row's key range [ks, ke)
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence, Tuple

import numpy as np

HEADS = 32
HEAD_DIM = 128


@dataclasses.dataclass
class IndexerWorkload:
    name: str
    q: np.ndarray
    weights: np.ndarray
    kv: np.ndarray
    kv_scale: np.ndarray
    ks: np.ndarray
    ke: np.ndarray
    k: int
    seed: int

    @property
    def num_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_kv(self) -> int:
        return int(self.kv.shape[0])

    def pairs_scored(self) -> int:
        """Sum over rows of the number of positions in each row's range."""
        lo = np.clip(self.ks.astype(np.int64), 0, self.num_kv)
        hi = np.clip(self.ke.astype(np.int64), 0, self.num_kv)
        return int(np.maximum(hi - lo, 0).sum())


def to_fp8_codes(x: np.ndarray) -> np.ndarray:
    """float values -> OCP E4M3 codes (round to nearest even), via torch's
    float8_e4m3fn conversion; values are clipped to the finite range first."""
    import torch
    t = torch.from_numpy(np.clip(np.asarray(x, np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def ranges(requests: Sequence[Tuple[int, int]]) -> Tuple[np.ndarray, np.ndarray, int]:
    """Causal key ranges of a ragged prefill batch of (query rows, key length)."""
    ks: List[int] = []
    ke: List[int] = []
    off = 0
    for nq, L in requests:
        assert 0 < nq <= L
        for i in range(nq):
            ks.append(off)
            ke.append(off + L - nq + i + 1)
        off += L
    return np.array(ks, np.int32), np.array(ke, np.int32), off


def make(requests: Sequence[Tuple[int, int]], k: int, seed: int, name: str = "", flat: bool = False,
         q_sigma: float = 1.0) -> IndexerWorkload:
    rng = np.random.default_rng(seed)
    ks, ke, n = ranges(requests)
    num_q = len(ks)
    q = to_fp8_codes(rng.standard_normal((num_q, HEADS, HEAD_DIM), dtype=np.float32) * q_sigma)
    w = (rng.standard_normal((num_q, HEADS), dtype=np.float32) / np.float32(np.sqrt(HEADS * HEAD_DIM)))
    if flat:
        # every key row identical: all of a row's scores tie (the page's
        # adversarial flat-score test)
        row = to_fp8_codes(rng.standard_normal((1, HEAD_DIM), dtype=np.float32))
        kv = np.repeat(row, n, axis=0)
        kv_scale = np.ones(n, np.float32)
    else:
        kv = to_fp8_codes(rng.standard_normal((n, HEAD_DIM), dtype=np.float32))
        kv_scale = rng.uniform(0.5, 1.5, n).astype(np.float32)
    return IndexerWorkload(name or f"ix_{seed}", q, w.astype(np.float32), kv, kv_scale, ks, ke, k, seed)


# The page's Validation shapes (request lists @ k) and its performance shape.
CONFIGS = {
    "single_32x32k_k2048": dict(requests=[(32, 32768)], k=2048, seed=7001),
    "ragged_3req_k2048": dict(requests=[(16, 8192), (16, 24576), (8, 4096)], k=2048, seed=7002),
    "single_32x32k_k512": dict(requests=[(32, 32768)], k=512, seed=7003),
    "short_8x1k_k2048": dict(requests=[(8, 1024)], k=2048, seed=7004),
    "odd_widths_k512": dict(requests=[(9, 4099), (5, 1023)], k=512, seed=7005),
    "flat_8x16k_k2048": dict(requests=[(8, 16384)], k=2048, seed=7006, flat=True),
    "prefill_8192x256k_k2048": dict(requests=[(8192, 262144)], k=2048, seed=7010),
    "prefill_1024x64k_k2048": dict(requests=[(1024, 65536)], k=2048, seed=7011),
}


def make_config(name: str) -> IndexerWorkload:
    c = dict(CONFIGS[name])
    return make(c.pop("requests"), c.pop("k"), c.pop("seed"), name=name, **c)
