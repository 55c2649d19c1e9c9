"""Seeded synthetic inputs for the fused top-k + page-table transform.

This module only *makes inputs*: it holds none of the selection or transform
arithmetic, so both the CPU oracle and the HIP path can be fed from it without
sharing any of the method's code.  Every generator is driven by numpy's PCG64
with an explicit seed, and returns host (numpy) arrays:

    scores      (B, W)  float32, row-major
    seq_lens    (B,)    int32
    page_table  (B, P)  int32, row-major

Shapes and value distributions follow the workloads the pages measure or
describe (SGLang PR #26788 "DeepSeek-V4 DSA indexer: faster top-k + page-table
transform", Performance section and commit notes: k = 512..2048, seq 8K..256K+,
batch up to 8192, page_size 64; flash-float-jit-kernels README latency table:
top-2048 out of contexts up to 1M at low batch).  The real model tensors those
pages measured on are not available; these seeded stand-ins have the same
shapes and the distributions written next to each config below.

Poisoning, so that a leak is visible in any check:
  * score positions at or beyond a row's seq_len hold +inf (a kernel reading
    past seq_len would select them first);
  * page-table entries no valid position maps to hold INT32_MIN.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

INT32_MIN = np.int32(-(2**31))


@dataclasses.dataclass
class Workload:
    name: str
    description: str
    scores: np.ndarray       # (B, W) float32
    seq_lens: np.ndarray     # (B,) int32
    page_table: np.ndarray   # (B, P) int32
    k: int
    page_size: int
    want_raw: bool
    seed: int

    @property
    def batch(self) -> int:
        return int(self.scores.shape[0])

    @property
    def width(self) -> int:
        return int(self.scores.shape[1])

    @property
    def pages_per_row(self) -> int:
        return int(self.page_table.shape[1])


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def poison_scores(scores: np.ndarray, seq_lens: np.ndarray) -> None:
    """Fill positions >= clamp(seq_len, 0, W) with +inf, in place."""
    W = scores.shape[1]
    for b, L in enumerate(seq_lens.tolist()):
        L = min(max(int(L), 0), W)
        scores[b, L:] = np.inf


def identity_table(B: int, P: int, seq_lens: np.ndarray, page_size: int) -> np.ndarray:
    pt = np.broadcast_to(np.arange(P, dtype=np.int32), (B, P)).copy()
    _poison_table(pt, seq_lens, page_size)
    return pt


def permutation_table(rng: np.random.Generator, B: int, P: int, seq_lens: np.ndarray,
                      page_size: int) -> np.ndarray:
    pt = np.empty((B, P), dtype=np.int32)
    for b in range(B):
        pt[b] = rng.permutation(P).astype(np.int32)
    _poison_table(pt, seq_lens, page_size)
    return pt


def _poison_table(pt: np.ndarray, seq_lens: np.ndarray, page_size: int) -> None:
    W_pages = pt.shape[1]
    for b, L in enumerate(seq_lens.tolist()):
        L = max(int(L), 0)
        used = min(-(-L // page_size), W_pages)
        pt[b, used:] = INT32_MIN


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


# ----------------------------------------------------------------------------
# The five benchmark workloads (C1..C5).  Seed = 1000 * config + sub-index.
# ----------------------------------------------------------------------------

def c1(seed: int = 1000) -> Workload:
    """batch 1, seq 16384, k 512, i.i.d. N(0,1), page_size 64, identity table, raw output on."""
    rng = _rng(seed)
    B, W, k, ps = 1, 16384, 512, 64
    scores = rng.standard_normal((B, W), dtype=np.float32)
    seq = np.full(B, W, dtype=np.int32)
    pt = identity_table(B, W // ps, seq, ps)
    return Workload("c1_b1_L16K_k512", "batch=1 seq=16384 k=512 N(0,1) ps=64 identity table, raw on",
                    scores, seq, pt, k, ps, True, seed)


def c2(seed: int = 2000) -> Workload:
    """Decode batch 64, ragged seq_lens ~ U{4096..65536}, k 2048.

    score[b,i] = sum_{h<8} relu(z[b,i,h]) * w[b,h], z ~ N(0,1), w ~ U(0,1): the
    shape of an indexer score (weighted sum of per-head relu'd dot products) with
    unit scale.  page_size 64, a random permutation page table per row.
    """
    rng = _rng(seed)
    B, W, k, ps, H = 64, 65536, 2048, 64, 8
    seq = rng.integers(4096, 65536, size=B, endpoint=True).astype(np.int32)
    w = rng.random((B, H), dtype=np.float32)
    scores = np.zeros((B, W), dtype=np.float32)
    for h in range(H):
        z = rng.standard_normal((B, W), dtype=np.float32)
        scores += np.maximum(z, np.float32(0)) * w[:, h:h + 1]
    poison_scores(scores, seq)
    pt = permutation_table(rng, B, W // ps, seq, ps)
    return Workload("c2_b64_ragged4K-64K_k2048",
                    "batch=64 seq~U[4096,65536] k=2048 sum_h relu(N(0,1))*U(0,1) ps=64 permuted table",
                    scores, seq, pt, k, ps, False, seed)


def c3(batch: int = 1, seed: Optional[int] = None) -> Workload:
    """Low batch, 1M-token rows, k 2048: N(0,1) plus slow sinusoidal drift.

    score[b,i] = z + 0.5 * sin(2*pi*i/65536 + phi_b), phi_b ~ U(0, 2*pi).  The
    period (16 cycles per 1M row) is this generator's reading of "slow".  The
    drift concentrates the top-k in the high-phase stretches of the row.
    page_size 64, random permutation page table per row.
    """
    sub = {1: 1, 4: 2, 8: 3}[batch]
    seed = 3000 + sub if seed is None else seed
    rng = _rng(seed)
    B, W, k, ps = batch, 1 << 20, 2048, 64
    phi = rng.random(B) * (2.0 * np.pi)
    i = np.arange(W, dtype=np.float64)
    scores = np.empty((B, W), dtype=np.float32)
    for b in range(B):
        z = rng.standard_normal(W, dtype=np.float32).astype(np.float64)
        scores[b] = (z + 0.5 * np.sin(2.0 * np.pi * i / 65536.0 + phi[b])).astype(np.float32)
    seq = np.full(B, W, dtype=np.int32)
    pt = permutation_table(rng, B, W // ps, seq, ps)
    return Workload(f"c3_b{batch}_L1M_k2048",
                    f"batch={batch} seq=1048576 k=2048 N(0,1)+0.5*sin drift ps=64 permuted table",
                    scores, seq, pt, k, ps, False, seed)


def c4a(seed: int = 4001, batch: int = 2048) -> Workload:
    """Bandwidth regime: batch 2048, seq 65536, k 512, N(0,1), page_size 64, identity table."""
    rng = _rng(seed)
    B, W, k, ps = batch, 65536, 512, 64
    scores = rng.standard_normal((B, W), dtype=np.float32)
    seq = np.full(B, W, dtype=np.int32)
    pt = identity_table(B, W // ps, seq, ps)
    return Workload(f"c4a_b{B}_L64K_k512", f"batch={B} seq=65536 k=512 N(0,1) ps=64 identity table",
                    scores, seq, pt, k, ps, False, seed)


def c4b(seed: int = 4002) -> Workload:
    """Bandwidth regime, second shape: batch 128, seq 131072, k 512, N(0,1), identity table."""
    rng = _rng(seed)
    B, W, k, ps = 128, 131072, 512, 64
    scores = rng.standard_normal((B, W), dtype=np.float32)
    seq = np.full(B, W, dtype=np.int32)
    pt = identity_table(B, W // ps, seq, ps)
    return Workload("c4b_b128_L128K_k512", "batch=128 seq=131072 k=512 N(0,1) ps=64 identity table",
                    scores, seq, pt, k, ps, False, seed)


def tie_table(rng: np.random.Generator, count: int = 256) -> np.ndarray:
    """The first `count` distinct bf16-rounded N(0,1) draws, in order of appearance."""
    seen: Dict[int, None] = {}
    while len(seen) < count:
        draws = bf16_rne(rng.standard_normal(1024, dtype=np.float32))
        for bits in draws.view(np.uint32).tolist():
            if bits not in seen:
                seen[bits] = None
                if len(seen) == count:
                    break
    return np.array(list(seen.keys()), dtype=np.uint32).view(np.float32)


def c5(seed: int = 5000) -> Workload:
    """Adversarial ties: batch 128, width 131072, k 1024, page_size 16.

    Scores take only 256 distinct bf16-rounded values (hundreds of exact copies
    of each, so the k-th value is tied many times over), then each entry becomes
    -inf with probability 0.05.  Rows b = 7 (mod 8) are short, seq_len ~ U{0..k-1}
    (row 7 forced to 0 and row 15 to k-1), so they exercise the -1 padding; the
    rest use the full width.  Random permutation page table per row.
    """
    rng = _rng(seed)
    B, W, k, ps = 128, 131072, 1024, 16
    table = tie_table(rng)
    scores = table[rng.integers(0, table.size, size=(B, W))]
    scores[rng.random((B, W)) < 0.05] = -np.inf
    seq = np.full(B, W, dtype=np.int32)
    for b in range(7, B, 8):
        seq[b] = rng.integers(0, k)  # [0, k-1]
    seq[7] = 0
    seq[15] = k - 1
    poison_scores(scores, seq)
    pt = permutation_table(rng, B, W // ps, seq, ps)
    return Workload("c5_b128_W128K_k1024_ties", "batch=128 width=131072 k=1024 256 bf16 values, 5% -inf, "
                    "short rows, ps=16 permuted table", scores, seq, pt, k, ps, False, seed)


def mixed(seed: int = 6000) -> Workload:
    """Mixed long/short decode batch: batch 32 of width 1,048,576, rows 0..3 at
    the full width and rows 4..31 at 16384, k 2048, N(0,1), page_size 64,
    random permutation page table per row.  The batch is below half a row per
    CU, yet its widest rows do not all fit the split kernel resident at once:
    the case a dispatcher that only knows the batch shape has to place.
    (SGLang PR #26788's commit notes report such valleys for half-long batches
    and a length-aware schedule as the fix.)"""
    rng = _rng(seed)
    B, W, k, ps = 32, 1 << 20, 2048, 64
    seq = np.full(B, 16384, dtype=np.int32)
    seq[:4] = W
    scores = rng.standard_normal((B, W), dtype=np.float32)
    poison_scores(scores, seq)
    pt = permutation_table(rng, B, W // ps, seq, ps)
    return Workload("mixed_b32_4x1M_28x16K_k2048", "batch=32 width=1048576: 4 rows of 1M, 28 of 16K, k=2048 N(0,1) "
                    "ps=64 permuted table", scores, seq, pt, k, ps, False, seed)


CONFIGS = {
    "c1": c1,
    "c2": c2,
    "c3_b1": lambda: c3(1),
    "c3_b4": lambda: c3(4),
    "c3_b8": lambda: c3(8),
    "c4a": c4a,
    "c4b": c4b,
    "c5": c5,
    "mixed": mixed,
}


def make(name: str) -> Workload:
    return CONFIGS[name]()


# ----------------------------------------------------------------------------
# Small generic generators used by the tests (edge cases, adversarial rows).
# ----------------------------------------------------------------------------

def custom(seed: int, batch: int, width: int, k: int, page_size: int,
           seq_lens: Optional[List[int]] = None, kind: str = "normal",
           table: str = "perm", want_raw: bool = True, extra_pages: int = 0) -> Workload:
    """A seeded workload of arbitrary shape.

    kind: "normal" (N(0,1)), "ties" (values from a few bf16 levels), "const"
    (every valid entry equal), "neginf" (every valid entry -inf), "zeros" (a mix
    of +0.0 and -0.0), "asc" / "desc" (strictly increasing / decreasing in the
    position), "int" (small integers, heavy ties), "wide" (log-uniform
    magnitudes of both signs, including subnormals and +-inf), "crowded"
    (97 % of entries 1.0, 2 % 4.0, 1 % -2.0: hundreds of equal keys next to a
    few far larger and smaller ones).
    table: "identity" or "perm".
    """
    rng = _rng(seed)
    B, W = batch, width
    if seq_lens is None:
        seq = np.full(B, W, dtype=np.int32)
    else:
        seq = np.asarray(seq_lens, dtype=np.int32)
    shape = (B, W)
    if kind == "normal":
        scores = rng.standard_normal(shape, dtype=np.float32)
    elif kind == "ties":
        levels = bf16_rne(rng.standard_normal(6, dtype=np.float32))
        scores = levels[rng.integers(0, levels.size, size=shape)]
    elif kind == "const":
        scores = np.full(shape, np.float32(rng.standard_normal()), dtype=np.float32)
    elif kind == "neginf":
        scores = np.full(shape, -np.inf, dtype=np.float32)
    elif kind == "zeros":
        scores = np.where(rng.random(shape) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    elif kind == "asc":
        scores = np.broadcast_to(np.arange(W, dtype=np.float32) * np.float32(0.25) - np.float32(W / 8),
                                 shape).copy()
    elif kind == "desc":
        scores = np.broadcast_to(np.float32(W / 8) - np.arange(W, dtype=np.float32) * np.float32(0.25),
                                 shape).copy()
    elif kind == "int":
        scores = rng.integers(-3, 4, size=shape).astype(np.float32)
    elif kind == "crowded":
        scores = np.ones(shape, dtype=np.float32)
        r = rng.random(shape)
        scores[r < 0.02] = np.float32(4.0)
        scores[(r >= 0.02) & (r < 0.03)] = np.float32(-2.0)
    elif kind == "wide":
        mag = np.exp2(rng.uniform(-149.0, 127.9, size=shape)).astype(np.float32)
        sign = np.where(rng.random(shape) < 0.5, np.float32(-1), np.float32(1))
        scores = (mag * sign).astype(np.float32)
        special = rng.random(shape)
        scores[special < 0.01] = np.inf
        scores[(special >= 0.01) & (special < 0.02)] = -np.inf
        scores[(special >= 0.02) & (special < 0.03)] = np.float32(0.0)
        scores[(special >= 0.03) & (special < 0.04)] = np.float32(-0.0)
    else:
        raise ValueError(kind)
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    poison_scores(scores, seq)
    P = -(-W // page_size) + extra_pages
    if table == "identity":
        pt = identity_table(B, P, seq, page_size)
    else:
        pt = permutation_table(rng, B, P, seq, page_size)
    return Workload(f"custom_{kind}_b{B}_W{W}_k{k}_ps{page_size}", kind, scores, seq, pt, k, page_size,
                    want_raw, seed)
