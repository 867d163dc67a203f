"""Seeded synthetic inputs for the strip-wise linear cross-entropy.

This module only *draws* inputs: hidden states ``h`` [N, H], the projection
weight ``W`` [V, H], int32 targets with ``ignore_index`` holes, and the fold
order of vocabulary shards.  It holds none of the arithmetic of the loss or
its gradients, so that the CPU oracle and the GPU path can both consume the
same bytes without sharing any code of the method itself.

Determinism: every array is produced from ``numpy.random.SeedSequence`` keyed
by (workload seed, stream id, chunk id).  Rows of ``h`` and ``W`` are generated
in fixed chunks of ``CHUNK_ROWS`` rows, so any subset of rows can be
regenerated on its own (the sampled oracle checks at full size rely on this)
and the result does not depend on how many rows were asked for.

bf16 workloads store the values as float32 arrays that are exactly
representable in bfloat16 (round-to-nearest-even applied once, here), so a
``.to(torch.bfloat16)`` on the device side and a float64 view on the oracle
side both see the same numbers.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

IGNORE_INDEX = -100
CHUNK_ROWS = 1024

_STREAM_HIDDEN = 1
_STREAM_WEIGHT = 2
_STREAM_TARGETS = 3
_STREAM_IGNORE = 4


@dataclass(frozen=True)
class Workload:
    """Shape, value distribution and reduction of one synthetic problem."""

    name: str
    n_tokens: int  # N
    hidden: int  # H
    vocab: int  # V
    strip: int  # Vs, the vocabulary strip width folded per step
    dtype: str  # "f32" or "bf16"
    hidden_scale: float  # h = hidden_scale * N(0, 1)
    weight_std: float  # W ~ N(0, weight_std^2)
    targets: str  # "uniform" or "zipf"
    zipf_s: float = 0.0
    ignore_frac: float = 0.0  # fraction of targets replaced by IGNORE_INDEX
    reduction: str = "mean"  # "mean" or "sum"
    grad_out: float = 1.0  # upstream gradient of the reduced loss
    shards: int = 0  # >0: W is folded as this many equal shards in ring order
    ring_start: int = 0  # first shard visited (ring order r, r+1, ... mod shards)
    seed: int = 1234

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def flops(self) -> float:
        """Algorithmic FLOP of one forward + backward: 8*N*H*V."""
        return 8.0 * self.n_tokens * self.hidden * self.vocab

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _w(name, n, h, v, vs, dtype, hs, ws, tg, **kw) -> Workload:
    return Workload(name, n, h, v, vs, dtype, hs, ws, tg, **kw)


# The five workloads, smallest first.  Seeds are 1234 + position.
WORKLOADS = {
    w.name: w
    for w in [
        _w("tiny_f32", 256, 128, 1024, 256, "f32", 1.0, 1.0 / math.sqrt(128), "uniform",
           seed=1234),
        _w("bf16_n4k_h2k_v152k", 4096, 2048, 151936, 8192, "bf16", 1.0, 0.02, "uniform",
           ignore_frac=0.10, seed=1235),
        _w("bf16_n16k_h6k_v155k_zipf_sum", 16384, 6144, 155136, 16384, "bf16",
           4.0 / math.sqrt(6144), 0.02, "zipf", zipf_s=1.1, reduction="sum",
           grad_out=1.0 / 16384, seed=1236),
        _w("bf16_n128k_h2k_v152k", 131072, 2048, 151936, 8192, "bf16", 1.0, 0.02, "uniform",
           seed=1237),
        _w("bf16_n64k_h6k_v262k_ring8", 65536, 6144, 262144, 32768, "bf16", 1.0,
           20.0 / math.sqrt(6144), "zipf", zipf_s=1.1, ignore_frac=0.05, shards=8,
           ring_start=3, seed=1238),
        # the second page's Ring-DTP benchmark shape (appendix C: N = 16384,
        # H = 7168, V = 200000, FP32) as one device's whole problem; the page
        # states no value distributions, so logits ~ N(0, 1): h ~ N(0, 1),
        # W ~ N(0, 1/H), uniform targets, mean reduction
        _w("f32_n16k_h7k_v200k", 16384, 7168, 200000, 8192, "f32", 1.0,
           1.0 / math.sqrt(7168), "uniform", seed=1239),
    ]
}
WORKLOAD_ORDER = list(WORKLOADS)

# Shapes measured beside the workloads above (their parity is covered by
# dedicated small-shape tests): the strip-free backward's comparison shape.
EXTRA_WORKLOADS = {
    w.name: w
    for w in [
        _w("bf16_n4k_h512_v32k", 4096, 512, 32768, 8192, "bf16", 1.0, 0.02, "uniform",
           ignore_frac=0.10, seed=1240),
    ]
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value (ties to even), returned as float32.

    Inputs here are finite normals, so NaN/Inf handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r & np.uint32(0xFFFF0000)).view(np.float32)


def _normal_chunk(w: Workload, stream: int, chunk: int, rows: int, cols: int,
                  scale: float) -> np.ndarray:
    x = _rng(w.seed, stream, chunk).standard_normal((rows, cols), dtype=np.float32)
    x *= np.float32(scale)
    return round_to_bf16(x) if w.dtype == "bf16" else x


def _matrix(w: Workload, stream: int, total_rows: int, scale: float,
            rows: np.ndarray | None, threads: int) -> np.ndarray:
    cols = w.hidden
    if rows is None:
        out = np.empty((total_rows, cols), dtype=np.float32)
        n_chunks = (total_rows + CHUNK_ROWS - 1) // CHUNK_ROWS

        def fill(c: int) -> None:
            r0 = c * CHUNK_ROWS
            r1 = min(total_rows, r0 + CHUNK_ROWS)
            out[r0:r1] = _normal_chunk(w, stream, c, CHUNK_ROWS, cols, scale)[: r1 - r0]

        if threads > 1 and n_chunks > 1:
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(fill, range(n_chunks)))
        else:
            for c in range(n_chunks):
                fill(c)
        return out
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= total_rows):
        raise IndexError("row index out of range")
    out = np.empty((rows.size, cols), dtype=np.float32)
    for c in np.unique(rows // CHUNK_ROWS):
        block = _normal_chunk(w, stream, int(c), CHUNK_ROWS, cols, scale)
        sel = np.nonzero(rows // CHUNK_ROWS == c)[0]
        out[sel] = block[rows[sel] - c * CHUNK_ROWS]
    return out


def hidden(w: Workload, rows: np.ndarray | None = None, threads: int = 8) -> np.ndarray:
    """Hidden states h [N, H] (or the given rows of it), float32 values."""
    return _matrix(w, _STREAM_HIDDEN, w.n_tokens, w.hidden_scale, rows, threads)


def weight(w: Workload, rows: np.ndarray | None = None, threads: int = 8) -> np.ndarray:
    """Projection weight W [V, H] (or the given vocabulary rows), float32 values."""
    return _matrix(w, _STREAM_WEIGHT, w.vocab, w.weight_std, rows, threads)


def zipf_ids(rng: np.random.Generator, n: int, vocab: int, s: float) -> np.ndarray:
    """Token ids drawn from a Zipf(s) law truncated to ranks 1..vocab.

    P(rank k) = k^-s / sum_{j<=vocab} j^-s, sampled by inverse CDF; the id is
    rank - 1, so the most frequent ids are the smallest.
    """
    ranks = np.arange(1, vocab + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-s))
    cdf /= cdf[-1]
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, vocab - 1).astype(np.int32)


def targets(w: Workload) -> np.ndarray:
    """int32 targets [N]; a seeded subset of round(ignore_frac*N) is IGNORE_INDEX."""
    rng = _rng(w.seed, _STREAM_TARGETS)
    if w.targets == "uniform":
        t = rng.integers(0, w.vocab, size=w.n_tokens, dtype=np.int64).astype(np.int32)
    elif w.targets == "zipf":
        t = zipf_ids(rng, w.n_tokens, w.vocab, w.zipf_s)
    else:
        raise ValueError(f"unknown target law {w.targets!r}")
    n_ignore = int(round(w.ignore_frac * w.n_tokens))
    if n_ignore:
        pos = _rng(w.seed, _STREAM_IGNORE).permutation(w.n_tokens)[:n_ignore]
        t[pos] = IGNORE_INDEX
    return t


def fold_order(w: Workload) -> list[tuple[int, int]]:
    """(v_begin, v_len) of every vocabulary strip, in the order they are folded.

    Without shards the strips of width ``strip`` are visited in natural order,
    the last one ragged.  With ``shards`` the vocabulary is cut into that many
    equal shards visited in ring order starting at ``ring_start``; each shard is
    then cut into strips of width ``strip``.
    """
    def cut(v0: int, v1: int) -> list[tuple[int, int]]:
        return [(a, min(w.strip, v1 - a)) for a in range(v0, v1, w.strip)]

    if w.shards <= 0:
        return cut(0, w.vocab)
    if w.vocab % w.shards:
        raise ValueError("vocab must split into equal shards")
    size = w.vocab // w.shards
    out: list[tuple[int, int]] = []
    for k in range(w.shards):
        s = (w.ring_start + k) % w.shards
        out += cut(s * size, (s + 1) * size)
    return out


def small(name: str, n: int, h: int, v: int, vs: int, dtype: str = "bf16", *,
          weight_std: float = 0.05, hidden_scale: float = 1.0, target_law: str = "uniform",
          ignore_frac: float = 0.0, reduction: str = "mean", grad_out: float = 1.0,
          shards: int = 0, ring_start: int = 0, seed: int = 7) -> Workload:
    """A small workload of arbitrary shape (parity and edge cases)."""
    return Workload(name, n, h, v, vs, dtype, hidden_scale, weight_std, target_law,
                    zipf_s=1.1, ignore_frac=ignore_frac, reduction=reduction,
                    grad_out=grad_out, shards=shards, ring_start=ring_start, seed=seed)
