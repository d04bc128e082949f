"""Seeded synthetic inputs for the per-decode-step sparse KV assembly path.

This module is the only code shared by the CPU oracle (``oracle/``) and the HIP
path (``token_level_gather_amd``).  It holds none of the method's arithmetic: it
draws KV rows, queries and Top-K index streams, and nothing else.  Slot lookup,
the sparse diff, LRU eviction, the gathers and attention live on each side
separately.

What the inputs stand in for
----------------------------
The pages measure whole models (GLM-5.3 and DeepSeek DSA decode at 16K-1M
context, per-GPU batch 192 at 16K with 20 % / 40 % Top-K miss: "XM-Sparse",
TL;DR and testbed sections; the SGLang/Tair hierarchical sparse attention
summary, third paragraph).  No weights, prompts or datasets are used here: KV
rows and queries are i.i.d. N(0, 1) rounded to bf16, and the Top-K selector's
output is replaced by index streams with a controlled carry-over between steps.

Recipe
------
* KV rows: 576 values per token (512 latent + 64 rope dims of an MLA layer),
  N(0, 1) drawn as float32 and rounded to bf16 (round to nearest, ties to even).
  Rows of unit (request r, layer l) come from ``SeedSequence([seed, 0, r, l])``
  in token order, so any unit can be generated on its own.
* Queries: 16 heads x 576 dims, N(0, 1) -> bf16, all requests of one
  (layer, step) from ``SeedSequence([seed, 2, l, t])``.
* Top-K streams, per unit from ``SeedSequence([seed, 1, r, l])``:
  - step 0 draws K distinct tokens from the workload's fresh distribution;
  - step t > 0 keeps ``K - round(f*K)`` tokens, a uniform random subset of the
    previous step's set, and draws ``round(f*K)`` fresh tokens from the fresh
    distribution restricted to tokens *not* in the previous set;
  - the K indices of a step are a seeded random permutation of kept + fresh
    (a selector's output is in score order, not token order).
* Fresh distributions: ``uniform`` over [0, N); ``zipf`` draws
  ``round(0.1 * n_fresh)`` tokens uniformly from the last 512 positions and the
  rest from P(p) proportional to (p + 1) ** -1.1 over p in [0, N) by rejection
  from ``Generator.zipf(1.1) - 1``.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

HEADS = 16
HEAD_DIM = 576
V_DIM = 512
ROW_BYTES = HEAD_DIM * 2

STREAM_POOL = 0
STREAM_TOPK = 1
STREAM_QUERY = 2


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and index-stream recipe of one synthetic decode workload."""

    name: str
    batch: int          # B requests
    layers: int         # L layers
    context: int        # N tokens per (request, layer)
    slots: int          # S hot-buffer slots per (request, layer)
    topk: int           # K selected tokens per step
    steps: int          # decode steps in the workload
    fresh_rate: float   # f: fraction of each step's Top-K drawn fresh
    dist: str = "uniform"   # "uniform" | "zipf"
    seed: int = 20261202
    zipf_s: float = 1.1
    forced_frac: float = 0.1
    forced_window: int = 512
    heads: int = HEADS
    head_dim: int = HEAD_DIM
    v_dim: int = V_DIM

    @property
    def n_fresh(self) -> int:
        return int(round(self.fresh_rate * self.topk))

    @property
    def n_keep(self) -> int:
        return self.topk - self.n_fresh

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def pool_bytes(self) -> int:
        return self.batch * self.layers * self.context * self.head_dim * 2

    def shrunk(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workload shapes this path is measured and tested on.
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("ctx4k_b1_k256", batch=1, layers=1, context=4096, slots=512,
                 topk=256, steps=16, fresh_rate=0.2, seed=20261202),
        Workload("ctx16k_b64_k2048", batch=64, layers=1, context=16384,
                 slots=4096, topk=2048, steps=32, fresh_rate=0.2,
                 seed=20261203),
        Workload("ctx16k_b192_k2048_f20", batch=192, layers=1, context=16384,
                 slots=4096, topk=2048, steps=32, fresh_rate=0.2,
                 seed=20261204),
        Workload("ctx16k_b192_k2048_f40", batch=192, layers=1, context=16384,
                 slots=4096, topk=2048, steps=32, fresh_rate=0.4,
                 seed=20261204),
        Workload("ctx128k_b32_l8_zipf", batch=32, layers=8, context=131072,
                 slots=4096, topk=2048, steps=16, fresh_rate=0.2, dist="zipf",
                 seed=20261205),
        Workload("ctx1m_b4_l4", batch=4, layers=4, context=1048576, slots=8192,
                 topk=2048, steps=16, fresh_rate=0.2, seed=20261206),
    ]
}

BENCH_WORKLOAD = "ctx16k_b64_k2048"


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) and return the raw uint16 bits.

    Inputs here are finite normals, so the NaN/overflow cases of a general
    conversion do not arise.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


# ---------------------------------------------------------------- KV rows

def fill_unit_rows(out: np.ndarray, wl: Workload, req: int, layer: int,
                   chunk_rows: int = 8192) -> None:
    """Write unit (req, layer)'s N rows of bf16 bits into ``out`` ([N][576] uint16)."""
    assert out.shape == (wl.context, wl.head_dim) and out.dtype == np.uint16
    rng = _rng(wl.seed, STREAM_POOL, req, layer)
    for r0 in range(0, wl.context, chunk_rows):
        r1 = min(wl.context, r0 + chunk_rows)
        out[r0:r1] = f32_to_bf16_bits(
            rng.standard_normal((r1 - r0, wl.head_dim), dtype=np.float32))


def fill_pool(pool: np.ndarray, wl: Workload, threads: Optional[int] = None) -> None:
    """Fill the whole host pool ``pool`` ([B][L][N][576] uint16) in place.

    Units are independent streams, so the bytes do not depend on ``threads``.
    """
    assert pool.shape == (wl.batch, wl.layers, wl.context, wl.head_dim)
    units = [(r, l) for r in range(wl.batch) for l in range(wl.layers)]
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if threads <= 1:
        for r, l in units:
            fill_unit_rows(pool[r, l], wl, r, l)
        return
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda u: fill_unit_rows(pool[u[0], u[1]], wl, u[0], u[1]), units))


def unit_rows(wl: Workload, req: int, layer: int) -> np.ndarray:
    out = np.empty((wl.context, wl.head_dim), dtype=np.uint16)
    fill_unit_rows(out, wl, req, layer)
    return out


# ---------------------------------------------------------------- queries

def queries(wl: Workload, layer: int, step: int) -> np.ndarray:
    """Queries of every request at (layer, step): [B][16][576] bf16 bits."""
    rng = _rng(wl.seed, STREAM_QUERY, layer, step)
    x = rng.standard_normal((wl.batch, wl.heads, wl.head_dim), dtype=np.float32)
    return f32_to_bf16_bits(x)


# ---------------------------------------------------------------- Top-K streams

def _take_new(cands: np.ndarray, taken: np.ndarray, need: int) -> np.ndarray:
    """First ``need`` candidates (in draw order) that are not taken and not repeated."""
    cands = cands[~taken[cands]]
    if cands.size == 0:
        return cands
    _, first = np.unique(cands, return_index=True)
    cands = cands[np.sort(first)]
    return cands[:need]


def _draw_uniform(rng, lo: int, hi: int, count: int, taken: np.ndarray) -> np.ndarray:
    got: List[np.ndarray] = []
    n = 0
    if hi - lo - int(taken[lo:hi].sum()) < count:
        raise ValueError("not enough free tokens to draw from")
    while n < count:
        cands = rng.integers(lo, hi, size=max(64, 2 * (count - n)), dtype=np.int64)
        new = _take_new(cands, taken, count - n)
        taken[new] = True
        got.append(new)
        n += new.size
    return np.concatenate(got) if got else np.zeros(0, np.int64)


def _draw_zipf(rng, wl: Workload, count: int, taken: np.ndarray) -> np.ndarray:
    n_forced = int(round(wl.forced_frac * count))
    lo = max(0, wl.context - wl.forced_window)
    forced = _draw_uniform(rng, lo, wl.context, n_forced, taken)
    got = [forced]
    n = 0
    need = count - n_forced
    while n < need:
        cands = rng.zipf(wl.zipf_s, size=max(256, 4 * (need - n))) - 1
        cands = cands[cands < wl.context].astype(np.int64)
        new = _take_new(cands, taken, need - n)
        taken[new] = True
        got.append(new)
        n += new.size
    return np.concatenate(got)


def _draw_fresh(rng, wl: Workload, count: int, taken: np.ndarray) -> np.ndarray:
    if wl.dist == "uniform":
        return _draw_uniform(rng, 0, wl.context, count, taken)
    if wl.dist == "zipf":
        return _draw_zipf(rng, wl, count, taken)
    raise ValueError(f"unknown fresh distribution {wl.dist!r}")


def unit_topk_stream(wl: Workload, req: int, layer: int, steps: int) -> np.ndarray:
    """Top-K index stream of one unit: [steps][K] int32, unique and in [0, N) per step."""
    rng = _rng(wl.seed, STREAM_TOPK, req, layer)
    out = np.empty((steps, wl.topk), dtype=np.int32)
    taken = np.zeros(wl.context, dtype=bool)
    prev = _draw_fresh(rng, wl, wl.topk, taken)
    out[0] = rng.permutation(prev)
    for t in range(1, steps):
        kept = rng.choice(prev, size=wl.n_keep, replace=False)
        taken[:] = False
        taken[prev] = True          # fresh tokens come from outside the previous set
        fresh = _draw_fresh(rng, wl, wl.n_fresh, taken)
        cur = np.concatenate([kept, fresh])
        out[t] = rng.permutation(cur)
        prev = cur
    return out


def topk_streams(wl: Workload, steps: Optional[int] = None,
                 requests: Optional[List[int]] = None,
                 threads: Optional[int] = None) -> np.ndarray:
    """All Top-K streams: [steps][L][B'][K] int32 for the requested requests."""
    steps = wl.steps if steps is None else steps
    reqs = list(range(wl.batch)) if requests is None else list(requests)
    out = np.empty((steps, wl.layers, len(reqs), wl.topk), dtype=np.int32)
    jobs = [(i, r, l) for i, r in enumerate(reqs) for l in range(wl.layers)]

    def run(job):
        i, r, l = job
        out[:, l, i, :] = unit_topk_stream(wl, r, l, steps)

    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if threads <= 1 or len(jobs) == 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, jobs))
    return out


PAD_PATTERNS = ("tail", "scatter", "empty", "none")


def pad_topk_streams(streams: np.ndarray, seed: int, patterns=PAD_PATTERNS) -> np.ndarray:
    """Padded copies of Top-K streams ([T][L][B][K]) for a selector that returns
    fewer than K tokens: request b uses ``patterns[b % len(patterns)]``:

    * ``tail``: only the first ``v`` entries are tokens, the rest -1, with ``v``
      drawn per step uniformly from [0, K] (a sequence shorter than K; v = 0
      and v = K included);
    * ``scatter``: each entry is -1 with probability 0.3;
    * ``empty``: every entry -1 on odd steps, no padding on even ones;
    * ``none``: no padding.
    """
    out = streams.copy()
    T, L, B, K = out.shape
    rng = np.random.default_rng(np.random.SeedSequence([seed, 3]))
    for t in range(T):
        for l in range(L):
            for b in range(B):
                kind = patterns[b % len(patterns)]
                row = out[t, l, b]
                if kind == "tail":
                    v = int(rng.integers(0, K + 1))
                    row[v:] = -1
                elif kind == "scatter":
                    row[rng.random(K) < 0.3] = -1
                elif kind == "empty":
                    if t % 2 == 1:
                        row[:] = -1
    return out
