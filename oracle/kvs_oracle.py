"""Plain, slow CPU oracle of one decode step of Top-K-driven sparse KV assembly.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It is independent
of the HIP path: no shared kernels, headers, helpers or constants.  Its only
input from elsewhere is the seeded data drawn by ``kvs_workload``.

What is computed, and from which passage
----------------------------------------
The pages describe the mechanism in prose only:

* "Sparse Attention-Driven KVCache Management for Domestic AI Supernodes"
  (talk abstract and agenda, "Sparse-Driven System Design"): the full history
  of KV data lives in a host memory pool, hot data is cached on the device, an
  index mapping links the two, Top-K indices drive token-level access, and
  the data the current step needs is assembled on demand by an index-based
  copy.
* SGLang/Tair hierarchical sparse attention summary, first paragraph: the GPU
  keeps only a Top-k LRU buffer of hot entries; third paragraph: only the sparse
  changes are transferred (the "Sparse Diff Kernel"); second paragraph: DSA
  selects the Top-k tokens and attention is computed over them only.
* "XM-Sparse", HiSparse integration section: KV management follows the request
  lifecycle publish -> fetch -> write-back -> free.

The pages leave the exact rules open; this oracle reads them as follows:

* LRU order: victims are the slots not holding a token of the current Top-K
  set, taken in ascending ``(last_used_step, slot)`` order; empty slots carry
  ``last_used = -1`` and therefore go first, lowest slot first.
* The j-th miss in Top-K array order is paired with the j-th victim.
* The step counter of a unit is the number of valid steps it has taken; hit
  slots and newly filled slots get ``last_used = t``.
* KV rows are MLA rows of 576 bf16 values; scores use all 576 dims, values are
  dims 0..511, scale 1/sqrt(576); softmax and sums in float64 here.
* Padded Top-K (``padded=True``): a selector may return fewer than K tokens
  (a sequence shorter than K); the value -1 marks an empty entry.  An empty
  entry is neither a hit nor a miss: it reads no map, takes no slot, does not
  count as "a token of the current Top-K set" for the LRU, gathers a zero row
  and is left out of the softmax.  A step whose entries are all empty still
  counts as a step; its output is zero and its log-sum-exp -inf.
* Lifecycle "publish" of a decode step's new row (``append``): the row
  replaces the token's row in the host pool and, if the token is resident in
  the hot buffer, that slot's copy too, so hot copies always equal the pool.

There is no approximation in the method: every step is an exact definition,
so the oracle is that definition written out.  The LRU victim choice sorts the
candidate slots with ``numpy.lexsort`` (a library sort standing in for
"ascending (last_used, slot)").
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

ROW_DIM = 576
V_DIM = 512


PAD = -1         # an empty Top-K entry when the step is padded
SLOT_PAD = -2    # slot_of of an empty entry (-1 = miss, >= 0 = hit slot)


class KvsError(ValueError):
    """An invalid Top-K input (out of range or duplicate); state is left unchanged."""


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    u32 = bits.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def attention_fp64(q_bits: np.ndarray, rows_bits: np.ndarray, scale: float,
                   v_dim: int = V_DIM):
    """Softmax attention of H query heads over the K gathered rows, in float64.

    q_bits: [H][D] bf16 bits; rows_bits: [K][D] bf16 bits (keys are the whole
    rows, values their first ``v_dim`` dims).  Returns (out [H][v_dim], lse [H])
    with lse the natural-log log-sum-exp of the scaled scores.  Over no rows at
    all (every entry of a padded step empty) the output is zero and lse -inf.
    """
    if rows_bits.shape[0] == 0:
        h = q_bits.shape[0]
        return np.zeros((h, v_dim)), np.full(h, -np.inf)
    q = bf16_bits_to_f64(q_bits)
    kv = bf16_bits_to_f64(rows_bits)
    z = (q @ kv.T) * scale                      # [H][K]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    s = e.sum(axis=1, keepdims=True)
    p = e / s
    out = p @ kv[:, :v_dim]
    lse = (m + np.log(s))[:, 0]
    return out, lse


@dataclasses.dataclass
class StepRecord:
    """Everything one unit-step produces, for comparison with the device."""

    t: int
    slot_of: np.ndarray      # [K] slot of topk[i] before the step, -1 = miss, -2 = empty
    miss_pos: np.ndarray     # [n_miss] Top-K positions of the misses, ascending
    victims: np.ndarray      # [n_miss] slot given to the j-th miss
    evicted: np.ndarray      # [n_miss] token that slot held before (-1 = empty)
    cbuf: np.ndarray         # [K][576] uint16: gathered rows in Top-K order
    out: Optional[np.ndarray]  # [H][512] float64
    lse: Optional[np.ndarray]  # [H] float64

    @property
    def n_miss(self) -> int:
        return int(self.miss_pos.size)

    @property
    def n_hit(self) -> int:
        return int((self.slot_of >= 0).sum())

    @property
    def n_pad(self) -> int:
        return int((self.slot_of == SLOT_PAD).sum())


class OracleUnit:
    """State of one (request, layer) unit: index maps, LRU stamps and a hot copy."""

    def __init__(self, context: int, slots: int, topk: int, keep_hot: bool = True):
        if not (1 <= topk <= slots):
            raise KvsError("need 1 <= K <= S")
        self.N, self.S, self.K = int(context), int(slots), int(topk)
        self.keep_hot = keep_hot
        self.reset()

    def reset(self) -> None:
        """Lifecycle "free": forget every resident token.  The step counter keeps running."""
        self.tok2slot = np.full(self.N, -1, dtype=np.int64)
        self.slot2tok = np.full(self.S, -1, dtype=np.int64)
        self.last_used = np.full(self.S, -1, dtype=np.int64)
        self.hot = np.zeros((self.S, ROW_DIM), dtype=np.uint16) if self.keep_hot else None
        if not hasattr(self, "t"):
            self.t = 0

    # -- one decode step ---------------------------------------------------
    def step(self, topk: np.ndarray, pool_rows: np.ndarray,
             q_bits: Optional[np.ndarray] = None, scale: float = 1.0 / 24.0,
             v_dim: int = V_DIM, padded: bool = False) -> StepRecord:
        """Run one step for this unit.

        topk: [K] token indices; pool_rows: [N][576] bf16 bits of this unit's
        host pool; q_bits: [H][576] bf16 bits or None to skip attention.
        padded: entries equal to PAD (-1) are empty.
        """
        topk = np.asarray(topk, dtype=np.int64)
        K = self.K
        if topk.shape != (K,):
            raise KvsError("topk has the wrong length")
        valid = (topk != PAD) if padded else np.ones(K, dtype=bool)
        vt = topk[valid]
        # 1. validate (unique, in range); invalid input leaves the state alone
        if vt.size and (vt.min() < 0 or vt.max() >= self.N):
            raise KvsError("Top-K index out of range")
        if np.unique(vt).size != vt.size:
            raise KvsError("duplicate Top-K index")
        t = self.t

        # 2. lookup + diff: hit iff the token maps to a slot; misses in array order
        slot_of = np.full(K, SLOT_PAD, dtype=np.int64)
        slot_of[valid] = self.tok2slot[vt]
        hit = slot_of >= 0
        miss_pos = np.flatnonzero(slot_of == -1)
        n_miss = miss_pos.size

        # 3. touch the hit slots
        self.last_used[slot_of[hit]] = t

        # 4. victims: non-hit slots in ascending (last_used, slot) order
        hit_slots = set(slot_of[hit].tolist())
        cand = np.array([s for s in range(self.S) if s not in hit_slots], dtype=np.int64)
        order = np.lexsort((cand, self.last_used[cand]))   # primary key last_used
        victims = cand[order[:n_miss]]

        # 5. map update: the j-th miss takes the j-th victim
        evicted = np.full(n_miss, -1, dtype=np.int64)
        for j in range(n_miss):
            v = victims[j]
            tok = topk[miss_pos[j]]
            old = self.slot2tok[v]
            if old >= 0:
                self.tok2slot[old] = -1
                evicted[j] = old
            self.slot2tok[v] = tok
            self.tok2slot[tok] = v
            self.last_used[v] = t

        # 6. index copy: hits from the hot copy (before write-back), misses from the
        #    pool; then write the misses back into their victim slots
        cbuf = np.zeros((K, ROW_DIM), dtype=np.uint16)   # empty entries stay zero
        for i in range(K):
            if hit[i]:
                cbuf[i] = self.hot[slot_of[i]] if self.keep_hot else pool_rows[topk[i]]
            elif valid[i]:
                cbuf[i] = pool_rows[topk[i]]
        if self.keep_hot:
            for j in range(n_miss):
                self.hot[victims[j]] = pool_rows[topk[miss_pos[j]]]

        # 7. Top-K attention over the gathered rows
        out = lse = None
        if q_bits is not None:
            out, lse = attention_fp64(q_bits, cbuf[valid], scale, v_dim)

        self.t = t + 1
        return StepRecord(t=t, slot_of=slot_of, miss_pos=miss_pos, victims=victims,
                          evicted=evicted, cbuf=cbuf, out=out, lse=lse)

    # -- lifecycle "publish" of one new row --------------------------------
    def append(self, pool_rows: np.ndarray, pos: int, row: np.ndarray) -> None:
        """Write ``row`` ([576] bf16 bits) as token ``pos`` of this unit's host pool
        (``pool_rows``, modified in place) and into its hot slot if it is resident."""
        if not 0 <= pos < self.N:
            raise KvsError("append position out of range")
        pool_rows[pos] = row
        s = self.tok2slot[pos]
        if s >= 0 and self.keep_hot:
            self.hot[s] = row

    # -- views ------------------------------------------------------------
    def resident(self) -> set:
        return set(self.slot2tok[self.slot2tok >= 0].tolist())


def run_unit(context: int, slots: int, topk_stream: np.ndarray, pool_rows: np.ndarray,
             q_stream: Optional[np.ndarray] = None, scale: float = 1.0 / 24.0,
             keep_hot: bool = True, padded: bool = False) -> List[StepRecord]:
    """Replay a whole Top-K stream ([T][K]) through one fresh unit."""
    unit = OracleUnit(context, slots, topk_stream.shape[1], keep_hot=keep_hot)
    recs = []
    for t in range(topk_stream.shape[0]):
        q = None if q_stream is None else q_stream[t]
        recs.append(unit.step(topk_stream[t], pool_rows, q, scale, padded=padded))
    return recs
