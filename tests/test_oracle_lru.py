"""Pins of the oracle's lookup / sparse diff / LRU / map update / gather steps.

Each check comes from something other than the oracle itself: a trace worked
by hand, a textbook LRU cache (K = 1), an independent order-array formulation,
set algebra on the resident set, and closed forms (cold start, repeated Top-K,
no eviction when the buffer holds the whole context).
"""
import collections
import json
import os

import numpy as np
import pytest

from oracle import KvsError, OracleUnit, run_unit

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lru_trace_n8_s4_k2.json")
GOLDEN_PADDED = os.path.join(os.path.dirname(__file__), "golden",
                             "lru_trace_padded_n8_s4_k3.json")


def _tagged_pool(n_ctx: int) -> np.ndarray:
    """Pool whose row r is filled with the value r + 1, so a row names its token."""
    return np.repeat(np.arange(1, n_ctx + 1, dtype=np.uint16)[:, None], 576, axis=1)


def test_golden_trace_worked_by_hand():
    g = json.load(open(GOLDEN))
    pool = _tagged_pool(g["context"])
    u = OracleUnit(g["context"], g["slots"], g["topk"])
    for st in g["steps"]:
        rec = u.step(np.array(st["topk"]), pool)
        assert rec.t == st["t"]
        assert rec.slot_of.tolist() == st["slot_of"]
        assert rec.miss_pos.tolist() == st["miss_pos"]
        assert rec.victims.tolist() == st["victims"]
        assert rec.evicted.tolist() == st["evicted"]
        assert u.last_used.tolist() == st["last_used"]
        assert u.slot2tok.tolist() == st["slot2tok"]
        # cbuf rows carry their token's tag; "h<s>" rows must come from hot slot s,
        # whose content before the step is the token the trace says slot s held
        for i, src in enumerate(st["cbuf_src"]):
            tok = st["topk"][i]
            assert int(rec.cbuf[i, 0]) == tok + 1
            if src[0] == "h":
                assert rec.slot_of[i] == int(src[1:])
            else:
                assert src == f"p{tok}" and rec.slot_of[i] == -1
    assert u.tok2slot.tolist() == g["final_tok2slot"]


class TextbookLRU:
    """Classic LRU cache over S numbered slots, empty slots evicted first (lowest first)."""

    def __init__(self, slots):
        self.od = collections.OrderedDict((("empty", s), s) for s in range(slots))
        self.where = {}

    def access(self, tok):
        if tok in self.where:
            key = ("tok", tok)
            self.od.move_to_end(key)
            return self.where[tok], None
        key, slot = self.od.popitem(last=False)      # least recently used
        evicted = key[1] if key[0] == "tok" else -1
        if evicted >= 0:
            del self.where[evicted]
        self.where[tok] = slot
        self.od[("tok", tok)] = slot
        return slot, evicted


@pytest.mark.parametrize("seed", range(6))
def test_k1_equals_textbook_lru(seed):
    rng = np.random.default_rng(seed)
    n_ctx, slots = 40, int(rng.integers(1, 9))
    pool = _tagged_pool(n_ctx)
    u = OracleUnit(n_ctx, slots, 1)
    ref = TextbookLRU(slots)
    for _ in range(200):
        tok = int(rng.integers(0, min(n_ctx, slots * 2 + 2)))
        rec = u.step(np.array([tok]), pool)
        slot, evicted = ref.access(tok)
        assert u.tok2slot[tok] == slot
        if rec.n_miss:
            assert rec.victims[0] == slot and rec.evicted[0] == evicted
        else:
            assert evicted is None and rec.slot_of[0] == slot
        for t, s in ref.where.items():
            assert u.slot2tok[s] == t


def order_array_model(n_ctx, slots, stream):
    """Independent formulation: keep the slots in an explicit LRU order list.

    After every step the list is sorted by (last_used, slot) by construction:
    untouched slots keep their relative order at the front, and the slots touched
    this step (hits and victims, all stamped with the newest step) follow in
    ascending slot order.  Victims are the first non-hit entries of the list.
    """
    order = list(range(slots))
    tok2slot = {}
    slot2tok = [-1] * slots
    out = []
    for topk in stream:
        hits = {tok2slot[x] for x in topk if x in tok2slot}
        misses = [x for x in topk if x not in tok2slot]
        nonhit = [s for s in order if s not in hits]
        victims = nonhit[: len(misses)]
        rest = nonhit[len(misses):]
        for x, v in zip(misses, victims):
            if slot2tok[v] >= 0:
                del tok2slot[slot2tok[v]]
            slot2tok[v] = x
            tok2slot[x] = v
        order = rest + sorted(hits | set(victims))
        out.append((list(victims), list(slot2tok)))
    return out


@pytest.mark.parametrize("seed", range(25))
def test_matches_order_array_model(seed):
    rng = np.random.default_rng(100 + seed)
    n_ctx = int(rng.integers(2, 50))
    slots = int(rng.integers(1, 17))
    k = int(rng.integers(1, min(slots, n_ctx) + 1))
    width = int(rng.integers(k, n_ctx + 1))      # narrow windows give many hits
    stream = [rng.choice(width, size=k, replace=False) for _ in range(25)]
    pool = _tagged_pool(n_ctx)
    recs = run_unit(n_ctx, slots, np.array(stream), pool)
    model = order_array_model(n_ctx, slots, [list(map(int, s)) for s in stream])
    for rec, (victims, slot2tok) in zip(recs, model):
        assert rec.victims.tolist() == victims
    u = OracleUnit(n_ctx, slots, k)
    for s, (_, slot2tok) in zip(stream, model):
        u.step(s, pool)
        assert u.slot2tok.tolist() == slot2tok


@pytest.mark.parametrize("seed", range(10))
def test_invariants_and_set_algebra(seed):
    rng = np.random.default_rng(seed)
    n_ctx, slots = 64, int(rng.integers(4, 33))
    k = int(rng.integers(1, slots + 1))
    pool = rng.integers(0, 65536, size=(n_ctx, 576), dtype=np.uint16)
    u = OracleUnit(n_ctx, slots, k)
    for t in range(30):
        topk = rng.choice(int(rng.integers(k, n_ctx + 1)), size=k, replace=False)
        before = u.resident()
        lu_before = u.last_used.copy()
        rec = u.step(topk, pool)
        hits = set(topk.tolist()) & before
        misses = [int(x) for x in topk if int(x) not in before]
        # I1 and the brute-force diff
        assert rec.n_hit == len(hits) and rec.n_hit + rec.n_miss == k
        assert [int(topk[i]) for i in rec.miss_pos] == misses
        # I2: resident set update
        evicted = {int(e) for e in rec.evicted if e >= 0}
        assert u.resident() == (before | set(misses)) - evicted
        assert len(u.resident()) <= slots
        assert evicted.isdisjoint(topk.tolist())
        # I3: the two maps are mutual inverses
        for s in range(slots):
            if u.slot2tok[s] >= 0:
                assert u.tok2slot[u.slot2tok[s]] == s
        assert int((u.tok2slot >= 0).sum()) == int((u.slot2tok >= 0).sum())
        # I4: every Top-K token is resident and stamped with t
        for x in topk:
            assert u.tok2slot[x] >= 0 and u.last_used[u.tok2slot[x]] == t
        # I7: every victim sorts before every non-victim non-hit slot
        hit_slots = {int(s) for s in rec.slot_of if s >= 0}
        vic = set(rec.victims.tolist())
        others = [s for s in range(slots) if s not in hit_slots and s not in vic]
        for v in rec.victims:
            for s in others:
                assert (lu_before[v], v) < (lu_before[s], s)
        # I5 / I6: gathered rows and hot rows are the pool's bytes
        assert np.array_equal(rec.cbuf, pool[topk])
        for s in range(slots):
            if u.slot2tok[s] >= 0:
                assert np.array_equal(u.hot[s], pool[u.slot2tok[s]])


def test_cold_start_closed_form():
    n_ctx, slots, k = 100, 30, 12
    pool = _tagged_pool(n_ctx)
    u = OracleUnit(n_ctx, slots, k)
    topk = np.random.default_rng(0).choice(n_ctx, size=k, replace=False)
    rec = u.step(topk, pool)
    assert rec.n_miss == k and rec.victims.tolist() == list(range(k))
    assert (rec.evicted == -1).all()
    for i, x in enumerate(topk):
        assert u.tok2slot[x] == i


def test_repeated_topk_hits_everything():
    n_ctx, slots, k = 100, 30, 12
    pool = _tagged_pool(n_ctx)
    u = OracleUnit(n_ctx, slots, k)
    topk = np.arange(k)[::-1].copy()
    u.step(topk, pool)
    t2s, s2t = u.tok2slot.copy(), u.slot2tok.copy()
    rec = u.step(np.random.default_rng(1).permutation(topk), pool)
    assert rec.n_miss == 0 and rec.victims.size == 0
    assert np.array_equal(u.tok2slot, t2s) and np.array_equal(u.slot2tok, s2t)
    assert (u.last_used[:k] == 1).all() and (u.last_used[k:] == -1).all()


def test_buffer_holding_whole_context_never_evicts():
    n_ctx = slots = 20
    k = 7
    pool = _tagged_pool(n_ctx)
    u = OracleUnit(n_ctx, slots, k)
    rng = np.random.default_rng(3)
    first_touch = []
    for _ in range(15):
        topk = rng.choice(n_ctx, size=k, replace=False)
        rec = u.step(topk, pool)
        assert (rec.evicted == -1).all()
        for i in rec.miss_pos:
            first_touch.append(int(topk[i]))
    for s, x in enumerate(first_touch):
        assert u.slot2tok[s] == x


def test_invalid_topk_raises_and_leaves_state():
    pool = _tagged_pool(16)
    u = OracleUnit(16, 8, 4)
    u.step(np.array([1, 2, 3, 4]), pool)
    snap = (u.tok2slot.copy(), u.slot2tok.copy(), u.last_used.copy(), u.t)
    for bad in ([1, 2, 3, 16], [-1, 2, 3, 4], [5, 5, 6, 7]):
        with pytest.raises(KvsError):
            u.step(np.array(bad), pool)
        assert np.array_equal(u.tok2slot, snap[0]) and np.array_equal(u.slot2tok, snap[1])
        assert np.array_equal(u.last_used, snap[2]) and u.t == snap[3]


def test_free_then_cold_refill():
    pool = _tagged_pool(32)
    u = OracleUnit(32, 8, 4)
    for t in range(3):
        u.step(np.array([t, t + 5, t + 10, t + 20]), pool)
    u.reset()
    assert u.t == 3 and not u.resident()
    rec = u.step(np.array([1, 2, 3, 4]), pool)
    assert rec.t == 3 and rec.n_miss == 4 and rec.victims.tolist() == [0, 1, 2, 3]


# ---------------------------------------------------------------- padded Top-K

def test_golden_padded_trace_worked_by_hand():
    g = json.load(open(GOLDEN_PADDED))
    pool = _tagged_pool(g["context"])
    u = OracleUnit(g["context"], g["slots"], g["topk"])
    for st in g["steps"]:
        rec = u.step(np.array(st["topk"]), pool, padded=True)
        assert rec.t == st["t"]
        assert rec.slot_of.tolist() == st["slot_of"]
        assert rec.miss_pos.tolist() == st["miss_pos"]
        assert rec.victims.tolist() == st["victims"]
        assert rec.evicted.tolist() == st["evicted"]
        assert u.last_used.tolist() == st["last_used"]
        assert u.slot2tok.tolist() == st["slot2tok"]
        for i, src in enumerate(st["cbuf_src"]):
            if src == "z":
                assert not rec.cbuf[i].any()
            else:
                assert int(rec.cbuf[i, 0]) == st["topk"][i] + 1
                if src[0] == "h":
                    assert rec.slot_of[i] == int(src[1:])
    assert u.tok2slot.tolist() == g["final_tok2slot"]


@pytest.mark.parametrize("seed", range(20))
def test_padded_matches_order_array_model_on_valid_tokens(seed):
    # the list model knows nothing of padding: it sees only each step's valid tokens
    rng = np.random.default_rng(300 + seed)
    n_ctx = int(rng.integers(2, 50))
    slots = int(rng.integers(1, 17))
    k = int(rng.integers(1, min(slots, n_ctx) + 1))
    width = int(rng.integers(k, n_ctx + 1))
    stream = []
    for _ in range(25):
        row = rng.choice(width, size=k, replace=False).astype(np.int64)
        row[rng.random(k) < rng.choice([0.0, 0.3, 1.0])] = -1
        stream.append(row)
    pool = _tagged_pool(n_ctx)
    recs = run_unit(n_ctx, slots, np.array(stream), pool, padded=True)
    model = order_array_model(n_ctx, slots, [[int(x) for x in r if x >= 0] for r in stream])
    u = OracleUnit(n_ctx, slots, k)
    for row, rec, (victims, slot2tok) in zip(stream, recs, model):
        assert rec.victims.tolist() == victims
        assert rec.n_hit + rec.n_miss + rec.n_pad == k and rec.n_pad == int((row < 0).sum())
        assert (rec.slot_of[row < 0] == -2).all()
        assert not rec.cbuf[row < 0].any()
        assert np.array_equal(rec.cbuf[row >= 0], pool[row[row >= 0]])
        u.step(row, pool, padded=True)
        assert u.slot2tok.tolist() == slot2tok


def test_padded_without_pads_is_the_unpadded_step():
    rng = np.random.default_rng(5)
    pool = rng.integers(0, 65536, size=(60, 576), dtype=np.uint16)
    a, b = OracleUnit(60, 20, 8), OracleUnit(60, 20, 8)
    for _ in range(12):
        topk = rng.choice(40, size=8, replace=False)
        ra, rb = a.step(topk, pool), b.step(topk, pool, padded=True)
        for f in ("slot_of", "miss_pos", "victims", "evicted", "cbuf"):
            assert np.array_equal(getattr(ra, f), getattr(rb, f))
    assert np.array_equal(a.last_used, b.last_used) and np.array_equal(a.tok2slot, b.tok2slot)


def test_padded_invalid_entries_still_raise():
    pool = _tagged_pool(16)
    u = OracleUnit(16, 8, 4)
    u.step(np.array([1, -1, 3, -1]), pool, padded=True)
    snap = (u.tok2slot.copy(), u.last_used.copy(), u.t)
    for bad in ([-2, 2, 3, 4], [1, -1, 16, -1], [5, -1, 5, 7]):
        with pytest.raises(KvsError):
            u.step(np.array(bad), pool, padded=True)
        assert np.array_equal(u.tok2slot, snap[0]) and np.array_equal(u.last_used, snap[1])
        assert u.t == snap[2]
    with pytest.raises(KvsError):          # without padding, -1 is out of range
        u.step(np.array([1, -1, 3, 4]), pool)


# ---------------------------------------------------------------- append (publish of a new row)

def test_append_updates_pool_and_resident_hot_copy():
    rng = np.random.default_rng(9)
    pool = rng.integers(0, 65536, size=(32, 576), dtype=np.uint16)
    u = OracleUnit(32, 8, 4)
    u.step(np.array([3, 9, 12, 20]), pool)
    new_res = rng.integers(0, 65536, size=576, dtype=np.uint16)     # token 9: resident
    new_cold = rng.integers(0, 65536, size=576, dtype=np.uint16)    # token 30: not resident
    slot9 = int(u.tok2slot[9])
    u.append(pool, 9, new_res)
    u.append(pool, 30, new_cold)
    assert np.array_equal(pool[9], new_res) and np.array_equal(pool[30], new_cold)
    assert np.array_equal(u.hot[slot9], new_res)
    rec = u.step(np.array([9, 30, 3, 12]), pool)
    assert rec.slot_of[0] == slot9                      # served from the hot copy
    assert np.array_equal(rec.cbuf[0], new_res) and np.array_equal(rec.cbuf[1], new_cold)
    with pytest.raises(KvsError):
        u.append(pool, 32, new_res)
