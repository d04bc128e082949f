"""Parity of the HIP path (through the C ABI) with the CPU oracle on MI355X.

Bit-exact: slot lookup, sparse diff (miss positions), victims, evicted tokens,
the index maps, LRU stamps and order, the gathered compute-buffer bytes and the
hot-buffer bytes of every occupied slot.  Attention: per (step, layer,
request) max-abs <= 2e-2 and relative L2 <= 1e-2 against the float64 oracle,
and the log-sum-exp within 2e-3.

Small shapes check every unit after every step; full-size workloads check
sampled requests after every step (units are independent, so the oracle only
needs the sampled units).
"""
import numpy as np
import pytest

import kvs_workload as W
from oracle import KvsError as OracleError
from oracle import OracleUnit

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
REL_L2 = 1e-2
LSE_ABS = 2e-3


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def _pool(wl, host=None, **kw):
    import token_level_gather_amd as kvs
    return kvs.Pool(wl.batch, wl.layers, wl.context, wl.slots, wl.topk, scale=wl.scale,
                    host=host, **kw)


def _u16(t):
    torch = _torch()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Harness:
    """Drives one pool through a workload and checks sampled units each step."""

    def __init__(self, wl, steps, check_reqs, fill="all", padded=False, **pool_kw):
        import token_level_gather_amd as kvs
        torch = _torch()
        self.wl, self.steps = wl, steps
        self.check_reqs = list(check_reqs)
        self.padded = padded
        if padded:
            pool_kw["flags"] = pool_kw.get("flags", 0) | kvs.KVS_FLAG_PADDED_TOPK
        self.direct = bool(pool_kw.get("flags", 0) & kvs.KVS_FLAG_DIRECT_HOT)
        self.pool = _pool(wl, **pool_kw)
        host = self.pool.host.array
        if fill == "all":
            W.fill_pool(host, wl)
        else:   # only the checked requests need real rows; other units read whatever is there
            from concurrent.futures import ThreadPoolExecutor
            units = [(b, l) for b in self.check_reqs for l in range(wl.layers)]
            with ThreadPoolExecutor(min(16, len(units))) as ex:
                list(ex.map(lambda u: W.fill_unit_rows(host[u[0], u[1]], wl, u[0], u[1]), units))
        self.topk = W.topk_streams(wl, steps)
        if padded:
            self.topk = W.pad_topk_streams(self.topk, wl.seed)
        self.oracle = {(b, l): OracleUnit(wl.context, wl.slots, wl.topk)
                       for b in self.check_reqs for l in range(wl.layers)}
        self.out = torch.empty((wl.batch, 16, 512), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((wl.batch, 16), dtype=torch.float32, device="cuda")
        self.max_abs = 0.0
        self.max_rel = 0.0
        # oracle totals over the checked units: unit steps, hits, misses, evictions
        self.totals = np.zeros(4, dtype=np.int64)

    def device_step(self, t, l, topk=None):
        torch = _torch()
        tk = self.topk[t, l] if topk is None else topk
        q = W.queries(self.wl, l, t)
        self.q = q
        self.pool.step(l, torch.from_numpy(np.ascontiguousarray(tk)).cuda(),
                       torch.from_numpy(q.view(np.int16)).cuda(), self.out, self.lse)
        torch.cuda.synchronize()
        return tk, q

    def check(self, t, l, tk, q):
        wl = self.wl
        out = _u16(self.out)
        lse = self.lse.cpu().numpy()
        for b in self.check_reqs:
            u = self.oracle[(b, l)]
            rec = u.step(tk[b], self.pool.host.array[b, l], q[b], wl.scale, padded=self.padded)
            st = self.pool.read_state(b, l)
            n = rec.n_miss
            self.totals += [1, rec.n_hit, n, int((rec.evicted >= 0).sum())]
            tag = f"step {t} layer {l} req {b}"
            assert st["counts"].tolist() == [rec.n_hit, n, int((rec.evicted >= 0).sum()), 1], tag
            assert np.array_equal(st["slot_of"], rec.slot_of), tag
            assert np.array_equal(st["miss_pos"][:n], rec.miss_pos), tag
            assert np.array_equal(st["victims"][:n], rec.victims), tag
            assert np.array_equal(st["evicted"][:n], rec.evicted), tag
            assert np.array_equal(st["tok2slot"], u.tok2slot), tag
            assert np.array_equal(st["slot2tok"], u.slot2tok), tag
            assert np.array_equal(st["last_used"], u.last_used), tag
            order = np.lexsort((np.arange(wl.slots), u.last_used))
            assert np.array_equal(st["lru_order"], order), tag
            assert st["step"] == u.t, tag
            tkb = np.asarray(tk[b], dtype=np.int64)
            want_rs = np.where(tkb >= 0, u.tok2slot[np.maximum(tkb, 0)], -1)
            assert np.array_equal(st["row_slot"], want_rs), tag + " row_slot"
            if not self.direct:   # direct mode assembles no compute buffer
                row = wl.topk * 1152
                cbuf = _u16(self.pool.cbuf[b * row:(b + 1) * row]).reshape(wl.topk, 576)
                assert np.array_equal(cbuf, rec.cbuf), tag + " cbuf bytes"
            hrow = wl.slots * 1152
            hu = b * wl.layers + l
            hot = _u16(self.pool.hot[hu * hrow:(hu + 1) * hrow]).reshape(wl.slots, 576)
            occ = u.slot2tok >= 0
            assert np.array_equal(hot[occ], u.hot[occ]), tag + " hot bytes"
            got = _bf16_to_f64(out[b])
            if rec.n_hit + rec.n_miss == 0:   # every entry empty: zero output, lse -inf
                assert not got.any() and np.all(lse[b] == -np.inf), tag
                continue
            err = got - rec.out
            max_abs = float(np.abs(err).max())
            rel = float(np.linalg.norm(err) / np.linalg.norm(rec.out))
            assert max_abs <= MAX_ABS and rel <= REL_L2, f"{tag}: max_abs {max_abs} rel {rel}"
            assert float(np.abs(lse[b] - rec.lse).max()) <= LSE_ABS, tag + " lse"
            self.max_abs = max(self.max_abs, max_abs)
            self.max_rel = max(self.max_rel, rel)

    def run(self):
        for t in range(self.steps):
            for l in range(self.wl.layers):
                tk, q = self.device_step(t, l)
                self.check(t, l, tk, q)
        rc, stats = self.pool.sync_status()
        assert rc == 0
        if sorted(self.check_reqs) == list(range(self.wl.batch)):
            self.check_stats(stats)
        return stats

    def check_stats(self, stats):
        """The library's running totals equal the oracle's, summed over every unit."""
        got = [stats.unit_steps, stats.hits, stats.misses, stats.evictions]
        assert got == self.totals.tolist(), (got, self.totals.tolist())
        assert stats.host_bytes == 1152 * int(self.totals[2])

    def close(self):
        self.pool.release()
        self.pool.host.free()


def _case(wl, steps, reqs, fill="all", padded=False, **pool_kw):
    h = Harness(wl, steps, reqs, fill, padded, **pool_kw)
    try:
        stats = h.run()
        print(f"{wl.name}: steps {steps} max_abs {h.max_abs:.3g} max_rel {h.max_rel:.3g} "
              f"miss rate {stats.misses / max(1, stats.hits + stats.misses):.3f}", flush=True)
        return h, stats
    finally:
        h.close()


# ---------------------------------------------------------------- small shapes, every unit

def test_4k_context_single_request_all_steps():
    wl = W.WORKLOADS["ctx4k_b1_k256"]
    _case(wl, wl.steps, [0])


@pytest.mark.parametrize("shape", [
    dict(batch=3, layers=1, context=5000, slots=700, topk=300, fresh_rate=0.3),   # ragged tiles
    dict(batch=2, layers=3, context=3000, slots=1100, topk=1025, fresh_rate=0.2),  # multi-layer
    dict(batch=4, layers=1, context=900, slots=64, topk=64, fresh_rate=0.5),      # S == K
    dict(batch=2, layers=1, context=2000, slots=40, topk=1, fresh_rate=1.0),      # K == 1
    dict(batch=2, layers=1, context=130, slots=130, topk=130, fresh_rate=0.0),    # N == S == K
    dict(batch=5, layers=2, context=20000, slots=16384, topk=8192, fresh_rate=0.4),  # limits
])
def test_small_shapes_every_unit(shape):
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="small", steps=6, **shape)
    _case(wl, wl.steps, range(wl.batch))


# One shape per instantiation of the diff kernel's per-thread bounds (Top-K
# entries per thread KPT, slots per thread SPT, each a power of two; 1024
# threads): every (KPT, SPT) pair that some K <= S within the limits selects.
# Each shape evicts occupied slots in at least two of its steps.
DIFF_INSTANTIATIONS = {
    # (KPT, SPT): (K, S, N, fresh rate, steps)
    (1, 1): (1000, 1024, 6000, 0.5, 6),
    (1, 2): (700, 2000, 9000, 1.0, 6),
    (1, 4): (1024, 4000, 20000, 1.0, 7),
    (1, 8): (1024, 5000, 40000, 1.0, 8),
    (1, 16): (1024, 9500, 60000, 1.0, 12),
    (2, 2): (2048, 2048, 9000, 0.3, 5),
    (2, 4): (1500, 3000, 12000, 0.8, 5),
    (2, 8): (2048, 8192, 40000, 1.0, 7),
    (2, 16): (2048, 12000, 50000, 1.0, 9),
    (4, 4): (4096, 4096, 20000, 0.3, 5),
    (4, 8): (3000, 6000, 20000, 0.6, 6),
    (4, 16): (4096, 16384, 60000, 1.0, 7),
    (8, 8): (8192, 8192, 30000, 0.2, 5),
    (8, 16): (6000, 16000, 60000, 0.8, 6),
}


def _per_thread(n):
    x = (n + 1023) // 1024
    p = 1
    while p < x:
        p *= 2
    return p


def test_diff_instantiation_table_covers_every_pair():
    # every (KPT, SPT) pair reachable under the limits K <= S <= 16384, K <= 8192
    reach = {(_per_thread(k), _per_thread(s)) for k in range(1, 8193, 97)
             for s in range(k, 16385, 89)} | {(8, 16), (8, 8)}
    assert reach == set(DIFF_INSTANTIATIONS)
    for (kpt, spt), (k, s, n, f, steps) in DIFF_INSTANTIATIONS.items():
        assert (_per_thread(k), _per_thread(s)) == (kpt, spt) and k <= s <= n


@pytest.mark.parametrize("inst", sorted(DIFF_INSTANTIATIONS), ids=lambda x: f"kpt{x[0]}_spt{x[1]}")
def test_diff_every_instantiation_evicts(inst):
    K, S, N, f, steps = DIFF_INSTANTIATIONS[inst]
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name=f"inst{inst[0]}x{inst[1]}", batch=2,
                                                  layers=1, context=N, slots=S, topk=K,
                                                  steps=steps, fresh_rate=f)
    _, stats = _case(wl, wl.steps, range(wl.batch))
    assert stats.evictions > 0


@pytest.mark.parametrize("mode", ["default", "direct", "padded"])
def test_topk_3000_slots_6000_every_unit(mode):
    # 2048 < K <= 4096 and 4096 < S <= 8192, with evictions from the third step
    import token_level_gather_amd as kvs
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="k3000", batch=3, layers=2, context=20000,
                                                  slots=6000, topk=3000, steps=8, fresh_rate=0.4)
    flags = kvs.KVS_FLAG_DIRECT_HOT if mode == "direct" else 0
    _, stats = _case(wl, wl.steps, range(wl.batch), padded=mode == "padded", flags=flags)
    assert stats.evictions > 0


# ---------------------------------------------------------------- separate launches

@pytest.mark.parametrize("mode", ["default", "direct", "padded", "padded_direct"])
@pytest.mark.parametrize("shape", [
    dict(batch=3, layers=1, context=5000, slots=700, topk=300, fresh_rate=0.3),
    dict(batch=2, layers=3, context=3000, slots=1100, topk=1025, fresh_rate=0.2),
    dict(batch=3, layers=2, context=20000, slots=6000, topk=3000, fresh_rate=0.4),
    # more tiles than 256 workgroups: shares of 3 and 2 tiles cross request
    # boundaries (17 x 32 tiles on 182 workgroups; 9 x 33 on 149, a 52-token last tile)
    dict(batch=17, layers=1, context=6000, slots=2100, topk=2048, fresh_rate=0.3),
    dict(batch=9, layers=1, context=5000, slots=2200, topk=2100, fresh_rate=0.25),
], ids=["k300", "k1025_l3", "k3000", "b17_k2048", "b9_k2100"])
def test_separate_attention_every_unit(shape, mode):
    # gather, attention over the complete compute buffer and merge as separate
    # launches: the same results as the assembling launch, checked the same way.
    # The gather's two host-read forms both run: k300 and k1025_l3 have few
    # fetch workgroups with misses (every read of a pass issued at once), k3000,
    # b17 and b9 enough for one read per thread (0.45-1.1 MB in flight).
    import token_level_gather_amd as kvs
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="separate", steps=6, **shape)
    flags = kvs.KVS_FLAG_SEPARATE_ATTENTION | (_direct() if "direct" in mode else 0)
    _case(wl, wl.steps, range(wl.batch), padded="padded" in mode, flags=flags)


@pytest.mark.parametrize("mode", ["default", "separate"])
def test_batch_above_256_every_unit(mode):
    # 300 requests: more diff workgroups and merge rows than CUs, one fetch and
    # one hit workgroup per request in the assembling launch (600 in all), and
    # the separate attention's 600 tiles shared by 200 workgroups across
    # request boundaries
    import token_level_gather_amd as kvs
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="b300", batch=300, layers=1, context=1500,
                                                slots=300, topk=128, steps=4, fresh_rate=0.3)
    flags = kvs.KVS_FLAG_SEPARATE_ATTENTION if mode == "separate" else 0
    _case(wl, wl.steps, range(wl.batch), flags=flags)


@pytest.mark.parametrize("topk,splits", [
    (300, 1),    # 5 tiles in one split: two full pairs and an odd tail
    (300, 2),    # 2 + 3 tiles
    (300, 5),    # one tile per split (no full pair, tail only)
    (1025, 4),   # 4, 4, 4, 5 tiles: even splits and a ragged last tile
    (1025, 17),  # every split a single tile, the last one a 1-token tile
])
def test_attention_split_counts(topk, splits):
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="splits", batch=3, context=4000,
                                                  slots=1100, topk=topk, steps=3,
                                                  fresh_rate=0.3)
    h, _ = _case(wl, wl.steps, range(wl.batch), attn_splits=splits)
    assert h.pool.sizes.attn_splits == splits


@pytest.mark.parametrize("shape", [
    dict(batch=4, layers=1, context=3000, slots=700, topk=300, fresh_rate=0.3),
    dict(batch=8, layers=2, context=5000, slots=1100, topk=1025, fresh_rate=0.2),
    dict(batch=4, layers=1, context=200, slots=64, topk=64, fresh_rate=0.5),
])
def test_padded_topk_every_unit(shape):
    # requests cycle through tail / scatter / all-empty / no padding
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="padded", steps=6, **shape)
    _case(wl, wl.steps, range(wl.batch), padded=True)


@pytest.mark.parametrize("fetch_blocks,splits", [
    (1, 1),      # fewer fetch workgroups than requests: still one per request
    (3, 2),      # one per request
    (64, 17),    # capped at ceil(K / 64) = 17 per request; many hit splits with no tile
    (7, 5),      # 3 per request; passes x, x + 3, ...
])
def test_assemble_fetch_and_hit_counts(fetch_blocks, splits):
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="assemble_counts", batch=3, context=4000,
                                                  slots=1100, topk=1025, steps=5,
                                                  fresh_rate=0.6)
    h, _ = _case(wl, wl.steps, range(wl.batch), fetch_blocks=fetch_blocks, attn_splits=splits)
    assert h.pool.sizes.attn_splits == splits


def test_padded_topk_explicit_splits():
    # whole tiles and whole splits of empty entries (tail padding, 4 splits)
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="padded_splits", batch=4, context=5000,
                                                  slots=1100, topk=1025, steps=5,
                                                  fresh_rate=0.3)
    _case(wl, wl.steps, range(wl.batch), padded=True, attn_splits=4)


# ---------------------------------------------------------------- rows read in place

@pytest.mark.parametrize("mode", ["default", "direct", "padded", "more_fetch"])
def test_steps_without_misses_every_unit(mode):
    # Steps whose Top-K is all resident (the previous step's set, reordered):
    # every request has no miss, so its fetch workgroups take shares of the
    # hit tiles in the assembling launch.  Normal steps before and after.
    import token_level_gather_amd as kvs
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="all_hit", batch=3, layers=2, context=3000,
                                                  slots=800, topk=300, steps=8, fresh_rate=0.3)
    kw = {}
    if mode == "direct":
        kw["flags"] = kvs.KVS_FLAG_DIRECT_HOT
    if mode == "more_fetch":   # more fetch than hit workgroups per request
        kw.update(fetch_blocks=15, attn_splits=2)
    h = Harness(wl, wl.steps, range(wl.batch), padded=mode == "padded", **kw)
    rng = np.random.default_rng(7)
    try:
        for t in range(wl.steps):
            for l in range(wl.layers):
                tk = h.topk[t, l]
                if t in (3, 4, 6):   # the previous step's Top-K in a new order
                    prev = h.topk[t - 1, l]
                    tk = np.stack([prev[b][rng.permutation(wl.topk)] for b in range(wl.batch)])
                    h.topk[t, l] = tk
                tk, q = h.device_step(t, l, topk=tk)
                h.check(t, l, tk, q)
                if t in (3, 4, 6):
                    for b in range(wl.batch):
                        assert h.pool.read_state(b, l)["counts"][1] == 0   # no miss
        rc, stats = h.pool.sync_status()
        assert rc == 0
        h.check_stats(stats)
    finally:
        h.close()


def test_probe_hit_copy_copies_only_the_hit_rows():
    # kvs_probe_hit_copy (measurement helper) repeats the index copy of the
    # last step's hits: hit rows of the compute buffer equal their hot rows
    # again, miss rows are left alone and empty entries get zero rows; it
    # refuses a pool that has run no step and one without compute buffer
    import token_level_gather_amd as kvs
    torch = _torch()
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="probe", batch=3, layers=2, context=3000,
                                                  slots=800, topk=300, steps=3, fresh_rate=0.3)
    h = Harness(wl, wl.steps, range(wl.batch), padded=True)
    try:
        with pytest.raises(kvs.KvsError):
            h.pool.probe_hit_copy(0)
        for t in range(wl.steps):
            for l in range(wl.layers):
                h.check(t, l, *h.device_step(t, l))
        l = wl.layers - 1
        row = wl.topk * 576
        before = _u16(h.pool.cbuf[:wl.batch * row * 2]).reshape(wl.batch, wl.topk, 576)
        h.pool.cbuf[:wl.batch * row * 2].fill_(0x5a)
        h.pool.probe_hit_copy(l)
        torch.cuda.synchronize()
        after = _u16(h.pool.cbuf[:wl.batch * row * 2]).reshape(wl.batch, wl.topk, 576)
        for b in range(wl.batch):
            slot_of = h.pool.read_state(b, l)["slot_of"]
            hit = slot_of >= 0
            assert np.array_equal(after[b][hit], before[b][hit])
            assert np.all(after[b][slot_of == -1] == 0x5a5a)   # misses: untouched
            assert np.all(after[b][slot_of == -2] == 0)        # empty entries: zero rows
        with pytest.raises(kvs.KvsError):
            h.pool.probe_hit_copy(wl.layers)
    finally:
        h.close()
    d = Harness(wl, 1, [0], flags=kvs.KVS_FLAG_DIRECT_HOT)
    try:
        d.check(0, 0, *d.device_step(0, 0))
        with pytest.raises(kvs.KvsError):
            d.pool.probe_hit_copy(0)
    finally:
        d.close()


def _direct():
    import token_level_gather_amd as kvs
    return kvs.KVS_FLAG_DIRECT_HOT


@pytest.mark.parametrize("shape", [
    dict(batch=3, layers=1, context=5000, slots=700, topk=300, fresh_rate=0.3),
    dict(batch=2, layers=3, context=3000, slots=1100, topk=1025, fresh_rate=0.2),
    dict(batch=2, layers=1, context=2000, slots=40, topk=1, fresh_rate=1.0),
    dict(batch=5, layers=2, context=20000, slots=16384, topk=8192, fresh_rate=0.4),
])
def test_direct_hot_every_unit(shape):
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="direct", steps=6, **shape)
    _case(wl, wl.steps, range(wl.batch), flags=_direct())


@pytest.mark.parametrize("splits", [1, 5])
def test_direct_hot_padded(splits):
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="direct_padded", batch=8, layers=2,
                                                  context=5000, slots=1100, topk=300, steps=5,
                                                  fresh_rate=0.3)
    _case(wl, wl.steps, range(wl.batch), padded=True, flags=_direct(), attn_splits=splits)


def test_zipf_stream_small():
    wl = W.WORKLOADS["ctx128k_b32_l8_zipf"].shrunk(batch=3, layers=2, context=20000, steps=6)
    _case(wl, wl.steps, range(wl.batch))


# ---------------------------------------------------------------- lifecycle and errors

@pytest.mark.parametrize("direct", [False, True])
def test_free_request_then_cold_refill(direct):
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(batch=3, context=4000, slots=600, topk=256,
                                                  steps=8)
    h = Harness(wl, wl.steps, range(3), flags=_direct() if direct else 0)
    try:
        for t in range(4):
            h.check(t, 0, *h.device_step(t, 0))
        h.pool.free_request(1)
        h.oracle[(1, 0)].reset()
        for t in range(4, 8):
            h.check(t, 0, *h.device_step(t, 0))
        st = h.pool.read_state(1, 0)
        assert st["step"] == 8
    finally:
        h.close()


@pytest.mark.parametrize("direct", [False, True])
@pytest.mark.parametrize("padded", [False, True])
@pytest.mark.parametrize("kind", ["range", "negative", "duplicate"])
def test_invalid_topk_leaves_request_untouched(kind, padded, direct):
    # with padding only -1 is empty: -5 stays out of range, and a token repeated
    # beside empty entries is still a duplicate
    import token_level_gather_amd as kvs
    torch = _torch()
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(batch=3, context=3000, slots=500, topk=200,
                                                  steps=6)
    h = Harness(wl, wl.steps, range(3), padded=padded, flags=_direct() if direct else 0)
    try:
        for t in range(2):
            h.check(t, 0, *h.device_step(t, 0))
        before = h.pool.read_state(1, 0)
        bad = h.topk[2, 0].copy()
        if kind == "range":
            bad[1, 17] = wl.context
        elif kind == "negative":
            bad[1, 0] = -5
        else:
            src = int(np.flatnonzero(bad[1] >= 0)[0])
            bad[1, (src + 9) % wl.topk] = bad[1, src]
        with pytest.raises(OracleError):
            h.oracle[(1, 0)].step(bad[1], h.pool.host.array[1, 0], padded=padded)
        h.device_step(2, 0, topk=bad)
        rc, _ = h.pool.sync_status()
        assert rc == (kvs.KVS_EDUP if kind == "duplicate" else kvs.KVS_ERANGE)
        after = h.pool.read_state(1, 0)
        for key in ("tok2slot", "slot2tok", "last_used", "lru_order", "step"):
            assert np.array_equal(np.asarray(before[key]), np.asarray(after[key])), key
        assert after["counts"][3] == 0
        assert not torch.any(h.out[1].float() != 0).item()
        assert torch.isinf(h.lse[1]).all().item()
        # the other requests took the step normally
        for b in (0, 2):
            rec = h.oracle[(b, 0)].step(bad[b], h.pool.host.array[b, 0], padded=padded)
            assert np.array_equal(h.pool.read_state(b, 0)["slot2tok"], h.oracle[(b, 0)].slot2tok)
            assert rec.t == 2
        # the status was cleared and the request continues from its old state
        assert h.pool.sync_status()[0] == 0
        h.check_reqs = [1]
        h.check(3, 0, *h.device_step(3, 0))
    finally:
        h.close()


# ---------------------------------------------------------------- full-size workloads, sampled

@pytest.mark.parametrize("name,reqs", [
    ("ctx16k_b64_k2048", [0, 37, 63]),
    ("ctx16k_b192_k2048_f20", [0, 191]),
    ("ctx16k_b192_k2048_f40", [5, 100]),
])
def test_full_size_16k_sampled(name, reqs):
    wl = W.WORKLOADS[name]
    _case(wl, wl.steps, reqs, fill="checked")


def test_full_size_16k_direct_hot_sampled():
    wl = W.WORKLOADS["ctx16k_b64_k2048"]
    _case(wl, wl.steps, [1, 40, 62], fill="checked", flags=_direct())


@pytest.mark.parametrize("name,reqs,steps", [
    ("ctx128k_b32_l8_zipf", [0, 31], 16),   # every step; evictions from step ~7
    # the workload's 16 steps plus 8: with 8192 slots and ~410 fresh tokens a
    # step, occupied slots are first evicted at step 15
    ("ctx1m_b4_l4", [0, 3], 24),
])
def test_full_size_long_context_sampled(name, reqs, steps):
    wl = W.WORKLOADS[name]
    h, stats = _case(wl, steps, reqs, fill="checked")
    assert h.totals[3] > 0, "the sampled units never evicted an occupied slot"
    assert stats.evictions > 0


def test_publish_rows_then_fetch():
    """Lifecycle "publish": rows written with kvs_publish are what later misses fetch."""
    import token_level_gather_amd as kvs
    torch = _torch()
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(batch=2, layers=2, context=3000, slots=400,
                                                  topk=200, steps=6, fresh_rate=0.5)
    h = Harness(wl, wl.steps, range(2))
    try:
        for t in range(2):
            for l in range(wl.layers):
                h.check(t, l, *h.device_step(t, l))
        rng = np.random.default_rng(7)
        published = {}
        for b in range(2):
            for l in range(wl.layers):
                resident = set(h.oracle[(b, l)].resident())
                free = [x for x in range(wl.context) if x not in resident]
                start = int(rng.choice(free[: len(free) - 40]))
                n = 1
                while n < 32 and start + n not in resident and start + n < wl.context:
                    n += 1
                rows = W.f32_to_bf16_bits(rng.standard_normal((n, 576)).astype(np.float32))
                h.pool.publish(b, l, start, rows)
                assert np.array_equal(h.pool.host.array[b, l, start:start + n], rows)
                # make the next step select the first published token (a miss)
                if start not in h.topk[2, l, b]:
                    h.topk[2, l, b, 0] = start
                published[(b, l)] = (start, rows[0])
        # the next step fetches the published bytes
        for l in range(wl.layers):
            h.check(2, l, *h.device_step(2, l))
            row = wl.topk * 1152
            for b in range(2):
                start, first = published[(b, l)]
                pos = int(np.flatnonzero(h.topk[2, l, b] == start)[0])
                got = h.pool.cbuf[b * row:(b + 1) * row].view(torch.int16).cpu().numpy()
                assert np.array_equal(got.view(np.uint16).reshape(wl.topk, 576)[pos], first)
        for t in range(3, wl.steps):
            for l in range(wl.layers):
                h.check(t, l, *h.device_step(t, l))
        for bad in ((2, 0, 0, 1), (0, 2, 0, 1), (0, 0, -1, 1), (0, 0, wl.context - 1, 2)):
            with pytest.raises(kvs.KvsError):
                h.pool.publish(bad[0], bad[1], bad[2], np.zeros((bad[3], 576), np.uint16))
    finally:
        h.close()


# ---------------------------------------------------------------- device-side publish

def _bf16_rows(rng, n):
    return W.f32_to_bf16_bits(rng.standard_normal((n, 576)).astype(np.float32))


@pytest.mark.parametrize("direct", [False, True])
def test_append_rows_then_hit_and_fetch(direct):
    # one new row per request: a token resident in the hot buffer (the next
    # step hits it and must read the new bytes from the hot copy), a token that
    # is not (the next step fetches it from the pool), and two requests with
    # nothing to append
    torch = _torch()
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="append", batch=4, layers=2, context=3000,
                                                  slots=400, topk=200, steps=6, fresh_rate=0.3)
    h = Harness(wl, wl.steps, range(wl.batch), flags=_direct() if direct else 0)
    try:
        for t in range(2):
            for l in range(wl.layers):
                h.check(t, l, *h.device_step(t, l))
        rng = np.random.default_rng(77)
        host = h.pool.host.array
        for l in range(wl.layers):
            st0, st1 = h.pool.read_state(0, l), h.pool.read_state(1, l)
            res_tok = next(int(x) for x in h.topk[2, l, 0] if st0["tok2slot"][x] >= 0)
            cold_tok = next(int(x) for x in h.topk[2, l, 1] if st1["tok2slot"][x] < 0)
            rows = _bf16_rows(rng, wl.batch)
            pos = np.array([res_tok, cold_tok, -1, -1], dtype=np.int64)
            before = host[2:, l].copy()
            h.pool.append(l, torch.from_numpy(rows.view(np.int16)).cuda(),
                          torch.from_numpy(pos).cuda())
            torch.cuda.synchronize()
            assert np.array_equal(host[0, l, res_tok], rows[0])
            assert np.array_equal(host[1, l, cold_tok], rows[1])
            assert np.array_equal(host[2:, l], before)
            slot = int(st0["tok2slot"][res_tok])
            hrow = wl.slots * 1152
            hot0 = _u16(h.pool.hot[l * hrow:(l + 1) * hrow]).reshape(wl.slots, 576)
            assert np.array_equal(hot0[slot], rows[0])
            h.oracle[(0, l)].append(host[0, l], res_tok, rows[0])
            h.oracle[(1, l)].append(host[1, l], cold_tok, rows[1])
        for t in range(2, wl.steps):
            for l in range(wl.layers):
                h.check(t, l, *h.device_step(t, l))
        rc, _ = h.pool.sync_status()
        assert rc == 0
        # out-of-range positions: nothing written, KVS_ERANGE latched
        snap = host[:, 0].copy()
        bad = np.array([wl.context, -2, -1, -1], dtype=np.int64)
        h.pool.append(0, torch.from_numpy(_bf16_rows(rng, wl.batch).view(np.int16)).cuda(),
                      torch.from_numpy(bad).cuda())
        import token_level_gather_amd as kvs
        rc, _ = h.pool.sync_status()
        assert rc == kvs.KVS_ERANGE
        assert np.array_equal(host[:, 0], snap)
    finally:
        h.close()


def test_publish_device_rows_then_fetch():
    torch = _torch()
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="publish_dev", batch=2, layers=2,
                                                  context=3000, slots=400, topk=200, steps=3,
                                                  fresh_rate=0.3)
    h = Harness(wl, wl.steps, range(wl.batch))
    try:
        rng = np.random.default_rng(78)
        rows = _bf16_rows(rng, 50)
        h.pool.publish_device(1, 1, 1000, torch.from_numpy(rows.view(np.int16)).cuda())
        torch.cuda.synchronize()
        assert np.array_equal(h.pool.host.array[1, 1, 1000:1050], rows)
        # step 0 of unit (1, 1) selects all 50 published tokens
        row = h.topk[0, 1, 1]
        keep = [int(x) for x in row if not 1000 <= x < 1050][: wl.topk - 50]
        h.topk[0, 1, 1] = np.array(list(range(1000, 1050)) + keep, dtype=np.int32)
        h.run()
    finally:
        h.close()


# ---------------------------------------------------------------- optional outputs, empty starts

def test_step_without_lse_matches_step_with_it():
    # two pools on the same host rows and inputs: lse = NULL must not change out
    import token_level_gather_amd as kvs
    torch = _torch()
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="nolse", batch=3, context=3000, slots=500,
                                                  topk=200, steps=4, fresh_rate=0.3)
    host = kvs.HostPool(wl.batch, wl.layers, wl.context)
    W.fill_pool(host.array, wl)
    pa = _pool(wl, host=host)
    pb = _pool(wl, host=host)
    try:
        topk = W.topk_streams(wl)
        out_a = torch.empty((wl.batch, 16, 512), dtype=torch.bfloat16, device="cuda")
        out_b = torch.empty_like(out_a)
        lse = torch.empty((wl.batch, 16), dtype=torch.float32, device="cuda")
        for t in range(wl.steps):
            tk = torch.from_numpy(topk[t, 0]).cuda()
            q = torch.from_numpy(W.queries(wl, 0, t).view(np.int16)).cuda()
            pa.step(0, tk, q, out_a, lse)
            pb.step(0, tk, q, out_b)
            torch.cuda.synchronize()
            assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), t
        assert pa.sync_status()[0] == 0 and pb.sync_status()[0] == 0
    finally:
        pa.release()
        pb.release()
        host.free()


@pytest.mark.parametrize("direct", [False, True])
def test_padded_request_starting_empty(direct):
    # request 0 has no entry at all on its first two steps, then ragged tails:
    # its running max starts from -inf in every split
    import token_level_gather_amd as kvs
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="empty_start", batch=3, context=4000,
                                                  slots=700, topk=300, steps=5, fresh_rate=0.3)
    flags = kvs.KVS_FLAG_DIRECT_HOT if direct else 0
    h = Harness(wl, wl.steps, range(wl.batch), padded=True, flags=flags)
    try:
        h.topk[0:2, :, 0, :] = -1
        h.topk[2, :, 0, 250:] = -1
        h.topk[3, :, 0, 1:] = -1
        h.run()
    finally:
        h.close()


# ---------------------------------------------------------------- measurement helper

def test_host_read_probe_reads_every_byte():
    # the probe's per-thread XOR fold, recomputed from the host bytes: thread t
    # folds the 16-byte chunks t, t + 65536, ... of the buffer
    import token_level_gather_amd as kvs
    torch = _torch()
    host = kvs.HostPool(1, 1, 3000)   # 3000 rows x 1152 B: 216,000 chunks, a ragged last pass
    try:
        rng = np.random.default_rng(11)
        host.array[...] = rng.integers(0, 65536, size=host.array.shape, dtype=np.uint16)
        sink = torch.empty(kvs.PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
        kvs.probe_host_read(host.ptr, host.nbytes, sink)
        torch.cuda.synchronize()
        words = host.array.reshape(-1).view(np.uint32).reshape(-1, 4)
        per_chunk = np.bitwise_xor.reduce(words, axis=1)
        n = per_chunk.size
        pad = (-n) % kvs.PROBE_SINK_WORDS
        folded = np.bitwise_xor.reduce(
            np.concatenate([per_chunk, np.zeros(pad, np.uint32)]).reshape(-1, kvs.PROBE_SINK_WORDS),
            axis=0)
        assert np.array_equal(sink.cpu().numpy().view(np.uint32), folded)
    finally:
        host.free()


def test_pool_context_manager_releases_and_frees_its_host_pool():
    import token_level_gather_amd as kvs
    torch = _torch()
    wl = W.WORKLOADS["ctx4k_b1_k256"]
    with kvs.Pool(wl.batch, wl.layers, wl.context, wl.slots, wl.topk, scale=wl.scale) as pool:
        W.fill_pool(pool.host.array, wl)
        out = torch.empty((1, 16, 512), dtype=torch.bfloat16, device="cuda")
        tk = torch.from_numpy(W.topk_streams(wl, 1)[0, 0]).cuda()
        q = torch.from_numpy(W.queries(wl, 0, 0).view(np.int16)).cuda()
        pool.step(0, tk, q, out)
        assert pool.sync_status()[0] == 0
    assert pool.handle is None and pool.host.ptr is None


# ---------------------------------------------------------------- state checker

@pytest.mark.parametrize("case", ["small", "padded", "direct", "zipf", "free_refill"])
def test_state_check_passes_on_valid_runs(case):
    import token_level_gather_amd as kvs
    base = W.WORKLOADS["ctx16k_b64_k2048"]
    flags = kvs.KVS_FLAG_CHECK | (kvs.KVS_FLAG_DIRECT_HOT if case == "direct" else 0)
    if case == "zipf":
        wl = W.WORKLOADS["ctx128k_b32_l8_zipf"].shrunk(batch=3, layers=2, context=20000, steps=5)
    else:
        wl = base.shrunk(name="check", batch=3, layers=2, context=4000, slots=500, topk=300,
                         steps=6, fresh_rate=0.4)
    h = Harness(wl, wl.steps, range(wl.batch), padded=case == "padded", flags=flags)
    try:
        if case == "free_refill":
            for t in range(3):
                for l in range(wl.layers):
                    h.check(t, l, *h.device_step(t, l))
            h.pool.free_request(1)
            for l in range(wl.layers):
                h.oracle[(1, l)].reset()
            for t in range(3, wl.steps):
                for l in range(wl.layers):
                    h.check(t, l, *h.device_step(t, l))
            assert h.pool.sync_status()[0] == 0
        else:
            h.run()   # asserts a clean status at the end
    finally:
        h.close()


def _meta_offsets(pool):
    # byte offsets of the per-unit arrays inside the pool's meta buffer: the
    # library lays out tok2slot [U][N] int32, slot2tok [U][Sp] int32, last_used
    # [U][Sp] int32 and the LRU order [U][Sp] uint16 in that order, each
    # 256-byte aligned, with Sp = S rounded up to 16 (white-box knowledge, used
    # only to corrupt state on purpose)
    def up(x):
        return (x + 255) // 256 * 256
    U = pool.B * pool.L
    t2s = 0
    s2t = up(t2s + U * pool.N * 4)
    lu = up(s2t + U * _slot_stride(pool.S) * 4)
    order = up(lu + U * _slot_stride(pool.S) * 4)
    return s2t, lu, order


def _slot_stride(slots):
    """Entries between two units' slot arrays in the meta buffer (white-box)."""
    return (slots + 15) // 16 * 16


@pytest.mark.parametrize("what", ["maps", "order"])
def test_state_check_catches_corruption(what):
    import token_level_gather_amd as kvs
    torch = _torch()
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="corrupt", batch=2, context=3000, slots=400,
                                                  topk=200, steps=3, fresh_rate=0.3)
    h = Harness(wl, wl.steps, [0], flags=kvs.KVS_FLAG_CHECK)
    try:
        h.device_step(0, 0)
        assert h.pool.sync_status()[0] == 0
        st = h.pool.read_state(0, 0)
        assert np.array_equal(np.sort(st["lru_order"]), np.arange(wl.slots))
        s2t_off, _, order_off = _meta_offsets(h.pool)
        if what == "maps":   # two occupied slots swap tokens: the maps stop being inverses
            occ = np.flatnonzero(st["slot2tok"] >= 0)[:2]
            w = h.pool.meta[s2t_off:s2t_off + wl.slots * 4].view(torch.int32)
            a, b = int(occ[0]), int(occ[1])
            w[a], w[b] = int(st["slot2tok"][b]), int(st["slot2tok"][a])
        else:                # the oldest and the newest order entries swap places
            o = h.pool.meta[order_off:order_off + wl.slots * 2].view(torch.int16)
            first, last = int(st["lru_order"][0]), int(st["lru_order"][-1])
            o[0], o[wl.slots - 1] = last, first
        torch.cuda.synchronize()
        h.device_step(0, 0)   # the same Top-K again: every entry hits, nothing is evicted
        assert h.pool.sync_status()[0] == kvs.KVS_ECORRUPT
    finally:
        h.close()


# ---------------------------------------------------------------- random small configurations

@pytest.mark.parametrize("seed", range(16))
def test_random_small_configs_every_unit(seed):
    # seeded draws of shape, miss rate, padding, direct mode, split count and
    # workgroup order; every unit checked against the oracle after every step
    import token_level_gather_amd as kvs
    rng = np.random.default_rng(9000 + seed)
    K = int(rng.choice([1, 7, 64, 65, 200, 513, 1024, 3000, 4096]))
    S = int(K + rng.integers(0, 3 * K + 64))
    S = min(S, 8192 if K > 1024 else 16384)   # the slot limit; large K stays under 8192
    N = int(max(S, K) + rng.integers(0, 4000))
    B = int(rng.integers(1, 6))
    L = int(rng.integers(1, 3))
    ntiles = (K + 63) // 64
    splits = int(rng.integers(1, min(ntiles, 64) + 1)) if rng.random() < 0.5 else 0
    flags = 0
    if rng.random() < 0.5:
        flags |= kvs.KVS_FLAG_DIRECT_HOT
    if rng.random() < 0.3:
        flags |= kvs.KVS_FLAG_HITS_FIRST
    if rng.random() < 0.3:
        flags |= kvs.KVS_FLAG_SEPARATE_ATTENTION
    padded = bool(rng.random() < 0.4)
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(
        name=f"rand{seed}", batch=B, layers=L, context=N, slots=S, topk=K, steps=4,
        fresh_rate=float(rng.choice([0.0, 0.2, 0.6, 1.0])), seed=20261300 + seed)
    print(f"random config {seed}: B={B} L={L} N={N} S={S} K={K} splits={splits} "
          f"flags={flags} padded={padded} fresh={wl.fresh_rate}", flush=True)
    _case(wl, wl.steps, range(B), padded=padded, flags=flags, attn_splits=splits)


@pytest.mark.parametrize("separate", [False, True])
@pytest.mark.parametrize("direct", [False, True])
def test_invalid_topk_single_split_writes_zero_output(direct, separate):
    # one split: with separate launches the attention writes out / lse itself
    # (no combine), also for a request whose Top-K is rejected
    import token_level_gather_amd as kvs
    torch = _torch()
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(batch=3, context=3000, slots=500, topk=200,
                                                  steps=4)
    flags = (_direct() if direct else 0) | (kvs.KVS_FLAG_SEPARATE_ATTENTION if separate else 0)
    h = Harness(wl, wl.steps, range(3), attn_splits=1, flags=flags)
    try:
        assert h.pool.sizes.attn_splits == 1
        for t in range(2):
            h.check(t, 0, *h.device_step(t, 0))
        bad = h.topk[2, 0].copy()
        bad[1, 5] = wl.context
        h.out.fill_(1.0)
        h.lse.fill_(1.0)
        h.device_step(2, 0, topk=bad)
        assert h.pool.sync_status()[0] == kvs.KVS_ERANGE
        assert not torch.any(h.out[1].float() != 0).item()
        assert torch.isinf(h.lse[1]).all().item() and (h.lse[1] < 0).all().item()
        for b in (0, 2):   # the valid requests were finished by the attention itself
            rec = h.oracle[(b, 0)].step(bad[b], h.pool.host.array[b, 0], h.q[b], wl.scale)
            got = _bf16_to_f64(_u16(h.out)[b])
            assert np.abs(got - rec.out).max() <= MAX_ABS
        h.check_reqs = [1]
        h.check(3, 0, *h.device_step(3, 0))
    finally:
        h.close()


# ---------------------------------------------------------------- host-checked arguments

def test_step_rejects_misaligned_pointers_before_any_work():
    # q and out are accessed in 16-byte vectors, topk and lse as 4-byte words:
    # a misaligned pointer is rejected on the host and nothing is enqueued
    import ctypes

    import token_level_gather_amd as kvs
    torch = _torch()
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(batch=2, context=3000, slots=500, topk=200,
                                                  steps=2)
    h = Harness(wl, wl.steps, range(2))
    try:
        lib = kvs.lib()
        B, K = wl.batch, wl.topk
        tk = torch.from_numpy(h.topk[0, 0]).cuda()
        q = torch.from_numpy(W.queries(wl, 0, 0).view(np.int16)).cuda()
        raw_tk = torch.empty(B * K + 4, dtype=torch.int32, device="cuda")
        raw_tk[1:1 + B * K].copy_(tk.view(-1))
        raw_q = torch.empty(B * 16 * 576 * 2 + 64, dtype=torch.uint8, device="cuda")
        raw_out = torch.empty(B * 16 * 512 * 2 + 64, dtype=torch.uint8, device="cuda")
        raw_lse = torch.empty(B * 16 * 4 + 64, dtype=torch.uint8, device="cuda")
        s = torch.cuda.current_stream().cuda_stream
        good = (tk.data_ptr(), q.data_ptr(), h.out.data_ptr(), h.lse.data_ptr())
        bad_cases = {
            "topk+4 is aligned": None,
            "topk+2": (tk.data_ptr() + 2, good[1], good[2], good[3]),
            "q+8": (good[0], raw_q.data_ptr() + 8, good[2], good[3]),
            "q+2": (good[0], raw_q.data_ptr() + 2, good[2], good[3]),
            "out+8": (good[0], good[1], raw_out.data_ptr() + 8, good[3]),
            "out+2": (good[0], good[1], raw_out.data_ptr() + 2, good[3]),
            "lse+2": (good[0], good[1], good[2], raw_lse.data_ptr() + 2),
        }
        for name, args in bad_cases.items():
            if args is None:
                continue
            rc = lib.kvs_step(h.pool.handle, 0, args[0], args[1], args[2], args[3], s)
            assert rc == kvs.KVS_EINVAL, name
            g = ctypes.c_void_p()
            rc = lib.kvs_graph_capture(h.pool.handle, 0, args[0], args[1], args[2], args[3],
                                       ctypes.byref(g))
            assert rc == kvs.KVS_EINVAL and g.value is None, name
        torch.cuda.synchronize()
        assert h.pool.read_state(0, 0)["step"] == 0, "a rejected call enqueued work"
        # an offset that keeps the alignment is accepted: topk at +4 bytes
        rc = lib.kvs_step(h.pool.handle, 0, raw_tk.data_ptr() + 4, good[1], good[2], good[3], s)
        assert rc == kvs.KVS_OK
        torch.cuda.synchronize()
        assert h.pool.sync_status()[0] == 0
        h.check_reqs = [0, 1]
        rec = h.oracle[(0, 0)].step(h.topk[0, 0, 0], h.pool.host.array[0, 0])
        assert np.array_equal(h.pool.read_state(0, 0)["slot2tok"], h.oracle[(0, 0)].slot2tok)
        assert rec.t == 0
    finally:
        h.close()


def test_create_pool_rejects_host_memory_and_short_allocations():
    import ctypes

    import token_level_gather_amd as kvs
    torch = _torch()
    lib = kvs.lib()
    cfg = kvs.make_config(batch=1, layers=1, context=4096, slots=512, topk=256)
    sz = kvs.query_sizes(cfg)
    host = kvs.HostPool(1, 1, 4096)
    try:
        def dev(n):
            return torch.empty(int(n) + 256, dtype=torch.uint8, device="cuda")
        hot, meta, cbuf, scr = dev(sz.hot_bytes), dev(sz.meta_bytes), dev(sz.cbuf_bytes), \
            dev(sz.scratch_bytes)
        ok = [host.ptr, hot.data_ptr(), meta.data_ptr(), cbuf.data_ptr(), scr.data_ptr()]
        caps = [host.nbytes, hot.numel(), meta.numel(), cbuf.numel(), scr.numel()]
        s = torch.cuda.current_stream().cuda_stream

        def create(ptrs, capacity):
            handle = ctypes.c_void_p()
            bufs = kvs.kvs_buffers(*ptrs, *capacity)
            rc = lib.kvs_create_pool(ctypes.byref(cfg), ctypes.byref(bufs), s,
                                     ctypes.byref(handle))
            if rc == kvs.KVS_OK:
                assert lib.kvs_release(handle) == kvs.KVS_OK
            else:
                assert handle.value is None
            return rc

        assert create(ok, caps) == kvs.KVS_OK
        # pinned host memory (GPU-addressable, but not device memory) as a device buffer
        for i in (1, 2, 3, 4):
            ptrs = list(ok)
            ptrs[i] = host.ptr
            assert create(ptrs, caps) == kvs.KVS_EINVAL, i
        # a device pointer 4 KiB before the end of its allocation (the caching
        # allocator's segment, one hipMalloc): the pool's hot buffer does not fit
        seg = next(sg for sg in torch.cuda.memory_snapshot()
                   if sg["address"] <= hot.data_ptr() < sg["address"] + sg["total_size"])
        near_end = seg["address"] + seg["total_size"] - 4096
        ptrs = list(ok)
        ptrs[1] = near_end
        assert create(ptrs, caps) == kvs.KVS_ENOMEM
    finally:
        host.free()


@pytest.mark.parametrize("bad_slot", ["past_end", "below_minus_one"])
def test_corrupt_map_entry_latches_ecorrupt(bad_slot):
    # a token-to-slot entry no step can write (>= S, or < -1) is reported as
    # corrupted state; that request is skipped (state unchanged, zero output),
    # the others take the step
    import token_level_gather_amd as kvs
    torch = _torch()
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="corrupt_slot", batch=3, context=3000,
                                                  slots=500, topk=200, steps=4, fresh_rate=0.3)
    h = Harness(wl, wl.steps, range(3))
    try:
        for t in range(2):
            h.check(t, 0, *h.device_step(t, 0))
        assert h.pool.sync_status()[0] == 0
        before = h.pool.read_state(1, 0)
        # a token of the next step's Top-K for request 1 (unit 1 * L + 0)
        tok = int(h.topk[2, 0, 1, 7])
        value = wl.slots + 3 if bad_slot == "past_end" else -5
        t2s = h.pool.meta[:3 * wl.context * 4].view(torch.int32)   # tok2slot [U][N] comes first
        t2s[1 * wl.context + tok] = value
        torch.cuda.synchronize()
        h.device_step(2, 0)
        assert h.pool.sync_status()[0] == kvs.KVS_ECORRUPT
        after = h.pool.read_state(1, 0)
        for key in ("slot2tok", "last_used", "lru_order", "step"):
            assert np.array_equal(np.asarray(before[key]), np.asarray(after[key])), key
        assert after["tok2slot"][tok] == value
        assert after["counts"][3] == 0
        assert not torch.any(h.out[1].float() != 0).item()
        for b in (0, 2):
            h.oracle[(b, 0)].step(h.topk[2, 0, b], h.pool.host.array[b, 0])
            assert np.array_equal(h.pool.read_state(b, 0)["slot2tok"], h.oracle[(b, 0)].slot2tok)
        assert h.pool.sync_status()[0] == 0
    finally:
        h.close()
