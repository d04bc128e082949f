"""The device-checked debug build (libkvs_checked.so) on MI355X.

Valid runs: the same parity bar as the normal build (bit-exact state and
bytes, attention within tolerance) and the same output bits as libkvs.so,
with a clean status.  Invalid state that the normal build trusts (an LRU order
entry past the slots or a slot listed twice, a slot-to-token entry outside
[-1, N), an appended token whose slot lies outside [-1, S)) is planted from
the host and must come back as KVS_EBOUNDS naming the access and the index,
with the request left untouched.  Those cases run against the checked build
only: it verifies the state before any access that would use it.
"""
import numpy as np
import pytest

import kvs_workload as W
from test_gpu_parity import Harness, _meta_offsets, _slot_stride, _torch, _u16

pytestmark = pytest.mark.gpu


def _checked():
    import token_level_gather_amd as kvs
    return kvs.load_library(kvs.CHECKED_LIB_PATH)


def _small(name, **kw):
    base = dict(batch=3, layers=2, context=4000, slots=500, topk=300, steps=5, fresh_rate=0.4)
    base.update(kw)
    return W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name=name, **base)


@pytest.mark.parametrize("case", ["default", "padded", "direct", "separate", "separate_direct",
                                  "separate_wide", "zipf", "k3000"])
def test_checked_build_matches_oracle(case):
    import token_level_gather_amd as kvs
    flags = 0
    if "direct" in case:
        flags |= kvs.KVS_FLAG_DIRECT_HOT
    if "separate" in case:
        flags |= kvs.KVS_FLAG_SEPARATE_ATTENTION
    if case == "zipf":
        wl = W.WORKLOADS["ctx128k_b32_l8_zipf"].shrunk(batch=3, layers=2, context=20000, steps=5)
    elif case == "separate_wide":   # enough fetch workgroups for one host read per thread
        wl = _small("checked_separate_wide", batch=17, layers=1, context=6000, slots=2100,
                    topk=2048, steps=3, fresh_rate=0.3)
    elif case == "k3000":   # 3 Top-K entries and 6 slots per diff thread
        wl = _small("checked_k3000", batch=2, layers=1, context=9000, slots=6000, topk=3000,
                    steps=4)
    else:
        wl = _small(f"checked_{case}")
    h = Harness(wl, wl.steps, range(wl.batch), padded=case == "padded", flags=flags,
                library=_checked())
    try:
        h.run()   # every unit against the oracle after every step; clean status at the end
    finally:
        h.close()


def test_checked_build_output_bits_equal_normal_build():
    torch = _torch()
    wl = _small("checked_bits", steps=4)
    outs = []
    for library in (None, _checked()):
        h = Harness(wl, wl.steps, [], library=library)
        got = []
        try:
            for t in range(wl.steps):
                for l in range(wl.layers):
                    h.device_step(t, l)
                    got.append((_u16(h.out).copy(), h.lse.cpu().numpy().copy()))
            assert h.pool.sync_status()[0] == 0
        finally:
            h.close()
        outs.append(got)
    for (o0, l0), (o1, l1) in zip(*outs):
        assert np.array_equal(o0, o1)
        assert np.array_equal(l0.view(np.uint32), l1.view(np.uint32))
    torch.cuda.synchronize()


def _planted(h, plant, expect_site):
    """Two clean steps, then `plant()` corrupts request 1's unit (layer 0) and
    returns the index the check must report; one more step: KVS_EBOUNDS with
    that site and index, request 1 untouched with a zero output, requests 0
    and 2 still equal to the oracle."""
    import token_level_gather_amd as kvs
    torch = _torch()
    for t in range(2):
        h.check(t, 0, *h.device_step(t, 0))
    assert h.pool.sync_status()[0] == 0
    expect_index = plant()
    torch.cuda.synchronize()
    before = h.pool.read_state(1, 0)
    h.device_step(2, 0)
    rc, st = h.pool.sync_status()
    assert rc == kvs.KVS_EBOUNDS
    assert (st.fault_site, st.fault_index) == (expect_site, expect_index)
    after = h.pool.read_state(1, 0)
    for key in ("tok2slot", "slot2tok", "last_used", "lru_order", "step"):
        assert np.array_equal(np.asarray(before[key]), np.asarray(after[key])), key
    assert after["counts"][3] == 0
    assert not torch.any(h.out[1].float() != 0).item()
    for b in (0, 2):
        h.oracle[(b, 0)].step(h.topk[2, 0, b], h.pool.host.array[b, 0])
        assert np.array_equal(h.pool.read_state(b, 0)["slot2tok"], h.oracle[(b, 0)].slot2tok)
    assert h.pool.sync_status()[0] == 0   # cleared by the previous sync


@pytest.mark.parametrize("slots", [500, 6000])   # slot tokens read per slot / per order entry
@pytest.mark.parametrize("kind", ["past_end", "repeated"])
def test_checked_build_rejects_bad_lru_order(kind, slots):
    import token_level_gather_amd as kvs
    torch = _torch()
    wl = _small(f"bad_order_{kind}", layers=1, slots=slots, context=9000, steps=3)
    h = Harness(wl, wl.steps, [0, 2], library=_checked())
    try:
        _, _, order_off = _meta_offsets(h.pool)
        sp = _slot_stride(wl.slots)
        base = (1 * wl.layers + 0) * sp
        order = h.pool.meta[order_off:order_off + wl.batch * wl.layers * sp * 2] \
            .view(torch.int16)

        def plant():
            if kind == "past_end":
                order[base + 7] = wl.slots + 5
                return wl.slots + 5
            dup = int(order[base + 8].item())   # position 9 repeats the slot at position 8
            order[base + 9] = dup
            return dup

        _planted(h, plant, kvs.KVS_SITE_LRU_ORDER)
    finally:
        h.close()


@pytest.mark.parametrize("value", ["past_context", "below_minus_one"])
def test_checked_build_rejects_bad_slot_token(value):
    import token_level_gather_amd as kvs
    torch = _torch()
    wl = _small(f"bad_s2t_{value}", layers=1, steps=3)
    h = Harness(wl, wl.steps, [0, 2], library=_checked())
    try:
        s2t_off, _, _ = _meta_offsets(h.pool)
        u = 1 * wl.layers + 0
        bad = wl.context + 7 if value == "past_context" else -3
        sp = _slot_stride(wl.slots)
        s2t = h.pool.meta[s2t_off:s2t_off + wl.batch * wl.layers * sp * 4] \
            .view(torch.int32)

        def plant():
            s2t[u * sp + 11] = bad
            return bad

        _planted(h, plant, kvs.KVS_SITE_SLOT_TOKEN)
    finally:
        h.close()


def test_checked_build_rejects_bad_append_slot():
    # an appended token whose token-to-slot entry lies past the slots: the row
    # is neither written to the pool nor to the hot buffer
    import token_level_gather_amd as kvs
    torch = _torch()
    wl = _small("bad_append", layers=1, steps=2)
    h = Harness(wl, wl.steps, [0], library=_checked())
    try:
        h.check(0, 0, *h.device_step(0, 0))
        assert h.pool.sync_status()[0] == 0
        tok = 3999
        t2s = h.pool.meta[:wl.batch * wl.layers * wl.context * 4].view(torch.int32)
        t2s[1 * wl.context + tok] = wl.slots + 2
        pool_row = h.pool.host.array[1, 0, tok].copy()
        rows = torch.full((wl.batch, 576), 0x3f80, dtype=torch.int16, device="cuda")
        pos = torch.tensor([-1, tok, -1], dtype=torch.int64, device="cuda")
        torch.cuda.synchronize()
        h.pool.append(0, rows, pos)
        rc, stats = h.pool.sync_status()
        assert rc == kvs.KVS_EBOUNDS
        assert (stats.fault_site, stats.fault_index) == (kvs.KVS_SITE_APPEND, wl.slots + 2)
        assert np.array_equal(h.pool.host.array[1, 0, tok], pool_row)
    finally:
        h.close()
