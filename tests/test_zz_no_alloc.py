"""kvs_step_static (per-step scratch in the library's static per-GPU array)
against kvs_step (scratch from the caller) through the C ABI.

Two pools share one host pool and the same inputs; one takes every step with
kvs_step, the other with kvs_step_static.  The kernels are the same, so the
outputs must agree bit for bit; both are also checked against the oracle.  A
second, smaller workload follows the first in the same process, so the static
array's leftover contents from the larger run must not leak into it.
"""
import ctypes

import numpy as np
import pytest

import kvs_workload as W
from oracle import OracleUnit

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
REL_L2 = 1e-2


def _run_pair(wl, flags=0):
    import torch

    import token_level_gather_amd as kvs
    B, L = wl.batch, wl.layers
    host = kvs.HostPool(B, L, wl.context)
    W.fill_pool(host.array, wl)
    ref = kvs.Pool(B, L, wl.context, wl.slots, wl.topk, scale=wl.scale, host=host, flags=flags)
    sta = kvs.Pool(B, L, wl.context, wl.slots, wl.topk, scale=wl.scale, host=host, flags=flags)
    try:
        assert sta.sizes.scratch_bytes <= kvs.STATIC_SCRATCH_BYTES
        topk = W.topk_streams(wl)
        oracle = {(b, l): OracleUnit(wl.context, wl.slots, wl.topk)
                  for b in range(B) for l in range(L)}
        out_r = torch.empty((B, 16, 512), dtype=torch.bfloat16, device="cuda")
        out_s = torch.empty_like(out_r)
        lse_r = torch.empty((B, 16), dtype=torch.float32, device="cuda")
        lse_s = torch.empty_like(lse_r)
        for t in range(wl.steps):
            for l in range(L):
                q_np = W.queries(wl, l, t)
                tk = torch.from_numpy(topk[t, l]).cuda()
                q = torch.from_numpy(q_np.view(np.int16)).cuda()
                ref.step(l, tk, q, out_r, lse_r)
                sta.step_static(l, tk, q, out_s, lse_s)
                torch.cuda.synchronize()
                assert torch.equal(out_r.view(torch.int16), out_s.view(torch.int16)), (t, l)
                assert torch.equal(lse_r, lse_s), (t, l)
                got = out_s.view(torch.int16).cpu().numpy().view(np.uint16)
                for b in range(B):
                    rec = oracle[(b, l)].step(topk[t, l, b], host.array[b, l], q_np[b], wl.scale)
                    sr, ss = ref.read_state(b, l), sta.read_state(b, l)
                    for key in ("tok2slot", "slot2tok", "last_used", "lru_order", "slot_of",
                                "miss_pos", "victims", "counts", "row_slot", "step"):
                        assert np.array_equal(np.asarray(sr[key]), np.asarray(ss[key])), key
                    assert np.array_equal(ss["tok2slot"], oracle[(b, l)].tok2slot)
                    assert np.array_equal(ss["miss_pos"][:rec.n_miss], rec.miss_pos)
                    g = (got[b].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                    err = g - rec.out
                    assert np.abs(err).max() <= MAX_ABS
                    assert np.linalg.norm(err) / np.linalg.norm(rec.out) <= REL_L2
        rr, sr_ = ref.sync_status(), sta.sync_status()
        assert rr[0] == 0 and sr_[0] == 0
        assert (rr[1].hits, rr[1].misses) == (sr_[1].hits, sr_[1].misses)
    finally:
        ref.release()
        sta.release()
        host.free()


def test_static_scratch_matches_caller_scratch_then_smaller_input():
    base = W.WORKLOADS["ctx16k_b64_k2048"]
    # first: 6 requests, 2 layers, K = 1025 over 4 splits' worth of tiles
    big = base.shrunk(name="static_big", batch=6, layers=2, context=6000, slots=1500,
                      topk=1025, steps=5, fresh_rate=0.3)
    _run_pair(big)
    # second, right after, with smaller inputs (fewer requests, smaller K)
    small = base.shrunk(name="static_small", batch=2, layers=1, context=3000, slots=400,
                        topk=200, steps=4, fresh_rate=0.5)
    _run_pair(small)


def test_static_scratch_direct_mode():
    import token_level_gather_amd as kvs
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="static_direct", batch=3, layers=2,
                                                  context=4000, slots=700, topk=300, steps=4,
                                                  fresh_rate=0.3)
    _run_pair(wl, flags=kvs.KVS_FLAG_DIRECT_HOT)


def test_static_scratch_rejects_pools_beyond_its_size():
    import torch

    import token_level_gather_amd as kvs
    # 1024 requests x K = 64: one split of 16 x 512 fp32 partials per request
    # alone is 32 MiB, past the static array
    pool = kvs.Pool(1024, 1, 64, 64, 64)
    try:
        assert pool.sizes.scratch_bytes > kvs.STATIC_SCRATCH_BYTES
        tk = torch.arange(64, dtype=torch.int32, device="cuda").repeat(1024, 1)
        q = torch.zeros((1024, 16, 576), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((1024, 16, 512), dtype=torch.bfloat16, device="cuda")
        rc = kvs.lib().kvs_step_static(pool.handle, 0, tk.data_ptr(), q.data_ptr(),
                                       out.data_ptr(), None,
                                       torch.cuda.current_stream().cuda_stream)
        assert rc == kvs.KVS_ENOMEM
        torch.cuda.synchronize()
        assert pool.read_state(0, 0)["step"] == 0   # nothing was enqueued
        assert kvs.lib().kvs_step_static(None, 0, None, None, None, None, None) == kvs.KVS_EINVAL
    finally:
        pool.close()
