"""HIP-graph capture of kvs_step: replays equal eager steps bit for bit and the oracle.

Each layer's step is captured once over fixed buffers; before every replay the
step's Top-K and queries are copied into those buffers by ordinary (eager)
stream work.  Every replay is checked: state, miss lists and gathered bytes
against the oracle and against an eager pool run on the same inputs (same
kernels, so the attention output must match the eager one bit for bit).
"""
import numpy as np
import pytest

import kvs_workload as W
from oracle import OracleUnit

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", ["default", "padded", "direct", "padded_direct"])
def test_graph_replay_equals_eager_and_oracle(mode):
    import torch

    import token_level_gather_amd as kvs
    padded = "padded" in mode
    flags = (kvs.KVS_FLAG_PADDED_TOPK if padded else 0) | \
        (kvs.KVS_FLAG_DIRECT_HOT if "direct" in mode else 0)
    wl = W.WORKLOADS["ctx16k_b64_k2048"].shrunk(name="graph", batch=4, layers=2, context=5000,
                                                  slots=700, topk=300, steps=8, fresh_rate=0.3)
    B, L = wl.batch, wl.layers
    host = kvs.HostPool(B, L, wl.context)
    W.fill_pool(host.array, wl)
    pg = kvs.Pool(B, L, wl.context, wl.slots, wl.topk, scale=wl.scale, host=host, flags=flags)
    pe = kvs.Pool(B, L, wl.context, wl.slots, wl.topk, scale=wl.scale, host=host, flags=flags)
    try:
        topk = W.topk_streams(wl)
        if padded:
            topk = W.pad_topk_streams(topk, wl.seed)
        tk_s = [torch.empty((B, wl.topk), dtype=torch.int32, device="cuda") for _ in range(L)]
        q_s = [torch.empty((B, 16, 576), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
        out_g = [torch.empty((B, 16, 512), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
        lse_g = [torch.empty((B, 16), dtype=torch.float32, device="cuda") for _ in range(L)]
        out_e = torch.empty((B, 16, 512), dtype=torch.bfloat16, device="cuda")
        lse_e = torch.empty((B, 16), dtype=torch.float32, device="cuda")
        graphs = [pg.capture(l, tk_s[l], q_s[l], out_g[l], lse_g[l]) for l in range(L)]
        torch.cuda.synchronize()
        # capture ran nothing: the pool is still empty
        assert pg.read_state(0, 0)["step"] == 0
        oracle = {(b, l): OracleUnit(wl.context, wl.slots, wl.topk)
                  for b in range(B) for l in range(L)}
        for t in range(wl.steps):
            for l in range(L):
                q = W.queries(wl, l, t)
                tk = torch.from_numpy(topk[t, l]).cuda()
                qt = torch.from_numpy(q.view(np.int16)).cuda().view(torch.bfloat16)
                tk_s[l].copy_(tk)
                q_s[l].copy_(qt)
                graphs[l].launch()
                pe.step(l, tk, qt, out_e, lse_e)
                torch.cuda.synchronize()
                assert torch.equal(out_g[l].view(torch.int16), out_e.view(torch.int16)), (t, l)
                assert torch.equal(lse_g[l], lse_e), (t, l)
                if not flags & kvs.KVS_FLAG_DIRECT_HOT:   # direct mode has no compute buffer
                    assert torch.equal(pg.cbuf, pe.cbuf), (t, l)
                for b in range(B):
                    rec = oracle[(b, l)].step(topk[t, l, b], host.array[b, l], q[b], wl.scale,
                                              padded=padded)
                    sg = pg.read_state(b, l)
                    se = pe.read_state(b, l)
                    for key in ("tok2slot", "slot2tok", "last_used", "lru_order", "slot_of",
                                "row_slot"):
                        assert np.array_equal(sg[key], se[key]), (t, l, b, key)
                    assert np.array_equal(sg["tok2slot"], oracle[(b, l)].tok2slot)
                    assert np.array_equal(sg["victims"][:rec.n_miss], rec.victims)
                    assert sg["step"] == t + 1
                    got = (out_g[l][b].view(torch.int16).cpu().numpy().view(np.uint16)
                           .astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                    if rec.n_hit + rec.n_miss == 0:   # all entries empty
                        assert not got.any() and torch.all(lse_g[l][b] == -np.inf)
                        continue
                    err = got - rec.out
                    assert np.abs(err).max() <= 2e-2
                    assert np.linalg.norm(err) / np.linalg.norm(rec.out) <= 1e-2
        for g in graphs:
            g.destroy()
        assert pg.sync_status()[0] == 0
    finally:
        pg.release()
        pe.release()
        host.free()
