"""The seeded input generators: determinism, ranges and the carry-over recipe."""
import hashlib

import numpy as np
import pytest

import kvs_workload as W


def _small(name, **kw):
    base = W.WORKLOADS[name]
    shrink = dict(batch=3, layers=min(base.layers, 2), steps=6)
    shrink.update(kw)
    return base.shrunk(**shrink)


@pytest.mark.parametrize("name", sorted(W.WORKLOADS))
def test_topk_stream_recipe(name):
    wl = _small(name)
    s = W.topk_streams(wl, threads=1)
    assert s.shape == (wl.steps, wl.layers, wl.batch, wl.topk) and s.dtype == np.int32
    for l in range(wl.layers):
        for b in range(wl.batch):
            prev = None
            for t in range(wl.steps):
                cur = s[t, l, b]
                assert cur.min() >= 0 and cur.max() < wl.context
                assert np.unique(cur).size == wl.topk
                if prev is not None:
                    kept = np.intersect1d(prev, cur)
                    assert kept.size == wl.n_keep          # fresh ones avoid prev
                if wl.dist == "zipf":
                    recent = int((cur >= wl.context - wl.forced_window).sum())
                    n_fresh = wl.topk if t == 0 else wl.n_fresh
                    assert recent >= int(round(wl.forced_frac * n_fresh))
                prev = cur


def test_keep_fresh_counts():
    assert (W.WORKLOADS["ctx4k_b1_k256"].n_keep, W.WORKLOADS["ctx4k_b1_k256"].n_fresh) == (205, 51)
    assert W.WORKLOADS["ctx16k_b64_k2048"].n_fresh == 410
    assert W.WORKLOADS["ctx16k_b192_k2048_f40"].n_fresh == 819


def test_streams_are_deterministic_and_thread_independent():
    wl = _small("ctx16k_b64_k2048", batch=4)
    a = W.topk_streams(wl, threads=1)
    b = W.topk_streams(wl, threads=4)
    assert np.array_equal(a, b)
    c = W.topk_streams(wl, requests=[2])
    assert np.array_equal(a[:, :, 2:3], c)


def test_pool_rows_deterministic_and_unit_addressable():
    wl = W.WORKLOADS["ctx4k_b1_k256"].shrunk(batch=2, layers=2, context=300)
    pool = np.empty((2, 2, 300, 576), np.uint16)
    W.fill_pool(pool, wl, threads=3)
    pool2 = np.empty_like(pool)
    W.fill_pool(pool2, wl, threads=1)
    assert np.array_equal(pool, pool2)
    assert np.array_equal(pool[1, 0], W.unit_rows(wl, 1, 0))
    assert not np.array_equal(pool[0, 0], pool[1, 0])
    h = hashlib.sha256(pool.tobytes()).hexdigest()
    assert h == hashlib.sha256(pool2.tobytes()).hexdigest()


def test_pool_values_are_bf16_normals():
    wl = W.WORKLOADS["ctx4k_b1_k256"]
    rows = W.unit_rows(wl, 0, 0)
    x = (rows.astype(np.uint32) << 16).view(np.float32)
    assert abs(float(x.mean())) < 0.01 and abs(float(x.std()) - 1.0) < 0.01
    # bf16 -> float32 -> bf16 round trips exactly
    assert np.array_equal(W.f32_to_bf16_bits(x), rows)


def test_queries_shape_and_seed():
    wl = W.WORKLOADS["ctx4k_b1_k256"]
    q0 = W.queries(wl, 0, 0)
    assert q0.shape == (1, 16, 576) and q0.dtype == np.uint16
    assert np.array_equal(q0, W.queries(wl, 0, 0))
    assert not np.array_equal(q0, W.queries(wl, 0, 1))
