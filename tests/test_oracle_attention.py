"""Pins of the oracle's Top-K sparse decode attention and bf16 decoding.

Checked against other formulations: dense softmax attention over the whole
context with non-selected tokens masked out, torch's scaled_dot_product_attention
in float64 on the CPU, scipy's logsumexp, and closed forms (zero query, equal
rows, a single token, invariance under permuting the Top-K order).
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from kvs_workload import f32_to_bf16_bits
from oracle import OracleUnit, attention_fp64, bf16_bits_to_f64

SCALE = 1.0 / 24.0


def _bf16(rng, *shape):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def test_bf16_decoding_known_values():
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x0000, 0x8000, 0x4049, 0x7F7F], dtype=np.uint16)
    want = [1.0, -2.0, 0.25, 0.0, -0.0, 3.140625, 3.3895313892515355e38]
    assert bf16_bits_to_f64(bits).tolist() == want


def test_bf16_rounding_ties_to_even():
    # 1 + 2^-8 lies halfway between bf16 1.0 and 1 + 2^-7: ties go to the even 1.0;
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: goes to even 1 + 2^-6.
    x = np.array([1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, -(1 + 2**-8)], dtype=np.float32)
    got = bf16_bits_to_f64(f32_to_bf16_bits(x)).tolist()
    assert got == [1.0, 1 + 2**-6, 1 + 2**-7, -1.0]


@pytest.mark.parametrize("seed", range(4))
def test_equals_dense_masked_softmax_over_context(seed):
    rng = np.random.default_rng(seed)
    n_ctx, k = 300, 37
    pool = _bf16(rng, n_ctx, 576)
    q = _bf16(rng, 16, 576)
    topk = rng.choice(n_ctx, size=k, replace=False)
    out, lse = attention_fp64(q, pool[topk], SCALE)
    # dense attention over all N tokens, non-selected tokens masked to -inf
    qf = bf16_bits_to_f64(q)
    kv = bf16_bits_to_f64(pool)
    z = qf @ kv.T * SCALE
    mask = np.full(n_ctx, -np.inf)
    mask[topk] = 0.0
    zm = z + mask
    w = np.exp(zm - zm.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    dense = w @ kv[:, :512]
    np.testing.assert_allclose(out, dense, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, logsumexp(z[:, topk], axis=1), rtol=1e-12)


def test_equals_torch_sdpa_float64():
    rng = np.random.default_rng(7)
    k = 129
    rows = _bf16(rng, k, 576)
    q = _bf16(rng, 16, 576)
    out, _ = attention_fp64(q, rows, SCALE)
    qt = torch.from_numpy(bf16_bits_to_f64(q)).view(1, 16, 1, 576)
    kt = torch.from_numpy(bf16_bits_to_f64(rows)).view(1, 1, k, 576).expand(1, 16, k, 576)
    vt = kt[..., :512]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=SCALE)
    np.testing.assert_allclose(out, ref.view(16, 512).numpy(), rtol=1e-10, atol=1e-12)


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(1)
    rows = _bf16(rng, 50, 576)
    out, lse = attention_fp64(np.zeros((16, 576), np.uint16), rows, SCALE)
    mean = bf16_bits_to_f64(rows)[:, :512].mean(axis=0)
    np.testing.assert_allclose(out, np.broadcast_to(mean, (16, 512)), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse, np.log(50.0), rtol=1e-14)


def test_equal_rows_give_that_row():
    rng = np.random.default_rng(2)
    row = _bf16(rng, 1, 576)
    rows = np.repeat(row, 20, axis=0)
    out, _ = attention_fp64(_bf16(rng, 16, 576), rows, SCALE)
    np.testing.assert_allclose(out, np.broadcast_to(bf16_bits_to_f64(row)[0, :512], (16, 512)),
                               rtol=1e-13)


def test_single_token_gives_the_row():
    rng = np.random.default_rng(3)
    row = _bf16(rng, 1, 576)
    q = _bf16(rng, 16, 576)
    out, lse = attention_fp64(q, row, SCALE)
    assert np.array_equal(out, np.broadcast_to(bf16_bits_to_f64(row)[0, :512], (16, 512)))
    np.testing.assert_allclose(lse, bf16_bits_to_f64(q) @ bf16_bits_to_f64(row)[0] * SCALE,
                               rtol=1e-13)


def test_topk_order_does_not_matter():
    rng = np.random.default_rng(4)
    rows = _bf16(rng, 64, 576)
    q = _bf16(rng, 16, 576)
    a, la = attention_fp64(q, rows, SCALE)
    perm = rng.permutation(64)
    b, lb = attention_fp64(q, rows[perm], SCALE)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(la, lb, rtol=1e-13)


def test_step_attention_uses_gathered_rows():
    rng = np.random.default_rng(5)
    n_ctx, slots, k = 200, 64, 32
    pool = _bf16(rng, n_ctx, 576)
    u = OracleUnit(n_ctx, slots, k)
    for _ in range(5):
        topk = rng.choice(n_ctx, size=k, replace=False)
        q = _bf16(rng, 16, 576)
        rec = u.step(topk, pool, q, SCALE)
        out, lse = attention_fp64(q, pool[topk], SCALE)
        np.testing.assert_array_equal(rec.out, out)
        np.testing.assert_array_equal(rec.lse, lse)


@pytest.mark.parametrize("seed", range(3))
def test_padded_step_equals_dense_masked_softmax(seed):
    # empty entries are masked out of the softmax (as tokens outside the Top-K
    # set are in the dense form), not scored as zero rows
    rng = np.random.default_rng(40 + seed)
    n_ctx, slots, k = 300, 64, 48
    pool = _bf16(rng, n_ctx, 576)
    q = _bf16(rng, 16, 576)
    topk = rng.choice(n_ctx, size=k, replace=False).astype(np.int64)
    topk[rng.random(k) < 0.4] = -1
    sel = topk[topk >= 0]
    rec = OracleUnit(n_ctx, slots, k).step(topk, pool, q, SCALE, padded=True)
    qf, kv = bf16_bits_to_f64(q), bf16_bits_to_f64(pool)
    z = qf @ kv.T * SCALE
    zm = z + np.where(np.isin(np.arange(n_ctx), sel), 0.0, -np.inf)
    w = np.exp(zm - zm.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(rec.out, w @ kv[:, :512], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(rec.lse, logsumexp(z[:, sel], axis=1), rtol=1e-12)


def test_padded_single_valid_entry_gives_that_row():
    rng = np.random.default_rng(44)
    pool = _bf16(rng, 50, 576)
    q = _bf16(rng, 16, 576)
    topk = np.array([-1, -1, 17, -1, -1])
    rec = OracleUnit(50, 8, 5).step(topk, pool, q, SCALE, padded=True)
    assert np.array_equal(rec.out, np.broadcast_to(bf16_bits_to_f64(pool[17])[:512], (16, 512)))
    np.testing.assert_allclose(rec.lse, bf16_bits_to_f64(q) @ bf16_bits_to_f64(pool[17]) * SCALE,
                               rtol=1e-13)


def test_all_empty_step_gives_zero_output_and_minus_inf_lse():
    rng = np.random.default_rng(45)
    pool = _bf16(rng, 50, 576)
    u = OracleUnit(50, 8, 4)
    u.step(np.array([1, 2, 3, 4]), pool)
    t2s = u.tok2slot.copy()
    rec = u.step(np.full(4, -1), pool, _bf16(rng, 16, 576), SCALE, padded=True)
    assert not rec.out.any() and np.all(rec.lse == -np.inf)
    assert rec.t == 1 and u.t == 2 and np.array_equal(u.tok2slot, t2s)
    assert rec.n_miss == 0 and rec.n_hit == 0 and rec.n_pad == 4
