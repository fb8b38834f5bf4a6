"""Pins for the FP64 backward oracle (CPU only).

The pages give only the forward definition; its gradients (dQ, dK, dV of the
loss sum(dO * O)) are pinned here against things other than the backward code
itself: central finite differences of the forward oracle (which has its own
pins), closed forms, and invariances the definition implies.
"""
import numpy as np
import pytest

import oracle
from workloads import random_qkv, band_global_block_mask


def _loss(q, k, v, dout, scale, causal, key_len, bm, block):
    o, _ = oracle.attention_f64(q, k, v, scale, causal, key_len, bm, block)
    return float((o * dout).sum())


def _modes(N, rng):
    nb = (N + 1) // 2
    return {
        "dense": dict(causal=False, key_len=None, bm=None),
        "causal": dict(causal=True, key_len=None, bm=None),
        "padded": dict(causal=False, key_len=np.array([max(1, N - 2), N], dtype=np.int32), bm=None),
        "blocks": dict(causal=False, key_len=None, bm=(rng.random(nb * nb) < 0.6).astype(np.uint8)),
        "all": dict(causal=True, key_len=np.array([N, 0], dtype=np.int32),
                    bm=(rng.random(nb * nb) < 0.7).astype(np.uint8)),
    }


@pytest.mark.parametrize("H,H_kv", [(1, 1), (4, 2)])
@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks", "all"])
def test_gradients_match_finite_differences(H, H_kv, mode):
    N, d, scale, block = 5, 3, 0.6, 2
    q, _, _, rng = random_qkv(2, H, N, d, seed=500 + H, dtype="f32")
    _, k, v, rng = random_qkv(2, H_kv, N, d, seed=600 + H, dtype="f32", rng=rng)
    q, k, v = (x.astype(np.float64) for x in (q, k, v))
    dout = rng.standard_normal(q.shape)
    m = _modes(N, rng)[mode]
    dq, dk, dv = oracle.attention_bwd_f64(q, k, v, dout, scale, m["causal"], m["key_len"], m["bm"], block)
    h = 1e-6
    args = dict(q=q, k=k, v=v)
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        x = args[name]
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = dict(args, **{name: xp}), dict(args, **{name: xm})
            fd[idx] = (_loss(ap["q"], ap["k"], ap["v"], dout, scale, m["causal"], m["key_len"], m["bm"], block)
                       - _loss(am["q"], am["k"], am["v"], dout, scale, m["causal"], m["key_len"], m["bm"], block)) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=0, atol=1e-8, err_msg=f"d{name} {mode}")


def test_zero_upstream_gradient_gives_zero():
    q, k, v, _ = random_qkv(1, 2, 40, 8, seed=7, dtype="f32")
    for g in oracle.attention_bwd_f64(q, k, v, np.zeros_like(q), 0.3, True):
        assert not np.any(g)


def test_zero_scale_closed_form():
    """scale = 0: uniform weights over the allowed keys, so dQ = dK = 0 and
    dV_j = sum over the rows i that see key j of dO_i / (#keys row i sees)."""
    B, H, N, d = 1, 1, 12, 4
    q, k, v, rng = random_qkv(B, H, N, d, seed=8, dtype="f32")
    dout = rng.standard_normal(q.shape)
    dq, dk, dv = oracle.attention_bwd_f64(q, k, v, dout, 0.0, True)
    assert not np.any(dq) and not np.any(dk)
    expect = np.zeros((N, d))
    for i in range(N):
        expect[: i + 1] += dout[0, 0, i] / (i + 1)
    np.testing.assert_allclose(dv[0, 0], expect, rtol=0, atol=1e-14)


@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks"])
def test_key_and_value_shift_invariances(mode):
    """Adding one vector to every key shifts each score row by a constant, so
    the output (and the loss) does not move: the dK rows sum to zero.  Adding
    one vector c to every value adds c to every output row that has a key, so
    the dV rows sum to the dO rows of those rows."""
    N, d = 64, 8
    q, k, v, rng = random_qkv(2, 3, N, d, seed=9, dtype="bf16")
    dout = rng.standard_normal(q.shape)
    nb = (N + 15) // 16
    kl = np.array([40, 0], dtype=np.int32) if mode == "padded" else None
    bm = band_global_block_mask(nb, rng, n_global=1) if mode == "blocks" else None
    causal = mode == "causal"
    dq, dk, dv = oracle.attention_bwd_f64(q, k, v, dout, 0.35, causal, kl, bm, 16)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, rtol=0, atol=1e-12)
    _, lse = oracle.attention_f64(q, k, v, 0.35, causal, kl, bm, 16)
    has_key = np.isfinite(lse)[..., None]
    np.testing.assert_allclose(dv.sum(axis=2), (dout * has_key).sum(axis=2), rtol=0, atol=1e-12)


def test_grouped_heads_sum_the_group():
    """dK, dV of a shared key/value head are the sums over its group of the
    plain multi-head gradients computed on repeated key/value heads."""
    B, H, H_kv, N, d = 2, 6, 2, 30, 8
    q, _, _, rng = random_qkv(B, H, N, d, seed=10, dtype="f32")
    _, k, v, rng = random_qkv(B, H_kv, N, d, seed=11, dtype="f32", rng=rng)
    dout = rng.standard_normal(q.shape)
    kl = np.array([20, 30], dtype=np.int32)
    dq, dk, dv = oracle.attention_bwd_f64(q, k, v, dout, 0.4, True, kl)
    G = H // H_kv
    dq2, dk2, dv2 = oracle.attention_bwd_f64(q, np.repeat(k, G, 1), np.repeat(v, G, 1), dout, 0.4, True, kl)
    np.testing.assert_allclose(dq, dq2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(B, H_kv, G, N, d).sum(2), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, dv2.reshape(B, H_kv, G, N, d).sum(2), rtol=0, atol=1e-12)


def test_fully_masked_batch_has_no_gradient():
    q, k, v, rng = random_qkv(2, 2, 20, 4, seed=12, dtype="f32")
    dout = rng.standard_normal(q.shape)
    dq, dk, dv = oracle.attention_bwd_f64(q, k, v, dout, 0.5, False, np.array([20, 0], dtype=np.int32))
    for g in (dq, dk, dv):
        assert not np.any(g[1])
        assert np.any(g[0])


def _masks(N, block, B, rng):
    nb = (N + block - 1) // block
    return {
        "dense": dict(causal=False, key_len=None, bm=None),
        "causal": dict(causal=True, key_len=None, bm=None),
        "padded": dict(causal=False, key_len=np.array([N - 9, N, 3][:B], dtype=np.int32), bm=None),
        "blocks": dict(causal=False, key_len=None, bm=(rng.random(nb * nb) < 0.5).astype(np.uint8)),
        "all": dict(causal=True, key_len=np.array([N, 0, N - 4][:B], dtype=np.int32),
                    bm=(rng.random(nb * nb) < 0.6).astype(np.uint8)),
    }


@pytest.mark.parametrize("H,H_kv", [(2, 2), (4, 2), (3, 1)])
@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks", "all"])
def test_sampled_gradients_match_full_backward(H, H_kv, mode):
    # The sampled-row dQ and sampled-key dK/dV evaluations (used to check the
    # GPU backward at full workload sizes) against the full backward, which
    # is pinned by finite differences above.
    B, N, d, block, scale = 3, 37, 16, 8, 0.3
    q, _, _, rng = random_qkv(B, H, N, d, seed=900 + H, dtype="f32")
    _, k, v, rng = random_qkv(B, H_kv, N, d, seed=910 + H, dtype="f32", rng=rng)
    dout = rng.standard_normal(q.shape)
    m = _masks(N, block, B, rng)[mode]
    args = (m["causal"], m["key_len"], m["bm"], block)
    dq, dk, dv = oracle.attention_bwd_f64(q, k, v, dout, scale, *args)
    rows = rng.choice(B * H * N, size=25, replace=False)
    cols = np.concatenate([rng.choice(B * H_kv * N, size=15, replace=False), [0, B * H_kv * N - 1, 0]])
    dq_r = oracle.attention_bwd_rows_f64(q, k, v, dout, rows, scale, *args)
    dk_c, dv_c = oracle.attention_bwd_cols_f64(q, k, v, dout, cols, scale, *args)
    np.testing.assert_allclose(dq_r, dq.reshape(-1, d)[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk_c, dk.reshape(-1, d)[cols], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv_c, dv.reshape(-1, d)[cols], rtol=0, atol=1e-12)


def test_sampled_gradients_reject_bad_indices():
    q, k, v, rng = random_qkv(1, 2, 10, 4, seed=920, dtype="f32")
    dout = rng.standard_normal(q.shape)
    with pytest.raises(RuntimeError):
        oracle.attention_bwd_rows_f64(q, k, v, dout, [20], 0.5)
    with pytest.raises(RuntimeError):
        oracle.attention_bwd_cols_f64(q, k, v, dout, [-1], 0.5)
    assert oracle.attention_bwd_rows_f64(q, k, v, dout, [], 0.5).shape == (0, 4)
