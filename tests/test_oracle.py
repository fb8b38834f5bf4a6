"""Pins for the FP64 oracle (CPU only).

Every check here ties the oracle to something other than itself: hand-derived
closed forms, a 40-digit brute-force evaluation on tiny inputs, invariances the
definition implies, and torch's float64 softmax as a library cross-check.

Definition under test (page 'Ch.04 Attention optimisation: FlashAttention and
sparse attention', mdooai.com, 'Key points of the formulas'):
S = scale * Q K^T, A = row-softmax(S) with rows summing to one, O = A V,
disallowed logits at -inf before the softmax.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import brute
from workloads import random_qkv, band_global_block_mask

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _val(s):
    if s == "-inf":
        return -math.inf
    if s.startswith("ln"):
        return math.log(float(s[2:]))
    return float(Fraction(s))


# ---------------------------------------------------------------- fixtures


def test_hand_derived_three_keys():
    """Hand-derived rationals (tests/golden/hand_three_keys.json)."""
    g = json.load(open(os.path.join(GOLDEN, "hand_three_keys.json")))
    q = np.array(g["q"], dtype=np.float64)[None, None]
    k = np.array(g["k"], dtype=np.float64)[None, None]
    v = np.array(g["v"], dtype=np.float64)[None, None]
    scale = _val(g["scale"])
    for c in g["cases"]:
        o, lse = oracle.attention_f64(q, k, v, scale, c["causal"], c["key_len"],
                                      c["block_mask"], c["block"])
        O = np.array([[_val(x) for x in row] for row in c["O"]])
        L = np.array([_val(x) for x in c["LSE"]])
        np.testing.assert_allclose(o[0, 0], O, rtol=0, atol=1e-14, err_msg=c["name"])
        fin = np.isfinite(L)
        np.testing.assert_allclose(lse[0, 0][fin], L[fin], rtol=0, atol=1e-14, err_msg=c["name"])
        assert np.all(lse[0, 0][~fin] == -np.inf), c["name"]


def test_stored_brute_force_values():
    """40-digit values written by tests/golden/make_golden.py from oracle/brute.py."""
    g = json.load(open(os.path.join(GOLDEN, "brute_small.json")))
    q, k, v = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v"))
    for c in g["cases"]:
        o, lse = oracle.attention_f64(q, k, v, g["scale"], c["causal"], c["key_len"],
                                      c["block_mask"], c["block"])
        O = np.array(c["O"], dtype=np.float64)
        L = np.array(c["LSE"], dtype=np.float64)
        np.testing.assert_allclose(o, O, rtol=0, atol=1e-13, err_msg=c["name"])
        fin = np.isfinite(L)
        np.testing.assert_allclose(lse[fin], L[fin], rtol=0, atol=1e-13, err_msg=c["name"])
        assert np.all(lse[~fin] == -np.inf)
        assert np.all(o[~fin] == 0.0)


# ---------------------------------------------------------------- brute force


@pytest.mark.parametrize("N,d", [(1, 1), (2, 2), (3, 4), (5, 3), (8, 4), (4, 64)])
@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks", "all"])
def test_brute_force_tiny(N, d, mode):
    q, k, v, rng = random_qkv(2, 1, N, d, seed=100 + 7 * N + d, dtype="f32")
    scale = 1.0 / math.sqrt(d)
    causal = mode in ("causal", "all")
    key_len = rng.integers(0, N, size=2, endpoint=True) if mode in ("padded", "all") else None
    block = 2
    nb = (N + block - 1) // block
    bm = (rng.random(nb * nb) < 0.6).astype(np.uint8) if mode in ("blocks", "all") else None
    o, lse = oracle.attention_f64(q, k, v, scale, causal, key_len, bm, block)
    O, L = brute.attention_mp(q, k, v, scale, causal, key_len, bm, block)
    O = np.array(O, dtype=np.float64)
    L = np.array(L, dtype=np.float64)
    np.testing.assert_allclose(o, O, rtol=0, atol=1e-13)
    fin = np.isfinite(L)
    np.testing.assert_allclose(lse[fin], L[fin], rtol=0, atol=1e-13)
    assert np.all(lse[~fin] == -np.inf)
    assert np.all(o[~fin] == 0.0)


# ---------------------------------------------------------------- closed forms


def _allowed_matrix(N, b, causal, key_len, bm, block):
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    ok = np.ones((N, N), dtype=bool)
    if causal:
        ok &= j <= i
    if key_len is not None:
        ok &= j < key_len[b]
    if bm is not None:
        nb = (N + block - 1) // block
        ok &= np.asarray(bm).reshape(nb, nb)[i // block, j // block] != 0
    return ok


@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks"])
def test_zero_query_gives_mean_of_allowed_values(mode):
    """Q = 0: all allowed logits are 0, so O_i = mean of allowed V rows and
    LSE_i = log(#allowed)."""
    B, H, N, d = 2, 2, 300, 16
    _, k, v, rng = random_qkv(B, H, N, d, seed=3, dtype="bf16")
    q = np.zeros_like(k)
    causal = mode == "causal"
    key_len = np.array([0, 211], dtype=np.int32) if mode == "padded" else None
    bm = band_global_block_mask(3, rng, n_global=1) if mode == "blocks" else None
    o, lse = oracle.attention_f64(q, k, v, 0.125, causal, key_len, bm, 128)
    for b in range(B):
        ok = _allowed_matrix(N, b, causal, key_len, bm, 128)
        cnt = ok.sum(1)
        for h in range(H):
            for i in range(N):
                if cnt[i] == 0:
                    assert lse[b, h, i] == -np.inf and np.all(o[b, h, i] == 0)
                    continue
                mean = v[b, h][ok[i]].astype(np.float64).mean(0)
                np.testing.assert_allclose(o[b, h, i], mean, rtol=0, atol=1e-13)
                assert abs(lse[b, h, i] - math.log(cnt[i])) < 1e-13


def test_dominant_logit_selects_value_row():
    """q_i = a e0, k_j* = c e0 with scale*a*c = 40 and every other k_j . e0 = 0:
    O_i = V_j* and LSE_i = 40 up to (N-1) e^-40."""
    N, d = 64, 8
    rng = np.random.default_rng(5)
    v = rng.standard_normal((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d))
    k[..., 0] = 0.0
    q = np.zeros((1, 1, N, d))
    for i in range(N):
        q[0, 0, i, 0] = 8.0
    jstar = 37
    k[0, 0, jstar, 0] = 10.0
    o, lse = oracle.attention_f64(q, k, v, 0.5, False)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, jstar], (N, d)), rtol=0,
                               atol=1e-15 + N * math.exp(-40) * np.abs(v).max())
    np.testing.assert_allclose(lse[0, 0], 40.0 + math.log1p((N - 1) * math.exp(-40)), rtol=0, atol=1e-13)


def test_single_key_and_causal_first_row():
    """N = 1: O = V_0, LSE = s_00.  Causal row 0 of any N: O_0 = V_0 exactly."""
    q, k, v, _ = random_qkv(1, 3, 1, 32, seed=9, dtype="bf16")
    o, lse = oracle.attention_f64(q, k, v, 0.3, False)
    np.testing.assert_array_equal(o, v)
    s00 = 0.3 * np.einsum("bhnd,bhnd->bhn", q.astype(np.float64), k.astype(np.float64))
    np.testing.assert_allclose(lse, s00, rtol=0, atol=1e-14)
    q, k, v, _ = random_qkv(2, 2, 77, 16, seed=10, dtype="bf16")
    o, lse = oracle.attention_f64(q, k, v, 0.25, True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])


@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks"])
def test_identity_values_expose_attention_matrix(mode):
    """With d = N and V = I, O = A itself: every row sums to 1, A_ij > 0 exactly
    on the allowed set and A_ij = 0 elsewhere (pins mask semantics and the
    orientation of the block mask: row = query block, column = key block)."""
    N = 48
    q, k, _, rng = random_qkv(2, 1, N, N, seed=11, dtype="f32")
    v = np.broadcast_to(np.eye(N), (2, 1, N, N)).copy()
    causal = mode == "causal"
    key_len = np.array([17, 48], dtype=np.int32) if mode == "padded" else None
    bm = None
    block = 8
    if mode == "blocks":
        bm = np.zeros((6, 6), dtype=np.uint8)
        bm[0, 5] = bm[1, 0] = bm[2, 2] = bm[5, 1] = bm[5, 4] = bm[3, 0] = bm[3, 1] = 1
        bm = bm.reshape(-1)           # row 4 has no active block
    o, lse = oracle.attention_f64(q * 0.2, k, v, 1.0, causal, key_len, bm, block)
    for b in range(2):
        ok = _allowed_matrix(N, b, causal, key_len, bm, block)
        A = o[b, 0]
        assert np.all(A[~ok] == 0.0)
        assert np.all(A[ok] > 0.0)
        rows = ok.any(1)
        np.testing.assert_allclose(A[rows].sum(1), 1.0, rtol=0, atol=1e-14)
        assert np.all(lse[b, 0][~rows] == -np.inf)


def test_fully_masked_rows():
    q, k, v, _ = random_qkv(2, 2, 20, 8, seed=12, dtype="bf16")
    o, lse = oracle.attention_f64(q, k, v, 0.5, False, key_len=np.array([0, 20]))
    assert np.all(o[0] == 0) and np.all(lse[0] == -np.inf)
    assert np.all(np.isfinite(lse[1]))


# ---------------------------------------------------------------- invariances


def test_joint_key_value_permutation_invariance():
    q, k, v, rng = random_qkv(1, 2, 200, 32, seed=13, dtype="bf16")
    o, lse = oracle.attention_f64(q, k, v, 0.2, False)
    p = rng.permutation(200)
    o2, lse2 = oracle.attention_f64(q, k[:, :, p], v[:, :, p], 0.2, False)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)
    # within the valid prefix when keys are padded
    kl = np.array([150], dtype=np.int32)
    o, lse = oracle.attention_f64(q, k, v, 0.2, False, key_len=kl)
    p = np.concatenate([rng.permutation(150), np.arange(150, 200)])
    o2, lse2 = oracle.attention_f64(q, k[:, :, p], v[:, :, p], 0.2, False, key_len=kl)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)


def test_value_affine_equivariance():
    q, k, v, _ = random_qkv(1, 2, 130, 16, seed=14, dtype="bf16")
    o, lse = oracle.attention_f64(q, k, v, 0.25, True)
    o2, lse2 = oracle.attention_f64(q, k, 3.0 * v - 1.5, 0.25, True)
    np.testing.assert_allclose(o2, 3.0 * o - 1.5, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(lse2, lse)


def test_causal_prefix_property():
    q, k, v, _ = random_qkv(1, 2, 257, 16, seed=15, dtype="bf16")
    o, lse = oracle.attention_f64(q, k, v, 0.25, True)
    o2, lse2 = oracle.attention_f64(q[:, :, :100], k[:, :, :100], v[:, :, :100], 0.25, True)
    np.testing.assert_allclose(o2, o[:, :, :100], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse2, lse[:, :, :100], rtol=0, atol=1e-14)


def test_mask_equivalences():
    """key_len = N == no padding; all-ones block mask == dense; a lower-triangular
    block mask with 1-token blocks == causal."""
    N = 140
    q, k, v, _ = random_qkv(2, 1, N, 16, seed=16, dtype="bf16")
    o, lse = oracle.attention_f64(q, k, v, 0.25, False)
    o2, lse2 = oracle.attention_f64(q, k, v, 0.25, False, key_len=np.array([N, N]))
    np.testing.assert_array_equal(o2, o)
    nb = 2
    o3, lse3 = oracle.attention_f64(q, k, v, 0.25, False, block_mask=np.ones(nb * nb), block=128)
    np.testing.assert_array_equal(o3, o)
    oc, lc = oracle.attention_f64(q, k, v, 0.25, True)
    tri = np.tril(np.ones((N, N), dtype=np.uint8)).reshape(-1)
    o4, l4 = oracle.attention_f64(q, k, v, 0.25, False, block_mask=tri, block=1)
    np.testing.assert_array_equal(o4, oc)
    np.testing.assert_array_equal(l4, lc)


def test_lse_normalises_the_softmax():
    """sum_j exp(S_ij - LSE_i) = 1 over the allowed keys."""
    q, k, v, _ = random_qkv(1, 1, 90, 32, seed=17, dtype="bf16")
    _, lse = oracle.attention_f64(q, k, v, 0.3, True)
    S = 0.3 * q[0, 0].astype(np.float64) @ k[0, 0].astype(np.float64).T
    S[np.triu_indices(90, 1)] = -np.inf
    np.testing.assert_allclose(np.exp(S - lse[0, 0][:, None]).sum(1), 1.0, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- library cross-check


@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks"])
def test_matches_torch_float64_softmax(mode):
    """torch CPU float64 softmax(QK^T*scale + mask) @ V as a library cross-check."""
    torch = pytest.importorskip("torch")
    B, H, N, d = 2, 3, 260, 64
    q, k, v, rng = random_qkv(B, H, N, d, seed=18, dtype="bf16")
    causal = mode == "causal"
    key_len = np.array([200, 131], dtype=np.int32) if mode == "padded" else None
    bm = band_global_block_mask(3, rng, n_global=1) if mode == "blocks" else None
    o, lse = oracle.attention_f64(q, k, v, 0.125, causal, key_len, bm, 128)
    tq, tk, tv = (torch.from_numpy(x.astype(np.float64)) for x in (q, k, v))
    s = (tq @ tk.transpose(-1, -2)) * 0.125
    for b in range(B):
        ok = torch.from_numpy(_allowed_matrix(N, b, causal, key_len, bm, 128))
        s[b] = s[b].masked_fill(~ok, -math.inf)
    ref = torch.softmax(s, -1) @ tv
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-12)


def test_rows_entry_matches_full_evaluation():
    q, k, v, rng = random_qkv(2, 2, 200, 32, seed=19, dtype="bf16")
    kl = np.array([150, 200], dtype=np.int32)
    bm = band_global_block_mask(2, rng, n_global=0)
    o, lse = oracle.attention_f64(q, k, v, 0.2, True, kl, bm, 128)
    rows = rng.choice(2 * 2 * 200, 60, replace=False)
    orow, lrow = oracle.attention_rows_f64(q, k, v, rows, 0.2, True, kl, bm, 128)
    np.testing.assert_array_equal(orow, o.reshape(-1, 32)[rows])
    np.testing.assert_array_equal(lrow, lse.reshape(-1)[rows])


# ---------------------------------------------------------------- grouped-query attention
# Query heads share key/value heads in consecutive groups of H / H_kv (page on
# FlashAttention-2 adoption, tcdigital.jp, section on the synergy with MQA/GQA).


@pytest.mark.parametrize("H,H_kv", [(4, 2), (6, 3), (4, 1), (3, 3)])
@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks"])
def test_gqa_brute_force_tiny(H, H_kv, mode):
    """Grouped heads against the 40-digit brute force (which maps query head h
    to key/value head h // (H // H_kv) in its own loop)."""
    N, d = 5, 3
    q, _, _, rng = random_qkv(2, H, N, d, seed=300 + H + 10 * H_kv, dtype="f32")
    _, k, v, rng = random_qkv(2, H_kv, N, d, seed=400 + H + 10 * H_kv, dtype="f32", rng=rng)
    key_len = rng.integers(0, N, size=2, endpoint=True) if mode == "padded" else None
    bm = (rng.random(9) < 0.6).astype(np.uint8) if mode == "blocks" else None
    o, lse = oracle.attention_f64(q, k, v, 0.7, mode == "causal", key_len, bm, 2)
    O, L = brute.attention_mp(q, k, v, 0.7, mode == "causal", key_len, bm, 2)
    O, L = np.array(O, dtype=np.float64), np.array(L, dtype=np.float64)
    np.testing.assert_allclose(o, O, rtol=0, atol=1e-13)
    fin = np.isfinite(L)
    np.testing.assert_allclose(lse[fin], L[fin], rtol=0, atol=1e-13)
    assert np.all(lse[~fin] == -np.inf)


def test_gqa_equals_multi_head_with_repeated_key_values():
    """Each key/value head repeated over its group of consecutive query heads
    turns the grouped problem into plain multi-head attention."""
    B, H, H_kv, N, d = 2, 8, 2, 70, 16
    q, _, _, rng = random_qkv(B, H, N, d, seed=31, dtype="bf16")
    _, k, v, rng = random_qkv(B, H_kv, N, d, seed=32, dtype="bf16", rng=rng)
    kl = np.array([50, 70], dtype=np.int32)
    o, lse = oracle.attention_f64(q, k, v, 0.25, True, kl)
    kr, vr = np.repeat(k, H // H_kv, axis=1), np.repeat(v, H // H_kv, axis=1)
    o2, lse2 = oracle.attention_f64(q, kr, vr, 0.25, True, kl)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    rows = rng.choice(B * H * N, 40, replace=False)
    orow, lrow = oracle.attention_rows_f64(q, k, v, rows, 0.25, True, kl)
    np.testing.assert_array_equal(orow, o.reshape(-1, d)[rows])
    np.testing.assert_array_equal(lrow, lse.reshape(-1)[rows])


def test_gqa_rejects_bad_head_counts():
    q, k, v, _ = random_qkv(1, 4, 8, 4, seed=5, dtype="f32")
    with pytest.raises(ValueError):
        oracle.attention_f64(q, k[:, :3], v[:, :3], 0.5)
