"""The seeded inputs have the structure the workloads promise (CPU only)."""
import numpy as np

import oracle
from workloads import (WORKLOADS, ORDER, make_inputs, band_global_block_mask, bf16_round,
                       causal_prefix, allowed_pairs)


def test_block_sparse_mask_structure():
    inp = make_inputs(WORKLOADS["block_sparse"], B=1, H=1)
    nb = 4096 // 128
    m = inp["block_mask"].reshape(nb, nb)
    assert int(m.sum()) == 222
    for r in range(nb):
        band = [c for c in range(nb) if abs(r - c) <= 1]
        assert all(m[r, c] for c in band)
        outside = [c for c in range(nb) if abs(r - c) > 1 and m[r, c]]
        assert len(outside) == 4


def test_band_mask_without_globals_is_tridiagonal():
    m = band_global_block_mask(6, np.random.default_rng(0), n_global=0).reshape(6, 6)
    i, j = np.indices((6, 6))
    np.testing.assert_array_equal(m, (np.abs(i - j) <= 1).astype(np.uint8))


def test_padding_lengths_in_range():
    kl = make_inputs(WORKLOADS["bert_padded"], H=1, N=512)["key_len"]
    assert kl.shape == (16,) and kl.min() >= 256 and kl.max() <= 512


def test_bf16_workloads_are_representable():
    for key in ORDER:
        w = WORKLOADS[key]
        inp = make_inputs(w, N=64, H=1, B=1)
        if w.dtype == "bf16":
            for n in ("q", "k", "v"):
                np.testing.assert_array_equal(inp[n], bf16_round(inp[n]))


def test_allowed_pairs_counts():
    assert allowed_pairs(4, 1, 1, causal=True) == 10
    assert allowed_pairs(4, 2, 3) == 2 * 3 * 16
    assert allowed_pairs(6, 1, 1, key_len=np.array([3])) == 18


def test_causal_prefix_is_the_full_problems_rows():
    """Rows 0..N-1 of the first heads of the 16K causal workload attend only to
    keys 0..N-1: the slice's exact outputs equal those rows of the full problem."""
    w = WORKLOADS["long_causal"]
    pre = causal_prefix(w, N=256, H=2)
    full = make_inputs(w)
    rng = np.random.default_rng(3)
    h = rng.integers(0, 2, 12)
    i = rng.integers(0, 256, 12)
    rows_full = h * w.N + i
    rows_pre = h * 256 + i
    o_full, l_full = oracle.attention_rows_f64(full["q"], full["k"], full["v"], rows_full,
                                               float(w.scale), True)
    o_pre, l_pre = oracle.attention_rows_f64(pre["q"], pre["k"], pre["v"], rows_pre,
                                             float(w.scale), True)
    np.testing.assert_array_equal(o_full, o_pre)
    np.testing.assert_array_equal(l_full, l_pre)
