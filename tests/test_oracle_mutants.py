"""The oracle's pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a temporary copy of oracle/attn_ref.c (a
dropped scale, an off-by-one mask, a transposed block mask, a dropped
normalisation, a wrong operand, a sign error, ..., and the same kinds of
mistakes in the gradient code), builds it with gcc, swaps
it in for the real oracle and runs a few fast pins from test_oracle.py.  At
least one pin has to fail for every mutant.  CPU only.
"""
import ctypes
import os
import shutil
import subprocess

import pytest

import oracle
from oracle import build as obuild
import test_oracle as pins
import test_oracle_bwd as bwd_pins

MUTANTS = {
    "dropped_scale": ("s[j] = scale * dot;", "s[j] = dot;"),
    "causal_off_by_one": ("if (causal && j > i) return 0;", "if (causal && j >= i) return 0;"),
    "key_len_off_by_one": ("j >= (int64_t)key_len[b]", "j > (int64_t)key_len[b]"),
    "block_mask_transposed": ("block_mask[(i / blk) * nkb + (j / blk)]",
                              "block_mask[(j / blk) * nkb + (i / blk)]"),
    "no_normalisation": ("s[j] /= l;", "s[j] /= 1.0;"),
    "lse_without_max": ("*lse = m + log(l);", "*lse = log(l);"),
    "keys_as_values": ("softmax_row_times_v(S + i * N, vh,", "softmax_row_times_v(S + i * N, kh,"),
    "sign_error": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "masked_row_unguarded": ("if (m == -INFINITY) {", "if (0) {"),
    "dot_index": ("dot += qi[c] * kj[c];", "dot += qi[c] * kj[0];"),
    "value_index": ("o[c] += s[j] * vj[c];", "o[c] += s[j] * vj[0];"),
    "kv_heads_interleaved": ("return b * Hkv + h / (H / Hkv);", "return b * Hkv + h % Hkv;"),
    # backward (gradient) mistakes
    "bwd_no_delta": ("A[i * N + j] = a * (da - Dr[i]);", "A[i * N + j] = a * da;"),
    "bwd_dk_unscaled": ("dkh[j * d + c] += scale * ds * qh[i * d + c];",
                        "dkh[j * d + c] += ds * qh[i * d + c];"),
    "bwd_dq_wrong_operand": ("dqh[i * d + c] += scale * ds * kh[j * d + c];",
                             "dqh[i * d + c] += scale * ds * vh[j * d + c];"),
    "bwd_dv_wrong_row": ("dvh[j * d + c] += a * doh[i * d + c];", "dvh[j * d + c] += a * doh[j * d + c];"),
    "bwd_delta_sign": ("A[i * N + j] = a * (da - Dr[i]);", "A[i * N + j] = a * (da + Dr[i]);"),
}

FAST_PINS = [
    pins.test_hand_derived_three_keys,
    pins.test_stored_brute_force_values,
    pins.test_fully_masked_rows,
    lambda: pins.test_identity_values_expose_attention_matrix("blocks"),
    lambda: pins.test_identity_values_expose_attention_matrix("padded"),
    pins.test_gqa_equals_multi_head_with_repeated_key_values,
    lambda: bwd_pins.test_gradients_match_finite_differences(1, 1, "causal"),
    lambda: bwd_pins.test_key_and_value_shift_invariances("dense"),
    bwd_pins.test_grouped_heads_sum_the_group,
]


@pytest.fixture(scope="module")
def gcc():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return "gcc"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, gcc, tmp_path):
    src = open(obuild.SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found once"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run([gcc, "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(lib), str(path), "-lm"],
                   check=True)
    saved = oracle._lib
    oracle._lib = oracle._configure(ctypes.CDLL(str(lib)))
    caught = []
    try:
        for pin in FAST_PINS:
            try:
                pin()
            except (AssertionError, RuntimeError, ValueError, FloatingPointError):
                caught.append(getattr(pin, "__name__", "lambda"))
    finally:
        oracle._lib = saved
    assert caught, f"no pin caught mutant {name}"


def test_unmutated_oracle_passes_fast_pins():
    for pin in FAST_PINS:
        pin()
