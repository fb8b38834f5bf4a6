"""GPU parity of the materialised baseline attention (fa_fwd_baseline)
against the FP64 oracle.

With S and A held in fp32 the baseline meets the same bars as the tiled
kernels (fp32: 1e-5, bf16: 2e-2, fp16: 4e-3, LSE: 1e-3).  With S and A held
in the 16-bit input type each is rounded once more; the bars then follow
from that arithmetic (first order, round to nearest even, relative error
u = 2^-8 for bf16, 2^-11 for fp16):
  * S_ij rounded: each logit moves by at most u*|s_ij|, which moves the
    weights A_ij by a factor within exp(+-2*u*max|s|) and the log-sum-exp by
    at most u*max|s|;
  * A_ij rounded: another factor within 1 +- u;
  * O = sum_j A_ij v_j therefore moves by at most
    (exp(2*u*max|s| + u) - 1) * max|v|, plus half an ulp of O when O is
    rounded to the input type.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import io_aware_exact_03_amd as fa  # noqa: E402
import oracle  # noqa: E402
from workloads import WORKLOADS, make_inputs, random_qkv, band_global_block_mask, causal_prefix  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 4e-3, "bf16_f32out": 2e-2}
TOL_LSE = 1e-3
UNIT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "bf16_f32out": 2.0 ** -8}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def tdt(fmt):
    return {"bf16": torch.bfloat16, "f16": torch.float16, "bf16_f32out": torch.bfloat16}.get(fmt, torch.float32)


def run_baseline(inp, fmt, inter="f32"):
    q, k, v = (torch.from_numpy(np.ascontiguousarray(inp[n])).to(tdt(fmt)).cuda() for n in ("q", "k", "v"))
    kl = torch.from_numpy(inp["key_len"]).cuda() if inp.get("key_len") is not None else None
    bm = torch.from_numpy(inp["block_mask"]).cuda() if inp.get("block_mask") is not None else None
    out_dt = torch.float32 if fmt == "bf16_f32out" else q.dtype
    out = torch.full(q.shape, float("nan"), dtype=out_dt, device="cuda")
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    B, H, N, _ = q.shape
    codes = {"bf16": fa.DTYPE_BF16, "f16": fa.DTYPE_F16, "f32": fa.DTYPE_F32, "bf16_f32out": fa.DTYPE_BF16_F32OUT}
    inter_code = fa.DTYPE_F32 if inter == "f32" else (fa.DTYPE_F16 if fmt == "f16" else fa.DTYPE_BF16)
    need = fa.fa_fwd_baseline_workspace_size(B, H, N, codes[fmt], inter_code)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN bytes
    fa.baseline(q, k, v, causal=inp["causal"], key_len=kl, block_mask=bm, scale=float(inp["scale"]),
                inter=inter, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy()


def ref(inp):
    return oracle.attention_f64(inp["q"], inp["k"], inp["v"], float(np.float32(inp["scale"])), inp["causal"],
                                inp.get("key_len"), inp.get("block_mask"), 128)


def max_abs_logit(inp):
    """max |scale * q_i . k_j| over all pairs (an upper bound over the allowed ones)."""
    q = inp["q"].astype(np.float64)
    k = inp["k"].astype(np.float64)
    s = np.einsum("bhid,bhjd->bhij", q, k) * float(inp["scale"])
    return float(np.abs(s).max())


def bars(inp, fmt, inter):
    if inter == "f32":
        return TOL[fmt], TOL_LSE
    u = UNIT[fmt]
    smax, vmax = max_abs_logit(inp), float(np.abs(inp["v"]).max())
    o_bar = (math.expm1(2 * u * smax + u)) * vmax
    if fmt != "bf16_f32out":
        o_bar += u * vmax  # half an ulp of the rounded output
    return o_bar * 1.01 + 1e-6, u * smax * 1.01 + 1e-5


def check(o, lse, o_ref, lse_ref, tol_o, tol_l, what):
    fin = np.isfinite(lse_ref)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    if fin.any():
        err = np.abs(o[fin] - o_ref[fin]).max()
        lerr = np.abs(lse[fin] - lse_ref[fin]).max()
        assert err <= tol_o, f"{what}: max|dO| = {err:.3e} > {tol_o:.3e}"
        assert lerr <= tol_l, f"{what}: max|dLSE| = {lerr:.3e} > {tol_l:.3e}"
    assert np.all(lse[~fin] == -np.inf), f"{what}: fully masked rows need LSE = -inf"
    assert np.all(o[~fin] == 0.0), f"{what}: fully masked rows need O = 0"


def custom(B, H, N, d, seed, fmt, causal=False, key_len=None, block_mask=None, amp=1.0):
    draw = {"bf16_f32out": "bf16"}.get(fmt, fmt)
    q, k, v, _ = random_qkv(B, H, N, d, seed, draw, amp)
    return dict(q=q, k=k, v=v, causal=causal, scale=np.float32(1.0 / math.sqrt(d)),
                key_len=None if key_len is None else np.asarray(key_len, dtype=np.int32),
                block_mask=None if block_mask is None else np.asarray(block_mask, dtype=np.uint8))


def modes_for(N, seed):
    rng = np.random.default_rng(seed)
    nb = (N + 127) // 128
    return {
        "dense": dict(causal=False),
        "causal": dict(causal=True),
        "padded": dict(causal=False, key_len=[max(1, N // 3), N]),
        "blocks": dict(causal=False, block_mask=band_global_block_mask(nb, rng, n_global=1)),
        "all": dict(causal=True, key_len=[N, max(1, N - 5)], block_mask=band_global_block_mask(nb, rng, n_global=1)),
        "empty": dict(causal=False, key_len=[0, N]),  # batch entry 0: no allowed key anywhere
    }


def test_baseline_tiny_f32_workload():
    inp = make_inputs(WORKLOADS["tiny_f32"])
    o, lse = run_baseline(inp, "f32")
    check(o, lse, *ref(inp), TOL["f32"], TOL_LSE, "tiny_f32 baseline")


@pytest.mark.parametrize("fmt,inter", [("bf16", "f32"), ("bf16", "io"), ("f16", "f32"), ("f16", "io"),
                                       ("f32", "f32"), ("bf16_f32out", "f32"), ("bf16_f32out", "io")])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 7, 129, 300])
@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks", "all", "empty"])
def test_baseline_modes(fmt, inter, d, N, mode):
    inp = custom(2, 2, N, d, seed=31 * N + d, fmt=fmt, **modes_for(N, N + 3)[mode])
    o, lse = run_baseline(inp, fmt, inter)
    check(o, lse, *ref(inp), *bars(inp, fmt, inter), f"baseline {fmt}/{inter} d={d} N={N} {mode}")


@pytest.mark.parametrize("inter", ["f32", "io"])
def test_baseline_long_causal_slice(inter):
    """Rows 0..2047 of heads 0..3 of the 16K causal workload (the deviation
    study's slice)."""
    inp = causal_prefix(WORKLOADS["long_causal"], N=2048, H=4)
    o, lse = run_baseline(inp, "bf16", inter)
    check(o, lse, *ref(inp), *bars(inp, "bf16", inter), f"long_causal slice baseline/{inter}")


@pytest.mark.parametrize("name", ["gpt2_causal", "bert_padded"])
def test_baseline_short_workloads_full(name):
    inp = make_inputs(WORKLOADS[name])
    o, lse = run_baseline(inp, "bf16", "f32")
    check(o, lse, *ref(inp), TOL["bf16"], TOL_LSE, f"{name} baseline")


def test_baseline_long_causal_full_size_sampled():
    """All 16 heads of the 16K causal workload: a 17 GB fp32 score matrix in
    device memory, checked on sampled rows."""
    w = WORKLOADS["long_causal"]
    inp = make_inputs(w)
    o, lse = run_baseline(inp, "bf16", "f32")
    rng = np.random.default_rng(77)
    rows = np.array(sorted(set(rng.integers(0, w.B * w.H * w.N, 400).tolist()) | {0, w.N - 1, w.B * w.H * w.N - 1}),
                    dtype=np.int64)
    o_ref, lse_ref = oracle.attention_rows_f64(inp["q"], inp["k"], inp["v"], rows, float(inp["scale"]), True,
                                               None, None, 128)
    check(o.reshape(-1, w.d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, TOL["bf16"], TOL_LSE,
          "long_causal baseline")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
