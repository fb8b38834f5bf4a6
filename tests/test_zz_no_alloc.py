"""fa_fwd_noalloc (the forward whose key-range split uses the library's
static scratch instead of a caller workspace) against fa_fwd_ws with a
caller workspace: identical bits on consecutive calls, the second smaller
than the first (the scratch keeps the first call's partials), and within the
bf16 bar of the FP64 oracle on sampled rows."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import io_aware_exact_03_amd as fa  # noqa: E402
import oracle  # noqa: E402
from workloads import random_qkv, band_global_block_mask  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f16": 4e-3}
TOL_LSE = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs(B, H, N, d, seed, dtype, causal, key_len=None, block_mask=None):
    q, k, v, _ = random_qkv(B, H, N, d, seed, dtype, 0.5)
    return dict(q=q, k=k, v=v, causal=causal, scale=np.float32(1.0 / math.sqrt(d)),
                key_len=None if key_len is None else np.asarray(key_len, dtype=np.int32),
                block_mask=None if block_mask is None else np.asarray(block_mask, dtype=np.uint8))


def _call(inp, dtype, entry):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    q, k, v = (torch.from_numpy(inp[n]).to(tdt).cuda() for n in ("q", "k", "v"))
    B, H, N, d = q.shape
    kl = torch.from_numpy(inp["key_len"]).cuda() if inp["key_len"] is not None else None
    bm = torch.from_numpy(inp["block_mask"]).cuda() if inp["block_mask"] is not None else None
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    code = fa.DTYPE_BF16 if dtype == "bf16" else fa.DTYPE_F16
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, H, N, d,
            float(inp["scale"]), inp["causal"], kl.data_ptr() if kl is not None else None,
            bm.data_ptr() if bm is not None else None, stream, code]
    if entry == "noalloc":
        fa.fa_fwd_noalloc(*args)
    else:
        need = fa.fa_fwd_workspace_size(B, H, N, d, code)
        ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device="cuda")  # NaN bytes
        fa.fa_fwd_ws(*args, ws.data_ptr(), ws.numel())
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _rows(B, H, N, seed, per_head=24):
    rng = np.random.default_rng(seed)
    rows = []
    for bh in range(B * H):
        pick = {0, 1, 127, 128, N // 2, N - 1} | set(rng.integers(0, N, per_head).tolist())
        rows.extend(bh * N + i for i in sorted(x for x in pick if x < N))
    return np.array(rows, dtype=np.int64)


CASES = [
    # (B, H, N, d, dtype, causal, key_len, block mask?): the first needs the
    # whole scratch (4 shares of 32768 rows at d = 128); later ones are
    # smaller and find the earlier call's partials there
    (1, 2, 16384, 128, "bf16", True, None, False),
    (2, 1, 3000, 64, "bf16", False, [3000, 1700], True),
    (1, 3, 1000, 128, "f16", True, None, False),
    (4, 16, 1024, 64, "bf16", True, None, False),  # 512 query tiles: no split, no scratch
    (1, 4, 16384, 128, "bf16", True, None, False),  # 512 tiles of long causal heads: two shares, the whole scratch
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_matches_workspace_forward(case):
    B, H, N, d, dtype, causal, key_len, blocks = CASES[case]
    print(f"noalloc case {case}: B={B} H={H} N={N} d={d} {dtype} causal={causal}", flush=True)
    nb = (N + 127) // 128
    bm = band_global_block_mask(nb, np.random.default_rng(case), n_global=2) if blocks else None
    inp = _inputs(B, H, N, d, 5000 + case, dtype, causal, key_len, bm)
    code = fa.DTYPE_BF16 if dtype == "bf16" else fa.DTYPE_F16
    assert fa.fa_fwd_workspace_size(B, H, N, d, code) <= fa.NOALLOC_SCRATCH_BYTES
    o_s, lse_s = _call(inp, dtype, "noalloc")
    o_w, lse_w = _call(inp, dtype, "workspace")
    assert torch.equal(o_s.view(torch.int16), o_w.view(torch.int16)), "O differs from fa_fwd_ws"
    assert torch.equal(lse_s.view(torch.int32), lse_w.view(torch.int32)), "LSE differs from fa_fwd_ws"
    rows = _rows(B, H, N, seed=case)
    o_ref, lse_ref = oracle.attention_rows_f64(inp["q"], inp["k"], inp["v"], rows, float(inp["scale"]),
                                               causal, inp["key_len"], inp["block_mask"], 128)
    og = o_s.double().numpy().reshape(-1, d)[rows]
    lg = lse_s.double().numpy().reshape(-1)[rows]
    fin = np.isfinite(lse_ref)
    assert np.all(np.isfinite(og))
    assert np.abs(og[fin] - o_ref[fin]).max() <= TOL[dtype]
    assert np.abs(lg[fin] - lse_ref[fin]).max() <= TOL_LSE
    assert np.all(og[~fin] == 0) and np.all(lg[~fin] == -np.inf)


def test_noalloc_repeated_calls_shrinking():
    """Two calls in a row, the second smaller: each equals its fa_fwd_ws result."""
    big = _inputs(1, 2, 16384, 128, 6001, "bf16", True)
    small = _inputs(1, 1, 5000, 128, 6002, "bf16", True)
    for inp in (big, small):
        o_s, lse_s = _call(inp, "bf16", "noalloc")
        o_w, lse_w = _call(inp, "bf16", "workspace")
        assert torch.equal(o_s.view(torch.int16), o_w.view(torch.int16))
        assert torch.equal(lse_s.view(torch.int32), lse_w.view(torch.int32))
