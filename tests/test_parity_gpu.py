"""GPU parity of the HIP attention path against the FP64 oracle.

Every case draws seeded inputs from ``workloads``, runs the library through
its C ABI (the ctypes binding) and compares element by element with the
oracle on the same values.  Bars: max|dO| <= 1e-5 for the fp32 path,
max|dO| <= 2e-2 for bf16 I/O with fp32 accumulation, |dLSE| <= 1e-3; rows
whose oracle LSE is -inf (no allowed key) must be exactly O = 0,
LSE = -inf.  Output buffers are poisoned with NaN before each call so an
unwritten element fails.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import io_aware_exact_03_amd as fa  # noqa: E402
import oracle  # noqa: E402
from workloads import (WORKLOADS, make_inputs, random_qkv, band_global_block_mask, causal_prefix,  # noqa: E402
                       bf16_round, f16_round)

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2
TOL_LSE = 1e-3
# fp16 I/O: O is rounded to fp16 once (half an ulp is <= 2^-11 for |O| < 2,
# <= 2^-10 below 4) and each probability once (relative 2^-11, which moves O
# by at most 2^-11 * max|v| ~ 2.4e-3 for |v| <= 5, far less for random
# signs); 4e-3 covers both with margin.
TOL_F16 = 4e-3


_PREFIX = {}


def long_causal_prefix():
    """Rows 0..2047 of heads 0..3 of the 16K causal workload (drawn once)."""
    if "x" not in _PREFIX:
        _PREFIX["x"] = causal_prefix(WORKLOADS["long_causal"], N=2048, H=4)
    return dict(_PREFIX["x"])


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(dtype, torch.float32)
    return t.to(tdt).cuda()


def run(inp, dtype="bf16", Br=0, Bc=0, scale=None, causal=None, workspace=None):
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    kl = torch.from_numpy(inp["key_len"]).cuda() if inp.get("key_len") is not None else None
    bm = torch.from_numpy(inp["block_mask"]).cuda() if inp.get("block_mask") is not None else None
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    sc = float(inp["scale"] if scale is None else scale)
    cz = inp["causal"] if causal is None else causal
    fa.fwd(q, k, v, causal=cz, key_len=kl, block_mask=bm, scale=sc, Br=Br, Bc=Bc,
           out=out, lse=lse, workspace=workspace)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy()


def garbage_workspace(nbytes):
    """A workspace whose bytes are all 0xFF (NaN as fp32): any partial result
    the split forgets to write shows up as a non-finite output."""
    return torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device="cuda")


def ref(inp, scale=None, causal=None):
    sc = float(np.float32(inp["scale"] if scale is None else scale))
    return oracle.attention_f64(inp["q"], inp["k"], inp["v"], sc,
                                inp["causal"] if causal is None else causal,
                                inp.get("key_len"), inp.get("block_mask"), 128)


def check(o, lse, o_ref, lse_ref, tol, what=""):
    fin = np.isfinite(lse_ref)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    if fin.any():
        err = np.abs(o[fin] - o_ref[fin]).max()
        lerr = np.abs(lse[fin] - lse_ref[fin]).max()
        assert err <= tol, f"{what}: max|dO| = {err:.3e} > {tol}"
        assert lerr <= TOL_LSE, f"{what}: max|dLSE| = {lerr:.3e} > {TOL_LSE}"
    assert np.all(lse[~fin] == -np.inf), f"{what}: fully masked rows need LSE = -inf"
    assert np.all(o[~fin] == 0.0), f"{what}: fully masked rows need O = 0"
    return float(np.abs(o - o_ref).max()) if o.size else 0.0


def custom(B, H, N, d, seed, dtype="bf16", causal=False, key_len=None, block_mask=None,
           scale=None, amp=1.0):
    q, k, v, _ = random_qkv(B, H, N, d, seed, dtype, amp)
    return dict(q=q, k=k, v=v, causal=causal,
                key_len=None if key_len is None else np.asarray(key_len, dtype=np.int32),
                block_mask=None if block_mask is None else np.asarray(block_mask, dtype=np.uint8),
                scale=np.float32(1.0 / math.sqrt(d) if scale is None else scale))


def modes_for(N, seed):
    rng = np.random.default_rng(seed)
    nb = (N + 127) // 128
    return {
        "dense": dict(causal=False),
        "causal": dict(causal=True),
        "padded": dict(causal=False, key_len=[max(1, N // 3), N]),
        "blocks": dict(causal=False, block_mask=band_global_block_mask(nb, rng, n_global=1)),
        "all": dict(causal=True, key_len=[N, max(1, N - 5)],
                    block_mask=band_global_block_mask(nb, rng, n_global=1)),
    }


# ---------------------------------------------------------------- fp32 path


def test_tiny_f32_workload():
    inp = make_inputs(WORKLOADS["tiny_f32"])
    o, lse = run(inp, "f32")
    check(o, lse, *ref(inp), TOL_F32, "tiny_f32")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 45, 300])
@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks", "all"])
def test_f32_modes(d, N, mode):
    inp = custom(2, 2, N, d, seed=N + d, dtype="f32", **modes_for(N, N)[mode])
    o, lse = run(inp, "f32")
    check(o, lse, *ref(inp), TOL_F32, f"f32 d={d} N={N} {mode}")


# ---------------------------------------------------------------- bf16 path


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 7, 129, 300, 1000])
@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks", "all"])
def test_bf16_modes(d, N, mode):
    inp = custom(2, 3, N, d, seed=10 * N + d, **modes_for(N, N + 1)[mode])
    o, lse = run(inp)
    check(o, lse, *ref(inp), TOL_BF16, f"bf16 d={d} N={N} {mode}")


def test_gpt2_causal_workload_full():
    inp = make_inputs(WORKLOADS["gpt2_causal"])
    o, lse = run(inp)
    check(o, lse, *ref(inp), TOL_BF16, "gpt2_causal")


def test_bert_padded_workload_full():
    inp = make_inputs(WORKLOADS["bert_padded"])
    o, lse = run(inp)
    check(o, lse, *ref(inp), TOL_BF16, "bert_padded")


def sample_rows(B, H, N, seed, per_head=48):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 3, 31, 32, 63, 64, 127, 128, 129, N // 2, N - 2, N - 1]
    rows = []
    for bh in range(B * H):
        pick = set(i for i in fixed if i < N) | set(rng.integers(0, N, per_head).tolist())
        rows.extend(bh * N + i for i in sorted(pick))
    return np.array(rows, dtype=np.int64)


@pytest.mark.parametrize("name", ["long_causal", "block_sparse"])
def test_large_workloads_sampled_rows(name):
    w = WORKLOADS[name]
    inp = make_inputs(w)
    o, lse = run(inp)
    rows = sample_rows(w.B, w.H, w.N, seed=w.seed)
    o_ref, lse_ref = oracle.attention_rows_f64(inp["q"], inp["k"], inp["v"], rows,
                                               float(inp["scale"]), inp["causal"],
                                               inp["key_len"], inp["block_mask"], 128)
    check(o.reshape(-1, w.d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, TOL_BF16, name)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("name", ["long_causal", "block_sparse"])
def test_large_workloads_full(name, dtype):
    """Every row of O and LSE of the two long workloads (16K causal d = 128;
    4K block-sparse d = 64 with its seeded mask) against the full FP64
    oracle, on the same launch configuration the benchmark times; in bf16
    (the workloads' type) and with the same draws rounded to fp16 instead
    (the tuned kernel's fp16 instances, fp16 bar)."""
    w = WORKLOADS[name]
    inp = make_inputs(w)
    if dtype == "f16":
        for n in ("q", "k", "v"):
            inp[n] = f16_round(inp[n])
    o, lse = run(inp, dtype=dtype)
    o_ref, lse_ref = ref(inp)
    err = check(o, lse, o_ref, lse_ref, TOL_BF16 if dtype == "bf16" else TOL_F16, f"{name} {dtype}")
    fin = np.isfinite(lse_ref)
    print(f"{name} {dtype}: full comparison over {o.size} outputs: max|dO| = {err:.3e}, "
          f"max|dLSE| = {np.abs(lse[fin] - lse_ref[fin]).max():.3e}", flush=True)
    assert fin.all(), "every row of these workloads sees at least one key"


def _raw_call(entry, inp, dtype, lse_on=True):
    """Calls a named C entry point directly (pointers and sizes only)."""
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    B, H, N, d = q.shape
    kl = torch.from_numpy(inp["key_len"]).cuda() if inp.get("key_len") is not None else None
    bm = torch.from_numpy(inp["block_mask"]).cuda() if inp.get("block_mask") is not None else None
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr() if lse_on else None,
            B, H, N, d, float(inp["scale"]), bool(inp["causal"]),
            kl.data_ptr() if kl is not None else None, bm.data_ptr() if bm is not None else None, stream]
    if entry == "fa_fwd_ex":
        fa.fa_fwd_ex(*args, fa.DTYPE_F32 if dtype == "f32" else fa.DTYPE_BF16, 0, 0)
    else:
        getattr(fa, entry)(*args)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("dtype,entry", [("bf16", "fa_fwd"), ("f32", "fa_fwd_f32")])
@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks", "all"])
@pytest.mark.parametrize("d", [64, 128])
def test_named_entry_points(dtype, entry, mode, d):
    """fa_fwd and fa_fwd_f32 themselves: within the bar of the oracle and
    bit-identical to fa_fwd_ex with the default tile."""
    N = 300
    inp = custom(2, 3, N, d, seed=700 + d, dtype=dtype, **modes_for(N, 701)[mode])
    o, lse = _raw_call(entry, inp, dtype)
    o_ex, lse_ex = _raw_call("fa_fwd_ex", inp, dtype)
    assert torch.equal(o.view(torch.int16 if dtype == "bf16" else torch.int32),
                       o_ex.view(torch.int16 if dtype == "bf16" else torch.int32)), entry
    assert torch.equal(lse.view(torch.int32), lse_ex.view(torch.int32)), entry
    check(o.double().numpy(), lse.double().numpy(), *ref(inp), TOL_BF16 if dtype == "bf16" else TOL_F32,
          f"{entry} d={d} {mode}")
    # lse = NULL: O is unchanged and the LSE buffer is left as it was
    o2, lse2 = _raw_call(entry, inp, dtype, lse_on=False)
    assert torch.equal(o2.view(torch.int16 if dtype == "bf16" else torch.int32),
                       o.view(torch.int16 if dtype == "bf16" else torch.int32))
    assert torch.isnan(lse2).all()


@pytest.mark.parametrize("N,d,causal", [(65536, 128, True), (65533, 64, False), (40000, 128, True)])
def test_very_long_sequences_sampled_rows(N, d, causal):
    """Single-head sequences up to 64K tokens (the longest context the
    FlashAttention summary page reports, Path-256), ragged lengths included;
    checked on sampled rows, with the tile-study kernel on the same input."""
    inp = custom(1, 1, N, d, seed=90 + d, causal=causal, amp=0.5)
    rows = sample_rows(1, 1, N, seed=91, per_head=24)
    o_ref, lse_ref = oracle.attention_rows_f64(inp["q"], inp["k"], inp["v"], rows,
                                               float(inp["scale"]), causal, None, None, 128)
    o, lse = run(inp)
    check(o.reshape(-1, d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, TOL_BF16, f"N={N} d={d}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    if d == 128:
        o, lse = run(inp, Br=64, Bc=128)
        check(o.reshape(-1, d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, TOL_BF16,
              f"N={N} tile study")


# Causal grids whose work orders take every branch of the CU-balanced order.
CAUSAL_ORDER_SHAPES = [(4, 24, 512),    # 48 items per XCD: a full round, then a partial one kept in order
               (8, 16, 512),    # 64 per XCD: the second round dealt in reverse
               (1, 4, 2048),    # one head spans two XCDs
               (2, 5, 1536),    # 15 per XCD, heads of 12 items: shares do not hold whole heads
               (1, 3, 640)]     # 15 workgroups, not a multiple of the 8 XCDs


@pytest.mark.parametrize("B,H,N", CAUSAL_ORDER_SHAPES)
def test_causal_work_orders(B, H, N):
    """Every (head, query tile) of a causal grid is computed exactly once
    whatever branch of the work order the grid size selects (outputs start
    as NaN, so a tile left out shows)."""
    inp = custom(B, H, N, 64, seed=97 + N + H, causal=True)
    check(*run(inp), *ref(inp), TOL_BF16, f"B{B} H{H} N{N}")


def _multi_chunk_mask(nb):
    """Block-mask rows of five kinds, cycling with the query block: active
    blocks only in the last 64-block chunk, only in the middle chunk, none,
    a few straddling the chunk boundaries, and every 7th block."""
    m = np.zeros((nb, nb), dtype=np.uint8)
    for r in range(nb):
        kind = r % 5
        if kind == 0:
            m[r, nb - 2:] = 1
        elif kind == 1:
            m[r, 64 + r % (nb - 64)] = 1
        elif kind == 3:
            m[r, [r, 63, 64, 127, nb - 1]] = 1
        elif kind == 4:
            m[r, ::7] = 1
    return m.reshape(-1)


@pytest.mark.parametrize("d,causal", [(64, False), (64, True), (128, False), (128, True)])
def test_block_mask_rows_over_several_chunks(d, causal):
    """A 16640-token head has 130 mask blocks per row, which the kernels scan
    in chunks of 64: rows whose first active block lies in the second or
    third chunk, empty rows and rows straddling chunk boundaries, direct and
    with the key-range split (whose shares start inside later chunks);
    checked on sampled rows of every row kind."""
    N = 16640
    nb = N // 128
    inp = custom(1, 1, N, d, seed=95 + d, causal=causal, amp=0.5, block_mask=_multi_chunk_mask(nb))
    blocks = [0, 1, 2, 3, 4, 5, 63, 64, 65, 66, 67, 127, 128, 129]
    rows = np.array(sorted({min(N - 1, r * 128 + o) for r in blocks for o in (0, 77, 127)}), dtype=np.int64)
    o_ref, lse_ref = oracle.attention_rows_f64(inp["q"], inp["k"], inp["v"], rows, float(inp["scale"]), causal,
                                               None, inp["block_mask"], 128)
    assert np.isinf(lse_ref).any() and np.isfinite(lse_ref).any()
    need = fa.fa_fwd_workspace_size(1, 1, N, d, fa.DTYPE_BF16)
    assert need > 0
    for ws in (None, garbage_workspace(need)):
        o, lse = run(inp, workspace=ws)
        check(o.reshape(-1, d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, TOL_BF16,
              f"d={d} causal={causal} split={ws is not None}")


def test_block_mask_rows_past_four_chunks():
    """A 33024-token head (258 mask blocks per row, five 64-block chunks) at
    d = 64 without the causal mask: the tuned kernel there counts a row's
    active blocks over its first four chunks to set the waves' issue
    priority, so rows whose only active blocks lie past block 255 (and rows
    with none) must still be computed in full; sampled rows of every row
    kind, direct and with the key-range split."""
    N, d = 33024, 64
    nb = N // 128
    inp = custom(1, 1, N, d, seed=97, causal=False, amp=0.5, block_mask=_multi_chunk_mask(nb))
    assert inp["block_mask"].reshape(nb, nb)[0, :256].sum() == 0
    blocks = [0, 1, 2, 3, 4, 63, 64, 127, 128, 191, 192, 255, 256, 257]
    rows = np.array(sorted({min(N - 1, r * 128 + o) for r in blocks for o in (0, 127)}), dtype=np.int64)
    o_ref, lse_ref = oracle.attention_rows_f64(inp["q"], inp["k"], inp["v"], rows, float(inp["scale"]), False,
                                               None, inp["block_mask"], 128)
    assert np.isinf(lse_ref).any() and np.isfinite(lse_ref).any()
    need = fa.fa_fwd_workspace_size(1, 1, N, d, fa.DTYPE_BF16)
    for ws in (None, garbage_workspace(need)):
        o, lse = run(inp, workspace=ws)
        check(o.reshape(-1, d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, TOL_BF16,
              f"N={N} split={ws is not None}")


@pytest.mark.parametrize("H,N,Br", [(2, 4096, 0), (1, 4096, 0), (4, 4096, 64), (2, 4096, 32)])
def test_heads_spanning_several_xcds(H, N, Br):
    """Few heads: one head's query tiles are shared round-robin by several
    XCDs (2, 4 or 8 per head); every output against the oracle."""
    inp = custom(1, H, N, 128, seed=95 + H, causal=True, amp=0.5)
    o, lse = run(inp, Br=Br, Bc=64 if Br else 0)
    check(o, lse, *ref(inp), TOL_BF16, f"H={H} N={N} Br={Br}")


@pytest.mark.parametrize("Br", [16, 32, 64, 128])
@pytest.mark.parametrize("Bc", [16, 32, 64, 128])
def test_tile_sweep_slice(Br, Bc):
    """The 16 (Br, Bc) tiles on the first 2048 rows of heads 0-3 of the 16K
    causal workload (a self-contained causal prefix)."""
    inp = long_causal_prefix()
    if "ref" not in _PREFIX:
        _PREFIX["ref"] = ref(inp)
    o, lse = run(inp, Br=Br, Bc=Bc)
    check(o, lse, *_PREFIX["ref"], TOL_BF16, f"sweep Br={Br} Bc={Bc}")


@pytest.mark.parametrize("Br", [16, 32, 64, 128])
@pytest.mark.parametrize("Bc", [16, 32, 64, 128])
@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks", "all"])
def test_tile_study_d64(Br, Bc, mode):
    """The tile-study kernels at d = 64: every (Br, Bc) on a ragged length
    (300 = two full 128-row blocks and a 44-row tail) under every mask."""
    inp = custom(2, 3, 300, 64, seed=80 + Br + Bc, **modes_for(300, 81)[mode])
    o, lse = run(inp, Br=Br, Bc=Bc)
    check(o, lse, *ref(inp), TOL_BF16, f"d=64 Br={Br} Bc={Bc} {mode}")


def run_f32out(inp, Br=0, Bc=0, order=None):
    """bf16 inputs, fp32 output (O before its final rounding): the
    tile-study kernels in FA_DTYPE_BF16_F32OUT mode."""
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    kl = torch.from_numpy(inp["key_len"]).cuda() if inp.get("key_len") is not None else None
    bm = torch.from_numpy(inp["block_mask"]).cuda() if inp.get("block_mask") is not None else None
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    fa.fwd(q, k, v, causal=inp["causal"], key_len=kl, block_mask=bm, scale=float(inp["scale"]), Br=Br, Bc=Bc,
           out=out, lse=lse, tile_order=fa.ORDER_ASCENDING if order is None else order)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Br", [16, 32, 64, 128])
@pytest.mark.parametrize("Bc", [16, 32, 64, 128])
def test_bf16_f32out_tiles(d, Br, Bc):
    """fp32-output mode of the tile-study kernels: within the bf16 bar of the
    oracle, and exactly the bf16-output kernel's result once rounded to bf16
    (round to nearest even), on every (Br, Bc) and two mask mixes."""
    for mode in ("causal", "all"):
        inp = custom(2, 2, 300, d, seed=400 + Br + Bc + d, **modes_for(300, 401)[mode])
        o32, lse32 = run_f32out(inp, Br, Bc)
        check(o32.double().cpu().numpy(), lse32.double().cpu().numpy(), *ref(inp), TOL_BF16,
              f"f32out d={d} Br={Br} Bc={Bc} {mode}")
        o16, lse16 = run(inp, Br=Br, Bc=Bc)
        rounded = o32.to(torch.bfloat16).double().cpu().numpy()
        assert np.array_equal(rounded, o16), f"f32out rounded != bf16 output, d={d} Br={Br} Bc={Bc} {mode}"
        assert np.array_equal(lse32.double().cpu().numpy(), lse16)


def test_bf16_f32out_default_tile_and_orders():
    inp = long_causal_prefix()
    if "ref" not in _PREFIX:
        _PREFIX["ref"] = ref(inp)
    for order in (fa.ORDER_ASCENDING, fa.ORDER_DESCENDING, fa.ORDER_SHUFFLED):
        o, lse = run_f32out(inp, 0 if order == fa.ORDER_ASCENDING else 64, 0 if order == fa.ORDER_ASCENDING else 32,
                            order)
        check(o.double().cpu().numpy(), lse.double().cpu().numpy(), *_PREFIX["ref"], TOL_BF16, f"f32out order {order}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Br", [16, 32, 64, 128])
@pytest.mark.parametrize("Bc", [16, 32, 64, 128])
def test_bf16_acc16_tiles(d, Br, Bc):
    """The study mode that rounds the running output to bf16 after every key
    tile.  Each rounding moves the normalised output by at most u*max|v|
    (u = 2^-8: the partial output never exceeds its row sum times max|v|,
    and later rescaling and the final division only shrink that error), so
    with T key tiles visited the bar is the bf16 bar plus T*u*max|v|; LSE
    is untouched (the row sum stays fp32)."""
    for mode in ("causal", "all"):
        inp = custom(2, 2, 300, d, seed=600 + Br + Bc + d, **modes_for(300, 601)[mode])
        q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
        kl = torch.from_numpy(inp["key_len"]).cuda() if inp.get("key_len") is not None else None
        bm = torch.from_numpy(inp["block_mask"]).cuda() if inp.get("block_mask") is not None else None
        o, lse = fa.fwd(q, k, v, causal=inp["causal"], key_len=kl, block_mask=bm, scale=float(inp["scale"]),
                        Br=Br, Bc=Bc, acc16=True)
        torch.cuda.synchronize()
        tiles = -(-300 // Bc)
        bar = TOL_BF16 + tiles * 2.0 ** -8 * float(np.abs(inp["v"]).max())
        check(o.double().cpu().numpy(), lse.double().cpu().numpy(), *ref(inp), bar, f"acc16 d={d} Br={Br} Bc={Bc} {mode}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Br", [16, 32, 64, 128])
@pytest.mark.parametrize("Bc", [16, 32, 64, 128])
def test_f32_tiles(d, Br, Bc):
    """The fp32 kernels at every (Br, Bc): within 1e-5 of the oracle on a
    ragged length under every mask mix."""
    for mode in ("dense", "causal", "padded", "blocks", "all"):
        inp = custom(2, 2, 300, d, seed=500 + Br + Bc + d, dtype="f32", **modes_for(300, 501)[mode])
        o, lse = run(inp, "f32", Br=Br, Bc=Bc)
        check(o, lse, *ref(inp), TOL_F32, f"f32 d={d} Br={Br} Bc={Bc} {mode}")


# ---------------------------------------------------------------- closed forms on the GPU


@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks"])
def test_zero_query_gives_mean_of_allowed_values(mode):
    N = 300
    inp = custom(2, 2, N, 64, seed=21, **modes_for(N, 3)[mode])
    inp["q"] = np.zeros_like(inp["q"])
    o, lse = run(inp)
    check(o, lse, *ref(inp), TOL_BF16, f"Q=0 {mode}")


def test_dominant_logit_selects_value_row():
    N, d = 256, 64
    inp = custom(1, 2, N, d, seed=22)
    inp["k"][..., 0] = 0.0
    inp["q"][...] = 0.0
    inp["q"][..., 0] = 8.0
    jstar = 77
    inp["k"][:, :, jstar, 0] = 40.0 / (8.0 * 0.125)
    o, lse = run(inp)
    np.testing.assert_allclose(o, np.broadcast_to(inp["v"][:, :, jstar:jstar + 1], o.shape),
                               rtol=0, atol=TOL_BF16)
    np.testing.assert_allclose(lse, 40.0, rtol=0, atol=TOL_LSE)


def _score_profile(name, N):
    """Designed per-key logits (natural-log units, before any max shift)."""
    j = np.arange(N, dtype=np.float64)
    t = j // 64  # key tile of 64
    return {
        # the row max creeps up by ~0.9 (base 2) per key tile: a small
        # rescale of O on almost every tile
        "slow_rise": 0.01 * j,
        # every key tile's max is ~17 (base 2) above the last one's: O and l
        # shrink by ~2^-17 on every tile
        "jumps": 12.0 * t,
        # the first tile holds the max: no rescale after it
        "falling": -0.02 * j,
        # rises, steps and drops mixed
        "sawtooth": 6.0 * (t % 3) + 0.01 * j,
    }[name]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("profile", ["slow_rise", "jumps", "falling", "sawtooth"])
def test_running_maximum_profiles(profile, causal, dtype):
    """Logits whose per-tile maxima rise slowly, jump far from tile to tile,
    fall or alternate, up to ~180 (natural log): the running maximum, the
    rescale (taken or skipped per wave) and the running sum must give the
    oracle's O and LSE whatever path the maxima take, in the direct launch
    and in the key-range split."""
    B, H, N, d = 1, 2, 1024, 64
    rnd = {"bf16": bf16_round, "f16": f16_round}[dtype]
    rng = np.random.default_rng(40 + len(profile))
    q = 0.3 * rng.standard_normal((B, H, N, d))
    k = 0.3 * rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    scale = 0.125
    q[..., 0] = 8.0  # q . k ~ 8 * k[..., 0], times the scale: logit ~ k[..., 0]
    k[..., 0] = _score_profile(profile, N)
    inp = dict(q=rnd(q.astype(np.float32)), k=rnd(k.astype(np.float32)), v=rnd(v.astype(np.float32)),
               causal=causal, key_len=None, block_mask=None, scale=np.float32(scale))
    tol = TOL_BF16 if dtype == "bf16" else TOL_F16
    want = ref(inp)
    check(*run(inp, dtype), *want, tol, f"{profile} {dtype}")
    need = fa.fa_fwd_workspace_size(B, H, N, d, fa.DTYPE_BF16 if dtype == "bf16" else fa.DTYPE_F16)
    assert need > 0
    check(*run(inp, dtype, workspace=garbage_workspace(need)), *want, tol, f"{profile} {dtype} split")


def test_ones_value_column_gives_ones():
    """Rows of A sum to one, so a V column of ones gives an O column of ones
    (up to the bf16 rounding of P against the fp32 row sum)."""
    inp = custom(2, 2, 500, 128, seed=23, causal=True)
    inp["v"][..., 5] = 1.0
    o, _ = run(inp)
    assert np.abs(o[..., 5] - 1.0).max() <= 2.0 ** -7
    inp32 = custom(2, 2, 500, 128, seed=23, dtype="f32", causal=True)
    inp32["v"][..., 5] = 1.0
    o, _ = run(inp32, "f32")
    assert np.abs(o[..., 5] - 1.0).max() <= 1e-6


def test_fully_masked_rows():
    N = 200
    bm = np.ones((2, 2), dtype=np.uint8)
    bm[1, :] = 0                       # query block 1 sees nothing
    inp = custom(2, 2, N, 64, seed=24, key_len=[0, N], block_mask=bm.reshape(-1))
    o, lse = run(inp)
    assert np.all(o[0] == 0) and np.all(lse[0] == -np.inf)
    assert np.all(o[1, :, 128:] == 0) and np.all(lse[1, :, 128:] == -np.inf)
    check(o, lse, *ref(inp), TOL_BF16, "fully masked")


def test_key_value_permutation_invariance():
    N = 384
    inp = custom(1, 2, N, 64, seed=25)
    o, lse = run(inp)
    p = np.random.default_rng(0).permutation(N)
    inp2 = dict(inp, k=inp["k"][:, :, p].copy(), v=inp["v"][:, :, p].copy())
    o2, lse2 = run(inp2)
    assert np.abs(o2 - o).max() <= TOL_BF16
    assert np.abs(lse2 - lse).max() <= TOL_LSE


def test_causal_prefix_property():
    inp = custom(1, 2, 700, 128, seed=26, causal=True)
    o, lse = run(inp)
    short = dict(inp, q=inp["q"][:, :, :300].copy(), k=inp["k"][:, :, :300].copy(),
                 v=inp["v"][:, :, :300].copy())
    o2, lse2 = run(short)
    np.testing.assert_array_equal(o2, o[:, :, :300])
    np.testing.assert_array_equal(lse2, lse[:, :, :300])


def test_mask_equivalences():
    N = 256
    inp = custom(2, 2, N, 64, seed=27)
    o, lse = run(inp)
    o2, lse2 = run(dict(inp, key_len=np.array([N, N], dtype=np.int32)))
    o3, lse3 = run(dict(inp, block_mask=np.ones(4, dtype=np.uint8)))
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(o3, o)
    np.testing.assert_array_equal(lse3, lse)


def test_deterministic_bits():
    inp = make_inputs(WORKLOADS["gpt2_causal"], B=2)
    o1, l1 = run(inp)
    o2, l2 = run(inp)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 1.7])
def test_nonstandard_scales(scale):
    inp = custom(1, 2, 150, 64, seed=28, causal=True)
    o, lse = run(inp, scale=scale)
    check(o, lse, *ref(inp, scale=scale), TOL_BF16, f"scale={scale}")
    o, lse = run(inp, "f32", scale=scale)
    check(o, lse, *ref(inp, scale=scale), TOL_F32, f"f32 scale={scale}")


def test_adjacent_output_buffers():
    """LSE placed directly before O in one allocation is a valid layout."""
    inp = custom(2, 3, 100, 64, seed=30)
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    n_lse = 2 * 3 * 100
    raw = torch.empty(n_lse * 4 + q.numel() * 2, dtype=torch.uint8, device="cuda")
    lse = raw[: n_lse * 4].view(torch.float32).view(2, 3, 100)
    out = raw[n_lse * 4:].view(torch.bfloat16).view(q.shape)
    fa.fwd(q, k, v, out=out, lse=lse)
    torch.cuda.synchronize()
    check(out.double().cpu().numpy(), lse.double().cpu().numpy(), *ref(inp), TOL_BF16, "adjacent")


def test_no_lse_requested():
    inp = custom(1, 1, 100, 64, seed=29)
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, lse=False)
    torch.cuda.synchronize()
    assert lse is None
    o_ref, _ = ref(inp)
    assert np.abs(o.double().cpu().numpy() - o_ref).max() <= TOL_BF16


# ---------------------------------------------------------------- grouped-query attention


def gqa_custom(B, H, H_kv, N, d, seed, dtype="bf16", **kw):
    inp = custom(B, H, N, d, seed, dtype=dtype, **kw)
    _, k, v, _ = random_qkv(B, H_kv, N, d, seed + 1000, dtype)
    inp["k"], inp["v"] = k, v
    return inp


@pytest.mark.parametrize("H,H_kv", [(8, 2), (4, 1)])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks", "all"])
def test_gqa_bf16(H, H_kv, d, mode):
    N = 300
    inp = gqa_custom(2, H, H_kv, N, d, seed=40 + H + d, **modes_for(N, 41)[mode])
    o, lse = run(inp)
    check(o, lse, *ref(inp), TOL_BF16, f"gqa H={H} H_kv={H_kv} d={d} {mode}")


@pytest.mark.parametrize("B,H,H_kv,N,d", [(8, 8, 2, 512, 128), (16, 4, 4, 512, 64), (8, 16, 16, 640, 64),
                                         (16, 16, 16, 512, 128)])
def test_key_padded_unit_order(B, H, H_kv, N, d):
    """Key-padded grids whose per-XCD shares hold whole key/value-head units,
    so the tuned kernels deal the units to the XCDs round-robin (grouped
    heads, a ragged N, both head sizes); ragged key lengths with an entry
    that has no key and one that has all; every output against the
    oracle."""
    rng = np.random.default_rng(420 + B + H + d)
    kl = rng.integers(1, N + 1, B)
    kl[0], kl[-1] = 0, N
    inp = gqa_custom(B, H, H_kv, N, d, seed=421 + d, key_len=kl)
    o, lse = run(inp)
    check(o, lse, *ref(inp), TOL_BF16, f"B={B} H={H} H_kv={H_kv} N={N} d={d}")


@pytest.mark.parametrize("Br,Bc", [(64, 32), (16, 128)])
def test_gqa_tile_study_kernels(Br, Bc):
    inp = gqa_custom(1, 6, 3, 200, 128, seed=42, causal=True)
    o, lse = run(inp, Br=Br, Bc=Bc)
    check(o, lse, *ref(inp), TOL_BF16, f"gqa Br={Br} Bc={Bc}")


def test_gqa_f32():
    inp = gqa_custom(2, 4, 2, 150, 64, seed=43, dtype="f32", causal=True)
    o, lse = run(inp, "f32")
    check(o, lse, *ref(inp), TOL_F32, "gqa f32")


def test_gqa_matches_repeated_key_values_bitwise():
    """The grouped call and a plain call on key/value heads repeated over each
    group run the same arithmetic, so the results agree bit for bit."""
    inp = gqa_custom(2, 8, 2, 333, 128, seed=44, causal=True)
    o, lse = run(inp)
    rep = dict(inp, k=np.repeat(inp["k"], 4, axis=1), v=np.repeat(inp["v"], 4, axis=1))
    o2, lse2 = run(rep)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


# ---------------------------------------------------------------- fp16 I/O


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 129, 300])
@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks", "all"])
def test_f16_modes(d, N, mode):
    inp = custom(2, 2, N, d, seed=50 + N + d, dtype="f16", **modes_for(N, 51)[mode])
    o, lse = run(inp, "f16")
    check(o, lse, *ref(inp), TOL_F16, f"f16 d={d} N={N} {mode}")


def test_f16_gqa_and_negative_scale():
    inp = gqa_custom(1, 4, 2, 200, 128, seed=52, dtype="f16", causal=True)
    o, lse = run(inp, "f16", scale=-0.1)
    check(o, lse, *ref(inp, scale=-0.1), TOL_F16, "f16 gqa scale=-0.1")


def test_f16_long_causal_slice():
    """The 16K causal workload's B1 H4 N2048 prefix, rounded to fp16."""
    inp = causal_prefix(WORKLOADS["long_causal"], N=2048, H=4, fmt="f16")
    o, lse = run(inp, "f16")
    check(o, lse, *ref(inp), TOL_F16, "f16 long_causal slice")


# ---------------------------------------------------------------- tile order (deviation study)


@pytest.mark.parametrize("order", ["descending", "shuffled"])
@pytest.mark.parametrize("Br,Bc", [(16, 16), (64, 32), (128, 128)])
@pytest.mark.parametrize("N,d", [(300, 128), (1000, 128), (300, 64)])
@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks", "all"])
def test_nonascending_tile_order(order, Br, Bc, N, d, mode):
    # key-tile counts per workgroup span 1 .. 63, odd and even (the shuffled
    # visit map must be a permutation of each count)
    inp = custom(2, 2, N, d, seed=60 + N + Br, **modes_for(N, 61)[mode])
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    kl = torch.from_numpy(inp["key_len"]).cuda() if inp.get("key_len") is not None else None
    bm = torch.from_numpy(inp["block_mask"]).cuda() if inp.get("block_mask") is not None else None
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    fa.fwd(q, k, v, causal=inp["causal"], key_len=kl, block_mask=bm, scale=float(inp["scale"]),
           Br=Br, Bc=Bc, out=out, lse=lse, tile_order=ORDERS[order])
    torch.cuda.synchronize()
    check(out.double().cpu().numpy(), lse.double().cpu().numpy(), *ref(inp), TOL_BF16,
          f"{order} Br={Br} Bc={Bc} N={N} d={d} {mode}")


ORDERS = {"descending": fa.ORDER_DESCENDING, "shuffled": fa.ORDER_SHUFFLED}


@pytest.mark.parametrize("order", ["descending", "shuffled"])
def test_nonascending_tile_order_fully_masked_rows(order):
    inp = custom(2, 2, 200, 128, seed=62, key_len=[0, 130])
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    kl = torch.from_numpy(inp["key_len"]).cuda()
    out, lse = fa.fwd(q, k, v, key_len=kl, Br=32, Bc=64, tile_order=ORDERS[order])
    torch.cuda.synchronize()
    check(out.double().cpu().numpy(), lse.double().cpu().numpy(), *ref(inp), TOL_BF16, f"{order} masked")



# ---------------------------------------------------------------- key-range split (fa_fwd_ws)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 129, 300, 1000])
@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks", "all"])
def test_split_forward_modes(d, N, mode):
    """Small grids take the split: 2..8 query tiles -> 16 shares, so many
    shares are empty or fully masked (LSE_s = -inf, weight 0)."""
    inp = custom(2, 3, N, d, seed=100 + N + d, **modes_for(N, 101)[mode])
    need = fa.fa_fwd_workspace_size(2, 3, N, d, fa.DTYPE_BF16)
    assert need > 0
    o, lse = run(inp, workspace=garbage_workspace(need))
    check(o, lse, *ref(inp), TOL_BF16, f"split d={d} N={N} {mode}")


def test_split_forward_fully_masked_rows():
    inp = custom(2, 2, 200, 128, seed=102, key_len=[0, 130])
    o, lse = run(inp, workspace=True)
    check(o, lse, *ref(inp), TOL_BF16, "split masked")


@pytest.mark.parametrize("d", [64, 128])
def test_split_forward_f16_and_gqa(d):
    inp = custom(1, 4, 777, d, seed=103, dtype="f16", causal=True)
    o, lse = run(inp, dtype="f16", workspace=True)
    check(o, lse, *ref(inp), TOL_F16, f"split f16 d={d}")
    q, k, v, _ = random_qkv(2, 8, 500, d, 104, "bf16")
    k, v = k[:, :2].copy(), v[:, :2].copy()
    tq, tk, tv = (to_dev(x, "bf16") for x in (q, k, v))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = fa.fwd(tq, tk, tv, causal=True, scale=scale, workspace=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_f64(q, k, v, scale, True)
    check(o.double().cpu().numpy(), lse.double().cpu().numpy(), o_ref, l_ref, TOL_BF16, "split gqa")


@pytest.mark.parametrize("H,N,d,causal", [(2, 16384, 128, True), (1, 32768, 128, True), (2, 16384, 64, False),
                                           (4, 16384, 128, True), (4, 16384, 64, True), (4, 16384, 128, False)])
def test_split_forward_one_gpu_share_sampled_rows(H, N, d, causal):
    """The one-GPU share of a head-sharded 16K problem, and a single 32K
    head, at full size: sampled rows against the oracle, all rows finite,
    and the whole output within the bar of the unsplit kernel's.  H = 4 is
    a grid of exactly 512 query tiles: split in two with the causal mask,
    unsplit without it (the workspace is then unused)."""
    inp = custom(1, H, N, d, seed=105 + H, causal=causal, amp=0.5)
    need = fa.fa_fwd_workspace_size(1, H, N, d, fa.DTYPE_BF16)
    assert need > 0
    rows = sample_rows(1, H, N, seed=106, per_head=24)
    o_ref, lse_ref = oracle.attention_rows_f64(inp["q"], inp["k"], inp["v"], rows,
                                               float(inp["scale"]), causal, None, None, 128)
    o, lse = run(inp, workspace=garbage_workspace(need))
    check(o.reshape(-1, d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, TOL_BF16, f"split H={H} N={N}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    o1, lse1 = run(inp)
    assert np.abs(o - o1).max() <= TOL_BF16 and np.abs(lse - lse1).max() <= TOL_LSE
