"""GPU parity of the HIP backward pass (fa_bwd) against the FP64 backward
oracle, which is the chain rule on the attention definition and is pinned by
finite differences of the forward oracle (tests/test_oracle_bwd.py).

Inputs are seeded bf16 Q, K, V and dO; O and LSE come from the library's own
forward on the same inputs (as in training).  Bar: for each of dQ, dK, dV,
max|g - g_ref| <= 2e-2 * max(1, max|g_ref|): the forward's bf16 tolerance
taken relative to the gradient's scale (P and dS enter the products rounded
to bf16, relative 2^-9 each, and every gradient is rounded to bf16 once).
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import io_aware_exact_03_amd as fa  # noqa: E402
import oracle  # noqa: E402
from workloads import WORKLOADS, make_inputs, random_qkv, band_global_block_mask  # noqa: E402

pytestmark = pytest.mark.gpu

TOL_REL = 2e-2
# fp16 I/O: P, dS and the gradients are rounded to fp16 (relative 2^-11,
# four times finer than bf16's 2^-9), and O and dO carry fp16 rounding; the
# bf16 bar scaled by the same 2^-2, rounded up to one significant digit.
TOL_REL_F16 = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev(x, dtype="bf16"):
    t = torch.bfloat16 if dtype == "bf16" else torch.float16
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(t).cuda()


def run_case(B, H, H_kv, N, d, seed, causal=False, key_len=None, block_mask=None, scale=None,
             dtype="bf16", workspace=None):
    q, _, _, rng = random_qkv(B, H, N, d, seed, dtype)
    _, k, v, rng = random_qkv(B, H_kv, N, d, seed + 1, dtype, rng=rng)
    dout = rng.standard_normal(q.shape).astype(np.float32)
    scale = np.float32(1.0 / math.sqrt(d) if scale is None else scale)
    tq, tk, tv, tdo = dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(dout, dtype)
    dout_b = tdo.float().cpu().numpy()
    kl = torch.from_numpy(np.asarray(key_len, dtype=np.int32)).cuda() if key_len is not None else None
    bm = torch.from_numpy(np.asarray(block_mask, dtype=np.uint8)).cuda() if block_mask is not None else None
    o, lse = fa.fwd(tq, tk, tv, causal=causal, key_len=kl, block_mask=bm, scale=float(scale))
    dq = torch.full_like(tq, float("nan"))
    dk = torch.full_like(tk, float("nan"))
    dv = torch.full_like(tv, float("nan"))
    fa.bwd(tq, tk, tv, o, tdo, lse, causal=causal, key_len=kl, block_mask=bm, scale=float(scale),
           dq=dq, dk=dk, dv=dv, workspace=workspace)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd_f64(q, k, v, dout_b, float(scale), causal,
                                   None if key_len is None else np.asarray(key_len, dtype=np.int32),
                                   None if block_mask is None else np.asarray(block_mask, dtype=np.uint8))
    errs = {}
    for name, g, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        g = g.double().cpu().numpy()
        assert np.all(np.isfinite(g)), f"{name}: non-finite"
        err = float(np.abs(g - r).max())
        errs[name] = err
        bound = (TOL_REL if dtype == "bf16" else TOL_REL_F16) * max(1.0, float(np.abs(r).max()))
        assert err <= bound, f"{name}: max|dg| = {err:.3e} > {bound:.3e}"
    return errs


@pytest.mark.parametrize("B,H,N", [(4, 24, 512), (8, 16, 512), (1, 4, 2048), (2, 5, 1536), (1, 3, 640)])
def test_bwd_causal_work_orders(B, H, N):
    """Causal grids whose sizes select every branch of the CU-balanced work
    order of the dK/dV and dQ kernels (a full round then a partial one, a
    reversed round, a head over two XCDs, shares without whole heads, a grid
    that is not a multiple of 8); gradients start as NaN."""
    run_case(B, H, H, N, 64, seed=300 + N + H, causal=True)


def modes(N, seed):
    rng = np.random.default_rng(seed)
    nb = (N + 127) // 128
    return {
        "dense": dict(),
        "causal": dict(causal=True),
        "padded": dict(key_len=[max(1, N // 3), N]),
        "blocks": dict(block_mask=band_global_block_mask(nb, rng, n_global=1)),
        "all": dict(causal=True, key_len=[N, max(1, N - 5)],
                    block_mask=band_global_block_mask(nb, rng, n_global=1)),
    }


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 45, 300])
@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks", "all"])
def test_bwd_modes(d, N, mode):
    run_case(2, 2, 2, N, d, seed=70 + N + d, **modes(N, 71)[mode])


def key_lengths(B, N, rng):
    """Ragged key lengths for B batch entries: one with no key, one full."""
    kl = rng.integers(0, N + 1, B)
    kl[0], kl[-1] = 0, N
    return kl


@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks", "all"])
def test_bwd_two_per_cu_modes(mode):
    """d = 128 grids of 1040 key blocks (B13 H16 N520: five 128-key blocks
    per head, the last ragged) run the dK/dV kernel at two 4-wave
    workgroups per CU (smaller grids take the pair kernel); every mask
    mode, gradients start as NaN."""
    B, H, N = 13, 16, 520
    rng = np.random.default_rng(400)
    kw = {"dense": {}, "causal": dict(causal=True), "padded": dict(key_len=key_lengths(B, N, rng)),
          "blocks": dict(block_mask=band_global_block_mask(5, rng, n_global=1)),
          "all": dict(causal=True, key_len=key_lengths(B, N, rng),
                      block_mask=band_global_block_mask(5, rng, n_global=1))}[mode]
    run_case(B, H, H, N, 128, seed=401, **kw)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,H_kv", [(2, 2), (8, 2)])
def test_bwd_two_per_cu_split(causal, H, H_kv):
    """B4 N1000 d128 with the split workspace: 64 key blocks split 16 ways
    over their (query head, query tile) steps, a 1024-workgroup grid of the
    two-per-CU dK/dV kernel writing fp32 partials."""
    assert fa.fa_bwd_workspace_size(4, H, H_kv, 1000, 128) > 0
    run_case(4, H, H_kv, 1000, 128, seed=402, causal=causal, workspace=True)


@pytest.mark.parametrize("B,H,H_kv,N,d", [(8, 8, 2, 512, 128), (16, 4, 4, 512, 64), (8, 16, 16, 512, 64)])
def test_bwd_key_padded_unit_order(B, H, H_kv, N, d):
    """Key-padded grids whose per-XCD shares hold whole key/value-head units,
    so the dK/dV and dQ kernels deal the units to the XCDs round-robin;
    ragged key lengths with an entry that has no key; gradients start as
    NaN."""
    rng = np.random.default_rng(410 + B + H + d)
    run_case(B, H, H_kv, N, d, seed=411 + d, key_len=key_lengths(B, N, rng))


def test_bwd_two_per_cu_f16():
    run_case(13, 16, 16, 520, 128, seed=403, causal=True, dtype="f16")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 45, 300, 1000])
@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks", "all"])
def test_bwd_modes_split(d, N, mode):
    """Small grids with a workspace: the dK/dV steps and the dQ key range
    are both split (16 ways here), partials summed by the reduce kernels;
    the workspace starts full of NaN bytes."""
    need = fa.fa_bwd_workspace_size(2, 2, 2, N, d)
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    run_case(2, 2, 2, N, d, seed=110 + N + d, workspace=ws, **modes(N, 111)[mode])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [45, 300])
@pytest.mark.parametrize("mode", ["dense", "causal", "padded", "blocks", "all"])
def test_bwd_f16_modes(d, N, mode):
    run_case(2, 2, 2, N, d, seed=90 + N + d, dtype="f16", **modes(N, 91)[mode])


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_f16_grouped_heads(causal):
    run_case(1, 8, 2, 257, 128, seed=92, causal=causal, dtype="f16")


# Grouped heads on these small grids take the query-head split (fp32 partial
# dK, dV in a workspace, summed by a second kernel) unless no workspace is
# given; both paths are checked.
@pytest.mark.parametrize("split", [True, None])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,H_kv", [(8, 2), (4, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_grouped_heads(split, d, H, H_kv, causal):
    assert fa.fa_bwd_workspace_size(1, H, H_kv, 200, d) > 0
    run_case(1, H, H_kv, 200, d, seed=72, causal=causal, workspace=split)


@pytest.mark.parametrize("split", [True, None])
@pytest.mark.parametrize("mode", ["padded", "blocks", "all"])
def test_bwd_grouped_heads_masked(split, mode):
    run_case(2, 6, 2, 300, 64, seed=77, workspace=split, **modes(300, 78)[mode])


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_split_f16_and_stale_workspace(d):
    # fp16 through the split path, with a workspace full of garbage on entry
    need = fa.fa_bwd_workspace_size(2, 12, 3, 333, d)
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    run_case(2, 12, 3, 333, d, seed=79, causal=True, dtype="f16", workspace=ws)


def test_bwd_split_deterministic():
    q, k, v, rng = random_qkv(1, 8, 300, 64, 80, "bf16")
    k, v = k[:, :1].copy(), v[:, :1].copy()
    tq, tk, tv = dev(q), dev(k), dev(v)
    tdo = dev(rng.standard_normal(q.shape).astype(np.float32))
    o, lse = fa.fwd(tq, tk, tv, causal=True)
    a = fa.bwd(tq, tk, tv, o, tdo, lse, causal=True)
    b = fa.bwd(tq, tk, tv, o, tdo, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("workload", ["gpt2_causal", "bert_padded", "long_causal", "block_sparse"])
def test_bwd_full_size_sampled(workload):
    # The whole workload at its full size, in the launch configuration the
    # backward report times; dQ checked on sampled query rows, dK and dV on
    # sampled keys of two key/value heads, each against the FP64 oracle
    # evaluated for just those outputs.
    w = WORKLOADS[workload]
    inp = make_inputs(w)
    rng = np.random.default_rng(w.seed + 500)
    tq, tk, tv = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    tdo = dev(rng.standard_normal(inp["q"].shape, dtype=np.float32))
    kl = torch.from_numpy(inp["key_len"]).cuda() if inp["key_len"] is not None else None
    bm = torch.from_numpy(inp["block_mask"]).cuda() if inp["block_mask"] is not None else None
    scale = float(inp["scale"])
    o, lse = fa.fwd(tq, tk, tv, causal=w.causal, key_len=kl, block_mask=bm, scale=scale)
    dq, dk, dv = fa.bwd(tq, tk, tv, o, tdo, lse, causal=w.causal, key_len=kl, block_mask=bm, scale=scale)
    torch.cuda.synchronize()
    B, H, N, d = inp["q"].shape
    # 256 query rows over all heads (plus the first and last rows of the
    # grid); 40 keys (plus keys 0 and N-1) in each of two key/value heads
    # (H_kv = H here), the first and last head of the grid among them
    rows = np.unique(np.concatenate([[0, N - 1, B * H * N - 1], rng.choice(B * H * N, size=256, replace=False)]))
    cols = []
    for x in (0, B * H - 1) if B * H > 1 else (0,):
        keys = np.unique(np.concatenate([[0, N - 1], rng.choice(N, size=40, replace=False)]))
        cols.append(x * N + keys)
    cols = np.concatenate(cols)
    args = (scale, w.causal, inp["key_len"], inp["block_mask"])
    dout = tdo.float().cpu().numpy()
    ref_dq = oracle.attention_bwd_rows_f64(inp["q"], inp["k"], inp["v"], dout, rows, *args)
    ref_dk, ref_dv = oracle.attention_bwd_cols_f64(inp["q"], inp["k"], inp["v"], dout, cols, *args)
    rows_t, cols_t = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    got = {"dq": dq.reshape(-1, d)[rows_t], "dk": dk.reshape(-1, d)[cols_t], "dv": dv.reshape(-1, d)[cols_t]}
    for name, r in (("dq", ref_dq), ("dk", ref_dk), ("dv", ref_dv)):
        g = got[name].double().cpu().numpy()
        assert np.all(np.isfinite(g)), f"{workload} {name}: non-finite"
        err = float(np.abs(g - r).max())
        bound = TOL_REL * max(1.0, float(np.abs(r).max()))
        assert err <= bound, f"{workload} {name}: max|dg| = {err:.3e} > {bound:.3e}"


@pytest.mark.parametrize("workload", ["gpt2_causal", "bert_padded", "block_sparse", "long_causal"])
def test_bwd_full_size_every_element(workload):
    # The whole workload at its full size, in the launch configuration the
    # backward report times, compared element by element with the full FP64
    # backward oracle: every element of dQ, dK and dV.  (The oracle holds an
    # N x N array of doubles per head; the 16K causal workload costs it
    # 2-10 s of host time per head.)
    w = WORKLOADS[workload]
    inp = make_inputs(w)
    rng = np.random.default_rng(w.seed + 600)
    tq, tk, tv = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    tdo = dev(rng.standard_normal(inp["q"].shape, dtype=np.float32))
    kl = torch.from_numpy(inp["key_len"]).cuda() if inp["key_len"] is not None else None
    bm = torch.from_numpy(inp["block_mask"]).cuda() if inp["block_mask"] is not None else None
    scale = float(inp["scale"])
    o, lse = fa.fwd(tq, tk, tv, causal=w.causal, key_len=kl, block_mask=bm, scale=scale)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (tq, tk, tv))
    fa.bwd(tq, tk, tv, o, tdo, lse, causal=w.causal, key_len=kl, block_mask=bm, scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd_f64(inp["q"], inp["k"], inp["v"], tdo.float().cpu().numpy(), scale, w.causal,
                                   inp["key_len"], inp["block_mask"])
    for name, g, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        g = g.double().cpu().numpy()
        assert np.all(np.isfinite(g)), f"{workload} {name}: non-finite"
        err = float(np.abs(g - r).max())
        bound = TOL_REL * max(1.0, float(np.abs(r).max()))
        print(f"{workload} {name}: {g.size} elements, max|dg| = {err:.3e} (bar {bound:.3e})", flush=True)
        assert err <= bound, f"{workload} {name}: max|dg| = {err:.3e} > {bound:.3e}"


def test_bwd_larger_causal():
    run_case(1, 2, 2, 1000, 128, seed=73, causal=True)


def test_bwd_fully_masked_batch_entry():
    errs = run_case(2, 2, 2, 150, 64, seed=74, key_len=[0, 150])
    assert all(e < 1 for e in errs.values())


@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_bwd_nonstandard_scales(scale):
    run_case(1, 2, 2, 130, 64, seed=75, causal=True, scale=scale)


def test_bwd_deterministic():
    q, k, v, rng = random_qkv(1, 2, 257, 128, 76, "bf16")
    tq, tk, tv = dev(q), dev(k), dev(v)
    tdo = dev(rng.standard_normal(q.shape).astype(np.float32))
    o, lse = fa.fwd(tq, tk, tv, causal=True)
    a = fa.bwd(tq, tk, tv, o, tdo, lse, causal=True)
    b = fa.bwd(tq, tk, tv, o, tdo, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_gqa_full_size_sampled():
    # Grouped heads at the 16K causal shape (B1 H16 N16384 d128, four query
    # heads per key/value head; its 512-workgroup dK/dV grid runs the 8-wave
    # pair kernel): forward O and LSE on sampled rows, dQ on sampled rows,
    # dK and dV on sampled keys of the last key/value head (summed over its
    # four query heads by the oracle).
    B, H, Hkv, N, d = 1, 16, 4, 16384, 128
    rng = np.random.Generator(np.random.PCG64(3004))
    q = random_qkv(B, H, N, d, 0, "bf16", 0.5, rng=rng)[0]
    _, k, v, rng = random_qkv(B, Hkv, N, d, 0, "bf16", 0.5, rng=rng)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    tq, tk, tv = dev(q), dev(k), dev(v)
    tdo = dev(rng.standard_normal(q.shape, dtype=np.float32))
    o, lse = fa.fwd(tq, tk, tv, causal=True, scale=scale)
    dq, dk, dv = fa.bwd(tq, tk, tv, o, tdo, lse, causal=True, scale=scale)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, B * H * N - 1], rng.choice(B * H * N, size=128, replace=False)]))
    # (one key/value head: the oracle runs the forward of its four query
    # heads at full length for these keys)
    cols = (B * Hkv - 1) * N + np.unique(np.concatenate([[0, N - 1], rng.choice(N, 40, replace=False)]))
    o_ref, l_ref = oracle.attention_rows_f64(q, k, v, rows, scale, True)
    dout = tdo.float().cpu().numpy()
    ref = {"dq": oracle.attention_bwd_rows_f64(q, k, v, dout, rows, scale, True)}
    ref["dk"], ref["dv"] = oracle.attention_bwd_cols_f64(q, k, v, dout, cols, scale, True)
    rows_t, cols_t = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    o_s = o.reshape(-1, d)[rows_t].double().cpu().numpy()
    l_s = lse.reshape(-1)[rows_t].double().cpu().numpy()
    assert np.abs(o_s - o_ref).max() <= 2e-2
    assert np.abs(l_s - l_ref).max() <= 1e-3
    got = {"dq": dq.reshape(-1, d)[rows_t], "dk": dk.reshape(-1, d)[cols_t], "dv": dv.reshape(-1, d)[cols_t]}
    for name, r in ref.items():
        g = got[name].double().cpu().numpy()
        err = float(np.abs(g - r).max())
        bound = TOL_REL * max(1.0, float(np.abs(r).max()))
        assert err <= bound, f"GQA {name}: max|dg| = {err:.3e} > {bound:.3e}"



@pytest.mark.parametrize("d", [128, 64])
def test_bwd_long_causal_one_round_split(d):
    """B1 H8 N8192 causal: 512 dK/dV and 512 dQ workgroups of very unequal
    work (64 key blocks per head), which the workspace splits in two; dQ on
    sampled rows, dK and dV on sampled keys of two heads, against the FP64
    oracle, and the same gradients from the unsplit call within the bar."""
    B, H, N = 1, 8, 8192
    assert fa.fa_bwd_workspace_size(B, H, H, N, d) == 2 * 2 * B * H * N * d * 4 + 2 * B * H * N * d * 4
    rng = np.random.Generator(np.random.PCG64(3200 + d))
    q, k, v, rng = random_qkv(B, H, N, d, 0, "bf16", rng=rng)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    tq, tk, tv = dev(q), dev(k), dev(v)
    tdo = dev(rng.standard_normal(q.shape, dtype=np.float32))
    o, lse = fa.fwd(tq, tk, tv, causal=True, scale=scale)
    dq, dk, dv = fa.bwd(tq, tk, tv, o, tdo, lse, causal=True, scale=scale, workspace=True)
    dq1, dk1, dv1 = fa.bwd(tq, tk, tv, o, tdo, lse, causal=True, scale=scale, workspace=None)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, N - 1, B * H * N - 1], rng.choice(B * H * N, size=96, replace=False)]))
    cols = np.concatenate([x * N + np.unique(np.concatenate([[0, N - 1], rng.choice(N, 24, replace=False)]))
                           for x in (0, B * H - 1)])
    dout = tdo.float().cpu().numpy()
    ref = {"dq": oracle.attention_bwd_rows_f64(q, k, v, dout, rows, scale, True)}
    ref["dk"], ref["dv"] = oracle.attention_bwd_cols_f64(q, k, v, dout, cols, scale, True)
    rows_t, cols_t = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    got = {"dq": dq.reshape(-1, d)[rows_t], "dk": dk.reshape(-1, d)[cols_t], "dv": dv.reshape(-1, d)[cols_t]}
    for name, r in ref.items():
        g = got[name].double().cpu().numpy()
        err = float(np.abs(g - r).max())
        bound = TOL_REL * max(1.0, float(np.abs(r).max()))
        assert err <= bound, f"{name}: max|dg| = {err:.3e} > {bound:.3e}"
    for name, a, b in (("dq", dq, dq1), ("dk", dk, dk1), ("dv", dv, dv1)):
        diff = float((a.float() - b.float()).abs().max())
        bound = 2 * TOL_REL * max(1.0, float(b.float().abs().max()))
        assert np.isfinite(diff) and diff <= bound, f"{name}: split vs unsplit {diff:.3e}"


def test_mqa_block_sparse_full_size_sampled():
    # Multi-query attention at the block-sparse shape (B4 H16 N4096 d64, one
    # key/value head, the band + global mask): the backward splits each key
    # block's 16 query heads over 8 workgroups.  dQ on sampled rows, dK and
    # dV on sampled keys against the oracle summed over all 16 query heads.
    w = WORKLOADS["block_sparse"]
    B, H, N, d = w.B, w.H, w.N, w.d
    rng = np.random.Generator(np.random.PCG64(3105))
    q = random_qkv(B, H, N, d, 0, "bf16", rng=rng)[0]
    _, k, v, rng = random_qkv(B, 1, N, d, 0, "bf16", rng=rng)
    bm = band_global_block_mask((N + 127) // 128, rng, w.sparse_globals)
    assert fa.fa_bwd_workspace_size(B, H, 1, N, d) > 0
    scale = float(np.float32(1.0 / math.sqrt(d)))
    tq, tk, tv = dev(q), dev(k), dev(v)
    tdo = dev(rng.standard_normal(q.shape, dtype=np.float32))
    tbm = torch.from_numpy(bm).cuda()
    o, lse = fa.fwd(tq, tk, tv, block_mask=tbm, scale=scale)
    dq, dk, dv = fa.bwd(tq, tk, tv, o, tdo, lse, block_mask=tbm, scale=scale)
    torch.cuda.synchronize()
    rows = rng.choice(B * H * N, size=24, replace=False)
    cols = int(rng.integers(B)) * N + np.unique(np.concatenate([[0, N - 1], rng.choice(N, 10)]))
    dout = tdo.float().cpu().numpy()
    ref = {"dq": oracle.attention_bwd_rows_f64(q, k, v, dout, rows, scale, False, None, bm)}
    ref["dk"], ref["dv"] = oracle.attention_bwd_cols_f64(q, k, v, dout, cols, scale, False, None, bm)
    rows_t, cols_t = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    got = {"dq": dq.reshape(-1, d)[rows_t], "dk": dk.reshape(-1, d)[cols_t], "dv": dv.reshape(-1, d)[cols_t]}
    for name, r in ref.items():
        g = got[name].double().cpu().numpy()
        err = float(np.abs(g - r).max())
        bound = TOL_REL * max(1.0, float(np.abs(r).max()))
        assert err <= bound, f"MQA {name}: max|dg| = {err:.3e} > {bound:.3e}"



@pytest.mark.parametrize("H,N", [(2, 16384), (1, 32768)])
def test_bwd_one_gpu_share_split_sampled(H, N):
    # One GPU's share of a head-sharded problem (B1 H2 N16384) and a single
    # 32K head, causal, d = 128: the backward splits both the dK/dV steps and
    # the dQ key range.  dQ on sampled rows, dK and dV on sampled keys.
    B, d = 1, 128
    assert fa.fa_bwd_workspace_size(B, H, H, N, d) > 0
    rng = np.random.Generator(np.random.PCG64(3200 + H))
    q, k, v, rng = random_qkv(B, H, N, d, 0, "bf16", 0.5, rng=rng)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    tq, tk, tv = dev(q), dev(k), dev(v)
    tdo = dev(rng.standard_normal(q.shape, dtype=np.float32))
    o, lse = fa.fwd(tq, tk, tv, causal=True, scale=scale)
    dq, dk, dv = fa.bwd(tq, tk, tv, o, tdo, lse, causal=True, scale=scale)
    torch.cuda.synchronize()
    rows = rng.choice(B * H * N, size=24, replace=False)
    cols = int(rng.integers(B * H)) * N + np.unique(np.concatenate([[0, N - 1], rng.choice(N, 6)]))
    dout = tdo.float().cpu().numpy()
    ref = {"dq": oracle.attention_bwd_rows_f64(q, k, v, dout, rows, scale, True)}
    ref["dk"], ref["dv"] = oracle.attention_bwd_cols_f64(q, k, v, dout, cols, scale, True)
    rows_t, cols_t = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    got = {"dq": dq.reshape(-1, d)[rows_t], "dk": dk.reshape(-1, d)[cols_t], "dv": dv.reshape(-1, d)[cols_t]}
    for name, r in ref.items():
        g = got[name].double().cpu().numpy()
        err = float(np.abs(g - r).max())
        bound = TOL_REL * max(1.0, float(np.abs(r).max()))
        assert err <= bound, f"H={H} N={N} {name}: max|dg| = {err:.3e} > {bound:.3e}"
