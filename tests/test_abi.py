"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/fa.h declares, and rejects bad arguments with the documented
status before any HIP call (so nothing here touches a device)."""
import ctypes
import math
import os
import re

import pytest

import io_aware_exact_03_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# Fake but aligned, non-null device addresses: every call below must fail
# validation, which happens before the library makes any HIP call.
Q, K, V, O, LSE = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(["fa_fwd", "fa_fwd_f32", "fa_fwd_ex", "fa_fwd_study",
                                           "fa_fwd_gqa", "fa_fwd_ws", "fa_fwd_workspace_size",
                                           "fa_fwd_noalloc", "fa_fwd_baseline",
                                           "fa_fwd_baseline_workspace_size", "fa_bwd", "fa_bwd_ex",
                                           "fa_bwd_workspace_size", "fa_tile_shape",
                                           "fa_status_string", "fa_last_hip_error"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert fa.library_path().startswith(ROOT)


def test_binding_names_match_the_abi():
    for name in declared_functions():
        assert callable(getattr(fa, name)), name


def call(**kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=LSE, B=2, H=3, N=100, d=64, scale=0.125, causal=0,
                key_len=None, block_mask=None, stream=None, dtype=0, Br=0, Bc=0)
    args.update(kw)
    lib = fa._load()
    return lib.fa_fwd_ex(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"],
                         args["H"], args["N"], args["d"], args["scale"], args["causal"],
                         args["key_len"], args["block_mask"], args["stream"], args["dtype"],
                         args["Br"], args["Bc"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(B=0), 2), (dict(H=-1), 2), (dict(N=0), 2), (dict(B=1 << 20, H=1 << 10, N=1 << 10), 2),
    (dict(d=96), 3), (dict(d=0), 3), (dict(d=256), 3),
    (dict(q=Q + 8), 4), (dict(o=O + 2), 4), (dict(lse=LSE + 2), 4), (dict(key_len=0x60000002), 4),
    (dict(Br=48, Bc=64), 5), (dict(Br=128, Bc=256), 5), (dict(dtype=5), 5), (dict(dtype=-1), 5),
    (dict(dtype=2, Br=64, Bc=32), 5),
    (dict(dtype=1, Br=256, Bc=64), 5), (dict(dtype=3, Br=256, Bc=64), 5), (dict(dtype=4, Br=256, Bc=64), 5),
    (dict(dtype=6), 5),
    (dict(d=64, Br=16, Bc=256), 5),
    # fp32 output of the bf16-input mode: o is 4 bytes per element
    (dict(dtype=3, o=Q - 2 * 3 * 100 * 64 * 2 - 16), 7),
    (dict(Br=256, Bc=64, block_mask=0x70000000), 5),
    (dict(scale=math.inf), 7), (dict(scale=math.nan), 7),
    (dict(o=Q + 64), 7), (dict(lse=O + 16), 7), (dict(lse=O - 2 * 3 * 100 * 4 + 4), 7),
    # lse over an input: the kernel would write it while other workgroups read
    (dict(lse=Q + 4), 7), (dict(lse=K + 2 * 3 * 100 * 64 * 2 - 4), 7), (dict(lse=V - 2 * 3 * 100 * 4 + 4), 7),
    (dict(lse=K), 7),
])
def test_invalid_arguments_return_status_without_launch(kw, status):
    assert call(**kw) == status
    assert fa.fa_status_string(status) not in ("", "unknown status")


def call_gqa(**kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=LSE, B=2, H=4, H_kv=2, N=100, d=64, scale=0.125,
                causal=0, key_len=None, block_mask=None, stream=None, dtype=0, Br=0, Bc=0)
    args.update(kw)
    lib = fa._load()
    return lib.fa_fwd_gqa(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"],
                          args["H"], args["H_kv"], args["N"], args["d"], args["scale"],
                          args["causal"], args["key_len"], args["block_mask"], args["stream"],
                          args["dtype"], args["Br"], args["Bc"])


@pytest.mark.parametrize("kw,status", [
    (dict(H_kv=0), 2), (dict(H_kv=3), 2), (dict(H=4, H_kv=8), 2), (dict(H_kv=-2), 2),
    (dict(k=None), 1), (dict(d=80), 3), (dict(v=V + 4), 4),
    # o overlapping the (smaller) key/value tensors: [B, H_kv, N, d] bf16
    (dict(o=K + 2 * 2 * 100 * 64 * 2 - 16), 7),
])
def test_gqa_invalid_arguments_return_status_without_launch(kw, status):
    assert call_gqa(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(order=3), 7), (dict(order=-1), 7),
    # descending and shuffled orders only on the tile-study kernels (bf16, d = 128, explicit tile)
    (dict(order=1), 5), (dict(order=1, d=64, Br=256, Bc=64), 5),
    (dict(order=2), 5), (dict(order=2, d=64), 5), (dict(order=2, dtype=1, Br=64, Bc=64), 5),
    (dict(order=2, d=128, Br=32, Bc=32, o=None), 1),
    (dict(order=1, dtype=1), 5), (dict(order=1, Br=256, Bc=64), 5), (dict(order=1, dtype=2, Br=128, Bc=64), 5),
    (dict(order=1, d=128, Br=64, Bc=32, q=None), 1),
])
def test_study_order_validation(kw, status):
    args = dict(q=Q, k=K, v=V, o=O, lse=LSE, B=2, H=3, N=100, d=128, scale=0.125, causal=0,
                key_len=None, block_mask=None, stream=None, dtype=0, Br=0, Bc=0, order=0)
    args.update(kw)
    lib = fa._load()
    rc = lib.fa_fwd_study(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"],
                          args["H"], args["N"], args["d"], args["scale"], args["causal"],
                          args["key_len"], args["block_mask"], args["stream"], args["dtype"],
                          args["Br"], args["Bc"], args["order"])
    assert rc == status


DO, LSEB, DELTA, DQ, DK, DV = 0x60000000, 0x70000000, 0x71000000, 0x72000000, 0x74000000, 0x76000000


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(dout=None), 1), (dict(lse=None), 1), (dict(delta=None), 1),
    (dict(dk=None), 1),
    (dict(B=0), 2), (dict(H_kv=3), 2), (dict(N=0), 2),
    (dict(d=96), 3),
    (dict(dq=DQ + 8), 4), (dict(dout=DO + 2), 4), (dict(lse=LSEB + 2), 4),
    (dict(scale=math.nan), 7),
    (dict(dq=Q + 64), 7),                  # output over an input
    (dict(dk=DV + 16), 7),                 # outputs overlapping each other
    (dict(delta=LSEB + 4), 7),             # workspace over the logsumexp
])
@pytest.mark.parametrize("entry", ["fa_bwd", "fa_bwd_ex"])
def test_bwd_invalid_arguments_return_status_without_launch(kw, status, entry):
    args = dict(q=Q, k=K, v=V, o=O, dout=DO, lse=LSEB, delta=DELTA, dq=DQ, dk=DK, dv=DV, B=2, H=4,
                H_kv=2, N=100, d=64, scale=0.125, causal=0, key_len=None, block_mask=None,
                stream=None)
    args.update(kw)
    lib = fa._load()
    names = ("q", "k", "v", "o", "dout", "lse", "delta", "dq", "dk", "dv", "B", "H", "H_kv", "N", "d",
             "scale", "causal", "key_len", "block_mask", "stream")
    if entry == "fa_bwd":
        rc = lib.fa_bwd(*[args[n] for n in names])
    else:
        rc = lib.fa_bwd_ex(*[args[n] for n in names], fa.DTYPE_F16, None, 0)
    assert rc == status


@pytest.mark.parametrize("dtype", [fa.DTYPE_F32, 3, -1])
def test_bwd_ex_rejects_unbuilt_dtypes(dtype):
    lib = fa._load()
    rc = lib.fa_bwd_ex(Q, K, V, O, DO, LSEB, DELTA, DQ, DK, DV, 2, 4, 2, 100, 64, 0.125, 0, None, None,
                       None, dtype, None, 0)
    assert rc == 5


WS = 0x78000000


BWS = 2 * 16 * 2 * 2 * 100 * 64 * 4 + 16 * 2 * 4 * 100 * 64 * 4


@pytest.mark.parametrize("ws,nbytes,status", [
    (WS, BWS - 1, 7),           # smaller than fa_bwd_workspace_size
    (WS + 8, BWS, 7),           # not 16-byte aligned
    (DQ + 64, BWS, 7),          # over an output
    (Q, BWS, 7),                # over an input
])
def test_bwd_workspace_validation(ws, nbytes, status):
    # B2 H4 H_kv2 N100 d64: a tiny grid, so both splits are used (16 each)
    assert fa.fa_bwd_workspace_size(2, 4, 2, 100, 64) == BWS
    lib = fa._load()
    rc = lib.fa_bwd_ex(Q, K, V, O, DO, LSEB, DELTA, DQ, DK, DV, 2, 4, 2, 100, 64, 0.125, 0, None, None,
                       None, fa.DTYPE_BF16, ws, nbytes)
    assert rc == status


def test_bwd_workspace_size():
    size = fa.fa_bwd_workspace_size
    # grids with at least 512 workgroups are not split
    assert size(1, 16, 16, 16384, 128) == 0 and size(8, 12, 12, 1024, 64) == 0
    # four key/value heads at 16K give 512 dK/dV workgroups of very unequal
    # causal work: two key-range splits (the causal case sets the size); the
    # dQ grid (16 x 128 tiles) needs none
    assert size(1, 16, 4, 16384, 128) == 2 * 2 * 4 * 16384 * 128 * 4
    # four heads at 16K: 512 dK/dV and 512 dQ workgroups, two splits each
    assert size(1, 4, 4, 16384, 128) == 2 * 2 * 4 * 16384 * 128 * 4 + 2 * 4 * 16384 * 128 * 4
    # 512 workgroups of short heads (32 key blocks): no split
    assert size(2, 8, 8, 4096, 128) == 0
    # multi-query 16K: 128 dK/dV workgroups -> 8 splits x (dK, dV) x N x d
    # floats; the dQ grid (16 x 128 tiles) needs none
    assert size(1, 16, 1, 16384, 128) == 8 * 2 * 16384 * 128 * 4
    # 2 x 2 x 32 = 128 key blocks -> 8 dK/dV splits; dQ grid 1024: none
    assert size(2, 16, 2, 4096, 64) == 8 * 2 * 2 * 2 * 4096 * 64 * 4
    # one GPU's share of a head-sharded 16K problem: 256 dK/dV workgroups
    # -> 4 splits; 256 dQ workgroups -> 4 key-range splits of dQ
    assert size(1, 2, 2, 16384, 128) == 4 * 2 * 2 * 16384 * 128 * 4 + 4 * 2 * 16384 * 128 * 4
    # invalid shapes report 0
    assert size(0, 4, 2, 100, 64) == 0 and size(1, 4, 3, 100, 64) == 0 and size(1, 4, 2, 100, 96) == 0


def test_status_strings_cover_every_code():
    seen = set()
    for code in range(8):
        s = fa.fa_status_string(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 8
    assert fa.fa_status_string(99) == "unknown status"
    assert fa.fa_last_hip_error() == 0


def test_python_wrappers_raise_with_status():
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd(Q, K, V, O, LSE, 1, 1, 16, 80, 0.1, 0, None, None, None)
    assert e.value.status == 3


def test_tile_table():
    for d in (64, 128):
        br, bc = fa.fa_tile_shape(fa.DTYPE_BF16, d)
        assert br in (128, 256) and bc in (32, 64)
        # the default is itself a built, explicitly selectable tile
        assert fa.fa_tile_shape(fa.DTYPE_BF16, d, False, br, bc) == (br, bc)
        # a block mask needs a tile no taller than one 128-token mask block
        br, bc = fa.fa_tile_shape(fa.DTYPE_BF16, d, block_sparse=True)
        assert br <= 128
    for d in (64, 128):
        for br in (16, 32, 64, 128):
            for bc in (16, 32, 64, 128):
                assert fa.fa_tile_shape(fa.DTYPE_BF16, d, False, br, bc) == (br, bc)
    assert fa.fa_tile_shape(fa.DTYPE_BF16, 64, False, 128, 64) == (128, 64)
    assert fa.fa_tile_shape(fa.DTYPE_BF16, 128, False, 256, 64) == (256, 64)
    assert fa.fa_tile_shape(fa.DTYPE_F32, 64) == (128, 32)
    for d in (64, 128):
        assert fa.fa_tile_shape(fa.DTYPE_F16, d) == (128, 64)
    with pytest.raises(fa.FaError):
        fa.fa_tile_shape(fa.DTYPE_F16, 128, False, 64, 32)
    with pytest.raises(fa.FaError):
        fa.fa_tile_shape(fa.DTYPE_BF16, 128, True, 256, 64)
    with pytest.raises(fa.FaError):
        fa.fa_tile_shape(fa.DTYPE_BF16, 64, False, 16, 256)



def test_fwd_workspace_size():
    size = fa.fa_fwd_workspace_size
    # enough workgroups already: no split (B*H*ceil(N/128) >= 512)
    assert size(1, 16, 16384, 128, fa.DTYPE_BF16) == 0 and size(4, 16, 4096, 64, fa.DTYPE_BF16) == 0
    # B1 H2 N16384: 256 query tiles -> 4 shares (1024 workgroups); O and LSE per share
    assert size(1, 2, 16384, 128, fa.DTYPE_BF16) == 4 * 2 * 16384 * (128 + 1) * 4
    assert size(1, 2, 16384, 128, fa.DTYPE_F16) == 4 * 2 * 16384 * (128 + 1) * 4
    # 300 tiles -> 2 shares (600 <= 1024 < 1200); 1 tile -> 16 shares (the cap)
    assert size(3, 1, 12800, 64, fa.DTYPE_BF16) == 2 * 3 * 12800 * 65 * 4
    assert size(1, 1, 100, 64, fa.DTYPE_BF16) == 16 * 100 * 65 * 4
    # exactly 512 tiles of long heads (64+ tiles each): two shares, which the
    # causal mask uses (the size covers it); short heads stay unsplit
    assert size(1, 4, 16384, 128, fa.DTYPE_BF16) == 2 * 4 * 16384 * (128 + 1) * 4
    assert size(2, 2, 16384, 64, fa.DTYPE_BF16) == 2 * 4 * 16384 * (64 + 1) * 4
    assert size(4, 16, 1024, 64, fa.DTYPE_BF16) == 0
    # fp32 is never split; invalid arguments report 0
    assert size(1, 2, 16384, 128, fa.DTYPE_F32) == 0
    assert size(0, 2, 100, 64, 0) == 0 and size(1, 2, 100, 96, 0) == 0


FWS = 0x7A000000


@pytest.mark.parametrize("ws,nbytes,status", [
    (FWS, 2 * 3 * 100 * 65 * 4 * 16 - 4, 7),   # smaller than needed
    (FWS + 4, 2 * 3 * 100 * 65 * 4 * 16, 7),   # not 16-byte aligned
    (O + 32, 2 * 3 * 100 * 65 * 4 * 16, 7),    # over the output
    (K, 2 * 3 * 100 * 65 * 4 * 16, 7),         # over an input
])
def test_fwd_workspace_validation(ws, nbytes, status):
    # B2 H3 N100 d64: 6 query tiles -> 16 shares
    assert fa.fa_fwd_workspace_size(2, 3, 100, 64, fa.DTYPE_BF16) == 2 * 3 * 100 * 65 * 4 * 16
    lib = fa._load()
    rc = lib.fa_fwd_ws(Q, K, V, O, LSE, 2, 3, 3, 100, 64, 0.125, 0, None, None, None, fa.DTYPE_BF16,
                       ws, nbytes)
    assert rc == status


def test_noalloc_scratch_covers_every_split_workspace():
    """The static scratch of fa_fwd_noalloc is the largest workspace the
    key-range split asks for: splits run only on grids of at most 512
    query tiles of 128 rows, with at most 1024 shares in all."""
    text = open(HEADER).read()
    m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) \* (\d+) \* (\d+) \* (\d+)\)", text)
    assert m, "FA_NOALLOC_SCRATCH_BYTES not found"
    limit = math.prod(int(x) for x in m.groups())
    assert limit == fa.NOALLOC_SCRATCH_BYTES
    worst = 0
    for d in (64, 128):
        for B in (1, 2, 3, 4, 8):
            for H in (1, 2, 3, 4, 6, 16):
                for N in (1, 100, 127, 128, 129, 1000, 4096, 8191, 16384, 32768, 40000, 65536):
                    need = fa.fa_fwd_workspace_size(B, H, N, d, fa.DTYPE_BF16)
                    assert need <= limit, (B, H, N, d, need)
                    worst = max(worst, need)
    assert worst == limit  # reached by B1 H2 N16384 d128 (4 shares of 32768 rows)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(H_kv=3), 2), (dict(N=0), 2), (dict(d=96), 3), (dict(o=O + 2), 4),
    (dict(scale=math.nan), 7), (dict(o=Q + 64), 7), (dict(lse=K + 16), 7), (dict(dtype=5), 5),
])
def test_noalloc_invalid_arguments_return_status_without_launch(kw, status):
    args = dict(q=Q, k=K, v=V, o=O, lse=LSE, B=1, H=2, H_kv=2, N=16384, d=128, scale=0.125, causal=1,
                key_len=None, block_mask=None, stream=None, dtype=0)
    args.update(kw)
    names = ("q", "k", "v", "o", "lse", "B", "H", "H_kv", "N", "d", "scale", "causal", "key_len",
             "block_mask", "stream", "dtype")
    assert fa._load().fa_fwd_noalloc(*[args[n] for n in names]) == status


WS = 0x7A000000


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(workspace=None), 1), (dict(B=0), 2), (dict(N=0), 2), (dict(d=80), 3),
    (dict(dtype=5), 5), (dict(dtype=4), 5), (dict(dtype=1, inter=0), 5), (dict(dtype=0, inter=2), 5),
    (dict(dtype=2, inter=0), 5),
    (dict(q=Q + 8), 4), (dict(workspace=WS + 4), 4), (dict(lse=LSE + 2), 4),
    (dict(scale=math.inf), 7), (dict(ws_bytes=2 * 3 * 100 * 100 * 4 - 1), 7),
    (dict(ws_bytes=2 * 3 * 100 * 100 * 2, inter=1), 7),
    (dict(o=Q + 64), 7), (dict(lse=V + 16), 7), (dict(workspace=O + 16), 7), (dict(lse=WS + 64), 7),
    (dict(B=1 << 12, H=1 << 12, N=1 << 10), 2),
])
def test_baseline_invalid_arguments_return_status_without_launch(kw, status):
    args = dict(q=Q, k=K, v=V, o=O, lse=LSE, B=2, H=3, N=100, d=64, scale=0.125, causal=0, key_len=None,
                block_mask=None, stream=None, dtype=0, inter=1, workspace=WS, ws_bytes=1 << 30)
    args.update(kw)
    names = ("q", "k", "v", "o", "lse", "B", "H", "N", "d", "scale", "causal", "key_len", "block_mask",
             "stream", "dtype", "inter", "workspace", "ws_bytes")
    assert fa._load().fa_fwd_baseline(*[args[n] for n in names]) == status


def test_baseline_workspace_size():
    assert fa.fa_fwd_baseline_workspace_size(2, 3, 100, fa.DTYPE_BF16, fa.DTYPE_F32) == 2 * 3 * 100 * 100 * 4
    assert fa.fa_fwd_baseline_workspace_size(2, 3, 100, fa.DTYPE_BF16, fa.DTYPE_BF16) == 2 * 3 * 100 * 100 * 2
    assert fa.fa_fwd_baseline_workspace_size(1, 16, 16384, fa.DTYPE_BF16_F32OUT, fa.DTYPE_F32) == 16 * 16384 ** 2 * 4
    assert fa.fa_fwd_baseline_workspace_size(1, 1, 10, fa.DTYPE_F32, fa.DTYPE_BF16) == 0
    assert fa.fa_fwd_baseline_workspace_size(0, 1, 10, fa.DTYPE_F32, fa.DTYPE_F32) == 0
