"""Python binding of the gfx950 exact-attention library (libfa.so).

The functions named after the C entry points (``fa_fwd``, ``fa_fwd_f32``,
``fa_fwd_ex``, ``fa_fwd_study``, ``fa_fwd_gqa``, ``fa_fwd_ws``, ``fa_fwd_workspace_size``,
``fa_fwd_noalloc``, ``fa_fwd_baseline``, ``fa_fwd_baseline_workspace_size``, ``fa_bwd``,
``fa_bwd_ex``, ``fa_bwd_workspace_size``, ``fa_tile_shape``,
``fa_status_string``,
``fa_last_hip_error``) only marshal arguments to include/fa.h and raise
``FaError`` on a non-zero status; every step of the attention itself runs in
the library's HIP kernels.  ``fwd`` and ``bwd`` are convenience wrappers
that allocate the outputs with torch and pass torch's current stream.  There is no
fallback: if libfa.so is missing or fails to load, every call raises.
"""
import ctypes
import math
import os

__all__ = ["FaError", "fa_fwd", "fa_fwd_f32", "fa_fwd_ex", "fa_fwd_study", "fa_fwd_gqa", "fa_fwd_ws", "fa_fwd_workspace_size",
           "fa_fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "fa_fwd_baseline", "fa_fwd_baseline_workspace_size",
           "baseline", "DTYPE_BF16_F32OUT", "DTYPE_BF16_ACC16", "fa_bwd", "fa_bwd_ex",
           "fa_bwd_workspace_size", "bwd",
           "fa_tile_shape", "ORDER_ASCENDING", "ORDER_DESCENDING", "ORDER_SHUFFLED",
           "fa_status_string", "fa_last_hip_error", "fwd", "library_path",
           "DTYPE_BF16", "DTYPE_F32", "DTYPE_F16", "MASK_BLOCK"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
DTYPE_BF16 = 0
DTYPE_F32 = 1
DTYPE_F16 = 2
DTYPE_BF16_F32OUT = 3
DTYPE_BF16_ACC16 = 4
ORDER_ASCENDING = 0
ORDER_DESCENDING = 1
ORDER_SHUFFLED = 2
MASK_BLOCK = 128
# FA_NOALLOC_SCRATCH_BYTES of include/fa.h: the static scratch of fa_fwd_noalloc
NOALLOC_SCRATCH_BYTES = 1024 * 128 * 129 * 4

FA_OK = 0
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_NULL_PTR", 2: "FA_ERR_INVALID_SHAPE",
                3: "FA_ERR_UNSUPPORTED_HEAD_DIM", 4: "FA_ERR_MISALIGNED",
                5: "FA_ERR_UNSUPPORTED_TILE", 6: "FA_ERR_HIP", 7: "FA_ERR_INVALID_ARG"}

_lib = None


class FaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        detail = ""
        if status == 6:
            detail = f" (hipError_t {fa_last_hip_error()})"
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: "
                         f"{fa_status_string(status)}{detail}")


def library_path():
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python __graft_entry__.py build` "
                           "or `python io_aware_exact_03_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    fwd_args = [vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_float, i32, vp, vp, vp]
    lib.fa_fwd.argtypes = fwd_args
    lib.fa_fwd.restype = i32
    lib.fa_fwd_f32.argtypes = fwd_args
    lib.fa_fwd_f32.restype = i32
    lib.fa_fwd_ex.argtypes = fwd_args + [i32, i32, i32]
    lib.fa_fwd_ex.restype = i32
    lib.fa_fwd_study.argtypes = fwd_args + [i32, i32, i32, i32]
    lib.fa_fwd_study.restype = i32
    lib.fa_fwd_gqa.argtypes = fwd_args[:7] + [i32] + fwd_args[7:] + [i32, i32, i32]
    lib.fa_fwd_gqa.restype = i32
    lib.fa_bwd.argtypes = [vp] * 10 + [i32] * 5 + [ctypes.c_float, i32, vp, vp, vp]
    lib.fa_bwd.restype = i32
    lib.fa_bwd_ex.argtypes = [vp] * 10 + [i32] * 5 + [ctypes.c_float, i32, vp, vp, vp, i32, vp,
                                                       ctypes.c_size_t]
    lib.fa_bwd_ex.restype = i32
    lib.fa_bwd_workspace_size.argtypes = [i32] * 5
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_fwd_ws.argtypes = [vp] * 5 + [i32] * 5 + [ctypes.c_float, i32, vp, vp, vp, i32, vp,
                                                     ctypes.c_size_t]
    lib.fa_fwd_ws.restype = i32
    lib.fa_fwd_noalloc.argtypes = [vp] * 5 + [i32] * 5 + [ctypes.c_float, i32, vp, vp, vp, i32]
    lib.fa_fwd_noalloc.restype = i32
    lib.fa_fwd_baseline.argtypes = fwd_args + [i32, i32, vp, ctypes.c_size_t]
    lib.fa_fwd_baseline.restype = i32
    lib.fa_fwd_baseline_workspace_size.argtypes = [i32] * 5
    lib.fa_fwd_baseline_workspace_size.restype = ctypes.c_size_t
    lib.fa_fwd_workspace_size.argtypes = [i32] * 5
    lib.fa_fwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_tile_shape.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.fa_tile_shape.restype = i32
    lib.fa_status_string.argtypes = [i32]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_hip_error.argtypes = []
    lib.fa_last_hip_error.restype = i32
    _lib = lib
    return lib


def _check(status, where):
    if status != FA_OK:
        raise FaError(status, where)


# ---------------------------------------------------------------- raw entry points
# Pointer arguments are integers (device addresses) or None; stream is a HIP
# stream handle as an integer (0 = default stream).


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, block_mask, stream):
    _check(_load().fa_fwd(q, k, v, o, lse, B, H, N, d, scale, int(bool(causal)),
                          key_len, block_mask, stream), "fa_fwd")


def fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, block_mask, stream):
    _check(_load().fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, int(bool(causal)),
                              key_len, block_mask, stream), "fa_fwd_f32")


def fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, block_mask, stream,
              dtype, Br, Bc):
    _check(_load().fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, int(bool(causal)),
                             key_len, block_mask, stream, dtype, Br, Bc), "fa_fwd_ex")


def fa_fwd_study(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, block_mask, stream,
                 dtype, Br, Bc, tile_order):
    _check(_load().fa_fwd_study(q, k, v, o, lse, B, H, N, d, scale, int(bool(causal)),
                                key_len, block_mask, stream, dtype, Br, Bc, tile_order),
           "fa_fwd_study")


def fa_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, key_len, block_mask, stream,
               dtype, Br, Bc):
    _check(_load().fa_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, scale, int(bool(causal)),
                              key_len, block_mask, stream, dtype, Br, Bc), "fa_fwd_gqa")


def fa_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv, N, d, scale, causal, key_len,
           block_mask, stream):
    _check(_load().fa_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv, N, d, scale,
                          int(bool(causal)), key_len, block_mask, stream), "fa_bwd")


def fa_bwd_ex(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv, N, d, scale, causal, key_len,
              block_mask, stream, dtype, workspace, workspace_bytes):
    _check(_load().fa_bwd_ex(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv, N, d, scale,
                             int(bool(causal)), key_len, block_mask, stream, dtype, workspace,
                             workspace_bytes), "fa_bwd_ex")


def fa_fwd_ws(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, key_len, block_mask, stream, dtype,
              workspace, workspace_bytes):
    _check(_load().fa_fwd_ws(q, k, v, o, lse, B, H, H_kv, N, d, scale, int(bool(causal)), key_len,
                             block_mask, stream, dtype, workspace, workspace_bytes), "fa_fwd_ws")


def fa_fwd_noalloc(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, key_len, block_mask, stream,
                   dtype):
    _check(_load().fa_fwd_noalloc(q, k, v, o, lse, B, H, H_kv, N, d, scale, int(bool(causal)), key_len,
                                  block_mask, stream, dtype), "fa_fwd_noalloc")


def fa_fwd_baseline(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, block_mask, stream, dtype,
                    inter_dtype, workspace, workspace_bytes):
    _check(_load().fa_fwd_baseline(q, k, v, o, lse, B, H, N, d, scale, int(bool(causal)), key_len,
                                   block_mask, stream, dtype, inter_dtype, workspace, workspace_bytes),
           "fa_fwd_baseline")


def fa_fwd_baseline_workspace_size(B, H, N, dtype, inter_dtype):
    return int(_load().fa_fwd_baseline_workspace_size(B, H, N, dtype, inter_dtype))


def fa_fwd_workspace_size(B, H, N, d, dtype):
    return int(_load().fa_fwd_workspace_size(B, H, N, d, dtype))


def fa_bwd_workspace_size(B, H, H_kv, N, d):
    return int(_load().fa_bwd_workspace_size(B, H, H_kv, N, d))


def fa_tile_shape(dtype, d, block_sparse=False, Br=0, Bc=0):
    br, bc = ctypes.c_int(0), ctypes.c_int(0)
    _check(_load().fa_tile_shape(dtype, d, int(bool(block_sparse)), Br, Bc, ctypes.byref(br),
                                 ctypes.byref(bc)), "fa_tile_shape")
    return br.value, bc.value


def fa_status_string(status):
    return _load().fa_status_string(status).decode()


def fa_last_hip_error():
    return int(_load().fa_last_hip_error())


# ---------------------------------------------------------------- torch convenience


def fwd(q, k, v, causal=False, key_len=None, block_mask=None, scale=None, Br=0, Bc=0,
        out=None, lse=None, stream=None, tile_order=ORDER_ASCENDING, workspace=None,
        acc16=False):
    """Attention forward on device tensors.

    q: contiguous [B, H, N, d] cuda tensor, bfloat16, float16 or float32; k, v: the
    same dtype, [B, H_kv, N, d] with H a multiple of H_kv (H_kv < H runs
    grouped-query attention through fa_fwd_gqa).
    key_len: int32 cuda tensor [B] or None.  block_mask: uint8 cuda tensor with
    ceil(N/128)^2 entries (row = query block) or None.  scale defaults to
    1/sqrt(d).  Br/Bc = 0 selects the tuned tile.  Returns (o, lse) with o like
    q and lse float32 [B, H, N]; `out`/`lse` may be passed preallocated (a
    float32 `out` with bfloat16 inputs selects the fp32-output mode of the
    tile-study kernels, O left unrounded), and
    lse=False skips the logsumexp (returned as None).  tile_order =
    ORDER_DESCENDING visits key tiles last-first, ORDER_SHUFFLED in a fixed
    permutation (tile-study kernels only).  ``acc16`` (bfloat16 only, a
    deviation-study mode): the running output is rounded to bf16 after every
    key tile (FA_DTYPE_BF16_ACC16).  ``workspace`` (tuned tile only):
    True allocates the key-range split workspace ``fa_fwd_workspace_size``
    asks for (grids too small for the GPU), a uint8 cuda tensor is used as
    it, "static" uses the library's own static scratch (fa_fwd_noalloc,
    nothing allocated), None (the default) runs unsplit.
    """
    import torch
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k and v must share a dtype")
    if q.dtype == torch.bfloat16:
        dtype = DTYPE_BF16_F32OUT if (out is not None and out.dtype == torch.float32) else DTYPE_BF16
        if acc16:
            if dtype != DTYPE_BF16:
                raise ValueError("acc16 takes a bfloat16 output")
            dtype = DTYPE_BF16_ACC16
    elif q.dtype == torch.float32:
        dtype = DTYPE_F32
    elif q.dtype == torch.float16:
        dtype = DTYPE_F16
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-d cuda tensor")
    B, H, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2:] != q.shape[2:]:
        raise ValueError("k and v must have the shape [B, H_kv, N, d] of q's B, N, d")
    H_kv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    want_lse = lse is not False
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    kl_ptr = None
    if key_len is not None:
        if key_len.dtype != torch.int32 or not key_len.is_cuda or key_len.numel() != B:
            raise ValueError("key_len must be an int32 cuda tensor of B entries")
        kl_ptr = key_len.data_ptr()
    bm_ptr = None
    if block_mask is not None:
        nb = (N + MASK_BLOCK - 1) // MASK_BLOCK
        if block_mask.dtype != torch.uint8 or not block_mask.is_cuda or block_mask.numel() != nb * nb:
            raise ValueError(f"block_mask must be a uint8 cuda tensor of {nb}x{nb} entries")
        bm_ptr = block_mask.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if isinstance(workspace, str):
        if workspace != "static" or tile_order != ORDER_ASCENDING or Br or Bc:
            raise ValueError('workspace="static" applies to the tuned tile in ascending order')
        fa_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                       lse.data_ptr() if want_lse else None, B, H, H_kv, N, d, float(scale),
                       causal, kl_ptr, bm_ptr, stream, dtype)
    elif workspace is not None and workspace is not False:
        if tile_order != ORDER_ASCENDING or Br or Bc:
            raise ValueError("the split workspace applies to the tuned tile in ascending order")
        if workspace is True:
            need = fa_fwd_workspace_size(B, H, N, d, dtype)
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 cuda tensor")
        fa_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                  lse.data_ptr() if want_lse else None, B, H, H_kv, N, d, float(scale),
                  causal, kl_ptr, bm_ptr, stream, dtype, workspace.data_ptr(), workspace.numel())
    elif tile_order != ORDER_ASCENDING:
        if H_kv != H:
            raise ValueError("tile_order applies to plain multi-head calls only")
        fa_fwd_study(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                     lse.data_ptr() if want_lse else None, B, H, N, d, float(scale),
                     causal, kl_ptr, bm_ptr, stream, dtype, Br, Bc, tile_order)
    elif H_kv == H:
        fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                  lse.data_ptr() if want_lse else None, B, H, N, d, float(scale),
                  causal, kl_ptr, bm_ptr, stream, dtype, Br, Bc)
    else:
        fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                   lse.data_ptr() if want_lse else None, B, H, H_kv, N, d, float(scale),
                   causal, kl_ptr, bm_ptr, stream, dtype, Br, Bc)
    return out, (lse if want_lse else None)


def baseline(q, k, v, causal=False, key_len=None, block_mask=None, scale=None, inter="f32",
             out=None, lse=None, workspace=None, stream=None):
    """Materialised attention (fa_fwd_baseline) on device tensors.

    q, k, v: contiguous [B, H, N, d] cuda tensors of one dtype (bfloat16,
    float16 or float32).  inter: "f32" holds S and A in float32, "io" in the
    input type.  out: optional preallocated output (float32 with bfloat16
    inputs keeps O unrounded).  workspace: optional uint8 cuda tensor of at
    least fa_fwd_baseline_workspace_size bytes (allocated here if None).
    Returns (o, lse).
    """
    import torch
    codes = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16, torch.float32: DTYPE_F32}
    if q.dtype not in codes or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype among bfloat16, float16, float32")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4 or t.shape != q.shape:
            raise ValueError(f"{name} must be a contiguous cuda tensor of q's shape")
    B, H, N, d = q.shape
    dtype = codes[q.dtype]
    if out is None:
        out = torch.empty_like(q)
    if q.dtype == torch.bfloat16 and out.dtype == torch.float32:
        dtype = DTYPE_BF16_F32OUT
    if inter not in ("f32", "io"):
        raise ValueError('inter must be "f32" or "io"')
    inter_code = DTYPE_F32 if inter == "f32" else codes[q.dtype]
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    need = fa_fwd_baseline_workspace_size(B, H, N, dtype, inter_code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    fa_fwd_baseline(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                    float(scale), causal, key_len.data_ptr() if key_len is not None else None,
                    block_mask.data_ptr() if block_mask is not None else None, stream, dtype, inter_code,
                    workspace.data_ptr(), workspace.numel())
    return out, lse


def bwd(q, k, v, o, dout, lse, causal=False, key_len=None, block_mask=None, scale=None,
        dq=None, dk=None, dv=None, delta=None, stream=None, workspace=True):
    """Gradients (dq, dk, dv) of sum(dout * o) for bf16 or fp16 attention.

    q, o, dout: contiguous bfloat16 or float16 [B, H, N, d] cuda tensors (one
    dtype for all); k, v: [B, H_kv, N, d]; lse: float32 [B, H, N] from
    ``fwd`` on the same inputs and options.  Outputs (and the float32
    [B, H, N] workspace ``delta``) are allocated with torch unless passed in.
    ``workspace``: True allocates the split workspace that
    ``fa_bwd_workspace_size`` asks for (grouped heads on small grids), a
    uint8 cuda tensor is used as it, None or False runs without one.
    """
    import torch
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("bwd takes bfloat16 or float16 tensors")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-d cuda tensor of q's dtype")
    B, H, N, d = q.shape
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must have q's shape")
    if k.shape != v.shape or k.shape[0] != B or k.shape[2:] != q.shape[2:]:
        raise ValueError("k and v must have the shape [B, H_kv, N, d] of q's B, N, d")
    H_kv = k.shape[1]
    if lse.dtype != torch.float32 or lse.shape != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if delta is None else delta
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.dtype != q.dtype or t.shape != like.shape or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous cuda tensor like {'q' if like is q else 'k'}")
    if delta.dtype != torch.float32 or delta.shape != (B, H, N) or not delta.is_contiguous():
        raise ValueError("delta must be a contiguous float32 [B, H, N] tensor")
    kl_ptr = key_len.data_ptr() if key_len is not None else None
    bm_ptr = block_mask.data_ptr() if block_mask is not None else None
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    ws_ptr, ws_bytes = None, 0
    if workspace is True:
        need = fa_bwd_workspace_size(B, H, H_kv, N, d)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        else:
            workspace = None
    if workspace is not None and workspace is not False:
        if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 cuda tensor")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    fa_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
              delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, H_kv, N, d,
              float(scale), causal, kl_ptr, bm_ptr, stream,
              DTYPE_F16 if q.dtype == torch.float16 else DTYPE_BF16, ws_ptr, ws_bytes)
    return dq, dk, dv
