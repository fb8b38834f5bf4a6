"""FP64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use it; the GPU library never imports, links or calls it,
and it shares no code with that library.

``attention_f64`` evaluates the plain definition from the page "Ch.04
Attention optimisation: FlashAttention and sparse attention" (mdooai.com,
sections "Core formula" / "Key points of the formulas"):
S = scale * Q K^T, disallowed logits set to -inf before the softmax,
A = row-softmax(S), O = A V, plus the row logsumexp (natural log).
The C implementation (attn_ref.c) materialises S one head at a time;
``attention_rows_f64`` does the same for a list of query rows only, for
sampled checks at sizes where a full pass would take too long.
``attention_bwd_f64`` gives the gradients of that definition (dQ, dK, dV for
a given dO), derived from it by the chain rule.

Inputs are widened exactly to float64 (float32 and bfloat16 values are
representable), so the oracle sees precisely the values the GPU receives.
"""
import ctypes

import numpy as np

from . import build as _build

_lib = None


def _configure(lib):
    """Declare the C entry points' signatures on a loaded library."""
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.attn_ref_f64.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64,
                                 ctypes.c_double, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p, i64]
    lib.attn_ref_f64.restype = ctypes.c_int
    lib.attn_ref_gqa_f64.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64, i64,
                                     ctypes.c_double, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p, i64]
    lib.attn_ref_gqa_f64.restype = ctypes.c_int
    lib.attn_ref_rows_f64.argtypes = [dp, dp, dp, i64, i64, i64, i64,
                                      ctypes.c_double, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p, i64,
                                      ctypes.c_void_p, i64, dp, dp]
    lib.attn_ref_rows_f64.restype = ctypes.c_int
    lib.attn_ref_rows_gqa_f64.argtypes = [dp, dp, dp, i64, i64, i64, i64, i64,
                                          ctypes.c_double, ctypes.c_int,
                                          ctypes.c_void_p, ctypes.c_void_p, i64,
                                          ctypes.c_void_p, i64, dp, dp]
    lib.attn_ref_rows_gqa_f64.restype = ctypes.c_int
    lib.attn_bwd_ref_gqa_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, i64, i64, i64, i64, i64,
                                         ctypes.c_double, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p, i64]
    lib.attn_bwd_ref_gqa_f64.restype = ctypes.c_int
    lib.attn_bwd_rows_gqa_f64.argtypes = [dp, dp, dp, dp, i64, i64, i64, i64, i64,
                                          ctypes.c_double, ctypes.c_int,
                                          ctypes.c_void_p, ctypes.c_void_p, i64,
                                          ctypes.c_void_p, i64, dp]
    lib.attn_bwd_rows_gqa_f64.restype = ctypes.c_int
    lib.attn_bwd_cols_gqa_f64.argtypes = [dp, dp, dp, dp, i64, i64, i64, i64, i64,
                                          ctypes.c_double, ctypes.c_int,
                                          ctypes.c_void_p, ctypes.c_void_p, i64,
                                          ctypes.c_void_p, i64, dp, dp]
    lib.attn_bwd_cols_gqa_f64.restype = ctypes.c_int
    lib.attn_ref_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = _configure(ctypes.CDLL(_build.ensure_built()))
    return _lib


def _f64(x):
    a = np.asarray(x)
    if a.dtype not in (np.float64, np.float32, np.float16):
        # bfloat16 arrive as float32 holding bf16 values; anything else is a bug
        raise TypeError(f"oracle inputs must be float arrays, got {a.dtype}")
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _prep(q, k, v, key_len, block_mask, block):
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.shape != v.shape or k.ndim != 4:
        raise ValueError("q must be [B, H, N, d] and k, v [B, H_kv, N, d]")
    B, H, N, d = q.shape
    if k.shape[0] != B or k.shape[2:] != (N, d) or k.shape[1] < 1 or H % k.shape[1]:
        raise ValueError("k, v must be [B, H_kv, N, d] with H a multiple of H_kv")
    kl = None
    if key_len is not None:
        kl = np.ascontiguousarray(key_len, dtype=np.int32)
        if kl.shape != (B,):
            raise ValueError("key_len must have shape [B]")
    bm = None
    if block_mask is not None:
        nb = (N + block - 1) // block
        bm = np.ascontiguousarray(block_mask, dtype=np.uint8)
        if bm.size != nb * nb:
            raise ValueError(f"block_mask must hold {nb}x{nb} entries")
    return q, k, v, kl, bm


def attention_f64(q, k, v, scale, causal=False, key_len=None, block_mask=None,
                  block=128):
    """O [B,H,N,d] float64 and LSE [B,H,N] float64 for the whole problem.

    ``scale`` is used as given (pass the same float32 value the GPU gets).
    k, v may have H_kv < H heads (grouped-query attention: query head h of a
    batch entry reads key/value head h // (H // H_kv)).
    """
    q, k, v, kl, bm = _prep(q, k, v, key_len, block_mask, block)
    B, H, N, d = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    rc = _load().attn_ref_gqa_f64(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, k.shape[1], N, d,
        float(scale), int(bool(causal)),
        kl.ctypes.data if kl is not None else None,
        bm.ctypes.data if bm is not None else None, block)
    if rc != 0:
        raise RuntimeError(f"attn_ref_f64 failed with code {rc}")
    return o, lse


def attention_rows_f64(q, k, v, rows, scale, causal=False, key_len=None,
                       block_mask=None, block=128):
    """Outputs for selected query rows only.

    ``rows`` holds flat row indices (b*H + h)*N + i.  Returns
    (o_rows [n, d], lse_rows [n]) in float64.
    """
    q, k, v, kl, bm = _prep(q, k, v, key_len, block_mask, block)
    B, H, N, d = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
    o = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    rc = _load().attn_ref_rows_gqa_f64(
        _ptr(q), _ptr(k), _ptr(v), B, H, k.shape[1], N, d, float(scale), int(bool(causal)),
        kl.ctypes.data if kl is not None else None,
        bm.ctypes.data if bm is not None else None, block,
        rows.ctypes.data, rows.size, _ptr(o), _ptr(lse))
    if rc != 0:
        raise RuntimeError(f"attn_ref_rows_f64 failed with code {rc}")
    return o, lse


def attention_bwd_f64(q, k, v, dout, scale, causal=False, key_len=None, block_mask=None,
                      block=128):
    """Gradients (dQ, dK, dV) in float64 of the loss sum(dout * O) for the
    attention definition above; k, v (and dK, dV) may have H_kv < H heads."""
    q, k, v, kl, bm = _prep(q, k, v, key_len, block_mask, block)
    dout = _f64(dout)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    B, H, N, d = q.shape
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    rc = _load().attn_bwd_ref_gqa_f64(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        B, H, k.shape[1], N, d, float(scale), int(bool(causal)),
        kl.ctypes.data if kl is not None else None,
        bm.ctypes.data if bm is not None else None, block)
    if rc != 0:
        raise RuntimeError(f"attn_bwd_ref_gqa_f64 failed with code {rc}")
    return dq, dk, dv


def attention_bwd_rows_f64(q, k, v, dout, rows, scale, causal=False, key_len=None,
                           block_mask=None, block=128):
    """dQ (float64, [n, d]) for selected query rows only; ``rows`` holds flat
    row indices (b*H + h)*N + i.  Same definition as attention_bwd_f64."""
    q, k, v, kl, bm = _prep(q, k, v, key_len, block_mask, block)
    dout = _f64(dout)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    B, H, N, d = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
    dq = np.empty((rows.size, d), dtype=np.float64)
    rc = _load().attn_bwd_rows_gqa_f64(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, k.shape[1], N, d, float(scale),
        int(bool(causal)), kl.ctypes.data if kl is not None else None,
        bm.ctypes.data if bm is not None else None, block, rows.ctypes.data, rows.size, _ptr(dq))
    if rc != 0:
        raise RuntimeError(f"attn_bwd_rows_gqa_f64 failed with code {rc}")
    return dq


def attention_bwd_cols_f64(q, k, v, dout, cols, scale, causal=False, key_len=None,
                           block_mask=None, block=128):
    """(dK, dV) (float64, [n, d] each) for selected keys only; ``cols`` holds
    flat key indices (b*H_kv + g)*N + j.  Same definition as
    attention_bwd_f64; costs one forward pass of the query heads that read
    the key/value heads involved."""
    q, k, v, kl, bm = _prep(q, k, v, key_len, block_mask, block)
    dout = _f64(dout)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    B, H, N, d = q.shape
    cols = np.ascontiguousarray(cols, dtype=np.int64).reshape(-1)
    dk = np.empty((cols.size, d), dtype=np.float64)
    dv = np.empty((cols.size, d), dtype=np.float64)
    rc = _load().attn_bwd_cols_gqa_f64(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, k.shape[1], N, d, float(scale),
        int(bool(causal)), kl.ctypes.data if kl is not None else None,
        bm.ctypes.data if bm is not None else None, block, cols.ctypes.data, cols.size,
        _ptr(dk), _ptr(dv))
    if rc != 0:
        raise RuntimeError(f"attn_bwd_cols_gqa_f64 failed with code {rc}")
    return dk, dv


def threads():
    """OpenMP threads the oracle's parallel regions use."""
    return int(_load().attn_ref_threads())


__all__ = ["attention_f64", "attention_rows_f64", "attention_bwd_f64", "attention_bwd_rows_f64",
           "attention_bwd_cols_f64", "threads"]
