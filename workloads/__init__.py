"""Seeded synthetic workloads for the attention forward path.

This module only draws inputs: random Q, K, V, per-sequence key lengths and
128 x 128 block masks.  It holds none of the attention arithmetic and is the
one module that both the GPU tests/benchmark and the oracle checks draw their
inputs from.

Recipe (shared by every configuration):
  * generator: numpy PCG64 seeded with the configuration's seed;
  * Q, K, V drawn in that order as float32 standard normals of shape
    [B, H, N, d], times ``amp`` (a power of two, so exact);
  * bf16 workloads round each value to bfloat16 with round-to-nearest-even
    (torch's float32 -> bfloat16 conversion) and keep it as float32 holding a
    bf16-representable value, so the oracle widens exactly what the GPU reads;
  * key lengths (padding workload) are drawn after Q, K, V as integers
    uniform in [lo, hi] inclusive, one per batch entry;
  * the block mask (sparse workload) is drawn after Q, K, V: for query block r
    the key blocks c with |r - c| <= 1 (a band three blocks wide, clipped at
    the edges) plus ``n_global`` distinct blocks chosen uniformly among those
    outside that band, rows in ascending order.  One mask for all (b, h).

The shapes follow the five workloads the attention library is measured on:
a tiny fp32 case, a GPT-2-small-shaped causal batch, a BERT-large-shaped
padded batch, a 16K-token causal context and a 4K-token block-sparse batch.
"""
from dataclasses import dataclass, field
import math

import numpy as np

MASK_BLOCK = 128  # block edge of the block-sparse mask, in tokens


@dataclass(frozen=True)
class Workload:
    key: str
    title: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "f32" or "bf16": the I/O type of the attention call
    causal: bool
    seed: int
    amp: float = 1.0
    key_len_range: tuple = None     # (lo, hi) inclusive, padding workload
    sparse_globals: int = 0         # >0: block-sparse workload
    notes: dict = field(default_factory=dict)

    @property
    def scale(self):
        """1/sqrt(d) rounded to float32: the value passed to the kernel."""
        return np.float32(1.0 / math.sqrt(self.d))


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "tiny non-causal fp32 attention",
                         1, 1, 128, 64, "f32", False, 1001),
    "gpt2_causal": Workload("gpt2_causal", "GPT-2-small-shaped causal attention",
                            8, 12, 1024, 64, "bf16", True, 1002),
    "bert_padded": Workload("bert_padded", "BERT-large-shaped attention with key padding",
                            16, 16, 512, 64, "bf16", False, 1003,
                            key_len_range=(256, 512)),
    "long_causal": Workload("long_causal", "16K-token causal attention, d=128",
                            1, 16, 16384, 128, "bf16", True, 1004, amp=0.5),
    "block_sparse": Workload("block_sparse", "block-sparse attention, band 3 + 4 global blocks",
                             4, 16, 4096, 64, "bf16", False, 1005, sparse_globals=4),
}
ORDER = ["tiny_f32", "gpt2_causal", "bert_padded", "long_causal", "block_sparse"]


def bf16_round(x):
    """float32 array -> float32 array of the nearest bfloat16 values (RNE)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def band_global_block_mask(nb, rng, n_global=4, radius=1):
    """uint8 [nb * nb] mask, row = query block, column = key block."""
    m = np.zeros((nb, nb), dtype=np.uint8)
    for r in range(nb):
        lo, hi = max(0, r - radius), min(nb - 1, r + radius)
        m[r, lo:hi + 1] = 1
        outside = np.array([c for c in range(nb) if c < lo or c > hi], dtype=np.int64)
        g = min(n_global, outside.size)
        if g:
            m[r, rng.choice(outside, g, replace=False)] = 1
    return m.reshape(-1)


def f16_round(x):
    """float32 array -> float32 array of the nearest IEEE half values (RNE)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def random_qkv(B, H, N, d, seed, dtype="bf16", amp=1.0, rng=None):
    """Q, K, V as float32 [B,H,N,d] (bf16- or fp16-representable when dtype is
    'bf16' or 'f16'; the unrounded float32 draw otherwise)."""
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(3):
        x = rng.standard_normal((B, H, N, d), dtype=np.float32)
        if amp != 1.0:
            x *= np.float32(amp)
        if dtype == "bf16":
            x = bf16_round(x)
        elif dtype == "f16":
            x = f16_round(x)
        out.append(x)
    return out[0], out[1], out[2], rng


def causal_prefix(w, N, H, fmt=None):
    """Rows 0..N-1 of heads 0..H-1 of causal workload ``w``'s full tensors.

    Under a causal mask these rows attend only to keys 0..N-1, so the slice
    is a self-contained problem whose exact outputs are those rows of the
    full problem.  ``fmt`` re-rounds the workload's float32 draw to another
    I/O format instead ("f32": unrounded, "f16": IEEE half, "bf16").
    Returns a dict like make_inputs.
    """
    if not w.causal or w.key_len_range is not None or w.sparse_globals:
        raise ValueError("causal_prefix needs a plain causal workload")
    q, k, v, _ = random_qkv(w.B, w.H, w.N, w.d, w.seed, fmt or w.dtype, w.amp)
    cut = lambda x: np.ascontiguousarray(x[:, :H, :N])
    return dict(q=cut(q), k=cut(k), v=cut(v), key_len=None, block_mask=None,
                scale=w.scale, causal=True)


def make_inputs(w, N=None, H=None, B=None):
    """Inputs of workload ``w`` (optionally with a smaller B/H/N, same recipe).

    Returns a dict: q, k, v (float32 ndarrays), key_len (int32 [B] or None),
    block_mask (uint8 [nb*nb] or None), scale (np.float32), causal (bool).
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    q, k, v, rng = random_qkv(B, H, N, w.d, w.seed, w.dtype, w.amp)
    key_len = None
    if w.key_len_range is not None:
        lo, hi = w.key_len_range
        key_len = rng.integers(min(lo, N), min(hi, N), size=B, endpoint=True).astype(np.int32)
    block_mask = None
    if w.sparse_globals:
        nb = (N + MASK_BLOCK - 1) // MASK_BLOCK
        block_mask = band_global_block_mask(nb, rng, w.sparse_globals)
    return dict(q=q, k=k, v=v, key_len=key_len, block_mask=block_mask,
                scale=w.scale, causal=w.causal)


def allowed_pairs(N, B, H, causal=False, key_len=None, block_mask=None,
                  block=MASK_BLOCK):
    """Count of (b, h, i, j) with key j visible to query i: the unit behind the
    algorithmic FLOP count 4*d per visible pair.  Counting only, no attention."""
    total = 0
    nb = (N + block - 1) // block
    for b in range(B):
        kl = N if key_len is None else int(min(max(key_len[b], 0), N))
        if block_mask is None:
            if causal:
                # sum over i of min(i+1, kl)
                full = min(kl, N)
                total_b = full * (full + 1) // 2 + (N - full) * full
            else:
                total_b = N * kl
        else:
            bm = np.asarray(block_mask).reshape(nb, nb)
            total_b = 0
            for r in range(nb):
                rows = min(block, N - r * block)
                for c in range(nb):
                    if not bm[r, c]:
                        continue
                    c0, c1 = c * block, min(N, (c + 1) * block)
                    for i in range(r * block, r * block + rows):
                        hi = min(c1, kl, i + 1 if causal else c1)
                        total_b += max(0, hi - c0)
        total += total_b * H
    return total
