"""Brute-force high-precision attention for tiny inputs -- TEST INFRASTRUCTURE.

An independent second evaluation of the attention definition on the page
"Ch.04 Attention optimisation: FlashAttention and sparse attention"
(mdooai.com, "Key points of the formulas"): S_ij = scale * q_i . k_j,
A_ij = exp(S_ij) / sum_j' exp(S_ij') over the allowed keys, O_i = sum_j A_ij v_j,
with disallowed keys dropped (their -inf logit contributes exp(-inf) = 0).

It works in mpmath at 40 significant digits with pure-Python loops and, unlike
the C oracle, neither materialises S nor subtracts the row maximum, so it
shares the definition but no code path with attn_ref.c.  Use only for N <= ~16
with bounded logits.  A row with no allowed key returns O = 0, LSE = -inf
(the reading the C oracle also takes).
"""
import mpmath

DPS = 40


def attention_mp(q, k, v, scale, causal=False, key_len=None, block_mask=None,
                 block=128):
    """q: nested lists or arrays [B][H][N][d], k and v [B][H_kv][N][d] (query
    head h reads key/value head h // (H // H_kv)); returns (O, LSE) as nested
    lists of mpmath.mpf.  block_mask is a flat sequence of ceil(N/block)^2."""
    with mpmath.workdps(DPS):
        B, H, N, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
        G = H // len(k[0])  # query heads per key/value head (grouped-query attention)
        nkb = (N + block - 1) // block
        sc = mpmath.mpf(float(scale))
        O, L = [], []
        for b in range(B):
            Ob, Lb = [], []
            for h in range(H):
                Oh, Lh = [], []
                for i in range(N):
                    num = [mpmath.mpf(0)] * d
                    den = mpmath.mpf(0)
                    for j in range(N):
                        if causal and j > i:
                            continue
                        if key_len is not None and j >= int(key_len[b]):
                            continue
                        if block_mask is not None and int(block_mask[(i // block) * nkb + j // block]) == 0:
                            continue
                        s = mpmath.fsum(mpmath.mpf(float(q[b][h][i][c])) * mpmath.mpf(float(k[b][h // G][j][c]))
                                        for c in range(d))
                        w = mpmath.exp(sc * s)
                        den += w
                        for c in range(d):
                            num[c] += w * mpmath.mpf(float(v[b][h // G][j][c]))
                    if den == 0:
                        Oh.append([mpmath.mpf(0)] * d)
                        Lh.append(mpmath.mpf("-inf"))
                    else:
                        Oh.append([x / den for x in num])
                        Lh.append(mpmath.log(den))
                Ob.append(Oh)
                Lb.append(Lh)
            O.append(Ob)
            L.append(Lb)
        return O, L
