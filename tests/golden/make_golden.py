"""Write tests/golden/brute_small.json from the 40-digit brute-force oracle.

Calls only oracle.brute (and the seeded input generator); run from the repo
root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import mpmath  # noqa: E402

from oracle import brute  # noqa: E402
from workloads import random_qkv  # noqa: E402

CASES = [
    dict(name="dense", causal=False, key_len=None, block_mask=None, block=128),
    dict(name="causal", causal=True, key_len=None, block_mask=None, block=128),
    dict(name="padded", causal=False, key_len=[4, 1], block_mask=None, block=128),
    # 3x3 blocks of 2 tokens; query block 1 has no active key block
    dict(name="block_mask", causal=False, key_len=None,
         block_mask=[1, 0, 1, 0, 0, 0, 0, 1, 1], block=2),
    dict(name="all_modes", causal=True, key_len=[5, 6],
         block_mask=[1, 0, 1, 1, 1, 0, 0, 1, 1], block=2),
]


def main():
    q, k, v, _ = random_qkv(2, 2, 6, 4, seed=7, dtype="bf16")
    scale = 0.5
    out = dict(
        citation=("Expected O and LSE of S = scale*Q K^T, A = row-softmax(S), O = A V with "
                  "disallowed logits at -inf, from the page 'Ch.04 Attention optimisation: "
                  "FlashAttention and sparse attention' (mdooai.com), 'Key points of the "
                  "formulas'; evaluated by oracle/brute.py in mpmath at %d digits." % brute.DPS),
        generator="tests/golden/make_golden.py",
        shape=list(q.shape), scale=scale,
        q=q.tolist(), k=k.tolist(), v=v.tolist(), cases=[])
    for c in CASES:
        O, L = brute.attention_mp(q, k, v, scale, c["causal"], c["key_len"],
                                  c["block_mask"], c["block"])
        out["cases"].append(dict(c, O=[[[[mpmath.nstr(x, 30) for x in row] for row in h] for h in b] for b in O],
                                 LSE=[[[mpmath.nstr(x, 30) for x in h] for h in b] for b in L]))
    path = os.path.join(HERE, "brute_small.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(path)


if __name__ == "__main__":
    main()
