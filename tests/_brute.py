"""Pure-Python brute-force attention for tiny inputs (an independent pin of the oracle).

Written with explicit loops, math.exp and math.fsum, with no numpy, so that it shares
no vectorised code path with oracle/attention.py.  Definition: "Phase 08" Concepts
list and Lab 01 step 1 (standard attention), screna.ai FlashAttention block
(S = QK^T, P = softmax(S), O = P V) and MHA/MQA/GQA block (grouped K/V heads).
"""

import math


def brute_attention(q, k, v, causal, scale, window=0, slopes=None):
    """q: nested lists [B][Hq][N][d]; k, v: [B][Hkv][N][d]. Returns (O, L) nested lists.
    window W: only keys j >= i - W + 1 (0 = none); slopes: ALiBi bias -slope[h] * |i - j|."""
    B = len(q)
    Hq = len(q[0])
    Hkv = len(k[0])
    G = Hq // Hkv
    O, L = [], []
    for b in range(B):
        Ob, Lb = [], []
        for h in range(Hq):
            kh = k[b][h // G]
            vh = v[b][h // G]
            Oh, Lh = [], []
            for i, qi in enumerate(q[b][h]):
                visible = [j for j in range(len(kh)) if ((not causal) or j <= i) and (not window or j >= i - window + 1)]
                bias = [0.0 if slopes is None else -slopes[h] * abs(i - j) for j in visible]
                scores = [scale * math.fsum(qi[t] * kh[j][t] for t in range(len(qi))) + bias[n]
                          for n, j in enumerate(visible)]
                top = max(scores)
                w = [math.exp(s - top) for s in scores]
                tot = math.fsum(w)
                d = len(vh[0])
                Oh.append([math.fsum(w[n] * vh[j][c] for n, j in enumerate(visible)) / tot for c in range(d)])
                Lh.append(top + math.log(tot))
            Ob.append(Oh)
            Lb.append(Lh)
        O.append(Ob)
        L.append(Lb)
    return O, L
