"""Plain fp64 CPU gradients of exact attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The GPU library never does.

What is differentiated is the function attention_ref defines ("Phase 08", Lab 01
step 1: standard attention; screna.ai FlashAttention and MHA/MQA/GQA blocks):
O = softmax(scale * Q K^T + mask) V per (batch, query head), query head h reading
K/V head h // (Hq // Hkv).  Given the upstream gradient dO of a loss with respect
to O, this returns the loss's gradients with respect to Q, K and V, computed the
textbook way with the full probability matrix materialised (the "Phase 08"
Concepts list names the FlashAttention backward as the consumer of O and L; the
pages give no formulas, so these are the standard chain-rule expressions):

    P   = softmax(S),  S = scale * Q K^T (masked entries -inf, their P = 0)
    dV  = P^T dO                          (summed over the query heads of a group)
    dP  = dO V^T
    dS  = P * (dP - rowsum(P * dP))       (softmax Jacobian applied row by row)
    dQ  = scale * dS K
    dK  = scale * dS^T Q                  (summed over the query heads of a group)

Pinned in tests/test_oracle_bwd.py by central finite differences of attention_ref,
closed forms and identities.
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def attention_bwd_ref(q, k, v, do, causal: bool, scale: float, chunk: int = 1024):
    """Gradients (dQ, dK, dV) of O = attention(Q, K, V) for upstream gradient dO.

    q, do [B, Hq, N, d]; k, v [B, Hkv, N, d].  Query rows are taken `chunk` at a time
    only to bound memory; each row's full probability vector is always formed.
    Rows with no visible key (none exist with equal query and key lengths) would
    contribute nothing.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    do = _f64(do)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape or do.shape != q.shape:
        raise ValueError("q/k/v/do shapes disagree")
    G = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    keys = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            kh, vh = k[b, g], v[b, g]
            for r0 in range(0, N, chunk):
                rows = np.arange(r0, min(N, r0 + chunk))
                s = scale * (q[b, h, rows] @ kh.T)
                if causal:
                    s = np.where(keys[None, :] <= rows[:, None], s, -np.inf)
                m = np.max(s, axis=1, keepdims=True)
                p = np.exp(s - m)
                p /= np.sum(p, axis=1, keepdims=True)
                dor = do[b, h, rows]
                dv[b, g] += p.T @ dor
                dp = dor @ vh.T
                ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
                dq[b, h, rows] = scale * (ds @ kh)
                dk[b, g] += scale * (ds.T @ q[b, h, rows])
    return dq, dk, dv


def attention_bwd_delta_ref(o, do):
    """D = rowsum(dO * O) per (batch, head, row): the value rowsum(P * dP) takes
    (since O = P V and dP = dO V^T), from O and dO alone."""
    return np.sum(_f64(o) * _f64(do), axis=-1)
