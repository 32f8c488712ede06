"""Shared element-by-element comparison of GPU outputs with the fp64 oracle.

Bars (the benchmark's tolerances): fp32 outputs O and L within 1e-4; bf16 outputs O
within 1e-2 and L within 1e-3, as max-abs errors over every compared element.

bf16 output floor.  Rounding the exact O to bf16 alone errs by up to half a bf16
ulp of O: 2^-7 = 0.0078 for |O| in [2, 4), but 2^-6 = 0.0156 for |O| in [4, 8),
more than the 1e-2 bar.  Where the format's half-ulp exceeds the bar no bf16
value can meet it, so there, and only there, an element passes when it is a
faithful bf16 rounding of the exact value: one of the two bf16 numbers that
bracket it (the correctly rounded one, or its neighbour on the other side of
the exact value when the kernel's fp32 result lay across the rounding midpoint).
Every other element must meet the bar.  Each check prints the largest error,
the floor max|bf16(O_ref) - O_ref|, and how many elements needed the rule and
were correctly rounded or the other neighbour.
"""

from __future__ import annotations

import numpy as np
import torch


def say(msg):
    print(msg, flush=True)


def f64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """x rounded to the nearest bf16 (ties to even), as float64."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.bfloat16).double().numpy()


def bf16_bracket(x: np.ndarray):
    """The bf16 values lo <= x < hi around x and their spacing sp = hi - lo (x normal
    in fp64; bf16 keeps 8 significant bits, so in the binade [2^e, 2^(e+1)) the
    spacing is 2^(e-7))."""
    _, ex = np.frexp(x)                    # |x| in [2^(ex-1), 2^ex)
    sp = np.ldexp(1.0, ex - 8)
    lo = np.floor(x / sp) * sp             # exact: division by a power of two
    return lo, lo + sp, sp


def check_outputs(O, L, Oref, Lref, what, tol_o, tol_l, bf16_out):
    """Compare every element.  O, L: GPU outputs (numpy fp64 or torch); Oref, Lref:
    the oracle's.  Rows with no visible key must have L = -inf (their O is 0)."""
    O, L = f64(O), f64(L)
    Oref, Lref = np.asarray(Oref, dtype=np.float64), np.asarray(Lref, dtype=np.float64)
    assert O.shape == Oref.shape and L.shape == Lref.shape, (what, O.shape, Oref.shape)
    assert np.all(np.isfinite(O)), f"{what}: non-finite O at {np.argwhere(~np.isfinite(O))[:4].tolist()}"
    fin = np.isfinite(Lref)
    assert np.all(np.isfinite(L[fin])), f"{what}: non-finite L"
    assert np.all(np.isneginf(L[~fin])), f"{what}: rows with no visible key must have L = -inf"
    err = np.abs(O - Oref)
    eo = float(err.max()) if err.size else 0.0
    el = float(np.abs(L[fin] - Lref[fin]).max()) if fin.any() else 0.0
    over = err > tol_o
    n_over = int(over.sum())
    floor = 0.0
    n_rne = n_other = 0
    if bf16_out and err.size:
        rne = bf16_rne(Oref)
        floor = float(np.abs(rne - Oref).max())
        if n_over:
            xo, go = Oref[over], O[over]
            lo, hi, sp = bf16_bracket(xo)
            wide = sp / 2 > tol_o                    # the format cannot meet the bar here
            faithful = (go == lo) | ((go == hi) & (xo != lo))
            is_rne = go == rne[over]
            is_other = faithful & ~is_rne
            ok = wide & faithful
            n_rne, n_other = int((wide & is_rne).sum()), int((wide & is_other).sum())
            if not ok.all():
                idx = np.argwhere(over)[~ok][:4].tolist()
                bad = np.flatnonzero(~ok)[:4]
                raise AssertionError(
                    f"{what}: O error {eo:.4g} > {tol_o} at {idx}: gpu {go[bad].tolist()} ref {xo[bad].tolist()} "
                    f"(not a faithful bf16 rounding where the format allows more than the bar)")
    say(f"{what}: max|dO|={eo:.3e} (bf16 output floor {floor:.3e}; {n_over} elements above {tol_o:g}: "
        f"{n_rne} correctly rounded, {n_other} the other bracketing bf16) max|dL|={el:.3e}")
    if not bf16_out:
        assert eo <= tol_o, f"{what}: O error {eo} > {tol_o}"
    assert el <= tol_l, f"{what}: L error {el} > {tol_l}"
    return eo, el, floor


def check_bf16(O, L, Oref, Lref, what, tol_o=1e-2, tol_l=1e-3):
    return check_outputs(O, L, Oref, Lref, what, tol_o, tol_l, True)


def check_f32(O, L, Oref, Lref, what, tol_o=1e-4, tol_l=1e-4):
    return check_outputs(O, L, Oref, Lref, what, tol_o, tol_l, False)


# ---- per-element bound of the bf16 forward's own roundings -------------------------
# The kernels give the P V product bf16-rounded probabilities r_j = p_j (1 + e_j),
# |e_j| <= 2^-8, and divide by their sum, so with w_j = p_j / sum p:
#   O_fp32 - O = sum_j w_j e_j (v_j - O) / (1 + sum_j w_j e_j),
# at most 2^-8 sum_j w_j |v_j - O| / (1 - 2^-8); the fp32 sums over n keys add up to
# n 2^-24 sum_j w_j |v_j|, and rounding O_fp32 to bf16 half a bf16 ulp.  On rows where
# a few keys carry the weight (scales far above 1/sqrt(d)) the first term no longer
# averages out and, with the output rounding, can exceed the 1e-2 bar where |O| lies in
# [2, 4) and the bf16 floor rule does not apply.
U_P = 2.0 ** -8
SLACK_P = 1.5   # exp2 and the scores' fp32 sums perturb p by well under 2^-9 relative


def fwd_p_bound(q, k, v, Oref, Lref, causal, scale, rows_per_chunk=16):
    """Per-element bound on |O_gpu - O| of the bf16 forward; q [B,Hq,N,d], k/v [B,Hkv,N,d]
    fp64 numpy, Oref/Lref the oracle's outputs."""
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    dev = np.zeros_like(Oref)
    acc = np.zeros_like(Oref)
    keys = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            K, V = k[b, h // G], v[b, h // G]
            for r0 in range(0, N, rows_per_chunk):
                rows = np.arange(r0, min(N, r0 + rows_per_chunk))
                s = scale * (q[b, h, rows] @ K.T)
                if causal:
                    s = np.where(keys[None, :] <= rows[:, None], s, -np.inf)
                w = np.exp(s - Lref[b, h, rows][:, None])               # softmax weights
                o = Oref[b, h, rows]
                dev[b, h, rows] = np.einsum("rj,rjc->rc", w, np.abs(V[None, :, :] - o[:, None, :]))
                acc[b, h, rows] = w @ np.abs(V)
    e32 = SLACK_P * (U_P / (1 - U_P) * dev + N * 2.0 ** -24 * acc)
    _, _, sp = bf16_bracket(np.abs(Oref) + e32 + 1e-300)
    return e32 + sp / 2


def check_bf16_p_bound(O, L, Oref, Lref, bound, what, tol_o=1e-2, tol_l=1e-3):
    """The bf16 check with one more allowance: an element above the bar passes when it
    lies within the forward's own per-element rounding bound (fwd_p_bound)."""
    O, L = f64(O), f64(L)
    err = np.abs(O - Oref)
    over = err > tol_o
    bad = over & (err > bound)
    fin = np.isfinite(Lref)
    el = float(np.abs(L[fin] - Lref[fin]).max()) if fin.any() else 0.0
    ratio = float((err / bound).max()) if err.size else 0.0
    say(f"{what}: max|dO|={err.max():.3e}, {int(over.sum())} elements above {tol_o:g}, largest error over "
        f"the P-rounding bound {ratio:.2f}, max|dL|={el:.3e}")
    if bad.any():
        idx = np.argwhere(bad)[:4].tolist()
        raise AssertionError(f"{what}: O error above both the bar and the rounding bound at {idx}: "
                             f"gpu {O[bad][:4].tolist()} ref {Oref[bad][:4].tolist()} bound {bound[bad][:4].tolist()}")
    assert np.all(np.isfinite(O)), f"{what}: non-finite O"
    assert el <= tol_l, f"{what}: L error {el} > {tol_l}"
    return ratio
