"""GPU parity of the backward (dQ, dK, dV) against the fp64 oracle, element by element.

The GPU backward consumes what a training step would: the bf16 inputs, the GPU
forward's bf16 O and fp32 L, and a bf16 upstream gradient dO.  The oracle
differentiates the exact function on the same bf16 inputs.  The pages give no
tolerance for gradients, so each element gets its own bound, derived from the
roundings the kernels make (bf16 keeps 8 significant bits: rounding x errs by at
most 2^-8 |x|):

  dV_j  <- sum_i bf16(P_ij) dO_i                      : 2^-8 sum_i P_ij |dO_i|
  dS_ij  = P_ij (dP_ij - D_i), rounded to bf16        : 2^-8 |dS_ij|
  D_i    = rowsum(dO_i * O_i) from the forward's bf16 O: |D_i - D_exact_i| = |dO_i . (O_i - O_exact_i)|
  dP_ij - D_i in fp32 (sums of d products)           : d 2^-24 (|dO_i| . |V_j| + |dO_i| . |O_i|)
  dQ_i  <- scale sum_j dS_ij K_j, dK_j <- scale sum_i dS_ij Q_i, each fed by both
  dS errors above; every output rounded to bf16        : 2^-8 |ref|

so, elementwise,
  |dV - ref| <= 2^-8 (P^T |dO| + |dV|)
  |dQ - ref| <= scale E |K| + 2^-8 |dQ|,   |dK - ref| <= scale E^T |Q| + 2^-8 |dK|,
  with E_ij = 2^-8 |dS_ij| + P_ij (|D_i - D_exact_i| + the fp32 term above),
summed over the query heads of a K/V group.  The check allows 1.5 times this bound
(second-order terms: fp32 accumulation over up to 8192 terms, exp2 rounding) and
prints the largest measured error over bound.  Small shapes compare every element;
the full-size workloads compare whole (batch, K/V head) slices.  Outputs are
pre-filled with NaN.
"""

import numpy as np
import pytest
import torch

from exact_io_aware_15_amd import fa_bwd, fa_fwd
from exact_io_aware_15_amd.workloads import CONFIGS, make_grad_output, make_inputs, make_prefill
from oracle import attention_bwd_ref

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SLACK = 1.5
U = 2.0 ** -8   # bf16 rounding, relative


def say(msg):
    print(msg, flush=True)


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def gpu_bwd(x, do, causal, scale=None):
    """(dq, dk, dv, o): the backward and the forward output it consumed."""
    q, k, v = (x[n].to(DEV) for n in "qkv")
    o, lse = fa_fwd(q, k, v, causal=causal, scale=scale)
    dq = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    dk = torch.full(k.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    dv = torch.full(v.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    fa_bwd(q, k, v, o, lse, do.to(DEV), causal=causal, scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return dq, dk, dv, o


def bwd_bounds(q, k, v, do, o_gpu, causal, scale, chunk=1024):
    """Per-element error bounds of the module docstring (fp64; same layouts as the
    gradients), from the exact probabilities on the same inputs and the forward's O."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    bq, bk, bv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
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
                p = np.exp(s - np.max(s, axis=1, keepdims=True))
                p /= np.sum(p, axis=1, keepdims=True)
                dor = do[b, h, rows]
                dp = dor @ vh.T
                dexact = np.sum(p * dp, axis=1, keepdims=True)
                ds = p * (dp - dexact)
                dD = np.sum(dor * (o_gpu[b, h, rows] - p @ vh), axis=1, keepdims=True)
                # fp32 sums of d products in dP and D: at most d * 2^-24 of their magnitude sums
                gam = d * 2.0 ** -24
                fp32 = gam * (np.abs(dor) @ np.abs(vh).T + np.sum(np.abs(dor * o_gpu[b, h, rows]), axis=1,
                                                                   keepdims=True))
                e = U * np.abs(ds) + p * (np.abs(dD) + fp32)
                bq[b, h, rows] = abs(scale) * (e @ np.abs(kh))
                bk[b, g] += abs(scale) * (e.T @ np.abs(q[b, h, rows]))
                bv[b, g] += U * (p.T @ np.abs(dor))
    return bq, bk, bv


def check(got, ref, bounds, what):
    worst = 0.0
    for name, g, r, bd in zip(("dQ", "dK", "dV"), got, ref, bounds):
        assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
        err = np.abs(g - r)
        bound = SLACK * (bd + U * np.abs(r))
        ratio = float(np.max(err / np.maximum(bound, 1e-300))) if r.size else 0.0
        worst = max(worst, ratio)
        say(f"{what} {name}: max|err|={float(err.max()):.3e} max|ref|={float(np.abs(r).max()):.3e} "
            f"largest err/bound={ratio:.3f}")
        bad = err > bound
        assert not bad.any(), (f"{what}: {name} exceeds its per-element bound at {np.argwhere(bad)[:4].tolist()}: "
                               f"err {err[bad][:4].tolist()} bound {bound[bad][:4].tolist()}")
    return worst


def compare(x, do, causal, scale, what, b=None, g=None):
    """Run the GPU backward and check every element (of one (batch, K/V head) slice when b, g are given)."""
    dq, dk, dv, o = gpu_bwd(x, do, causal, scale=scale)
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all().item()
    q, k, v, dof, of = f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(do), f64(o)
    got = [f64(dq), f64(dk), f64(dv)]
    if b is not None:
        G = q.shape[1] // k.shape[1]
        hs = slice(g * G, (g + 1) * G)
        q, dof, of = q[b:b + 1, hs], dof[b:b + 1, hs], of[b:b + 1, hs]
        k, v = k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1]
        got = [got[0][b:b + 1, hs], got[1][b:b + 1, g:g + 1], got[2][b:b + 1, g:g + 1]]
    ref = attention_bwd_ref(q, k, v, dof, causal, scale)
    bounds = bwd_bounds(q, k, v, dof, of, causal, scale)
    check(got, ref, bounds, what)
    return got


SMALL = [
    # B, Hq, Hkv, N, d, causal
    (1, 1, 1, 1, 64, False),
    (1, 1, 1, 17, 128, True),
    (1, 2, 1, 65, 64, True),
    (2, 2, 2, 127, 128, False),
    (1, 4, 2, 200, 128, True),
    (1, 4, 1, 300, 64, False),
    (2, 8, 1, 129, 128, True),
    (1, 2, 2, 513, 64, True),
    (1, 1, 1, 640, 128, True),
    (1, 6, 2, 200, 128, True),   # 3 query heads per K/V head
    (1, 5, 1, 150, 64, False),   # 5 query heads on one K/V head
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}_Hq{}_Hkv{}_N{}_d{}_{}".format(
    s[0], s[1], s[2], s[3], s[4], "causal" if s[5] else "full"))
def test_bwd_small_every_element(shape):
    B, Hq, Hkv, N, d, causal = shape
    say(f"bwd small {shape}")
    x = make_prefill(B, Hq, Hkv, N, d, "bf16", seed=300 + N + d)
    do = make_grad_output(B, Hq, N, d, seed=300 + N + d)
    compare(x, do, causal, 1.0 / np.sqrt(d), str(shape))


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.4])
def test_bwd_scale_edge_cases(scale):
    say(f"bwd scale {scale}")
    x = make_prefill(1, 2, 1, 150, 128, "bf16", seed=17)
    do = make_grad_output(1, 2, 150, 128, seed=17)
    for causal in (False, True):
        got = compare(x, do, causal, scale, f"scale={scale} causal={causal}")
        if scale == 0.0:
            # dQ and dK are exactly zero; dV is the plain average of dO over visible rows
            assert np.all(got[0] == 0) and np.all(got[1] == 0)


# (config, batch, K/V head) slices checked against the oracle at full size
FULL = [
    ("c2_bf16_B4_H16_N2048_d64", 3, 5),
    ("c3_bf16_causal_B1_H32_N8192_d128", 0, 31),
    ("c4_bf16_causal_gqa_B2_Hq32_Hkv8_N4096_d128", 1, 7),
    ("c4_bf16_causal_mqa_B2_Hq32_Hkv1_N4096_d128", 0, 0),
]


@pytest.mark.parametrize("name,b,g", FULL, ids=[f[0] for f in FULL])
def test_bwd_full_size_slice(name, b, g):
    cfg = CONFIGS[name]
    say(f"bwd full-size {name} b={b} g={g}")
    x = make_inputs(cfg)
    do = make_grad_output(cfg.B, cfg.Hq, cfg.N, cfg.d, seed=cfg.seed)
    compare(x, do, cfg.causal, cfg.scale, f"{name} b={b} g={g}", b=b, g=g)


def test_bwd_deterministic():
    say("bwd determinism")
    x = make_prefill(1, 4, 1, 500, 128, "bf16", seed=21)
    do = make_grad_output(1, 4, 500, 128, seed=21)
    a = gpu_bwd(x, do, True)[:3]
    c = gpu_bwd(x, do, True)[:3]
    for s, t in zip(a, c):
        assert torch.equal(s, t)
