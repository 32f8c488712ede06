"""GPU parity of the backward (dQ, dK, dV) against the fp64 oracle.

The GPU backward consumes what a training step would: the bf16 inputs, the GPU
forward's bf16 O and fp32 L, and a bf16 upstream gradient dO.  The oracle
differentiates the exact function on the same bf16 inputs.  No tolerance is given
for the backward; the bar used here is normwise per tensor,
max|gpu - ref| <= 2e-2 * max|ref|: the kernels round P and dS to bf16 before the
matrix products (relative 2^-9 each), use the bf16-rounded O in D = rowsum(dO * O),
and round the outputs to bf16 (2^-9), about 3 * 2^-9 = 0.6% of the largest
element in the worst case; the bar leaves a factor of three.  Small shapes
compare every element; the full-size workloads compare whole (batch, K/V head)
slices the oracle can afford.  Outputs are pre-filled with NaN.
"""

import numpy as np
import pytest
import torch

from exact_io_aware_15_amd import fa_bwd, fa_fwd
from exact_io_aware_15_amd.workloads import CONFIGS, make_grad_output, make_inputs, make_prefill
from oracle import attention_bwd_ref

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL = 2e-2


def say(msg):
    print(msg, flush=True)


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def gpu_bwd(x, do, causal, scale=None):
    q, k, v = (x[n].to(DEV) for n in "qkv")
    o, lse = fa_fwd(q, k, v, causal=causal, scale=scale)
    dq = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    dk = torch.full(k.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    dv = torch.full(v.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    fa_bwd(q, k, v, o, lse, do.to(DEV), causal=causal, scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(got, ref, what):
    worst = 0.0
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
        den = float(np.max(np.abs(r))) if r.size else 0.0
        err = float(np.max(np.abs(g - r))) if r.size else 0.0
        rel = err / den if den > 0 else err
        worst = max(worst, rel)
        say(f"{what} {name}: max|err|={err:.3e} max|ref|={den:.3e} ratio={rel:.2e}")
        assert rel <= REL, f"{what}: {name} error {err} > {REL} * {den}"
    return worst


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
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}_Hq{}_Hkv{}_N{}_d{}_{}".format(
    s[0], s[1], s[2], s[3], s[4], "causal" if s[5] else "full"))
def test_bwd_small_every_element(shape):
    B, Hq, Hkv, N, d, causal = shape
    say(f"bwd small {shape}")
    x = make_prefill(B, Hq, Hkv, N, d, "bf16", seed=300 + N + d)
    do = make_grad_output(B, Hq, N, d, seed=300 + N + d)
    got = [f64(t) for t in gpu_bwd(x, do, causal)]
    ref = attention_bwd_ref(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(do), causal, 1.0 / np.sqrt(d))
    check(got, ref, str(shape))


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.4])
def test_bwd_scale_edge_cases(scale):
    say(f"bwd scale {scale}")
    x = make_prefill(1, 2, 1, 150, 128, "bf16", seed=17)
    do = make_grad_output(1, 2, 150, 128, seed=17)
    for causal in (False, True):
        got = [f64(t) for t in gpu_bwd(x, do, causal, scale=scale)]
        ref = attention_bwd_ref(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(do), causal, scale)
        if scale == 0.0:
            # dQ and dK are exactly zero; dV is the plain average of dO over visible rows
            assert np.all(got[0] == 0) and np.all(got[1] == 0)
        check(got, ref, f"scale={scale} causal={causal}")


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
    dq, dk, dv = gpu_bwd(x, do, cfg.causal, scale=cfg.scale)
    G = cfg.Hq // cfg.Hkv
    hs = slice(g * G, (g + 1) * G)
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all().item()
    ref = attention_bwd_ref(f64(x["q"][b:b + 1, hs]), f64(x["k"][b:b + 1, g:g + 1]), f64(x["v"][b:b + 1, g:g + 1]),
                            f64(do[b:b + 1, hs]), cfg.causal, cfg.scale)
    got = [f64(dq[b:b + 1, hs]), f64(dk[b:b + 1, g:g + 1]), f64(dv[b:b + 1, g:g + 1])]
    check(got, ref, f"{name} b={b} g={g}")


def test_bwd_deterministic():
    say("bwd determinism")
    x = make_prefill(1, 4, 1, 500, 128, "bf16", seed=21)
    do = make_grad_output(1, 4, 500, 128, seed=21)
    a = gpu_bwd(x, do, True)
    c = gpu_bwd(x, do, True)
    for s, t in zip(a, c):
        assert torch.equal(s, t)
