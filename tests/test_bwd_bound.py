"""The per-element backward bound of tests/test_backward_gpu.py, checked on the CPU:
a numpy emulation of the kernels' roundings (bf16 P in dV, bf16 dS, D from the bf16
forward output, bf16 outputs) stays inside it, and a planted error does not."""

import numpy as np
import pytest
import torch

from exact_io_aware_15_amd.workloads import make_grad_output, make_prefill
from oracle import attention_bwd_ref
from test_backward_gpu import bwd_bounds, check


def bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


def emulate(q, k, v, do, causal, scale):
    """The backward with the kernels' roundings, in fp64 otherwise; also the bf16 forward O."""
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    dq, dk, dv, o = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(q)
    keys = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            s = scale * (q[b, h] @ k[b, g].T)
            if causal:
                s = np.where(keys[None, :] <= keys[:, None], s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            o[b, h] = bf16(p @ v[b, g])
            dp = do[b, h] @ v[b, g].T
            ds = bf16(p * (dp - np.sum(do[b, h] * o[b, h], axis=1, keepdims=True)))
            dv[b, g] += bf16(p).T @ do[b, h]
            dq[b, h] = scale * (ds @ k[b, g])
            dk[b, g] += scale * (ds.T @ q[b, h])
    return bf16(dq), bf16(dk), bf16(dv), o


@pytest.mark.parametrize("causal", [False, True])
def test_emulated_kernel_roundings_stay_inside_the_bound(causal):
    x = make_prefill(1, 4, 2, 96, 64, "bf16", seed=5)
    q, k, v = (x[n].double().numpy() for n in "qkv")
    do = make_grad_output(1, 4, 96, 64, seed=5).double().numpy()
    scale = 0.125
    dq, dk, dv, o = emulate(q, k, v, do, causal, scale)
    ref = attention_bwd_ref(q, k, v, do, causal, scale)
    bounds = bwd_bounds(q, k, v, do, o, causal, scale)
    worst = check([dq, dk, dv], ref, bounds, f"emulated causal={causal}")
    assert worst > 0.05   # the bound is not vacuous: the roundings use a visible part of it


def test_planted_error_on_a_small_element_fails():
    x = make_prefill(1, 2, 1, 64, 64, "bf16", seed=6)
    q, k, v = (x[n].double().numpy() for n in "qkv")
    do = make_grad_output(1, 2, 64, 64, seed=6).double().numpy()
    dq, dk, dv, o = emulate(q, k, v, do, True, 0.125)
    ref = attention_bwd_ref(q, k, v, do, True, 0.125)
    bounds = bwd_bounds(q, k, v, do, o, True, 0.125)
    # the smallest nonzero dK element, off by 5 % of itself: far below a normwise bar
    idx = np.unravel_index(np.argmin(np.where(np.abs(ref[1]) > 0, np.abs(ref[1]), np.inf)), ref[1].shape)
    bad = dk.copy()
    bad[idx] = ref[1][idx] * 1.05 + np.sign(ref[1][idx]) * 1e-3 * np.abs(ref[1]).max()
    with pytest.raises(AssertionError):
        check([dq, bad, dv], ref, bounds, "planted")
