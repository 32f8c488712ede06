"""The per-element bound of the bf16 forward's roundings (tests/_parity.py: fwd_p_bound),
checked on the CPU: a numpy emulation of the kernel's arithmetic (bf16-rounded
probabilities in the P V product, O divided by their sum, O rounded to bf16) stays inside
it on rows dominated by a few keys, using a visible part of it, and a planted error does
not."""

import numpy as np
import pytest

from _parity import bf16_rne, check_bf16_p_bound, fwd_p_bound
from exact_io_aware_15_amd.workloads import make_prefill
from oracle import attention_ref


def emulate(q, k, v, causal, scale):
    """O of the bf16 forward: r = bf16(p), O = bf16(sum r v / sum r); fp64 otherwise."""
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    o = np.zeros_like(q)
    keys = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, h] @ k[b, h // G].T)
            if causal:
                s = np.where(keys[None, :] <= keys[:, None], s, -np.inf)
            r = bf16_rne(np.exp(s - s.max(axis=1, keepdims=True)))
            o[b, h] = bf16_rne((r @ v[b, h // G]) / r.sum(axis=1, keepdims=True))
    return o


@pytest.mark.parametrize("causal", [False, True])
def test_emulated_roundings_stay_inside_the_bound(causal):
    # scale 0.9 at d = 128 on unit-variance inputs: a few keys carry each row's weight
    x = make_prefill(1, 2, 1, 400, 128, "bf16", seed=71)
    q, k, v = (x[n].double().numpy() for n in "qkv")
    O, L = attention_ref(q, k, v, causal, 0.9)
    Oe = emulate(q, k, v, causal, 0.9)
    bound = fwd_p_bound(q, k, v, O, L, causal, 0.9)
    ratio = check_bf16_p_bound(Oe, L, O, L, bound, f"emulated scale 0.9 causal={causal}")
    assert ratio > 0.3    # the roundings use a visible part of the bound


def test_bound_is_tight_where_the_weight_is_spread():
    # scale 1/sqrt(d) on the same inputs: the bound is small, close to the output rounding
    x = make_prefill(1, 1, 1, 256, 64, "bf16", seed=3)
    q, k, v = (x[n].double().numpy() for n in "qkv")
    O, L = attention_ref(q, k, v, True, 0.125)
    bound = fwd_p_bound(q, k, v, O, L, True, 0.125)
    assert np.median(bound) < 1e-2


def test_planted_error_fails():
    x = make_prefill(1, 1, 1, 200, 128, "bf16", seed=72)
    q, k, v = (x[n].double().numpy() for n in "qkv")
    O, L = attention_ref(q, k, v, True, 0.9)
    Oe = emulate(q, k, v, True, 0.9)
    bound = fwd_p_bound(q, k, v, O, L, True, 0.9)
    i = np.unravel_index(np.argmax(np.where(np.abs(O) < 1, bound, 0)), O.shape)
    Oe[i] = O[i] + max(1.5 * bound[i], 0.011)
    with pytest.raises(AssertionError):
        check_bf16_p_bound(Oe, L, O, L, bound, "planted")
