"""Pins of the fp64 backward oracle (CPU only): finite differences of the forward
definition, closed forms and identities."""

import numpy as np
import pytest

from oracle import attention_bwd_delta_ref, attention_bwd_ref, attention_ref


def _rand(shape, seed):
    return np.random.default_rng(2000 + seed).standard_normal(shape)


def _loss(q, k, v, do, causal, scale):
    o, _ = attention_ref(q, k, v, causal, scale)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(1, 1), (2, 1), (4, 2)])
def test_bwd_matches_central_finite_differences(causal, hq, hkv):
    # loss = sum(O * dO) has gradient dO with respect to O, so its gradients with
    # respect to Q, K, V are exactly what attention_bwd_ref returns
    B, N, d, scale = 1, 5, 3, 0.7
    q = _rand((B, hq, N, d), 1)
    k = _rand((B, hkv, N, d), 2)
    v = _rand((B, hkv, N, d), 3)
    do = _rand((B, hq, N, d), 4)
    dq, dk, dv = attention_bwd_ref(q, k, v, do, causal, scale)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            fp = _loss(q, k, v, do, causal, scale)
            x[idx] = old - eps
            fm = _loss(q, k, v, do, causal, scale)
            x[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_bwd_scale_zero_closed_form():
    # scale 0: P is uniform over the visible keys, dQ = dK = 0 and dV_j is the sum of
    # dO_i / (number of keys row i sees) over the rows that see key j
    B, H, N, d = 1, 2, 6, 4
    q, k, v, do = (_rand((B, H, N, d), s) for s in range(4))
    for causal in (False, True):
        dq, dk, dv = attention_bwd_ref(q, k, v, do, causal, 0.0)
        assert np.all(dq == 0) and np.all(dk == 0)
        want = np.zeros_like(dv)
        for i in range(N):
            seen = range(i + 1) if causal else range(N)
            for j in seen:
                want[:, :, j] += do[:, :, i] / len(seen)
        np.testing.assert_allclose(dv, want, rtol=1e-13, atol=1e-13)


def test_bwd_constant_keys_give_zero_dq():
    # identical keys: every score of a row is the same, softmax is flat whatever Q
    # is, so the loss does not depend on Q
    B, H, N, d = 1, 1, 7, 5
    q, v, do = _rand((B, H, N, d), 5), _rand((B, H, N, d), 6), _rand((B, H, N, d), 7)
    k = np.broadcast_to(_rand((1, 1, 1, d), 8), (B, H, N, d)).copy()
    for causal in (False, True):
        dq, _, _ = attention_bwd_ref(q, k, v, do, causal, 0.9)
        np.testing.assert_allclose(dq, 0.0, atol=1e-12)


def test_bwd_gqa_equals_mha_on_repeated_kv():
    B, Hq, Hkv, N, d = 2, 4, 2, 9, 4
    q, do = _rand((B, Hq, N, d), 9), _rand((B, Hq, N, d), 10)
    k, v = _rand((B, Hkv, N, d), 11), _rand((B, Hkv, N, d), 12)
    G = Hq // Hkv
    for causal in (False, True):
        dq, dk, dv = attention_bwd_ref(q, k, v, do, causal, 0.5)
        dq2, dk2, dv2 = attention_bwd_ref(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), do, causal, 0.5)
        np.testing.assert_allclose(dq, dq2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dk, dk2.reshape(B, Hkv, G, N, d).sum(axis=2), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dv, dv2.reshape(B, Hkv, G, N, d).sum(axis=2), rtol=1e-12, atol=1e-12)


def test_bwd_row_chunking_does_not_change_the_result():
    B, H, N, d = 1, 2, 13, 4
    q, k, v, do = (_rand((B, H, N, d), 20 + s) for s in range(4))
    a = attention_bwd_ref(q, k, v, do, True, 0.3)
    b = attention_bwd_ref(q, k, v, do, True, 0.3, chunk=4)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-13)


def test_delta_equals_rowsum_of_p_times_dp():
    B, H, N, d, scale = 1, 1, 8, 4, 0.6
    q, k, v, do = (_rand((B, H, N, d), 30 + s) for s in range(4))
    o, _ = attention_ref(q, k, v, True, scale)
    s = scale * q[0, 0] @ k[0, 0].T
    s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dp = do[0, 0] @ v[0, 0].T
    np.testing.assert_allclose(attention_bwd_delta_ref(o, do)[0, 0], np.sum(p * dp, axis=1), rtol=1e-12)
