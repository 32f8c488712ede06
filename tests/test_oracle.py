"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test fixes the oracle to a fact that the pages or mathematics determine:
hand-derived worked examples, closed forms, brute force on tiny inputs, and the
identities the method rests on.  None of these needs the GPU.
"""

import glob
import json
import math
import os

import numpy as np
import pytest

from oracle import attention_ref, decode_ref, gather_pages_ref, lse_merge_ref, online_ref
from tests._brute import brute_attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(1000 + seed)


def _rand(shape, seed):
    return _rng(seed).standard_normal(shape)


# --------------------------------------------------------------------------- golden

def _arr(x):
    return np.asarray(x, dtype=np.float64) if not isinstance(x, list) else np.array(
        json.loads(json.dumps(x).replace('"nan"', "NaN")), dtype=np.float64)


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLDEN, "*.json"))),
                         ids=lambda p: os.path.basename(p))
def test_golden_worked_examples(path):
    with open(path) as f:
        g = json.load(f)
    assert g["citation"] and g["derivation"]
    if "page_table" in g:
        O, L = decode_ref(_arr(g["q"]), _arr(g["kpages"]), _arr(g["vpages"]),
                          np.array(g["page_table"]), np.array(g["ctx_lens"]), g["scale"])
    else:
        O, L = attention_ref(_arr(g["q"]), _arr(g["k"]), _arr(g["v"]), g["causal"], g["scale"])
    np.testing.assert_allclose(O, _arr(g["O"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, _arr(g["L"]), rtol=0, atol=1e-13)


# --------------------------------------------------------------------------- brute force

TINY = [
    # B, Hq, Hkv, N, d, causal
    (1, 1, 1, 1, 1, False),
    (1, 1, 1, 5, 3, False),
    (1, 1, 1, 5, 3, True),
    (2, 2, 1, 4, 2, True),
    (1, 4, 2, 6, 4, False),
    (1, 4, 2, 6, 4, True),
    (2, 2, 2, 3, 4, True),
]


@pytest.mark.parametrize("shape", TINY)
def test_brute_force_tiny(shape):
    B, Hq, Hkv, N, d, causal = shape
    seed = hash(shape) % 997
    q = _rand((B, Hq, N, d), seed)
    k = _rand((B, Hkv, N, d), seed + 1)
    v = _rand((B, Hkv, N, d), seed + 2)
    scale = 0.37 + 0.5 * (seed % 3)
    Ob, Lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), causal, scale)
    O, L = attention_ref(q, k, v, causal, scale)
    np.testing.assert_allclose(O, np.array(Ob), rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, np.array(Lb), rtol=0, atol=1e-13)


def test_rows_subset_matches_full():
    q = _rand((1, 2, 37, 8), 1)
    k = _rand((1, 2, 37, 8), 2)
    v = _rand((1, 2, 37, 8), 3)
    rows = np.array([0, 5, 36, 17])
    for causal in (False, True):
        O, L = attention_ref(q, k, v, causal, 0.3)
        Os, Ls = attention_ref(q, k, v, causal, 0.3, rows=rows, chunk=3)
        np.testing.assert_allclose(Os, O[:, :, rows], rtol=0, atol=1e-14)
        np.testing.assert_allclose(Ls, L[:, :, rows], rtol=0, atol=1e-14)


# --------------------------------------------------------------------------- closed forms

def test_constant_keys_noncausal_gives_mean_of_v():
    N, d, scale = 23, 8, 0.41
    q = _rand((1, 1, N, d), 4)
    k0 = _rand((d,), 5)
    k = np.broadcast_to(k0, (1, 1, N, d)).copy()
    v = _rand((1, 1, N, d), 6)
    O, L = attention_ref(q, k, v, False, scale)
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(v[0, 0].mean(axis=0), (N, d)), atol=1e-13)
    np.testing.assert_allclose(L[0, 0], scale * q[0, 0] @ k0 + math.log(N), atol=1e-13)


def test_constant_keys_causal_gives_prefix_means():
    N, d, scale = 19, 4, 0.7
    q = _rand((1, 1, N, d), 7)
    k0 = _rand((d,), 8)
    k = np.broadcast_to(k0, (1, 1, N, d)).copy()
    v = _rand((1, 1, N, d), 9)
    O, L = attention_ref(q, k, v, True, scale)
    prefix = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    np.testing.assert_allclose(O[0, 0], prefix, atol=1e-13)
    np.testing.assert_allclose(L[0, 0], scale * q[0, 0] @ k0 + np.log(np.arange(1, N + 1)), atol=1e-13)


def test_scale_zero_gives_uniform_weights():
    N, d = 11, 3
    q, k, v = (_rand((1, 1, N, d), s) for s in (10, 11, 12))
    O, L = attention_ref(q, k, v, False, 0.0)
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(v[0, 0].mean(0), (N, d)), atol=1e-13)
    np.testing.assert_allclose(L[0, 0], math.log(N), atol=1e-13)
    Oc, Lc = attention_ref(q, k, v, True, 0.0)
    np.testing.assert_allclose(Lc[0, 0], np.log(np.arange(1, N + 1)), atol=1e-13)


def test_one_hot_dominant_logit_selects_v_row():
    # q = c e0, k_{j*} = a e0, other keys 0: the selected score exceeds the rest by
    # scale*c*a = 64 (c = 8, a = 64, scale = 1/8), so O = v_{j*} to within e^-64.
    N, d, jstar = 40, 16, 13
    c, a, scale = 8.0, 64.0, 0.125
    q = np.zeros((1, 1, N, d))
    q[..., 0] = c
    k = np.zeros((1, 1, N, d))
    k[0, 0, jstar, 0] = a
    v = _rand((1, 1, N, d), 13)
    O, L = attention_ref(q, k, v, False, scale)
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(v[0, 0, jstar], (N, d)), atol=1e-12)
    exact_L = math.log(math.exp(scale * c * a) + (N - 1))
    np.testing.assert_allclose(L[0, 0], exact_L, rtol=1e-15)
    # Causal: rows before j* cannot see it and average the zero-score prefix instead.
    Oc, _ = attention_ref(q, k, v, True, scale)
    prefix = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    np.testing.assert_allclose(Oc[0, 0, :jstar], prefix[:jstar], atol=1e-13)
    np.testing.assert_allclose(Oc[0, 0, jstar:], np.broadcast_to(v[0, 0, jstar], (N - jstar, d)), atol=1e-12)


def test_equal_dominant_keys_average_their_values():
    N, d, scale = 30, 8, 0.125
    q = np.zeros((1, 1, N, d))
    q[..., 0] = 8.0
    k = np.zeros((1, 1, N, d))
    winners = [3, 17, 29]
    k[0, 0, winners, 0] = 64.0
    v = _rand((1, 1, N, d), 14)
    O, L = attention_ref(q, k, v, False, scale)
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(v[0, 0, winners].mean(0), (N, d)), atol=1e-12)
    np.testing.assert_allclose(L[0, 0], 64.0 + math.log(3.0), atol=1e-12)


def test_single_key_returns_its_value():
    d, scale = 5, 0.9
    q, k, v = (_rand((2, 3, 1, d), s) for s in (15, 16, 17))
    for causal in (False, True):
        O, L = attention_ref(q, k, v, causal, scale)
        np.testing.assert_allclose(O, v, atol=1e-15)
        np.testing.assert_allclose(L, scale * np.sum(q * k, axis=-1), atol=1e-14)


def test_shift_of_all_keys_moves_only_lse():
    # Adding u to every key adds scale*q_i.u to every score of row i: softmax is
    # unchanged, L moves by exactly that amount.
    N, d, scale = 17, 6, 0.33
    q, k, v = (_rand((1, 2, N, d), s) for s in (18, 19, 20))
    u = _rand((d,), 21)
    for causal in (False, True):
        O1, L1 = attention_ref(q, k, v, causal, scale)
        O2, L2 = attention_ref(q, k + u, v, causal, scale)
        np.testing.assert_allclose(O2, O1, atol=1e-12)
        np.testing.assert_allclose(L2 - L1, scale * q @ u, atol=1e-12)


def test_output_is_convex_combination_of_values():
    N, d = 50, 4
    q, k, v = (_rand((1, 1, N, d), s) for s in (22, 23, 24))
    O, _ = attention_ref(q, 3 * k, v, True, 1.0)
    for i in range(N):
        lo = v[0, 0, : i + 1].min(axis=0)
        hi = v[0, 0, : i + 1].max(axis=0)
        assert np.all(O[0, 0, i] >= lo - 1e-12) and np.all(O[0, 0, i] <= hi + 1e-12)


# --------------------------------------------------------------------------- identities

@pytest.mark.parametrize("block_c", [1, 7, 64, 97])
@pytest.mark.parametrize("causal", [False, True])
def test_online_recurrence_equals_two_pass(block_c, causal):
    B, Hq, Hkv, N, d = 1, 4, 2, 97, 16
    q = _rand((B, Hq, N, d), 25)
    k = 1.5 * _rand((B, Hkv, N, d), 26)
    v = _rand((B, Hkv, N, d), 27)
    O, L = attention_ref(q, k, v, causal, 0.25)
    Oo, Lo = online_ref(q, k, v, causal, 0.25, block_c)
    np.testing.assert_allclose(Oo, O, atol=1e-12)
    np.testing.assert_allclose(Lo, L, atol=1e-12)


def test_lse_merge_of_any_key_partition_equals_unsplit():
    N, d, scale = 61, 8, 0.3
    q = _rand((1, 1, 5, d), 28)
    k = _rand((1, 1, N, d), 29)
    v = _rand((1, 1, N, d), 30)
    full_O, full_L = attention_ref(np.concatenate([q, np.zeros((1, 1, N - 5, d))], 2), k, v, False, scale)
    full_O, full_L = full_O[:, :, :5], full_L[:, :, :5]
    rng = _rng(31)
    for parts in (1, 2, 5, 61):
        cuts = np.sort(rng.choice(np.arange(1, N), size=parts - 1, replace=False)) if parts > 1 else []
        bounds = [0, *cuts, N]
        os_, ls_ = [], []
        for a, b in zip(bounds[:-1], bounds[1:]):
            # evaluate the 5 query rows against keys [a, b) by the definition
            s = scale * (q[0, 0] @ k[0, 0, a:b].T)
            m = s.max(1)
            p = np.exp(s - m[:, None])
            os_.append((p @ v[0, 0, a:b]) / p.sum(1)[:, None])
            ls_.append(m + np.log(p.sum(1)))
        # an empty part (no keys) must contribute nothing, even if its o is garbage
        os_.append(np.full((5, d), np.nan))
        ls_.append(np.full(5, -np.inf))
        O, L = lse_merge_ref(np.stack(os_), np.stack(ls_))
        np.testing.assert_allclose(O, full_O[0, 0], atol=1e-12)
        np.testing.assert_allclose(L, full_L[0, 0], atol=1e-12)


def test_lse_merge_all_empty():
    O, L = lse_merge_ref(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(O == 0) and np.all(np.isneginf(L))


@pytest.mark.parametrize("Hkv", [1, 2, 4])
def test_grouped_heads_equal_mha_on_repeated_kv(Hkv):
    B, Hq, N, d = 2, 8, 21, 8
    q = _rand((B, Hq, N, d), 32)
    k = _rand((B, Hkv, N, d), 33)
    v = _rand((B, Hkv, N, d), 34)
    G = Hq // Hkv
    for causal in (False, True):
        O, L = attention_ref(q, k, v, causal, 0.35)
        Om, Lm = attention_ref(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), causal, 0.35)
        np.testing.assert_array_equal(O, Om)
        np.testing.assert_array_equal(L, Lm)


def test_group_map_is_contiguous_blocks():
    # query head h must read K/V head h // G: give each K/V head a distinct constant
    # value row so O identifies the head that was read.
    B, Hq, Hkv, N, d = 1, 6, 3, 4, 2
    q = _rand((B, Hq, N, d), 35)
    k = _rand((B, Hkv, N, d), 36)
    v = np.zeros((B, Hkv, N, d))
    for g in range(Hkv):
        v[0, g] = g + 1.0
    O, _ = attention_ref(q, k, v, False, 1.0)
    for h in range(Hq):
        np.testing.assert_allclose(O[0, h], h // 2 + 1.0, atol=1e-14)


# --------------------------------------------------------------------------- decode

def _brute_gather(pages, table_row, n, g):
    ps = pages.shape[2]
    return np.array([pages[table_row[t // ps], g, t % ps] for t in range(n)], dtype=np.float64)


def _paged(kc, vc, page_size, rng, extra_pages=3):
    """Scatter contiguous per-sequence caches [S][Hkv, n, d] into a shuffled NaN pool."""
    S = len(kc)
    Hkv, _, d = kc[0].shape
    counts = [-(-x.shape[1] // page_size) for x in kc]
    P = sum(counts) + extra_pages
    perm = rng.permutation(P)
    kp = np.full((P, Hkv, page_size, d), np.nan)
    vp = np.full((P, Hkv, page_size, d), np.nan)
    maxp = max(max(counts), 1) + 2
    table = np.full((S, maxp), P - 1, dtype=np.int64)
    off = 0
    for s in range(S):
        n = kc[s].shape[1]
        for p in range(counts[s]):
            pid = perm[off]
            off += 1
            table[s, p] = pid
            lo, hi = p * page_size, min(n, (p + 1) * page_size)
            kp[pid, :, : hi - lo] = kc[s][:, lo:hi]
            vp[pid, :, : hi - lo] = vc[s][:, lo:hi]
    return kp, vp, table


def test_gather_matches_token_by_token_walk():
    rng = _rng(37)
    lens = [1, 16, 17, 40]
    kc = [rng.standard_normal((2, n, 4)) for n in lens]
    vc = [rng.standard_normal((2, n, 4)) for n in lens]
    kp, vp, table = _paged(kc, vc, 16, rng)
    for s, n in enumerate(lens):
        for g in range(2):
            np.testing.assert_array_equal(gather_pages_ref(kp, table[s], n, g), _brute_gather(kp, table[s], n, g))
            np.testing.assert_array_equal(gather_pages_ref(kp, table[s], n, g), kc[s][g])


def test_decode_equals_dense_attention_on_gathered_cache():
    rng = _rng(38)
    S, Hq, Hkv, d, ps = 5, 8, 2, 8, 16
    lens = [1, 15, 16, 33, 70]
    kc = [rng.standard_normal((Hkv, n, d)) for n in lens]
    vc = [rng.standard_normal((Hkv, n, d)) for n in lens]
    kp, vp, table = _paged(kc, vc, ps, rng)
    q = rng.standard_normal((S, Hq, d))
    O, L = decode_ref(q, kp, vp, table, np.array(lens), 0.3)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    for s, n in enumerate(lens):
        # the dense definition, with the query placed as the last of n rows
        qq = np.zeros((1, Hq, n, d))
        qq[:, :, n - 1] = q[s]
        Od, Ld = attention_ref(qq, kc[s][None], vc[s][None], False, 0.3, rows=[n - 1])
        np.testing.assert_allclose(O[s], Od[0, :, 0], atol=1e-12)
        np.testing.assert_allclose(L[s], Ld[0, :, 0], atol=1e-12)


def test_decode_equals_last_row_of_causal_prefill():
    rng = _rng(39)
    Hq, Hkv, n, d = 4, 2, 45, 8
    q = rng.standard_normal((1, Hq, n, d))
    k = rng.standard_normal((1, Hkv, n, d))
    v = rng.standard_normal((1, Hkv, n, d))
    Oc, Lc = attention_ref(q, k, v, True, 0.5)
    for t in (1, 16, 17, n):
        kp, vp, table = _paged([k[0, :, :t]], [v[0, :, :t]], 16, rng)
        O, L = decode_ref(q[:, :, t - 1], kp, vp, table, np.array([t]), 0.5)
        np.testing.assert_allclose(O[0], Oc[0, :, t - 1], atol=1e-12)
        np.testing.assert_allclose(L[0], Lc[0, :, t - 1], atol=1e-12)


def test_decode_invariant_to_page_permutation():
    rng = _rng(40)
    lens = [33, 7]
    kc = [rng.standard_normal((2, n, 8)) for n in lens]
    vc = [rng.standard_normal((2, n, 8)) for n in lens]
    q = rng.standard_normal((2, 4, 8))
    a = _paged(kc, vc, 16, np.random.default_rng(1))
    b = _paged(kc, vc, 16, np.random.default_rng(2))
    assert not np.array_equal(a[2], b[2])
    Oa, La = decode_ref(q, a[0], a[1], a[2], np.array(lens), 0.4)
    Ob, Lb = decode_ref(q, b[0], b[1], b[2], np.array(lens), 0.4)
    np.testing.assert_array_equal(Oa, Ob)
    np.testing.assert_array_equal(La, Lb)


def test_decode_empty_context():
    kp = np.full((2, 1, 16, 4), np.nan)
    O, L = decode_ref(np.ones((1, 2, 4)), kp, kp, np.array([[1]]), np.array([0]), 1.0)
    assert np.all(O == 0) and np.all(np.isneginf(L))


# ------------------------------------------------- sliding window and ALiBi (Lab 01 extensions)

from oracle import alibi_slopes_ref  # noqa: E402


@pytest.mark.parametrize("window", [1, 2, 3, 5, 100])
@pytest.mark.parametrize("alibi", [False, True])
def test_window_alibi_matches_brute_force(window, alibi):
    B, Hq, Hkv, N, d = 1, 2, 1, 6, 3
    q, k, v = _rand((B, Hq, N, d), 60), _rand((B, Hkv, N, d), 61), _rand((B, Hkv, N, d), 62)
    slopes = [0.5, 0.125] if alibi else None
    O, L = attention_ref(q, k, v, True, 0.8, window=window, alibi_slopes=slopes)
    Ob, Lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), True, 0.8, window=window, slopes=slopes)
    np.testing.assert_allclose(O, np.array(Ob), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(L, np.array(Lb), rtol=1e-13, atol=1e-13)


def test_alibi_noncausal_matches_brute_force():
    q, k, v = _rand((1, 2, 5, 3), 63), _rand((1, 2, 5, 3), 64), _rand((1, 2, 5, 3), 65)
    O, L = attention_ref(q, k, v, False, 0.6, alibi_slopes=[0.3, 2.0])
    Ob, Lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), False, 0.6, slopes=[0.3, 2.0])
    np.testing.assert_allclose(O, np.array(Ob), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(L, np.array(Lb), rtol=1e-13, atol=1e-13)


def test_window_one_selects_the_diagonal():
    # W = 1: each row sees only its own key, so O_i = V_i and L_i = scale q_i . k_i
    q, k, v = _rand((2, 3, 9, 4), 66), _rand((2, 3, 9, 4), 67), _rand((2, 3, 9, 4), 68)
    O, L = attention_ref(q, k, v, True, 0.7, window=1)
    np.testing.assert_allclose(O, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(L, 0.7 * np.sum(q * k, axis=-1), rtol=1e-14, atol=1e-14)


def test_window_at_least_n_is_plain_causal():
    q, k, v = _rand((1, 2, 11, 4), 69), _rand((1, 2, 11, 4), 70), _rand((1, 2, 11, 4), 71)
    a = attention_ref(q, k, v, True, 0.5, window=11)
    b = attention_ref(q, k, v, True, 0.5)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_alibi_zero_slope_is_plain_and_steep_slope_picks_diagonal():
    q, k, v = _rand((1, 2, 8, 4), 72), _rand((1, 2, 8, 4), 73), _rand((1, 2, 8, 4), 74)
    a = attention_ref(q, k, v, True, 0.5, alibi_slopes=[0.0, 0.0])
    b = attention_ref(q, k, v, True, 0.5)
    np.testing.assert_array_equal(a[0], b[0])
    # a slope of 1e4 per position drives every other key's weight below exp(-1e4) = 0
    O, _ = attention_ref(q, k, v, True, 0.5, alibi_slopes=[1e4, 1e4])
    np.testing.assert_allclose(O, v, rtol=0, atol=1e-15)


def test_alibi_shift_form_under_causal_mask():
    # with j <= i, -m |i - j| = m j - m i; the -m i part is constant along row i, so
    # the probabilities are those of the scores plus m j, and L is their logsumexp
    # minus m i
    N, d, m = 7, 3, 0.37
    q, k, v = _rand((1, 1, N, d), 75), _rand((1, 1, N, d), 76), _rand((1, 1, N, d), 77)
    O, L = attention_ref(q, k, v, True, 0.9, alibi_slopes=[m])
    s = 0.9 * q[0, 0] @ k[0, 0].T + m * np.arange(N)[None, :]
    s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    np.testing.assert_allclose(O[0, 0], (p @ v[0, 0]) / p.sum(axis=1, keepdims=True), rtol=1e-13, atol=1e-13)
    lse = s.max(axis=1) + np.log(p.sum(axis=1)) - m * np.arange(N)
    np.testing.assert_allclose(L[0, 0], lse, rtol=1e-13, atol=1e-13)


def test_alibi_slopes_are_the_geometric_sequence():
    s = alibi_slopes_ref(8)
    np.testing.assert_allclose(s, [0.5 ** (h + 1) for h in range(8)], rtol=0, atol=0)


def test_window_requires_causal():
    with pytest.raises(ValueError):
        attention_ref(np.zeros((1, 1, 2, 2)), np.zeros((1, 1, 2, 2)), np.zeros((1, 1, 2, 2)), False, 1.0, window=1)


# ------------------------------------------------- chunked prefill over a paged cache

from oracle import prefill_paged_ref  # noqa: E402
from exact_io_aware_15_amd.workloads import make_prefill_paged  # noqa: E402


def _chunked(S, Hq, Hkv, d, C, ctx, seed):
    x = make_prefill_paged(S, Hq, Hkv, d, C, 1, 64, seed=seed, fixed_ctx=ctx)
    return (x["q"].double().numpy(), x["kpages"].double().numpy(), x["vpages"].double().numpy(),
            x["page_table"].numpy(), x["ctx_lens"].numpy())


def test_prefill_paged_chunk_of_one_is_decode():
    q, kp, vp, pt, cl = _chunked(3, 4, 2, 8, 1, (1, 17, 40), 80)
    O, L = prefill_paged_ref(q, kp, vp, pt, cl, 0.3)
    Od, Ld = decode_ref(q[:, :, 0], kp, vp, pt, cl, 0.3)
    np.testing.assert_allclose(O[:, :, 0], Od, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(L[:, :, 0], Ld, rtol=1e-13, atol=1e-13)


def test_prefill_paged_whole_context_is_causal_prefill():
    # ctx == C: the chunk is the whole sequence, i.e. a causal prefill of the gathered K/V
    q, kp, vp, pt, cl = _chunked(2, 4, 2, 8, 21, (21, 21), 81)
    O, L = prefill_paged_ref(q, kp, vp, pt, cl, 0.4)
    for s in range(2):
        k = np.stack([gather_pages_ref(kp, pt[s], 21, g) for g in range(2)])[None]
        v = np.stack([gather_pages_ref(vp, pt[s], 21, g) for g in range(2)])[None]
        Oc, Lc = attention_ref(q[s][None], k, v, True, 0.4)
        np.testing.assert_allclose(O[s], Oc[0], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(L[s], Lc[0], rtol=1e-13, atol=1e-13)


def test_prefill_paged_matches_brute_force():
    q, kp, vp, pt, cl = _chunked(2, 2, 1, 3, 4, (6, 9), 82)
    O, L = prefill_paged_ref(q, kp, vp, pt, cl, 0.7)
    for s in range(2):
        n = int(cl[s])
        k = [[gather_pages_ref(kp, pt[s], n, 0).tolist()]]
        v = [[gather_pages_ref(vp, pt[s], n, 0).tolist()]]
        # the chunk rows are the last C rows of a causal attention over the whole sequence
        qq = np.zeros((1, 2, n, 3))
        qq[0, :, n - 4:] = q[s]
        Ob, Lb = brute_attention(qq.tolist(), k, v, True, 0.7)
        np.testing.assert_allclose(O[s], np.array(Ob)[0][:, n - 4:], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(L[s], np.array(Lb)[0][:, n - 4:], rtol=1e-13, atol=1e-13)


def test_prefill_paged_ignores_page_order():
    q, kp, vp, pt, cl = _chunked(2, 2, 2, 8, 5, (33, 50), 83)
    O, L = prefill_paged_ref(q, kp, vp, pt, cl, 0.5)
    perm = np.random.default_rng(5).permutation(kp.shape[0])
    inv = np.argsort(perm)
    pt2 = np.where(pt < kp.shape[0], inv[pt], pt)
    O2, L2 = prefill_paged_ref(q, kp[perm], vp[perm], pt2, cl, 0.5)
    np.testing.assert_allclose(O, O2, rtol=0, atol=0)
    np.testing.assert_allclose(L, L2, rtol=0, atol=0)


# ------------------------------------------------- INT8 group-scaled KV decode

from oracle import decode_int8_ref, dequant_pages_ref  # noqa: E402
from exact_io_aware_15_amd.workloads import make_decode_int8  # noqa: E402


def test_dequant_is_per_token_per_group_product():
    rng = np.random.default_rng(90)
    qv = rng.integers(-127, 128, size=(2, 1, 3, 8)).astype(np.int8)
    sc = rng.uniform(0.1, 1, size=(2, 1, 3, 2))
    got = dequant_pages_ref(qv, sc, 4)
    for idx in np.ndindex(qv.shape):
        p, h, t, c = idx
        assert got[idx] == float(qv[idx]) * sc[p, h, t, c // 4]


def test_int8_decode_with_unit_scales_is_the_bf16_decode_of_the_integers():
    x = make_decode_int8(3, 4, 2, 64, fixed_ctx=(5, 16, 33), seed=91)
    ones = np.ones(x["kscale"].shape)
    O, L = decode_int8_ref(x["q"].double().numpy(), x["kq"].numpy(), ones, x["vq"].numpy(), ones,
                           x["page_table"].numpy(), x["ctx_lens"].numpy(), 0.01)
    Od, Ld = decode_ref(x["q"].double().numpy(), x["kq"].numpy().astype(np.float64), x["vq"].numpy().astype(np.float64),
                        x["page_table"].numpy(), x["ctx_lens"].numpy(), 0.01)
    np.testing.assert_array_equal(O, Od)
    np.testing.assert_array_equal(L, Ld)


def test_int8_decode_uniform_v_scale_scales_the_output():
    # one common V scale s multiplies O by s and leaves L alone
    x = make_decode_int8(2, 2, 1, 64, fixed_ctx=(7, 40), seed=92)
    ks = np.where(np.isnan(x["kscale"].numpy()), 1.0, x["kscale"].numpy())
    args = (x["q"].double().numpy(), x["kq"].numpy(), ks, x["vq"].numpy())
    O1, L1 = decode_int8_ref(*args, np.ones(ks.shape), x["page_table"].numpy(), x["ctx_lens"].numpy(), 0.1)
    O2, L2 = decode_int8_ref(*args, np.full(ks.shape, 0.25), x["page_table"].numpy(), x["ctx_lens"].numpy(), 0.1)
    np.testing.assert_allclose(O2, 0.25 * O1, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(L1, L2)


def test_int8_inputs_poison_only_unused_slots():
    x = make_decode_int8(3, 2, 1, 64, fixed_ctx=(1, 16, 17), seed=93)
    ks = x["kscale"].numpy()
    for s, n in enumerate(x["ctx_lens"].tolist()):
        for t in range(n):
            page = x["page_table"][s, t // 16].item()
            assert np.all(np.isfinite(ks[page, :, t % 16]))
    assert np.all(np.isnan(ks[-1]))
