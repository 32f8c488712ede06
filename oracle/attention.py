"""Plain, slow, fp64 CPU definitions of exact attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
module.  The GPU library never does.

Everything is computed in float64 with numpy.  Inputs are the exact values the GPU
receives (bf16 or fp32), upcast.  Tensor layouts:

  prefill  q [B, Hq, N, d]   k, v [B, Hkv, N, d]   ->  O [B, Hq, N, d], L [B, Hq, N]
  decode   q [S, Hq, d]      kpages, vpages [num_pages, Hkv, page_size, d]
           page_table [S, max_pages] int, ctx_lens [S] int
                             ->  O [S, Hq, d], L [S, Hq]

Readings of the pages taken here (each is also listed with the design notes):
  * L is the natural logarithm of sum_j exp(scale * q_i . k_j) over the keys row i
    may see (the logsumexp named in the "FlashAttention backward" concept).
  * causal: query row i sees keys j <= i (queries and keys have the same length).
  * grouped heads: query head h reads K/V head h // (Hq // Hkv) (contiguous groups).
  * decode: the single query of sequence s sees its first ctx_lens[s] cached tokens,
    with no further mask; an empty context gives O = 0 and L = -inf.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "attention_ref",
    "alibi_slopes_ref",
    "decode_ref",
    "prefill_paged_ref",
    "dequant_pages_ref",
    "decode_int8_ref",
    "online_ref",
    "lse_merge_ref",
    "gather_pages_ref",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _group_size(hq: int, hkv: int) -> int:
    if hkv <= 0 or hq % hkv != 0:
        raise ValueError(f"Hq={hq} is not a multiple of Hkv={hkv}")
    return hq // hkv


def _softmax_rows(s: np.ndarray, v: np.ndarray):
    """Standard attention on one block of fully-formed score rows.

    "Phase 08" Concepts list, standard attention; screna.ai FlashAttention block
    (P = softmax(S), output P V).  s is [R, Nk] (masked entries are -inf), v is [Nk, d].
    Returns O [R, d] and L [R] with L = m + ln(sum exp(s - m)).
    Rows with no visible key give O = 0, L = -inf.
    """
    m = np.max(s, axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 for masked entries
    l = np.sum(p, axis=1)
    o = p @ v
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(empty[:, None], 0.0, o / np.where(empty, 1.0, l)[:, None])
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return o, lse


def attention_ref(q, k, v, causal: bool, scale: float, rows=None, chunk: int = 1024, window: int = 0,
                  alibi_slopes=None):
    """Standard (materialising) attention: S = scale * Q K^T, mask, softmax, P V.

    "Phase 08", Lab 01 step 1 (standard attention as the reference) and the
    Concepts list (full n x n score matrix); screna.ai FlashAttention block
    (S = QK^T, P = softmax(S)); MHA/MQA/GQA block (each group of query heads shares
    one K/V head).

    rows: optional 1-D array of query-row indices to evaluate (all rows if None).
    Each evaluated row's full score vector over all N keys is formed; rows are
    taken `chunk` at a time only to bound memory.

    Extensions named in the "Phase 08" Lab 01 extensions row (sliding-window
    attention as in Mistral, ALiBi bias):
      window: W >= 1 keeps, for query i, only keys j >= i - W + 1 (the last W
        positions up to and including i); causal only; 0 = no window.
      alibi_slopes: per query head slope m_h (sequence of Hq floats); the score of
        (i, j) gains -m_h * |i - j| (= m_h * (j - i) under the causal mask).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, Hq, N, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, Nk, dk) != (B, N, d) or v.shape != k.shape:
        raise ValueError("q/k/v shapes disagree")
    if window and not causal:
        raise ValueError("a sliding window is defined for causal attention only")
    G = _group_size(Hq, Hkv)
    slopes = None if alibi_slopes is None else _f64(alibi_slopes)
    row_idx = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = row_idx.shape[0]
    O = np.zeros((B, Hq, R, d), dtype=np.float64)
    L = np.zeros((B, Hq, R), dtype=np.float64)
    key_idx = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            kh = k[b, g]
            vh = v[b, g]
            for c0 in range(0, R, chunk):
                ri = row_idx[c0:c0 + chunk]
                s = scale * (q[b, h, ri] @ kh.T)  # [r, N], every key of every row
                if slopes is not None:
                    s = s - slopes[h] * np.abs(ri[:, None] - key_idx[None, :])
                if causal:
                    s = np.where(key_idx[None, :] <= ri[:, None], s, -np.inf)
                if window:
                    s = np.where(key_idx[None, :] >= ri[:, None] - window + 1, s, -np.inf)
                o, lse = _softmax_rows(s, vh)
                O[b, h, c0:c0 + chunk] = o
                L[b, h, c0:c0 + chunk] = lse
    return O, L


def alibi_slopes_ref(n_heads: int):
    """The geometric ALiBi slopes 2^(-8 (h + 1) / n) for heads h = 0 .. n-1 (n a power of
    two), the usual choice with the bias of the Lab 01 extensions row."""
    return np.array([2.0 ** (-8.0 * (h + 1) / n_heads) for h in range(n_heads)])


def gather_pages_ref(pages, page_table_row, ctx_len: int, kv_head: int) -> np.ndarray:
    """Contiguous [ctx_len, d] cache of one sequence and one K/V head.

    "Phase 08", Lab 03 step 1 (fixed-size token pages) and step 4 (the kernel reaches
    non-contiguous pages through an indirection table): logical token t of the
    sequence lives in page page_table_row[t // page_size], slot t % page_size.
    """
    pages = np.asarray(pages)
    page_size = pages.shape[2]
    n_pages = -(-ctx_len // page_size)
    ids = np.asarray(page_table_row[:n_pages], dtype=np.int64)
    blk = pages[ids, kv_head]  # [n_pages, page_size, d]
    return _f64(blk.reshape(n_pages * page_size, pages.shape[3])[:ctx_len])


def decode_ref(q, kpages, vpages, page_table, ctx_lens, scale: float):
    """One-query attention over a paged KV cache (decode), by the definition.

    Same definition as attention_ref for a single query row with no mask, applied to
    the sequence's cached K/V gathered from its pages ("Phase 08", Concepts list:
    KV cache, paged attention; Lab 03 step 4).
    """
    q = _f64(q)
    S, Hq, d = q.shape
    Hkv = np.asarray(kpages).shape[1]
    G = _group_size(Hq, Hkv)
    O = np.zeros((S, Hq, d), dtype=np.float64)
    L = np.zeros((S, Hq), dtype=np.float64)
    for s in range(S):
        n = int(ctx_lens[s])
        if n == 0:
            L[s, :] = -np.inf
            continue
        for g in range(Hkv):
            ks = gather_pages_ref(kpages, page_table[s], n, g)
            vs = gather_pages_ref(vpages, page_table[s], n, g)
            hs = slice(g * G, (g + 1) * G)
            sc = scale * (q[s, hs] @ ks.T)  # [G, n]
            o, lse = _softmax_rows(sc, vs)
            O[s, hs] = o
            L[s, hs] = lse
    return O, L


def dequant_pages_ref(qpages, scales, group: int):
    """fp64 values of group-scaled int8 pages: qpages [P, Hkv, page, d] int8 times
    scales [P, Hkv, page, d // group] (one scale per token and `group` consecutive
    channels).  screna.ai KV-cache quantization block (INT8 KV cache; group-wise
    scales)."""
    qv = _f64(qpages)
    sc = np.repeat(_f64(scales), group, axis=-1)
    return qv * sc


def decode_int8_ref(q, kq, kscale, vq, vscale, page_table, ctx_lens, scale: float, group: int = 32):
    """Paged decode over an INT8 group-scaled KV cache: the decode definition applied
    to the dequantized cache (screna.ai KV-cache quantization block; "Phase 08" Lab 03
    step 4)."""
    return decode_ref(q, dequant_pages_ref(kq, kscale, group), dequant_pages_ref(vq, vscale, group), page_table,
                      ctx_lens, scale)


def prefill_paged_ref(q, kpages, vpages, page_table, ctx_lens, scale: float):
    """Chunked prefill over a paged KV cache, by the definition.

    "Phase 08", Concepts list (chunked prefill: a long prompt is processed a chunk
    at a time; paged attention) and Lab 03 steps 1 and 4 (16-token pages reached
    through an indirection table).  Sequence s holds ctx_lens[s] cached tokens, the
    last C of which are the chunk's own tokens (their K/V already written to the
    cache); chunk row r is the token at position ctx_lens[s] - C + r and sees every
    cached token at a position <= its own (causal within the chunk, everything
    before it).  Requires ctx_lens[s] >= C.

    q [S, Hq, C, d] -> O [S, Hq, C, d], L [S, Hq, C].
    """
    q = _f64(q)
    S, Hq, C, d = q.shape
    Hkv = np.asarray(kpages).shape[1]
    G = _group_size(Hq, Hkv)
    O = np.zeros((S, Hq, C, d))
    L = np.zeros((S, Hq, C))
    for s in range(S):
        n = int(ctx_lens[s])
        if n < C:
            raise ValueError("every sequence must already hold its chunk (ctx_lens >= C)")
        pos = n - C + np.arange(C)
        keys = np.arange(n)
        for g in range(Hkv):
            ks = gather_pages_ref(kpages, page_table[s], n, g)
            vs = gather_pages_ref(vpages, page_table[s], n, g)
            for h in range(g * G, (g + 1) * G):
                sc = scale * (q[s, h] @ ks.T)  # [C, n]
                sc = np.where(keys[None, :] <= pos[:, None], sc, -np.inf)
                o, lse = _softmax_rows(sc, vs)
                O[s, h] = o
                L[s, h] = lse
    return O, L


def online_ref(q, k, v, causal: bool, scale: float, block_c: int):
    """The online-softmax recurrence, walked over key blocks of block_c columns.

    "Phase 08", Concepts list (online softmax; FlashAttention tiling) and the Lab 01
    talking points (the three-line update of running max m, normaliser l and
    output O).  Reading of that garbled formula: its index counts key/value tiles;
    the score of a tile is scale * Q K_t^T; the exponentials multiply V_t (the
    printed "v^T"); O is kept unnormalised and divided by l once at the end, and
    L = m + ln l.  All query rows of a head form one block (the recurrence is per row).
    Used only to pin the materialising definition (they must agree) -- it is not
    what the GPU is compared against.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = _group_size(Hq, Hkv)
    O = np.zeros((B, Hq, N, d))
    L = np.zeros((B, Hq, N))
    rows = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            acc = np.zeros((N, d))
            for j0 in range(0, N, block_c):
                j1 = min(N, j0 + block_c)
                s = scale * (q[b, h] @ k[b, g, j0:j1].T)
                if causal:
                    s = np.where(np.arange(j0, j1)[None, :] <= rows[:, None], s, -np.inf)
                m_new = np.maximum(m, np.max(s, axis=1))
                live = np.isfinite(m_new)
                ms = np.where(live, m_new, 0.0)
                alpha = np.where(live, np.exp(np.where(live, m, 0.0) - ms), 1.0)
                alpha = np.where(np.isfinite(m), alpha, 0.0)  # nothing accumulated yet
                p = np.exp(s - ms[:, None])
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ v[b, g, j0:j1]
                m = m_new
            with np.errstate(divide="ignore", invalid="ignore"):
                O[b, h] = np.where((l > 0)[:, None], acc / np.where(l > 0, l, 1.0)[:, None], 0.0)
                L[b, h] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return O, L


def lse_merge_ref(o_parts, lse_parts):
    """Merge attention results computed over disjoint key subsets.

    Each part c holds o_c (normalised over its own keys) and lse_c (its logsumexp).
    The whole-key result is L = ln sum_c exp(lse_c) and O = sum_c exp(lse_c - L) o_c:
    the same rescaling algebra as the online-softmax update of the "Phase 08" Lab 01
    talking points, applied once to whole parts.  Parts with lse_c = -inf (no keys)
    contribute nothing; if every part is empty, O = 0 and L = -inf.

    o_parts [C, ..., d], lse_parts [C, ...].
    """
    o = _f64(o_parts)
    lse = _f64(lse_parts)
    mx = np.max(lse, axis=0)
    live = np.isfinite(mx)
    mxs = np.where(live, mx, 0.0)
    w = np.exp(lse - mxs[None])  # exp(-inf) = 0 for empty parts
    tot = np.sum(w, axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        L = np.where(live, mxs + np.log(np.where(live, tot, 1.0)), -np.inf)
        wn = np.where(live[None], w / np.where(live, tot, 1.0)[None], 0.0)
    # 0 * (anything finite) parts are fine; an empty part's o may be garbage, so mask it.
    o = np.where(np.isfinite(lse)[..., None], o, 0.0)
    O = np.sum(wn[..., None] * o, axis=0)
    return O, L
