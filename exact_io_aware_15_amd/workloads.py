"""Seeded synthetic inputs for the attention kernels and their oracle.

This module draws and lays out inputs only: it holds none of the attention arithmetic.
Both sides of every parity check (the HIP library and the fp64 oracle) receive the
tensors made here, so both see bit-identical values.

Recipe (all workloads are synthetic, as the "Phase 08" Lab 01 datasets row states):
  * numpy.random.default_rng(seed) (PCG64); float32 standard normal draws.
  * prefill draw order: Q, then K, then V, each in [B, H, N, d] row-major order.
  * a value scale (0.5 for the long causal workload) multiplies the fp32 draws before
    rounding; the rounding to bf16 is round-to-nearest-even (torch's CPU cast).
  * decode draw order: q [S, Hq, d], then ctx_lens ~ U{lo..hi} (inclusive), then the K
    page pool, then the V page pool ([P + 1, Hkv, page, d]), then a permutation of the
    P real page ids.  Sequence s owns the next ceil(ctx_s / page) ids of that
    permutation, in order.  Page id P is an all-NaN poison page; unused page-table
    slots point at it, and the token slots past ctx_s in each sequence's last page
    are NaN too, so any read of data outside the context shows up in the output.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "PrefillConfig",
    "DecodeConfig",
    "CONFIGS",
    "make_prefill",
    "make_decode",
    "make_inputs",
]


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    dtype: str  # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    seed: int
    value_scale: float = 1.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def kind(self) -> str:
        return "prefill"


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    num_seqs: int
    Hq: int
    Hkv: int
    d: int
    ctx_lo: int
    ctx_hi: int
    seed: int
    page_size: int = 16
    max_pages_per_seq: int | None = None
    fixed_ctx: tuple = field(default=())  # explicit context lengths (overrides the draw)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def kind(self) -> str:
        return "decode"


# The five workloads (the MQA variant of the grouped-query one is listed separately).
CONFIGS = {
    "c1_f32_B1_H1_N256_d64": PrefillConfig("c1_f32_B1_H1_N256_d64", "f32", 1, 1, 1, 256, 64, False, 1),
    "c2_bf16_B4_H16_N2048_d64": PrefillConfig("c2_bf16_B4_H16_N2048_d64", "bf16", 4, 16, 16, 2048, 64, False, 2),
    "c3_bf16_causal_B1_H32_N8192_d128": PrefillConfig(
        "c3_bf16_causal_B1_H32_N8192_d128", "bf16", 1, 32, 32, 8192, 128, True, 3, 0.5),
    "c4_bf16_causal_gqa_B2_Hq32_Hkv8_N4096_d128": PrefillConfig(
        "c4_bf16_causal_gqa_B2_Hq32_Hkv8_N4096_d128", "bf16", 2, 32, 8, 4096, 128, True, 4),
    "c4_bf16_causal_mqa_B2_Hq32_Hkv1_N4096_d128": PrefillConfig(
        "c4_bf16_causal_mqa_B2_Hq32_Hkv1_N4096_d128", "bf16", 2, 32, 1, 4096, 128, True, 4),
    "c5_bf16_paged_decode_S64_Hq32_Hkv8_d128": DecodeConfig(
        "c5_bf16_paged_decode_S64_Hq32_Hkv8_d128", 64, 32, 8, 128, 1024, 16384, 5,
        page_size=16, max_pages_per_seq=1024),
}


def _normal(rng: np.random.Generator, shape, value_scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if value_scale != 1.0:
        x *= np.float32(value_scale)
    return x


def _to(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(x)
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t.contiguous()
    raise ValueError(dtype)


def make_prefill(B, Hq, Hkv, N, d, dtype="bf16", seed=0, value_scale=1.0):
    """q [B,Hq,N,d], k/v [B,Hkv,N,d] as CPU torch tensors (bf16 or fp32)."""
    rng = np.random.default_rng(seed)
    q = _to(_normal(rng, (B, Hq, N, d), value_scale), dtype)
    k = _to(_normal(rng, (B, Hkv, N, d), value_scale), dtype)
    v = _to(_normal(rng, (B, Hkv, N, d), value_scale), dtype)
    return {"q": q, "k": k, "v": v}


def make_alibi_slopes(n_heads: int) -> torch.Tensor:
    """fp32 ALiBi slopes 2^(-8 (h + 1) / n) for heads h = 0 .. n-1 (the geometric
    sequence usually paired with the bias), as a CPU tensor."""
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / n_heads) for h in range(n_heads)], dtype=torch.float32)


def make_grad_output(B, Hq, N, d, dtype="bf16", seed=0):
    """Upstream gradient dO [B, Hq, N, d] for the backward: N(0,1) from its own
    stream (seed + 7919, so it is independent of the forward inputs of the same seed)."""
    rng = np.random.default_rng(seed + 7919)
    return _to(_normal(rng, (B, Hq, N, d)), dtype)


def make_decode(num_seqs, Hq, Hkv, d, ctx_lo=1, ctx_hi=64, seed=0, page_size=16,
                max_pages_per_seq=None, fixed_ctx=(), dtype="bf16"):
    """Paged-KV decode inputs as CPU tensors.

    Returns q [S,Hq,d], kpages/vpages [P+1,Hkv,page,d] (page P = poison),
    page_table [S,max_pages] int32, ctx_lens [S] int32, num_pages = P + 1.
    """
    rng = np.random.default_rng(seed)
    q = _to(_normal(rng, (num_seqs, Hq, d)), dtype)
    if fixed_ctx:
        ctx = np.asarray(fixed_ctx, dtype=np.int64)
        if ctx.shape != (num_seqs,):
            raise ValueError("fixed_ctx must have one entry per sequence")
    else:
        ctx = rng.integers(ctx_lo, ctx_hi, size=num_seqs, endpoint=True).astype(np.int64)
    pages_per_seq = -(-ctx // page_size)
    P = int(pages_per_seq.sum())
    need = int(pages_per_seq.max()) if num_seqs else 0
    maxp = max(1, need) if max_pages_per_seq is None else int(max_pages_per_seq)
    if maxp < need:
        raise ValueError("max_pages_per_seq too small for the drawn context lengths")
    kp = _normal(rng, (P + 1, Hkv, page_size, d))
    vp = _normal(rng, (P + 1, Hkv, page_size, d))
    perm = rng.permutation(P).astype(np.int64)
    table = np.full((num_seqs, maxp), P, dtype=np.int32)
    off = 0
    for s in range(num_seqs):
        n = int(pages_per_seq[s])
        table[s, :n] = perm[off:off + n]
        off += n
        tail = int(ctx[s]) % page_size
        if n > 0 and tail:
            last = perm[off - 1]
            kp[last, :, tail:, :] = np.nan
            vp[last, :, tail:, :] = np.nan
    kp[P] = np.nan
    vp[P] = np.nan
    return {
        "q": q,
        "kpages": _to(kp, dtype),
        "vpages": _to(vp, dtype),
        "page_table": torch.from_numpy(table),
        "ctx_lens": torch.from_numpy(ctx.astype(np.int32)),
        "num_pages": P + 1,
        "page_size": page_size,
        "max_pages_per_seq": maxp,
    }


def make_prefill_paged(num_seqs, Hq, Hkv, d, chunk, ctx_lo, ctx_hi, seed=0, page_size=16, fixed_ctx=(),
                       dtype="bf16"):
    """Chunked-prefill inputs over a paged cache: the paged K/V pools, page table and
    ctx_lens of make_decode (context lengths drawn from [max(ctx_lo, chunk), ctx_hi]),
    and chunk queries q [S, Hq, chunk, d] from their own stream (seed + 104729)."""
    x = make_decode(num_seqs, Hq, Hkv, d, max(ctx_lo, chunk), ctx_hi, seed, page_size, None, fixed_ctx, dtype)
    rng = np.random.default_rng(seed + 104729)
    x["q"] = _to(_normal(rng, (num_seqs, Hq, chunk, d)), dtype)
    return x


def make_decode_int8(num_seqs, Hq, Hkv, d, ctx_lo=1, ctx_hi=64, seed=0, page_size=16, fixed_ctx=(),
                     group=32):
    """Paged decode inputs with an INT8 group-scaled KV cache: the q, page table and
    ctx_lens of make_decode (same seed), K/V pools [P+1, Hkv, page, d] int8 uniform in
    [-127, 127] and fp32 scales [P+1, Hkv, page, d // group] uniform in [1/256, 1/64]
    (so K/V values are O(1)).  Slots past each context and the padding page have NaN
    scales, which a kernel must never let through."""
    x = make_decode(num_seqs, Hq, Hkv, d, ctx_lo, ctx_hi, seed, page_size, None, fixed_ctx)
    P1 = x["num_pages"]
    rng = np.random.default_rng(seed + 15485863)
    kq = rng.integers(-127, 128, size=(P1, Hkv, page_size, d), dtype=np.int64).astype(np.int8)
    vq = rng.integers(-127, 128, size=(P1, Hkv, page_size, d), dtype=np.int64).astype(np.int8)
    ks = rng.uniform(1 / 256, 1 / 64, size=(P1, Hkv, page_size, d // group)).astype(np.float32)
    vs = rng.uniform(1 / 256, 1 / 64, size=(P1, Hkv, page_size, d // group)).astype(np.float32)
    # NaN scales wherever the bf16 pools of make_decode hold NaN (unused slots, padding page)
    bad = torch.isnan(x["kpages"][..., 0]).numpy()
    ks[bad] = np.nan
    vs[bad] = np.nan
    x.update({"kq": torch.from_numpy(kq), "vq": torch.from_numpy(vq), "kscale": torch.from_numpy(ks),
              "vscale": torch.from_numpy(vs), "group": group})
    del x["kpages"], x["vpages"]
    return x


def make_inputs(cfg):
    """Inputs for a registered configuration (PrefillConfig or DecodeConfig)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if cfg.kind == "prefill":
        return make_prefill(cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d, cfg.dtype, cfg.seed, cfg.value_scale)
    return make_decode(cfg.num_seqs, cfg.Hq, cfg.Hkv, cfg.d, cfg.ctx_lo, cfg.ctx_hi, cfg.seed,
                       cfg.page_size, cfg.max_pages_per_seq, cfg.fixed_ctx)
