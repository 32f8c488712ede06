"""Exact attention (FlashAttention forward and backward) and paged-KV decode for MI355X (gfx950).

Thin ctypes binding over libfa.so, whose C ABI is declared in include/fa.h.  The
functions below carry the C names and only marshal arguments: they check dtypes,
shapes, contiguity and devices, allocate outputs with torch when none are given,
and pass raw device pointers plus torch's current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no fallback path, and a
missing library raises.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "FAError",
    "lib",
    "load_library",
    "use_library",
    "DEBUG_SYNC_LIB_PATH",
    "fa_fwd",
    "fa_fwd_f32",
    "fa_fwd_ex",
    "fa_fwd_splitk",
    "fa_fwd_splitk_workspace_size",
    "fa_bwd",
    "fa_bwd_workspace_size",
    "fa_decode_paged",
    "fa_decode_paged_workspace_size",
    "fa_prefill_paged",
    "fa_decode_paged_int8",
    "fa_decode_paged_noalloc",
    "fa_decode_paged_noalloc_max_scratch",
    "fa_status_string",
    "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
# the same library built with every HBM -> LDS copy and LDS read stage fenced (tests
# compare it bitwise with libfa.so)
DEBUG_SYNC_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_debugsync.so")

FA_OK = 0
_lib = None
_loaded = {}


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {fa_status_string(status)}")


def lib() -> ctypes.CDLL:
    """The library every call below uses: libfa.so, loaded once.  Raises if it has not
    been built."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


class use_library:
    """Context manager: route the calls of this module through another build of the
    library (for instance load_library(DEBUG_SYNC_LIB_PATH)) inside the block."""

    def __init__(self, L: ctypes.CDLL):
        self.L = L

    def __enter__(self):
        global _lib
        self.prev, _lib = lib(), self.L
        return self.L

    def __exit__(self, *exc):
        global _lib
        _lib = self.prev
        return False


def load_library(path: str) -> ctypes.CDLL:
    """Load a build of the C ABI (once per path) and declare its signatures."""
    if path in _loaded:
        return _loaded[path]
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m exact_io_aware_15_amd.build`")
    L = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.fa_fwd.restype = i
    L.fa_fwd_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.fa_fwd_f32.restype = i
    L.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, vp]
    L.fa_fwd_ex.restype = i
    L.fa_fwd_splitk_workspace_size.argtypes = [i, i, i, i, i]
    L.fa_fwd_splitk_workspace_size.restype = sz
    L.fa_fwd_splitk.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    L.fa_fwd_splitk.restype = i
    L.fa_bwd_workspace_size.argtypes = [i, i, i, i, i]
    L.fa_bwd_workspace_size.restype = sz
    L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    L.fa_bwd.restype = i
    L.fa_decode_paged_int8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp, sz, vp]
    L.fa_decode_paged_int8.restype = i
    L.fa_prefill_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp]
    L.fa_prefill_paged.restype = i
    L.fa_decode_paged_workspace_size.argtypes = [i, i, i, i, i]
    L.fa_decode_paged_workspace_size.restype = sz
    L.fa_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, sz, vp]
    L.fa_decode_paged.restype = i
    L.fa_decode_paged_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    L.fa_decode_paged_noalloc.restype = i
    L.fa_decode_paged_noalloc_max_scratch.argtypes = []
    L.fa_decode_paged_noalloc_max_scratch.restype = sz
    L.fa_status_string.argtypes = [i]
    L.fa_status_string.restype = ctypes.c_char_p
    _loaded[path] = L
    return L


def fa_status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t: torch.Tensor, name: str, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _fwd(entry: str, dtype, q, k, v, causal, scale, out, lse):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, N, d] and k, v [B, Hkv, N, d]")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    _need(q, "q", dtype, (B, Hq, N, d), dev)
    _need(k, "k", dtype, (B, Hkv, N, d), dev)
    _need(v, "v", dtype, (B, Hkv, N, d), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    _need(out, "out", dtype, (B, Hq, N, d), dev)
    _need(lse, "lse", torch.float32, (B, Hq, N), dev)
    st = getattr(lib(), entry)(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, N, d,
                               int(bool(causal)), float(scale), _stream(q))
    if st != FA_OK:
        raise FAError(st, entry)
    return out, lse


def fa_fwd(q, k, v, causal=False, scale=None, out=None, lse=None):
    """bf16 forward: q [B,Hq,N,d], k/v [B,Hkv,N,d] -> (O bf16 [B,Hq,N,d], L fp32 [B,Hq,N])."""
    return _fwd("fa_fwd", torch.bfloat16, q, k, v, causal, scale, out, lse)


def fa_fwd_splitk_workspace_size(B, Hq, N, d, causal) -> int:
    return int(lib().fa_fwd_splitk_workspace_size(B, Hq, N, d, int(bool(causal))))


def fa_fwd_splitk(q, k, v, causal=False, scale=None, out=None, lse=None, workspace=None):
    """fa_fwd with the key range of each query block cut into chunks when the launch has
    fewer than 256 (query block, head) items; workspace: a uint8 device tensor of at least
    fa_fwd_splitk_workspace_size(...) bytes (allocated here when None)."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, N, d] and k, v [B, Hkv, N, d]")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    _need(q, "q", torch.bfloat16, (B, Hq, N, d), dev)
    _need(k, "k", torch.bfloat16, (B, Hkv, N, d), dev)
    _need(v, "v", torch.bfloat16, (B, Hkv, N, d), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=dev) if out is None else out
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev) if lse is None else lse
    _need(out, "out", torch.bfloat16, (B, Hq, N, d), dev)
    _need(lse, "lse", torch.float32, (B, Hq, N), dev)
    if workspace is None:
        workspace = torch.empty(max(1, fa_fwd_splitk_workspace_size(B, Hq, N, d, causal)), dtype=torch.uint8,
                                device=dev)
    st = lib().fa_fwd_splitk(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, N, d, int(bool(causal)),
                             float(scale), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_splitk")
    return out, lse


def fa_fwd_f32(q, k, v, causal=False, scale=None, out=None, lse=None):
    """fp32 forward, same layouts as fa_fwd."""
    return _fwd("fa_fwd_f32", torch.float32, q, k, v, causal, scale, out, lse)


def fa_fwd_ex(q, k, v, causal=True, scale=None, window=0, alibi_slopes=None, out=None, lse=None):
    """bf16 forward with a sliding window (causal, last `window` keys; 0 = none) and/or
    ALiBi slopes (fp32 [Hq] on the device, bias -m_h |i - j|; None = no bias)."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    _need(q, "q", torch.bfloat16, (B, Hq, N, d), dev)
    _need(k, "k", torch.bfloat16, (B, Hkv, N, d), dev)
    _need(v, "v", torch.bfloat16, (B, Hkv, N, d), dev)
    if alibi_slopes is not None:
        _need(alibi_slopes, "alibi_slopes", torch.float32, (Hq,), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=dev) if out is None else out
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev) if lse is None else lse
    _need(out, "out", torch.bfloat16, (B, Hq, N, d), dev)
    _need(lse, "lse", torch.float32, (B, Hq, N), dev)
    st = lib().fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, N, d, int(bool(causal)),
                         float(scale), int(window), _ptr(alibi_slopes), _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_ex")
    return out, lse


def fa_bwd_workspace_size(B, Hq, Hkv, N, d) -> int:
    return int(lib().fa_bwd_workspace_size(B, Hq, Hkv, N, d))


def fa_bwd(q, k, v, o, lse, dout, causal=False, scale=None, dq=None, dk=None, dv=None, workspace=None):
    """bf16 backward: q, o, dout [B,Hq,N,d]; k, v [B,Hkv,N,d]; lse fp32 [B,Hq,N] (from fa_fwd)
    -> (dQ [B,Hq,N,d], dK [B,Hkv,N,d], dV [B,Hkv,N,d]) in bf16."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, N, d] and k, v [B, Hkv, N, d]")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    bf = torch.bfloat16
    for t, n, shp in ((q, "q", (B, Hq, N, d)), (k, "k", (B, Hkv, N, d)), (v, "v", (B, Hkv, N, d)),
                      (o, "o", (B, Hq, N, d)), (dout, "dout", (B, Hq, N, d))):
        _need(t, n, bf, shp, dev)
    _need(lse, "lse", torch.float32, (B, Hq, N), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty((B, Hq, N, d), dtype=bf, device=dev) if dq is None else dq
    dk = torch.empty((B, Hkv, N, d), dtype=bf, device=dev) if dk is None else dk
    dv = torch.empty((B, Hkv, N, d), dtype=bf, device=dev) if dv is None else dv
    _need(dq, "dq", bf, (B, Hq, N, d), dev)
    _need(dk, "dk", bf, (B, Hkv, N, d), dev)
    _need(dv, "dv", bf, (B, Hkv, N, d), dev)
    need = fa_bwd_workspace_size(B, Hq, Hkv, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    st = lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                      B, Hq, Hkv, N, d, int(bool(causal)), float(scale), _ptr(workspace),
                      workspace.numel() * workspace.element_size(), _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_bwd")
    return dq, dk, dv


def fa_decode_paged_workspace_size(num_seqs, Hq, d, max_pages_per_seq, page_size=16) -> int:
    return int(lib().fa_decode_paged_workspace_size(num_seqs, Hq, d, max_pages_per_seq, page_size))


def fa_decode_paged(q, kpages, vpages, page_table, ctx_lens, scale=None, out=None, lse=None,
                    workspace=None):
    """Paged decode: q [S,Hq,d] bf16; kpages/vpages [P,Hkv,16,d] bf16; page_table [S,maxp] int32;
    ctx_lens [S] int32 -> (O bf16 [S,Hq,d], L fp32 [S,Hq])."""
    S, Hq, d = q.shape
    P, Hkv, page_size, dk = kpages.shape
    maxp = page_table.shape[1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    _need(q, "q", torch.bfloat16, (S, Hq, d), dev)
    _need(kpages, "kpages", torch.bfloat16, (P, Hkv, page_size, d), dev)
    _need(vpages, "vpages", torch.bfloat16, (P, Hkv, page_size, d), dev)
    _need(page_table, "page_table", torch.int32, (S, maxp), dev)
    _need(ctx_lens, "ctx_lens", torch.int32, (S,), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((S, Hq, d), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=dev)
    _need(out, "out", torch.bfloat16, (S, Hq, d), dev)
    _need(lse, "lse", torch.float32, (S, Hq), dev)
    need = fa_decode_paged_workspace_size(S, Hq, d, maxp, page_size)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    st = lib().fa_decode_paged(_ptr(q), _ptr(kpages), _ptr(vpages), _ptr(page_table), _ptr(ctx_lens),
                               _ptr(out), _ptr(lse), S, Hq, Hkv, d, page_size, maxp, P, float(scale),
                               _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_decode_paged")
    return out, lse


def fa_decode_paged_noalloc_max_scratch() -> int:
    return int(lib().fa_decode_paged_noalloc_max_scratch())


def fa_decode_paged_noalloc(q, kpages, vpages, page_table, ctx_lens, out, lse, scale=None):
    """fa_decode_paged with the library's own device scratch instead of a workspace.  The
    caller passes the outputs (O bf16 [S,Hq,d], L fp32 [S,Hq]); nothing is allocated."""
    S, Hq, d = q.shape
    P, Hkv, page_size, _ = kpages.shape
    maxp = page_table.shape[1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    _need(q, "q", torch.bfloat16, (S, Hq, d), dev)
    _need(kpages, "kpages", torch.bfloat16, (P, Hkv, page_size, d), dev)
    _need(vpages, "vpages", torch.bfloat16, (P, Hkv, page_size, d), dev)
    _need(page_table, "page_table", torch.int32, (S, maxp), dev)
    _need(ctx_lens, "ctx_lens", torch.int32, (S,), dev)
    _need(out, "out", torch.bfloat16, (S, Hq, d), dev)
    _need(lse, "lse", torch.float32, (S, Hq), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_decode_paged_noalloc(_ptr(q), _ptr(kpages), _ptr(vpages), _ptr(page_table), _ptr(ctx_lens),
                                       _ptr(out), _ptr(lse), S, Hq, Hkv, d, page_size, maxp, P, float(scale),
                                       _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_decode_paged_noalloc")
    return out, lse


def fa_prefill_paged(q, kpages, vpages, page_table, ctx_lens, scale=None, out=None, lse=None):
    """Chunked prefill: q [S,Hq,C,d] bf16 (the last C tokens of each sequence's cache);
    kpages/vpages [P,Hkv,16,d] bf16; page_table [S,maxp] int32; ctx_lens [S] int32 (>= C)
    -> (O bf16 [S,Hq,C,d], L fp32 [S,Hq,C])."""
    S, Hq, C, d = q.shape
    P, Hkv, page_size, _ = kpages.shape
    maxp = page_table.shape[1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    _need(q, "q", torch.bfloat16, (S, Hq, C, d), dev)
    _need(kpages, "kpages", torch.bfloat16, (P, Hkv, page_size, d), dev)
    _need(vpages, "vpages", torch.bfloat16, (P, Hkv, page_size, d), dev)
    _need(page_table, "page_table", torch.int32, (S, maxp), dev)
    _need(ctx_lens, "ctx_lens", torch.int32, (S,), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty((S, Hq, C, d), dtype=torch.bfloat16, device=dev) if out is None else out
    lse = torch.empty((S, Hq, C), dtype=torch.float32, device=dev) if lse is None else lse
    _need(out, "out", torch.bfloat16, (S, Hq, C, d), dev)
    _need(lse, "lse", torch.float32, (S, Hq, C), dev)
    st = lib().fa_prefill_paged(_ptr(q), _ptr(kpages), _ptr(vpages), _ptr(page_table), _ptr(ctx_lens), _ptr(out),
                                _ptr(lse), S, Hq, Hkv, d, C, page_size, maxp, P, float(scale), _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_prefill_paged")
    return out, lse


def fa_decode_paged_int8(q, kq, kscale, vq, vscale, page_table, ctx_lens, scale=None, out=None, lse=None,
                         workspace=None, group=32):
    """Paged decode over an INT8 cache: kq/vq [P,Hkv,16,d] int8, kscale/vscale [P,Hkv,16,d/group] fp32,
    other arguments as fa_decode_paged -> (O bf16 [S,Hq,d], L fp32 [S,Hq])."""
    S, Hq, d = q.shape
    P, Hkv, page_size, _ = kq.shape
    maxp = page_table.shape[1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    _need(q, "q", torch.bfloat16, (S, Hq, d), dev)
    _need(kq, "kq", torch.int8, (P, Hkv, page_size, d), dev)
    _need(vq, "vq", torch.int8, (P, Hkv, page_size, d), dev)
    _need(kscale, "kscale", torch.float32, (P, Hkv, page_size, d // group), dev)
    _need(vscale, "vscale", torch.float32, (P, Hkv, page_size, d // group), dev)
    _need(page_table, "page_table", torch.int32, (S, maxp), dev)
    _need(ctx_lens, "ctx_lens", torch.int32, (S,), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty((S, Hq, d), dtype=torch.bfloat16, device=dev) if out is None else out
    lse = torch.empty((S, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    _need(out, "out", torch.bfloat16, (S, Hq, d), dev)
    _need(lse, "lse", torch.float32, (S, Hq), dev)
    need = fa_decode_paged_workspace_size(S, Hq, d, maxp, page_size)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    st = lib().fa_decode_paged_int8(_ptr(q), _ptr(kq), _ptr(kscale), _ptr(vq), _ptr(vscale), _ptr(page_table),
                                    _ptr(ctx_lens), _ptr(out), _ptr(lse), S, Hq, Hkv, d, page_size, group, maxp, P,
                                    float(scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_decode_paged_int8")
    return out, lse
