"""The C-ABI library: it loads, exports every declared symbol, and rejects bad
arguments on the host before touching the GPU (CPU only: no call here reaches a launch)."""

import ctypes
import os
import re

import pytest

import exact_io_aware_15_amd as fa

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "fa.h")

OK, NULL, SHAPE, UNSUP, SCALE, ALIGN, WORKSPACE, HIP, SCRATCH = range(9)
P = ctypes.c_void_p(0x10000)      # aligned stand-in device pointer, never dereferenced
MIS = ctypes.c_void_p(0x10008)    # 8-byte aligned only
Z = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa.so is not built (python -m exact_io_aware_15_amd.build)")
    return fa.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert set(names) >= {"fa_fwd", "fa_fwd_f32", "fa_fwd_ex", "fa_prefill_paged", "fa_decode_paged_int8", "fa_bwd", "fa_bwd_workspace_size", "fa_decode_paged",
                          "fa_decode_paged_workspace_size", "fa_status_string"}
    for n in names:
        assert hasattr(L, n), n


def test_status_codes_match_header(L):
    text = open(HEADER).read()
    codes = dict((k, int(v)) for k, v in re.findall(r"#define (FA_\w+)\s+(\d+)", text))
    assert codes == {"FA_OK": 0, "FA_ERR_NULL": 1, "FA_ERR_SHAPE": 2, "FA_ERR_UNSUPPORTED": 3,
                     "FA_ERR_SCALE": 4, "FA_ERR_ALIGN": 5, "FA_ERR_WORKSPACE": 6, "FA_ERR_HIP": 7,
                     "FA_ERR_SCRATCH": 8}
    for c in range(9):
        assert fa.fa_status_string(c)
    assert fa.fa_status_string(99) == "unknown status"


def fwd(L, entry, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, N=16, d=64, causal=0, scale=0.125):
    return getattr(L, entry)(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, Z)


@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_f32"])
def test_fwd_validation(L, entry):
    assert fwd(L, entry, q=Z) == NULL
    assert fwd(L, entry, lse=Z) == NULL
    assert fwd(L, entry, d=96) == UNSUP
    assert fwd(L, entry, d=256) == UNSUP
    assert fwd(L, entry, Hq=3, Hkv=2) == SHAPE
    assert fwd(L, entry, Hkv=0) == SHAPE
    assert fwd(L, entry, N=-1) == SHAPE
    assert fwd(L, entry, B=-2) == SHAPE
    assert fwd(L, entry, causal=2) == SHAPE
    assert fwd(L, entry, scale=float("nan")) == SCALE
    assert fwd(L, entry, scale=float("inf")) == SCALE
    assert fwd(L, entry, k=MIS) == ALIGN
    assert fwd(L, entry, o=MIS) == ALIGN
    # every size is at least 1: an empty batch or sequence is a shape error
    assert fwd(L, entry, B=0) == SHAPE
    assert fwd(L, entry, N=0) == SHAPE
    assert fwd(L, entry, Hq=0) == SHAPE
    # dispatch limits: fewer than 2^31 work-items per launch
    rows = {"fa_fwd": 256, "fa_fwd_f32": 256 // 4}[entry]
    threads = {"fa_fwd": 512, "fa_fwd_f32": 256}[entry]
    blocks_max = (2**31 - 1) // threads
    assert fwd(L, entry, B=blocks_max // 2 + 1, Hq=2, Hkv=1, N=rows) == SHAPE
    # (the same sizes one workgroup fewer pass the size checks and stop at the NULL pointer;
    # no call here may reach a launch)
    assert fwd(L, entry, B=blocks_max // 2, Hq=2, Hkv=1, N=rows, q=Z) == NULL


def dec(L, q=P, kp=P, vp=P, pt=P, cl=P, o=P, lse=P, S=2, Hq=8, Hkv=2, d=128, ps=16, maxp=4, npages=9,
        scale=0.1, ws=P, wsb=1 << 30):
    return L.fa_decode_paged(q, kp, vp, pt, cl, o, lse, S, Hq, Hkv, d, ps, maxp, npages, scale, ws, wsb, Z)


def test_decode_validation(L):
    assert dec(L, q=Z) == NULL
    assert dec(L, pt=Z) == NULL
    assert dec(L, cl=Z) == NULL
    assert dec(L, d=80) == UNSUP
    assert dec(L, ps=32) == UNSUP
    assert dec(L, Hq=6, Hkv=4) == SHAPE
    assert dec(L, S=-1) == SHAPE
    assert dec(L, maxp=0) == SHAPE
    assert dec(L, maxp=128 * 65535 + 1) == SHAPE   # more splits than one grid dimension holds
    assert dec(L, scale=float("-inf")) == SCALE
    assert dec(L, vp=MIS) == ALIGN
    assert dec(L, ws=Z) == WORKSPACE
    need = fa.fa_decode_paged_workspace_size(2, 8, 128, 4, 16)
    assert dec(L, wsb=need - 1) == WORKSPACE
    assert dec(L, ws=MIS, wsb=need) == ALIGN
    assert dec(L, S=0) == SHAPE
    assert dec(L, Hq=0) == SHAPE
    assert dec(L, npages=0) == SHAPE
    # split grid: num_seqs * Hq * splits workgroups of 256 threads below 2^31 work-items
    assert dec(L, S=(2**31 - 1) // 256 // 8 + 1, Hq=8, Hkv=2, maxp=4, wsb=1 << 62) == SHAPE


def test_workspace_size(L):
    # one fp32 partial (d values + one logsumexp) per (sequence, head, split of 128 pages)
    for S, Hq, d, maxp in [(64, 32, 128, 1024), (1, 1, 64, 1), (3, 4, 64, 33)]:
        splits = -(-maxp // 128)
        o_bytes = S * Hq * splits * d * 4
        assert fa.fa_decode_paged_workspace_size(S, Hq, d, maxp, 16) == -(-o_bytes // 256) * 256 + S * Hq * splits * 4
    assert fa.fa_decode_paged_workspace_size(1, 1, 96, 1, 16) == 0
    assert fa.fa_decode_paged_workspace_size(1, 1, 64, 1, 8) == 0
    assert fa.fa_decode_paged_workspace_size(-1, 1, 64, 1, 16) == 0


def bwd(L, q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, Hq=2, Hkv=1, N=16, d=64, causal=0, scale=0.125,
        ws=P, wsb=1 << 30):
    return L.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, ws, wsb, Z)


def test_bwd_validation(L):
    assert bwd(L, q=Z) == NULL
    assert bwd(L, do=Z) == NULL
    assert bwd(L, dk=Z) == NULL
    assert bwd(L, d=96) == UNSUP
    assert bwd(L, Hq=3, Hkv=2) == SHAPE
    assert bwd(L, causal=5) == SHAPE
    assert bwd(L, scale=float("nan")) == SCALE
    assert bwd(L, dv=MIS) == ALIGN
    assert bwd(L, ws=Z) == WORKSPACE
    need = fa.fa_bwd_workspace_size(1, 2, 1, 16, 64)
    assert bwd(L, wsb=need - 1) == WORKSPACE
    assert bwd(L, ws=MIS, wsb=need) == ALIGN
    assert bwd(L, B=0) == SHAPE
    assert bwd(L, N=0) == SHAPE
    # the bf16 kernels address one (batch, head) slice through a 32-bit byte range
    assert bwd(L, N=2**24, d=128, B=1, Hq=1, Hkv=1) == SHAPE          # 2^24 * 128 * 2 = 4 GiB
    assert bwd(L, N=2**24 - 64, d=128, B=1, Hq=1, Hkv=1, q=Z) == NULL


def test_bwd_workspace_size(L):
    # D and L log2(e) per row (fp32, each padded to 256 B); head-chunk partials of dK
    # and dV only when fewer than 512 (128-key block, K/V head) pairs exist
    def dbytes(B, Hq, N):
        return 2 * (-(-B * Hq * N * 4 // 256) * 256)
    assert fa.fa_bwd_workspace_size(1, 32, 32, 8192, 128) == dbytes(1, 32, 8192)      # 2048 pairs
    assert fa.fa_bwd_workspace_size(2, 32, 8, 4096, 128) == dbytes(2, 32, 4096)       # 512 pairs
    # multi-query: 64 pairs -> 8 chunks of 4 heads
    assert fa.fa_bwd_workspace_size(2, 32, 1, 4096, 128) == dbytes(2, 32, 4096) + 2 * 8 * 2 * 1 * 4096 * 128 * 4
    assert fa.fa_bwd_workspace_size(1, 2, 1, 16, 96) == 0
    assert fa.fa_bwd_workspace_size(1, 3, 2, 16, 64) == 0


def fwd_ex(L, window=0, slopes=Z, causal=1, **kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, N=16, d=64, scale=0.125)
    args.update(kw)
    return L.fa_fwd_ex(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"], args["Hq"], args["Hkv"],
                       args["N"], args["d"], causal, args["scale"], window, slopes, Z)


def test_fwd_ex_validation(L):
    assert fwd_ex(L, window=-1) == SHAPE
    assert fwd_ex(L, window=4, causal=0) == UNSUP
    assert fwd_ex(L, slopes=ctypes.c_void_p(0x10002)) == ALIGN
    assert fwd_ex(L, q=Z) == NULL
    assert fwd_ex(L, d=80) == UNSUP
    assert fwd_ex(L, window=3, N=0) == SHAPE
    assert fwd_ex(L, B=0) == SHAPE
    assert fwd_ex(L, N=2**24, d=128, B=1, Hq=1, Hkv=1) == SHAPE
    assert fwd_ex(L, N=2**25, d=64, B=1, Hq=1, Hkv=1) == SHAPE
    assert fwd_ex(L, N=2**25 - 64, d=64, B=1, Hq=1, Hkv=1, q=Z) == NULL


def pp(L, q=P, kp=P, vp=P, pt=P, cl=P, o=P, lse=P, S=2, Hq=8, Hkv=2, d=128, C=5, ps=16, maxp=4, npages=9,
       scale=0.1):
    return L.fa_prefill_paged(q, kp, vp, pt, cl, o, lse, S, Hq, Hkv, d, C, ps, maxp, npages, scale, Z)


def test_prefill_paged_validation(L):
    assert pp(L, cl=Z) == NULL
    assert pp(L, d=96) == UNSUP
    assert pp(L, ps=8) == UNSUP
    assert pp(L, Hq=6, Hkv=4) == SHAPE
    assert pp(L, C=-1) == SHAPE
    assert pp(L, scale=float("nan")) == SCALE
    assert pp(L, o=MIS) == ALIGN
    assert pp(L, C=0) == SHAPE
    assert pp(L, S=0) == SHAPE
    assert pp(L, npages=0) == SHAPE
    # a chunk lies inside its sequence's cache: at most max_pages_per_seq * 16 tokens
    assert pp(L, C=4 * 16 + 1, maxp=4) == SHAPE
    assert pp(L, C=4 * 16, maxp=4, q=Z) == NULL


def d8(L, q=P, kq=P, ks=P, vq=P, vs=P, pt=P, cl=P, o=P, lse=P, S=2, Hq=8, Hkv=2, d=128, ps=16, group=32, maxp=4,
       npages=9, scale=0.1, ws=P, wsb=1 << 30):
    return L.fa_decode_paged_int8(q, kq, ks, vq, vs, pt, cl, o, lse, S, Hq, Hkv, d, ps, group, maxp, npages, scale, ws,
                                  wsb, Z)


def test_decode_int8_validation(L):
    assert d8(L, ks=Z) == NULL
    assert d8(L, group=64) == UNSUP
    assert d8(L, d=80) == UNSUP
    assert d8(L, Hq=6, Hkv=4) == SHAPE
    assert d8(L, vs=ctypes.c_void_p(0x10002)) == ALIGN
    assert d8(L, kq=MIS) == ALIGN
    assert d8(L, ws=Z) == WORKSPACE
    assert d8(L, S=0) == SHAPE
    assert d8(L, npages=0) == SHAPE


def test_fwd_bf16_slice_limit(L):
    # one (batch, head) slice of N x d bf16 values must span at most 2^32 - 1 bytes
    assert fwd(L, "fa_fwd", N=2**24, d=128, B=1, Hq=1, Hkv=1) == SHAPE
    assert fwd(L, "fa_fwd", N=2**24 - 1, d=128, B=1, Hq=1, Hkv=1, q=Z) == NULL
    assert fwd(L, "fa_fwd", N=2**25, d=64, B=1, Hq=1, Hkv=1) == SHAPE
    assert fwd(L, "fa_fwd", N=2**25 - 1, d=64, B=1, Hq=1, Hkv=1, q=Z) == NULL


def test_workspace_sizes_reject_empty(L):
    assert fa.fa_decode_paged_workspace_size(0, 8, 128, 4, 16) == 0
    assert fa.fa_bwd_workspace_size(0, 2, 1, 16, 64) == 0
    assert fa.fa_bwd_workspace_size(1, 2, 1, 0, 64) == 0


def na(L, q=P, kp=P, vp=P, pt=P, cl=P, o=P, lse=P, S=2, Hq=8, Hkv=2, d=128, ps=16, maxp=4, npages=9, scale=0.1):
    return L.fa_decode_paged_noalloc(q, kp, vp, pt, cl, o, lse, S, Hq, Hkv, d, ps, maxp, npages, scale, Z)


def test_decode_noalloc_validation(L):
    assert na(L, q=Z) == NULL
    assert na(L, d=80) == UNSUP
    assert na(L, ps=32) == UNSUP
    assert na(L, Hq=6, Hkv=4) == SHAPE
    assert na(L, S=0) == SHAPE
    assert na(L, scale=float("nan")) == SCALE
    assert na(L, lse=MIS) == ALIGN
    cap = L.fa_decode_paged_noalloc_max_scratch()
    assert cap == 32 << 20
    # sizes whose partials exceed the fixed scratch are rejected before any HIP call
    S, Hq, d = 64, 32, 128
    maxp = 128
    while fa.fa_decode_paged_workspace_size(S, Hq, d, maxp) <= cap:
        maxp += 128
    assert na(L, S=S, Hq=Hq, Hkv=8, d=d, maxp=maxp) == SCRATCH
    assert "scratch" in fa.fa_status_string(SCRATCH)


def splitk(L, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=4, N=8192, d=128, causal=1, scale=0.088, ws=P,
           ws_bytes=1 << 40):
    return L.fa_fwd_splitk(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, ws, ws_bytes, Z)


def test_fwd_splitk_workspace_size(L):
    # a launch with at least 256 (256-row query block, head) items is not split
    assert fa.fa_fwd_splitk_workspace_size(1, 32, 8192, 128, 1) == 0
    assert fa.fa_fwd_splitk_workspace_size(4, 16, 2048, 64, 0) == 0
    # one GPU's share of the c3 forward (4 heads: 128 items) is, in fp32 partials of
    # 256 rows x (d + 1) per chunk slot
    sz = fa.fa_fwd_splitk_workspace_size(1, 4, 8192, 128, 1)
    assert sz >= 2 * 4 * 32 * 256 * (128 + 1) * 4
    # out-of-range arguments
    for args in [(0, 4, 8192, 128, 1), (1, 0, 8192, 128, 1), (1, 4, 0, 128, 1), (1, 4, 8192, 96, 1),
                 (1, 4, 8192, 128, 2)]:
        assert L.fa_fwd_splitk_workspace_size(*args) == 0


def test_fwd_splitk_validation(L):
    need = fa.fa_fwd_splitk_workspace_size(1, 4, 8192, 128, 1)
    assert splitk(L, q=Z) == NULL
    assert splitk(L, d=96) == UNSUP
    assert splitk(L, Hq=3, Hkv=2) == SHAPE
    assert splitk(L, N=0) == SHAPE
    assert splitk(L, scale=float("nan")) == SCALE
    assert splitk(L, v=MIS) == ALIGN
    # a split launch needs its workspace: missing, short or misaligned
    assert splitk(L, ws=Z) == WORKSPACE
    assert splitk(L, ws_bytes=need - 1) == WORKSPACE
    assert splitk(L, ws=MIS, ws_bytes=need) == ALIGN
