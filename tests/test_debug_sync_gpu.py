"""The fast build of the tiled kernels against the debug-sync build (every HBM -> LDS
copy waited for and fenced with a workgroup barrier as soon as it is issued, every LDS
read stage waited for), bitwise, at full configuration sizes.  The fast build relies on
its per-tile waits alone (its LDS tile pointers tell the compiler that the copy in
flight writes only the other buffer); a read racing a copy would make the two builds
differ."""

import pytest
import torch

import exact_io_aware_15_amd as fa
from _parity import say
from exact_io_aware_15_amd.workloads import (CONFIGS, make_alibi_slopes, make_grad_output, make_inputs,
                                             make_prefill_paged)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def both(fn):
    """fn() through libfa.so, then through libfa_debugsync.so."""
    a = fn()
    torch.cuda.synchronize()
    with fa.use_library(fa.load_library(fa.DEBUG_SYNC_LIB_PATH)):
        b = fn()
        torch.cuda.synchronize()
    return a, b


def same(a, b, what):
    for x, y in zip(a, b):
        assert torch.equal(x, y), f"{what}: fast and debug-sync builds differ"
    say(f"{what}: bitwise equal")


FWD = ["c3_bf16_causal_B1_H32_N8192_d128", "c4_bf16_causal_gqa_B2_Hq32_Hkv8_N4096_d128",
       "c4_bf16_causal_mqa_B2_Hq32_Hkv1_N4096_d128", "c2_bf16_B4_H16_N2048_d64"]


@pytest.mark.parametrize("name", FWD)
def test_forward_fast_equals_debug_sync(name):
    cfg = CONFIGS[name]
    x = make_inputs(cfg)
    q, k, v = (x[n].to(DEV) for n in "qkv")
    same(*both(lambda: fa.fa_fwd(q, k, v, causal=cfg.causal, scale=cfg.scale)), f"fa_fwd {name}")


def test_window_alibi_fast_equals_debug_sync():
    cfg = CONFIGS["c3_bf16_causal_B1_H32_N8192_d128"]
    x = make_inputs(cfg)
    q, k, v = (x[n].to(DEV) for n in "qkv")
    sl = make_alibi_slopes(cfg.Hq).to(DEV)
    same(*both(lambda: fa.fa_fwd_ex(q, k, v, causal=True, scale=cfg.scale, window=4096, alibi_slopes=sl)),
         "fa_fwd_ex c3 window 4096 + ALiBi")


def test_chunked_prefill_fast_equals_debug_sync():
    x = make_prefill_paged(16, 32, 8, 128, 512, 512, 16384, seed=6)
    g = {kk: (vv.to(DEV) if torch.is_tensor(vv) else vv) for kk, vv in x.items()}
    same(*both(lambda: fa.fa_prefill_paged(g["q"], g["kpages"], g["vpages"], g["page_table"], g["ctx_lens"])),
         "fa_prefill_paged 16 x 512")


@pytest.mark.parametrize("name", FWD[:3])
def test_backward_fast_equals_debug_sync(name):
    cfg = CONFIGS[name]
    x = make_inputs(cfg)
    q, k, v = (x[n].to(DEV) for n in "qkv")
    do = make_grad_output(cfg.B, cfg.Hq, cfg.N, cfg.d, seed=cfg.seed).to(DEV)
    o, l = fa.fa_fwd(q, k, v, causal=cfg.causal, scale=cfg.scale)
    same(*both(lambda: fa.fa_bwd(q, k, v, o, l, do, causal=cfg.causal, scale=cfg.scale)), f"fa_bwd {name}")


def test_fwd_splitk_fast_equals_debug_sync():
    """The 4-head share of the causal N8192 forward, whose key tiles the split-K path cuts
    into chunks; the chunk partials and their merge both compared."""
    cfg = CONFIGS["c3_bf16_causal_B1_H32_N8192_d128"]
    x = make_inputs(cfg)
    q, k, v = (x[n][:, :4].contiguous().to(DEV) for n in "qkv")
    same(*both(lambda: fa.fa_fwd_splitk(q, k, v, causal=True, scale=cfg.scale)), "fa_fwd_splitk c3 4 heads")
