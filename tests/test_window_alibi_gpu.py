"""GPU parity of the sliding-window / ALiBi forward (fa_fwd_ex) against the fp64 oracle.

Same bars as the plain bf16 forward: O within 1e-2 and L within 1e-3 (max-abs),
with the bf16 output-floor rule of tests/_parity.py.  Every test compares every
output element, the full-size workloads included.  Outputs are pre-filled with NaN."""

import numpy as np
import pytest
import torch

from _parity import check_bf16, f64, say
from exact_io_aware_15_amd import fa_fwd, fa_fwd_ex
from exact_io_aware_15_amd.workloads import CONFIGS, make_alibi_slopes, make_inputs, make_prefill
from oracle import attention_ref

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_ex(x, causal, window, alibi, scale=None):
    q, k, v = (x[n].to(DEV) for n in "qkv")
    Hq = q.shape[1]
    slopes = make_alibi_slopes(Hq) if alibi else None
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device=DEV)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa_fwd_ex(q, k, v, causal=causal, scale=scale, window=window,
              alibi_slopes=None if slopes is None else slopes.to(DEV), out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse, (None if slopes is None else slopes.double().numpy())


def check(O, L, Oref, Lref, what):
    return check_bf16(O, L, Oref, Lref, what)


SMALL = [
    # B, Hq, Hkv, N, d, causal, window, alibi
    (1, 2, 1, 70, 64, True, 1, False),
    (1, 2, 2, 200, 128, True, 7, True),
    (1, 4, 2, 300, 128, True, 64, False),
    (2, 2, 1, 257, 64, True, 65, True),
    (1, 1, 1, 600, 128, True, 100, True),
    (1, 2, 1, 513, 128, True, 256, False),
    (1, 2, 1, 130, 64, True, 500, True),     # window wider than the sequence
    (1, 4, 4, 333, 128, True, 0, True),      # ALiBi only
    (2, 4, 2, 190, 64, False, 0, True),      # non-causal ALiBi: -m |i - j|
    (1, 6, 2, 420, 128, True, 150, True),    # 3 query heads per K/V head
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}_Hq{}_Hkv{}_N{}_d{}_{}_w{}_{}".format(
    s[0], s[1], s[2], s[3], s[4], "causal" if s[5] else "full", s[6], "alibi" if s[7] else "noalibi"))
def test_window_alibi_small_every_element(shape):
    B, Hq, Hkv, N, d, causal, window, alibi = shape
    say(f"window/alibi small {shape}")
    x = make_prefill(B, Hq, Hkv, N, d, "bf16", seed=400 + N + window)
    out, lse, slopes = run_ex(x, causal, window, alibi)
    Oref, Lref = attention_ref(f64(x["q"]), f64(x["k"]), f64(x["v"]), causal, 1.0 / np.sqrt(d),
                               window=window, alibi_slopes=slopes)
    check(f64(out), f64(lse), Oref, Lref, str(shape))


@pytest.mark.parametrize("scale", [0.0, -0.11, 0.3, 0.9])
@pytest.mark.parametrize("window", [0, 40])
def test_causal_alibi_scale_edge_cases(scale, window):
    # zero, negative and large softmax scales with causal ALiBi (with and without a
    # window): the bias enters independently of the scale's size and sign.  At 0.9 a
    # few keys dominate each row and |O| reaches 4, where the bf16 output's own
    # rounding exceeds 1e-2 (the output-floor rule applies there)
    say(f"causal alibi scale={scale} window={window}")
    x = make_prefill(1, 4, 2, 160, 128, "bf16", seed=57)
    out, lse, slopes = run_ex(x, True, window, True, scale=scale)
    Oref, Lref = attention_ref(f64(x["q"]), f64(x["k"]), f64(x["v"]), True, scale, window=window,
                               alibi_slopes=slopes)
    check(f64(out), f64(lse), Oref, Lref, f"scale={scale} window={window}")


def test_fwd_ex_without_options_is_fa_fwd_bitwise():
    x = make_prefill(1, 4, 2, 450, 128, "bf16", seed=31)
    q, k, v = (x[n].to(DEV) for n in "qkv")
    for causal in (False, True):
        a = fa_fwd(q, k, v, causal=causal)
        b = fa_fwd_ex(q, k, v, causal=causal, window=0, alibi_slopes=None)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


FULL = [
    ("c3_bf16_causal_B1_H32_N8192_d128", 4096, True),
    ("c4_bf16_causal_gqa_B2_Hq32_Hkv8_N4096_d128", 1000, True),
    ("c4_bf16_causal_mqa_B2_Hq32_Hkv1_N4096_d128", 512, False),
    ("c2_bf16_B4_H16_N2048_d64", 0, True),
]


@pytest.mark.parametrize("name,window,alibi", FULL, ids=[f"{f[0]}_w{f[1]}" for f in FULL])
def test_window_alibi_full_size_every_element(name, window, alibi):
    cfg = CONFIGS[name]
    say(f"window/alibi full-size {name} window={window} alibi={alibi}")
    x = make_inputs(cfg)
    out, lse, slopes = run_ex(x, cfg.causal, window, alibi, scale=cfg.scale)
    O, L = f64(out), f64(lse)
    del out, lse
    Oref, Lref = attention_ref(f64(x["q"]), f64(x["k"]), f64(x["v"]), cfg.causal, cfg.scale, window=window,
                               alibi_slopes=slopes)
    check(O, L, Oref, Lref, f"{name} window={window} alibi={alibi} (every element)")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("window", [0, 300])
def test_causal_alibi_steep_slopes_every_element(d, window):
    """Slopes 2, 1, 0.5, 0.25: a row's weight sits on its last few keys, so the bf16
    rounding of those few probabilities would reach O undamped (it averages out over
    many keys).  The tiles nearest each wave's diagonal carry P in two bf16 parts."""
    say(f"causal alibi steep slopes d={d} window={window}")
    x = make_prefill(2, 4, 2, 700, d, "bf16", seed=71 + d + window)
    q, k, v = (x[n].to(DEV) for n in "qkv")
    slopes = torch.tensor([2.0, 1.0, 0.5, 0.25], dtype=torch.float32)
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device=DEV)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa_fwd_ex(q, k, v, causal=True, window=window, alibi_slopes=slopes.to(DEV), out=out, lse=lse)
    torch.cuda.synchronize()
    Oref, Lref = attention_ref(f64(x["q"]), f64(x["k"]), f64(x["v"]), True, 1.0 / np.sqrt(d), window=window,
                               alibi_slopes=slopes.double().numpy())
    check(out, lse, Oref, Lref, f"steep slopes d={d} window={window}")
