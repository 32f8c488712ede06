"""GPU parity of the split-K forward (fa_fwd_splitk) against the fp64 oracle, on every
element: launches with few (query block, head) items, whose blocks are cut into key
chunks and merged, with ragged ends, GQA, both head dimensions, causal and not, and edge
scales; a launch with enough items to need no split equals fa_fwd bit for bit."""

import numpy as np
import pytest
import torch

from _parity import check_bf16, check_bf16_p_bound, f64, fwd_p_bound, say
from exact_io_aware_15_amd import fa_fwd, fa_fwd_splitk, fa_fwd_splitk_workspace_size
from exact_io_aware_15_amd.workloads import make_prefill
from oracle import attention_ref

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

SPLIT_SHAPES = [
    # B, Hq, Hkv, N, d, causal
    (1, 4, 4, 8192, 128, True),     # one GPU's share of the causal B1 H32 N8192 forward
    (1, 2, 1, 3000, 64, True),      # ragged last block, GQA
    (1, 3, 3, 2500, 128, False),
    (2, 2, 2, 700, 128, True),
    (1, 1, 1, 300, 64, True),
    (1, 1, 1, 64, 128, False),      # one tile: nothing to split
    (1, 6, 2, 1800, 128, True),     # 3 query heads per K/V head
]


def run(x, causal, scale=None):
    q, k, v = (x[n].to(DEV) for n in "qkv")
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device=DEV)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.full((max(1, fa_fwd_splitk_workspace_size(q.shape[0], q.shape[1], q.shape[2], q.shape[3], causal)),),
                    0xFF, dtype=torch.uint8, device=DEV)  # NaN-patterned workspace
    fa_fwd_splitk(q, k, v, causal=causal, scale=scale, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: "B{}_Hq{}_Hkv{}_N{}_d{}_{}".format(
    s[0], s[1], s[2], s[3], s[4], "causal" if s[5] else "full"))
def test_splitk_every_element(shape):
    B, Hq, Hkv, N, d, causal = shape
    say(f"split-K forward {shape}, workspace {fa_fwd_splitk_workspace_size(B, Hq, N, d, causal)} B")
    x = make_prefill(B, Hq, Hkv, N, d, "bf16", seed=40 + N + d, value_scale=0.5 if N == 8192 else 1.0)
    out, lse = run(x, causal)
    Oref, Lref = attention_ref(f64(x["q"]), f64(x["k"]), f64(x["v"]), causal, 1.0 / np.sqrt(d))
    check_bf16(f64(out), f64(lse), Oref, Lref, f"split-K {shape}")


@pytest.mark.parametrize("scale", [0.0, -0.0883883, 0.9])
def test_splitk_scale_edge_cases(scale):
    # at 0.9 (ten times 1/sqrt(d) on unit-variance inputs) a few keys carry each row's
    # weight and the bf16 probabilities' rounding can pass the 1e-2 bar where |O| is in
    # [2, 4): those elements are held to the forward's own per-element rounding bound,
    # as fa_fwd's are (tests/test_parity_gpu.py)
    say(f"split-K scale {scale}")
    x = make_prefill(1, 2, 1, 1500, 128, "bf16", seed=71)
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    for causal in (False, True):
        out, lse = run(x, causal, scale=scale)
        Oref, Lref = attention_ref(q, k, v, causal, scale)
        what = f"split-K scale={scale} causal={causal}"
        if scale == 0.9:
            check_bf16_p_bound(f64(out), f64(lse), Oref, Lref, fwd_p_bound(q, k, v, Oref, Lref, causal, scale), what)
        else:
            check_bf16(f64(out), f64(lse), Oref, Lref, what)


def test_unsplit_launch_equals_fa_fwd_bitwise():
    # 8 query blocks x 32 heads = 256 items: nothing is split and no workspace is needed
    assert fa_fwd_splitk_workspace_size(1, 32, 2048, 128, 1) == 0
    x = make_prefill(1, 32, 8, 2048, 128, "bf16", seed=77)
    out, lse = run(x, True)
    q, k, v = (x[n].to(DEV) for n in "qkv")
    o2, l2 = fa_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)
