"""The allocation-free paged decode (fa_decode_paged_noalloc) against the workspace
entry point (fa_decode_paged) through the C ABI: two calls in a row, the second with
a smaller input, each compared with the workspace call bitwise (same kernels) and with
the fp64 oracle at the bf16 bars."""

import numpy as np
import pytest
import torch

from _parity import check_bf16, f64, say
from exact_io_aware_15_amd import (fa_decode_paged, fa_decode_paged_noalloc, fa_decode_paged_noalloc_max_scratch,
                                   fa_decode_paged_workspace_size)
from exact_io_aware_15_amd.workloads import make_decode
from oracle import decode_ref

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to_dev(x):
    return {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in x.items()}


def test_noalloc_matches_workspace_entry_point_twice():
    cases = [
        # first call: 32 sequences up to 16K tokens (about 4 MB of partials); second: smaller
        make_decode(32, 32, 8, 128, 1024, 16384, seed=71),
        make_decode(5, 8, 2, 128, seed=72, fixed_ctx=(0, 1, 17, 700, 2049)),
    ]
    for i, x in enumerate(cases):
        g = to_dev(x)
        S, Hq, d = x["q"].shape
        say(f"no-alloc decode call {i}: S={S} Hq={Hq} maxp={x['page_table'].shape[1]}")
        assert fa_decode_paged_workspace_size(S, Hq, d, x["page_table"].shape[1]) <= fa_decode_paged_noalloc_max_scratch()
        o_ws = torch.full((S, Hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        l_ws = torch.full((S, Hq), float("nan"), dtype=torch.float32, device=DEV)
        fa_decode_paged(g["q"], g["kpages"], g["vpages"], g["page_table"], g["ctx_lens"], out=o_ws, lse=l_ws)
        o_na = torch.full_like(o_ws, float("nan"))
        l_na = torch.full_like(l_ws, float("nan"))
        fa_decode_paged_noalloc(g["q"], g["kpages"], g["vpages"], g["page_table"], g["ctx_lens"], o_na, l_na)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws), f"call {i}: O differs from the workspace entry point"
        assert torch.equal(torch.nan_to_num(l_na), torch.nan_to_num(l_ws)), f"call {i}: L differs"
        Oref, Lref = decode_ref(f64(x["q"]), x["kpages"].float().numpy(), x["vpages"].float().numpy(),
                                x["page_table"].numpy(), x["ctx_lens"].numpy(), 1.0 / np.sqrt(d))
        check_bf16(o_na, l_na, Oref, Lref, f"no-alloc call {i}")


def test_noalloc_rejects_sizes_past_the_scratch():
    from exact_io_aware_15_amd import FAError

    cap = fa_decode_paged_noalloc_max_scratch()
    # 64 sequences x 32 heads x 128 pages per split: maxp such that the partials exceed the scratch
    S, Hq, d = 64, 32, 128
    maxp = 128
    while fa_decode_paged_workspace_size(S, Hq, d, maxp) <= cap:
        maxp *= 2
    x = make_decode(S, Hq, 8, d, seed=73, fixed_ctx=tuple([16] * S))
    g = to_dev(x)
    table = torch.zeros((S, maxp), dtype=torch.int32, device=DEV)
    o = torch.empty((S, Hq, d), dtype=torch.bfloat16, device=DEV)
    l = torch.empty((S, Hq), dtype=torch.float32, device=DEV)
    with pytest.raises(FAError) as e:
        fa_decode_paged_noalloc(g["q"], g["kpages"], g["vpages"], table, g["ctx_lens"], o, l)
    assert e.value.status == 8
