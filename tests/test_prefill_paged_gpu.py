"""GPU parity of the chunked prefill over a paged cache (fa_prefill_paged) against
the fp64 oracle, every element.  Bars as for the bf16 forward: O within 1e-2, L within
1e-3, with the bf16 output-floor rule of tests/_parity.py.  The page pools carry NaN in every slot past a sequence's context and in the
padding page, so a read past the context fails the check."""

import numpy as np
import pytest
import torch

from _parity import check_bf16, f64, say
from exact_io_aware_15_amd import fa_decode_paged, fa_prefill_paged
from exact_io_aware_15_amd.workloads import make_prefill_paged
from oracle import prefill_paged_ref

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run(x, scale=None):
    g = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in x.items()}
    S, Hq, C, d = x["q"].shape
    out = torch.full((S, Hq, C, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((S, Hq, C), float("nan"), dtype=torch.float32, device=DEV)
    fa_prefill_paged(g["q"], g["kpages"], g["vpages"], g["page_table"], g["ctx_lens"], scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def oracle(x, scale):
    return prefill_paged_ref(f64(x["q"]), x["kpages"].float().numpy(), x["vpages"].float().numpy(),
                             x["page_table"].numpy(), x["ctx_lens"].numpy(), scale)


CASES = [
    # S, Hq, Hkv, d, chunk, ctx lens
    (3, 4, 2, 128, 1, (1, 17, 100)),
    (4, 8, 2, 128, 37, (37, 100, 1000, 4099)),
    (2, 4, 1, 64, 256, (256, 300)),
    (2, 32, 8, 128, 300, (300, 5000)),
    (2, 2, 2, 128, 513, (513, 2049)),
    (3, 8, 1, 64, 64, (64, 65, 1024)),
    # the kernel runs the tiles below a block's causal boundary in a loop of their own
    # (an even number of them) and the rest in the general loop: boundaries at tiles 1,
    # 2, 5 and 6 (64-key tiles), so the first loop is empty, even and odd-rounded
    (2, 8, 2, 128, 300, (363, 427)),
    (2, 4, 2, 64, 200, (327, 711)),
    (2, 6, 2, 128, 100, (100, 700)),  # 3 query heads per K/V head
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"S{c[0]}_Hq{c[1]}_Hkv{c[2]}_d{c[3]}_C{c[4]}")
def test_prefill_paged_every_element(case):
    S, Hq, Hkv, d, C, lens = case
    say(f"chunked prefill {case}")
    x = make_prefill_paged(S, Hq, Hkv, d, C, 1, 64, seed=500 + C, fixed_ctx=lens)
    out, lse = run(x)
    Oref, Lref = oracle(x, 1.0 / np.sqrt(d))
    check_bf16(out, lse, Oref, Lref, str(case))


def test_prefill_paged_chunk_of_one_matches_decode():
    x = make_prefill_paged(6, 8, 2, 128, 1, 1, 3000, seed=77)
    g = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in x.items()}
    o1, l1 = run(x)
    o2, l2 = fa_decode_paged(g["q"][:, :, 0].contiguous(), g["kpages"], g["vpages"], g["page_table"], g["ctx_lens"])
    torch.cuda.synchronize()
    assert float((o1[:, :, 0].float() - o2.float()).abs().max()) <= 1e-2
    assert float((l1[:, :, 0] - l2).abs().max()) <= 1e-3


def test_prefill_paged_full_size():
    # 16 sequences, 512-token chunks, contexts 512 .. 16384, Hq32 Hkv8 d128: every element
    say("chunked prefill full size")
    x = make_prefill_paged(16, 32, 8, 128, 512, 512, 16384, seed=6)
    out, lse = run(x)
    Oref, Lref = oracle(x, 1.0 / np.sqrt(128))
    check_bf16(out, lse, Oref, Lref, "full size (16 x 512-token chunks)")
