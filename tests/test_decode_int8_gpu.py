"""GPU parity of the INT8 group-scaled paged decode against the fp64 oracle (the decode
definition on the dequantized cache), every element.  Bars as for the bf16 decode:
O within 1e-2, L within 1e-3, with the bf16 output-floor rule of tests/_parity.py.  Slots past each context and the padding page carry NaN
scales (and arbitrary int8 values), so any leak fails the check."""

import numpy as np
import pytest
import torch

from _parity import check_bf16, say
from exact_io_aware_15_amd import fa_decode_paged_int8
from exact_io_aware_15_amd.workloads import make_decode_int8
from oracle import decode_int8_ref

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run(x, scale=None):
    g = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in x.items()}
    S, Hq, d = x["q"].shape
    out = torch.full((S, Hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((S, Hq), float("nan"), dtype=torch.float32, device=DEV)
    fa_decode_paged_int8(g["q"], g["kq"], g["kscale"], g["vq"], g["vscale"], g["page_table"], g["ctx_lens"],
                         scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def check(x, out, lse, what):
    d = x["q"].shape[-1]
    Oref, Lref = decode_int8_ref(x["q"].double().numpy(), x["kq"].numpy(), x["kscale"].numpy(), x["vq"].numpy(),
                                 x["vscale"].numpy(), x["page_table"].numpy(), x["ctx_lens"].numpy(),
                                 1.0 / np.sqrt(d))
    check_bf16(out, lse, Oref, Lref, what)


CASES = [
    # S, Hq, Hkv, d, ctx lens
    (6, 4, 4, 128, (1, 15, 16, 17, 100, 513)),
    (5, 8, 2, 64, (0, 1, 511, 512, 1000)),
    (4, 32, 8, 128, (2048, 3, 16 * 32 + 1, 777)),
    (3, 16, 2, 128, (5, 70, 1600)),
    (3, 8, 1, 64, (33, 1, 64)),
    (2, 2, 1, 128, (16384, 9999)),
    (3, 6, 2, 128, (40, 17, 2100)),   # 3 query heads per K/V head: one of 4 head slots idle
    (2, 12, 2, 64, (300, 4097)),      # 6 per K/V head: two workgroups, the second half full
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"S{c[0]}_Hq{c[1]}_Hkv{c[2]}_d{c[3]}")
def test_decode_int8_every_element(case):
    S, Hq, Hkv, d, lens = case
    say(f"int8 decode {case}")
    x = make_decode_int8(S, Hq, Hkv, d, seed=600 + S, fixed_ctx=lens)
    out, lse = run(x)
    check(x, out, lse, str(case))


def test_decode_int8_full_size():
    # the c5 shapes: 64 sequences, Hq32 Hkv8 d128, contexts U[1024, 16384]
    say("int8 decode full size")
    x = make_decode_int8(64, 32, 8, 128, 1024, 16384, seed=5)
    out, lse = run(x)
    check(x, out, lse, "full size")


def test_decode_int8_query_magnitudes():
    # the key products run on fp16 q under a power-of-two scale per head: heads whose q
    # is large, tiny, zero or ordinary must all match the oracle
    say("int8 decode query magnitudes")
    x = make_decode_int8(3, 8, 2, 128, seed=640, fixed_ctx=(300, 17, 2000))
    q = x["q"].float()
    factors = torch.tensor([64.0, 2.0 ** -20, 0.0, 1.0, 2.0 ** -120, 16.0, 1.0, 0.5])
    x["q"] = (q * factors[None, :, None]).to(torch.bfloat16)
    out, lse = run(x)
    check(x, out, lse, "query magnitudes")
