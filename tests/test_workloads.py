"""The seeded input generator: determinism, layout and poison placement (CPU only)."""

import numpy as np
import torch

from exact_io_aware_15_amd.workloads import CONFIGS, make_decode, make_prefill


def test_prefill_deterministic_and_rounded():
    a = make_prefill(1, 2, 1, 33, 64, "bf16", seed=3, value_scale=0.5)
    b = make_prefill(1, 2, 1, 33, 64, "bf16", seed=3, value_scale=0.5)
    for n in "qkv":
        assert a[n].dtype == torch.bfloat16 and torch.equal(a[n], b[n])
    assert a["q"].shape == (1, 2, 33, 64) and a["k"].shape == (1, 1, 33, 64)
    # the value scale is applied before rounding: 0.5 * N(0,1) has std ~0.5
    assert 0.4 < a["q"].float().std().item() < 0.6


def test_mqa_variant_shares_q_with_gqa():
    g = CONFIGS["c4_bf16_causal_gqa_B2_Hq32_Hkv8_N4096_d128"]
    m = CONFIGS["c4_bf16_causal_mqa_B2_Hq32_Hkv1_N4096_d128"]
    assert g.seed == m.seed and (g.B, g.Hq, g.N, g.d) == (m.B, m.Hq, m.N, m.d)
    a = make_prefill(1, 4, 2, 16, 8, seed=g.seed)
    b = make_prefill(1, 4, 1, 16, 8, seed=m.seed)
    assert torch.equal(a["q"], b["q"])


def test_decode_layout_and_poison():
    lens = (1, 16, 17, 40, 0)
    x = make_decode(5, 4, 2, 8, seed=9, page_size=16, fixed_ctx=lens)
    table = x["page_table"].numpy()
    P = x["num_pages"] - 1
    used = []
    for s, n in enumerate(lens):
        npg = -(-n // 16)
        used.extend(table[s, :npg].tolist())
        assert np.all(table[s, npg:] == P)
    assert sorted(used) == list(range(P))  # each real page owned exactly once
    kp = x["kpages"].float().numpy()
    assert np.all(np.isnan(kp[P]))
    for s, n in enumerate(lens):
        if n % 16:
            last = table[s, -(-n // 16) - 1]
            assert np.all(np.isnan(kp[last, :, n % 16:]))
            assert np.all(np.isfinite(kp[last, :, : n % 16]))
    assert x["ctx_lens"].dtype == torch.int32 and x["page_table"].dtype == torch.int32


def test_decode_context_draw_in_range():
    x = make_decode(64, 4, 1, 8, ctx_lo=1024, ctx_hi=16384, seed=5, page_size=16, max_pages_per_seq=1024)
    c = x["ctx_lens"].numpy()
    assert c.min() >= 1024 and c.max() <= 16384
    assert x["page_table"].shape == (64, 1024)
