"""CPU checks of the fp64 oracle against the pages' worked examples, closed forms,
invariants, brute-force finite differences and library special cases."""
import pytest

from tests.oracle_pins import ALL_PINS, oracle_impl


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle_impl())


def test_batched_matches_per_head():
    """attn_ref_fwd / attn_ref_bwd over [B,H,N,d] equal the per-head functions,
    with each batch entry using its own valid length."""
    import numpy as np
    import oracle
    from attn_inputs import make_inputs
    x = make_inputs(2, 3, 10, 4, seed=5, with_grad=True, seqlen_range=(3, 10))
    o, lse = oracle.attn_ref_fwd(x["q"], x["k"], x["v"], 0.5, True, x["seqlens"])
    dq, dk, dv = oracle.attn_ref_bwd(x["q"], x["k"], x["v"], x["do"], 0.5, True, x["seqlens"])
    for b in range(2):
        L = int(x["seqlens"][b])
        for h in range(3):
            oh, lh = oracle.attn_ref_head(x["q"][b, h], x["k"][b, h], x["v"][b, h], 0.5, True, L)
            assert np.array_equal(o[b, h], oh) and np.array_equal(lse[b, h], lh)
            g = oracle.attn_ref_bwd_head(x["q"][b, h], x["k"][b, h], x["v"][b, h],
                                         x["do"][b, h], 0.5, True, L)
            assert np.array_equal(dq[b, h], g[0]) and np.array_equal(dk[b, h], g[1])
            assert np.array_equal(dv[b, h], g[2])
            rows = [0, L - 1, 9]
            orow, lrow = oracle.attn_ref_rows(x["q"], x["k"], x["v"], b, h, rows, 0.5, True,
                                              x["seqlens"])
            assert np.array_equal(orow, oh[rows]) and np.array_equal(lrow, lh[rows])


def test_inputs_are_seeded_and_bf16_exact():
    """The generator is deterministic and the bf16 values upcast exactly."""
    import numpy as np
    import torch
    from attn_inputs import make_inputs
    a = make_inputs(1, 2, 8, 4, torch.bfloat16, seed=3, seqlen_range=(2, 8))
    b = make_inputs(1, 2, 8, 4, torch.bfloat16, seed=3, seqlen_range=(2, 8))
    assert torch.equal(a["q"], b["q"]) and torch.equal(a["seqlens"], b["seqlens"])
    from oracle.attention import _f64
    assert np.array_equal(_f64(a["q"]), a["q"].to(torch.float64).numpy())
