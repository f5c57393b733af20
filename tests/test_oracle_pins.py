"""CPU tests: the oracle against its pins (closed forms, library routines, brute force, invariants)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_selected_expert_oracle_equals_full_oracle():
    """The oracle over a layer whose stacks hold only the routed experts gives the
    same result, bit for bit, as over the complete stacks."""
    import numpy as np
    import moe_inputs as mi
    import oracle
    from helpers import oracle_layer_selected, pick_tokens
    for cfg in (mi.TINY, mi.LayerConfig("sel", 61, 61, d_in=256, d_ff=192, n_experts=9, top_k=3,
                                        renormalize=False, bits_gate_up=4, bits_down=6,
                                        sb_dtype=mi.BF16, x_dtype=mi.BF16, router_dtype=mi.BF16,
                                        resid_dtype=mi.BF16, n_shared=1, d_ff_shared=128,
                                        shared_gate=True)):
        w = mi.gen_layer_weights(cfg, 2, threads=2)
        x, resid, _ = pick_tokens(cfg, 2, 3, w["router"])
        full = oracle.layer(cfg, w, x, resid)
        sel = oracle_layer_selected(cfg, 2, x, resid)
        assert np.array_equal(full["route"]["ids"], sel["route"]["ids"])
        assert np.array_equal(full["out"], sel["out"])
        assert np.array_equal(full["ffn"]["act"], sel["ffn"]["act"])
