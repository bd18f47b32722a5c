"""The CPU oracle against its pins (brute force, torch conv1d, closed forms, invariants)."""

import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.load())


def test_oracle_rejects_malformed_problems():
    import numpy as np
    import workloads

    wl = workloads.custom("bad", n_seq=2, d_inner=32, qk_channels=0, T=2, accept_offsets=True)
    inp = workloads.make_inputs(wl)
    for slot, nat in (([0, 2], [0, 0]), ([0, 1], [0, 2]), ([0, 1], [-1, 0])):
        inp.slot_idx = np.array(slot, np.int32)
        inp.num_accept_tokens = np.array(nat, np.int32)
        with pytest.raises(ValueError):
            oracle.run_inputs(inp)
    wl = workloads.custom("bad_pair", x_dtype="f32", state_dtype="bf16", T=2)
    with pytest.raises(ValueError):
        oracle.run_inputs(workloads.make_inputs(wl))
