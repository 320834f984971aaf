"""The FP64 oracle against what the pages and mathematics fix (CPU only)."""
import numpy as np
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_oracle_rejects_bad_arguments(orc):
    x, s0 = oracle_pins.rand_inputs(1, B=1, T=4, H=1, dk=2, dv=2)
    bad_cu = np.array([0, 3, 2], dtype=np.int32)         # decreasing offsets
    with pytest.raises(ValueError):
        orc.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], None, bad_cu)
    with pytest.raises(ValueError):
        orc.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], None, None, chains=[5])


def test_chain_subset_matches_full(orc):
    x, s0 = oracle_pins.rand_inputs(2, B=2, T=9, H=3)
    o, s = orc.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], s0)
    chains = [4, 1]
    oc, sc = orc.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], s0, chains=chains)
    for c in chains:
        n, h = divmod(c, 3)
        np.testing.assert_array_equal(oc[n, :, h], o[n, :, h])
        np.testing.assert_array_equal(sc[n, h], s[n, h])
    # chains not evaluated keep the initial state and zero outputs
    np.testing.assert_array_equal(sc[0, 0], s0[0, 0])
    assert not oc[0, :, 0].any()


def test_zero_length_sequences(orc):
    cu = np.array([0, 0, 3, 3], dtype=np.int32)
    x, _ = oracle_pins.rand_inputs(3, B=1, T=3, H=1, dk=4, dv=4, state=False)
    s0 = np.random.default_rng(0).standard_normal((3, 1, 4, 4))
    o, s = orc.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], s0, cu)
    np.testing.assert_array_equal(s[0], s0[0])            # empty sequence: state passes through
    np.testing.assert_array_equal(s[2], s0[2])


@pytest.mark.parametrize("pin", oracle_pins.BACKWARD_PINS, ids=lambda p: p.__name__)
def test_backward_pin(orc, pin):
    pin(orc)


def test_backward_chain_subset(orc):
    x, s0, g, gs = oracle_pins._bwd_inputs(46, B=2, T=7, H=3, dk=3, dv=2)
    full = orc.backward(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], g, s0, gs)
    part = orc.backward(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], g, s0, gs, chains=[4])
    n, h = divmod(4, 3)
    for key in ("dq", "dk", "dv", "dalpha", "db", "dw"):
        np.testing.assert_array_equal(part[key][n, :, h], full[key][n, :, h])
    np.testing.assert_array_equal(part["d_initial_state"][n, h], full["d_initial_state"][n, h])
