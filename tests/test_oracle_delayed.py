"""Pins of the oracle's delayed per-tensor scaling ("Why FP8 training is
stable", Failure 1: the scale applied this step comes from a short history
of recent max-abs values).  The pages print no delayed-scaling numbers; the
pins are a reduction to the pinned per-tensor quantizer, the window's closed
form, and the failure shape the page describes."""
import numpy as np
import pytest

import oracle

E4M3, E5M2, PT = oracle.E4M3, oracle.E5M2, oracle.PER_TENSOR


def _x(seed, scale=1.0, shape=(64, 96)):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_history_one_same_tensor_twice_is_current_scaling(fmt):
    x = _x(1, 7.0)
    st = oracle.DelayedState(1, init_scale=0.25)
    c1, used1, _ = oracle.quantize_delayed(x, fmt, st)
    assert used1 == np.float32(0.25)
    ref1, _, _ = oracle.quantize(x, fmt, PT, oracle.GIVEN, np.float32([0.25]))
    assert np.array_equal(c1, ref1)                   # step 1: the initial scale
    c2, used2, _ = oracle.quantize_delayed(x, fmt, st)
    ref2, s2, _ = oracle.quantize(x, fmt, PT)         # current scaling of x
    assert used2.view(np.uint32) == s2[0].view(np.uint32)
    assert np.array_equal(c2, ref2)


def test_window_max_and_ring():
    """s for step t+1 = fl32(max(last H amaxes, 1e-12) / MAX); the ring
    overwrites the oldest entry."""
    H = 3
    amaxes = [2.0, 0.5, 8.0, 1.0, 0.25, 0.125, 4.0]
    st = oracle.DelayedState(H, init_scale=1.0)
    for t, a in enumerate(amaxes):
        x = np.zeros((4, 32), np.float32)
        x[1, 3] = -a
        _, used, _ = oracle.quantize_delayed(x, E4M3, st)
        window = amaxes[max(0, t - H + 1): t + 1]
        assert st.scale[0] == np.float32(max(window)) / np.float32(448.0)
        assert st.pos[0] == (t + 1) % H
        if t > 0:
            prev = amaxes[max(0, t - H): t]
            assert used == np.float32(max(prev)) / np.float32(448.0)


def test_empty_history_uses_the_floor():
    st = oracle.DelayedState(2, init_scale=1.0)
    oracle.quantize_delayed(np.zeros((2, 8), np.float32), E5M2, st)
    assert st.scale[0] == np.float32(1e-12) / np.float32(57344.0)


def test_spike_saturates_under_delayed_scaling():
    """The failure shape on the page: after steady steps, an unusually large
    activation meets a scale derived from the history and saturates, while
    current scaling of the same tensor would not."""
    st = oracle.DelayedState(4, init_scale=1.0)
    for k in range(5):
        oracle.quantize_delayed(_x(10 + k), E4M3, st)
    spike = _x(99)
    spike[3, :16] *= 100.0
    codes, used, _ = oracle.quantize_delayed(spike, E4M3, st)
    sat = np.count_nonzero((codes & 0x7F) == 0x7E)
    cur, _, _ = oracle.quantize(spike, E4M3, PT)
    # current scaling maps only the values within half an FP8 step of the amax to MAX
    assert sat >= 10 and np.count_nonzero((cur & 0x7F) == 0x7E) <= 3
    # and the next step's scale has caught up with the spike
    assert st.scale[0] == np.float32(np.abs(spike).max()) / np.float32(448.0)


def test_nonfinite_inputs_and_ring_position():
    x = _x(5)
    x[0, 0] = np.nan
    x[1, 1] = -np.inf
    st = oracle.DelayedState(2, init_scale=0.5)
    codes, _, nf = oracle.quantize_delayed(x, E4M3, st)
    assert nf == 1 and codes[0, 0] == 0x7F and codes[1, 1] == 0xFE
    assert st.history[0] == np.float32(np.abs(x[np.isfinite(x)]).max())
    # a position outside [0, H) is taken modulo H
    odd = oracle.DelayedState(3)
    odd.pos[0] = 7
    oracle.quantize_delayed(x, E4M3, odd)
    assert odd.pos[0] == 2 and odd.history[1] > 0 and odd.history[0] == 0
