"""Pins of the oracle's exact gradient sum of squares (for norm clipping).
The pages print no norm values; the exact integer sum is pinned by Python's
arbitrary-precision integers, the FP64 norm by numpy float64 sums."""
import numpy as np
import pytest

import oracle


def _py_exact(grads):
    tot = 0
    for g in grads:
        f = np.asarray(g).view(np.float16).astype(np.float64)
        f = f[np.isfinite(f)]
        G = (np.abs(f) * 2.0 ** 24).astype(np.int64)          # exact: < 2^40
        tot += sum(int(v) * int(v) for v in G.tolist())
    return tot


@pytest.mark.parametrize("S", [65536.0, 1.0, 2.0 ** -10, 3.0])
def test_exact_integer_sum_and_norm(S):
    rng = np.random.default_rng(8)
    grads = [rng.integers(0, 0x7C00, n, dtype=np.uint32).astype(np.uint16) |
             (rng.integers(0, 2, n).astype(np.uint16) << 15) for n in (1, 77, 4096, 100000)]
    grads[2][5] = 0x7C00          # Inf and NaN are left out of the sum
    grads[3][9] = 0x7E01
    outs, found, (lo, hi), nsq = oracle.unscale_check_sumsq(grads, S)
    X = _py_exact(grads)
    assert (hi << 64) | lo == X and found == 1
    inv = np.float32(1.0) / np.float32(S)
    y = np.concatenate([o.astype(np.float64) for o in outs])
    y = y[np.isfinite(y)]
    ref = float(np.sum(y * y)) if S != 3.0 else float(X) * 2.0 ** -48 * float(inv) ** 2
    assert abs(nsq - ref) <= 1e-12 * ref


def test_accumulates_across_calls_and_fp16_extremes():
    a = np.array([0x7BFF, 0xFBFF, 0x0001, 0x8001, 0x0400], np.uint16)  # +-65504, +-2^-24, 2^-14
    _, _, acc1, _ = oracle.unscale_check_sumsq([a], 1.0)
    _, _, acc2, n2 = oracle.unscale_check_sumsq([a], 1.0, sumsq=acc1)
    X = _py_exact([a])
    assert (acc1[1] << 64) | acc1[0] == X
    assert (acc2[1] << 64) | acc2[0] == 2 * X
    assert n2 == float(2 * X) * 2.0 ** -48          # exact here
    # the largest possible square, 2^31 times, needs the upper word
    big = np.full(1 << 16, 0x7BFF, np.uint16)
    acc = (0, 0)
    for _ in range(4):
        _, _, acc, _ = oracle.unscale_check_sumsq([big], 1.0, sumsq=acc)
    assert (acc[1] << 64) | acc[0] == 4 * (1 << 16) * (65504 * 2 ** 24) ** 2
    assert acc[1] > 0


def test_round_to_nearest_even_conversion_of_the_total():
    """fl64 of the 128-bit total rounds to nearest even: 2^60 + 2^7 + 1 needs
    rounding (53 significant bits), checked against Python's int -> float."""
    target = (1 << 60) + (1 << 7) + 1
    # one FP16 value 1.0 contributes (2^24)^2 = 2^48; build the total through
    # the running-sum input instead
    _, _, acc, nsq = oracle.unscale_check_sumsq([np.zeros(0, np.uint16)], 1.0,
                                                sumsq=(target & (2**64 - 1), target >> 64))
    assert nsq == float(target) * 2.0 ** -48
    tie = (1 << 60) + (1 << 7)                          # exactly halfway: to even
    _, _, _, nsq2 = oracle.unscale_check_sumsq([np.zeros(0, np.uint16)], 1.0,
                                               sumsq=(tie, 0))
    assert nsq2 == float(tie) * 2.0 ** -48 == 2.0 ** 12
