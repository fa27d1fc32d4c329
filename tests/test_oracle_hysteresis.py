"""Pins of the oracle's second scaler policy (hysteresis, consecutive
hysteresis, min_loss_scale, window), "Numerical Precision, Mixed Precision,
and Loss Scaling", loss-scaler constants paragraph: the DeepSpeed fp16 block
starts at 2^16 like GradScaler, grows after a 1000-step window, and has
hysteresis 2, consecutive_hysteresis false and min_loss_scale 1.  The page
prints no trajectory for it; the pins are the reduction to the GradScaler
policy (pinned by the page trace), closed forms, and the two statements the
page makes when it compares the policies."""
import numpy as np
import pytest

import oracle

DS = dict(growth=2.0, backoff=0.5, window=1000, hysteresis=2, consecutive=False, min_scale=1.0)


def _run(flags, S0=65536.0, **kw):
    cfg = dict(DS, **kw)
    st = oracle.HysteresisState(S0, h=cfg["hysteresis"])
    traj = []
    for f in flags:
        st.found_inf.value = int(f)
        oracle.update_scale_hysteresis(st, **cfg)
        traj.append((float(st.S), st.tracker.value, st.h.value, st.skips.value))
    return traj


def _run_pt(flags, S0=65536.0, interval=2000):
    st = oracle.ScalerState(S0)
    traj = []
    for f in flags:
        st.found_inf.value = int(f)
        oracle.update_scale(st, 2.0, 0.5, interval)
        traj.append((float(st.S), st.tracker.value, st.skips.value))
    return traj


@pytest.mark.parametrize("p,interval", [(0.001, 2000), (0.02, 50), (0.3, 3), (0.9, 7)])
def test_reduces_to_gradscaler_policy(p, interval):
    """Hysteresis 1 and no floor (min_scale 0) is the GradScaler policy,
    whose oracle is pinned by the page's trace and closed forms."""
    flags = np.random.default_rng(int(p * 1000)).random(6000) < p
    a = _run(flags, window=interval, hysteresis=1, min_scale=0.0)
    b = _run_pt(flags, interval=interval)
    assert [(s, t, k) for s, t, _, k in a] == b


def test_page_trace_through_the_reduction():
    """The 5-step trace of "Loss scaling, FP8, and the failure that never
    crashes" (init 1024, interval 3, Inf at step 4)."""
    traj = _run([0, 0, 0, 1, 0], S0=1024.0, window=3, hysteresis=1, min_scale=0.0)
    assert [s for s, *_ in traj] == [1024.0, 1024.0, 2048.0, 1024.0, 1024.0]


def test_every_step_overflows_collapses_to_the_floor():
    """From 2^16 with hysteresis 2: the first overflow only spends the
    budget, each later one halves, S reaches min_loss_scale 1 at step 17 and
    stays there; every step is skipped."""
    traj = _run([1] * 40)
    S = [s for s, *_ in traj]
    assert S[0] == 65536.0
    assert S[1:17] == [2.0 ** (15 - k) for k in range(16)]
    assert all(s == 1.0 for s in S[16:])
    assert traj[-1][3] == 40


def test_no_floor_collapses_like_gradscaler_but_one_step_later():
    traj = _run([1] * 200, min_scale=0.0)
    S = [s for s, *_ in traj]
    assert S[165] == 2.0 ** -149 and S[166] == 0.0          # one later than GradScaler's 165/166 (0-based 164/165)


@pytest.mark.parametrize("consecutive", [False, True])
def test_alternating_overflow_and_clean(consecutive):
    """Overflow, clean, overflow, ...: with consecutive hysteresis the clean
    step refills the budget and S never drops; without it the budget stays
    spent and S halves at every overflow after the first."""
    traj = _run([1, 0] * 20, consecutive=consecutive)
    S = [s for s, *_ in traj]
    if consecutive:
        assert set(S) == {65536.0}
    else:
        assert S[0] == S[1] == 65536.0
        for k in range(1, 17):
            assert S[2 * k] == S[2 * k + 1] == 2.0 ** (16 - k)
        assert S[-1] == 1.0
    assert traj[-1][3] == 20


def test_growth_every_window_refills_the_budget():
    """Clean steps double S every 1000 steps; an isolated overflow spends
    the budget (S kept) and restarts the window; the next growth refills
    it, so a later isolated overflow again keeps S."""
    flags = [0] * 2500 + [1] + [0] * 1000 + [1] + [0] * 10
    traj = _run(flags)
    S = [s for s, *_ in traj]
    assert S[998] == 65536.0 and S[999] == 131072.0 and S[1999] == 262144.0
    assert traj[2500] == (262144.0, 0, 1, 1)         # kept, budget spent
    assert traj[3500] == (524288.0, 0, 2, 1)         # 1000 clean steps: growth, refill
    assert traj[3501] == (524288.0, 0, 1, 2)         # isolated overflow keeps S again


def test_growth_twice_as_eager_as_gradscaler():
    """The page's comparison: with a window half GradScaler's 2000-step
    interval, this policy tries a larger scale twice as often."""
    flags = [0] * 6000
    ds = _run(flags)
    pt = _run_pt(flags)
    assert ds[-1][0] == 2.0 ** 22 and pt[-1][0] == 2.0 ** 19


def test_skip_rate_differs_from_the_same_start():
    """The page's other comparison: moving a training setup from one policy
    to the other changes how often steps are skipped, even from the same
    starting scale.  Model: a step overflows exactly when S >= 2^17.
    GradScaler: 2000 clean + 1 skipped per cycle; the hysteresis-2 policy:
    1000 clean + 2 skipped per cycle."""
    def simulate(update, st, n):
        skips = 0
        for _ in range(n):
            st.found_inf.value = int(float(st.S) >= 2.0 ** 17)
            skips += st.found_inf.value
            update(st)
        return skips
    n = 30000
    pt = simulate(lambda st: oracle.update_scale(st, 2.0, 0.5, 2000), oracle.ScalerState(65536.0), n)
    ds = simulate(lambda st: oracle.update_scale_hysteresis(st, **DS),
                  oracle.HysteresisState(65536.0, h=2), n)
    # GradScaler overflows at steps 2000 + 2001k (0-based); the other policy
    # at 1000 + 1002k and 1001 + 1002k
    assert pt == n // 2001 == 14
    assert ds == 2 * ((n - 1000) // 1002) + min(2, (n - 1000) % 1002) == 58
