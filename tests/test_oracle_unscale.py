"""Pins of the oracle's fused unscale + non-finite check and of the
grow/backoff scale state machine (CPU only)."""
import numpy as np
import pytest

import oracle
from conftest import load_golden


def _floats(s):
    return [float(v) for v in s.split(",")]


# ------------------------------------------------------------------ unscale
def test_worked_example_1e8_via_1024():
    """'Loss scaling, FP8, and the failure that never crashes', worked
    example: 1e-8 vanishes in FP16, survives scaled by 1024, and the FP32
    division by 1024 recovers 1.0011717677116394e-08."""
    g = load_golden("worked_example_1e-8.txt")
    grad = np.float32(float(g["gradient"]))
    S = float(g["scale"])
    direct = np.float16(grad)                       # numpy's IEEE half cast
    scaled = np.float16(grad * np.float32(S))
    assert float(direct) == float(g["unscaled_fp16"])
    assert float(scaled) == float(g["scaled_fp16"])
    assert scaled.view(np.uint16) == 0x00AC          # an FP16 subnormal
    outs, found = oracle.unscale_check([np.array([scaled]).view(np.uint16)], S)
    assert float(outs[0][0]) == float(g["recovered_fp32"])
    assert found == 0


def test_precision_py_scaled_roundtrip():
    """'Mixed precision and FP8 training', precision.py: [1e-8, 1e-6, 2e-5]
    stored in FP16 after x2^16 and divided back."""
    g = load_golden("precision_py.txt")
    grads = np.array(_floats(g["gradients"]), np.float32)
    S = float(g["scale"])
    direct = grads.astype(np.float16)
    assert direct.astype(np.float64).tolist() == _floats(g["fp16_direct"])
    stored = (grads * np.float32(S)).astype(np.float16)
    outs, found = oracle.unscale_check([stored], S)
    assert outs[0].astype(np.float64).tolist() == _floats(g["scaled_recovered"])
    assert found == 0
    # with S = 1 the oracle returns the plain widening (first printed row)
    outs1, _ = oracle.unscale_check([direct], 1.0)
    assert outs1[0].astype(np.float64).tolist() == _floats(g["fp16_direct"])


SCALES = [2.0 ** k for k in range(-20, 41)] + [3.0, 1000.0, 65535.0, 1e-30, 7e-39, 1e-45,
                                               3.0e38, np.inf, 0.0]


@pytest.mark.parametrize("S", SCALES)
def test_unscale_all_fp16_patterns_vs_numpy(S):
    """Every FP16 bit pattern against numpy's float16->float32 widening and
    float32 multiply by float32(1/S); NaN outputs canonical; flag set iff
    some output is not finite."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    outs, found = oracle.unscale_check([h], S)
    o = outs[0]
    with np.errstate(all="ignore"):
        inv = np.float32(1.0) / np.float32(S) if S != 0 else np.float32(np.inf)
        ref = h.view(np.float16).astype(np.float32) * inv
    nan = np.isnan(ref)
    assert np.array_equal(o[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert (o[nan].view(np.uint32) == oracle.CANONICAL_NAN_BITS).all()
    assert found == int(not np.isfinite(ref).all())


def test_unscale_seeded_nonpower_scales():
    rng = np.random.default_rng(77)
    h = rng.integers(0, 65536, size=1 << 16, dtype=np.uint32).astype(np.uint16)
    for S in rng.uniform(1.0, 1e6, size=200).astype(np.float32):
        outs, _ = oracle.unscale_check([h], float(S))
        with np.errstate(all="ignore"):
            ref = h.view(np.float16).astype(np.float32) * (np.float32(1) / S)
        ok = ~np.isnan(ref)
        assert np.array_equal(outs[0][ok].view(np.uint32), ref[ok].view(np.uint32))


def test_found_inf_is_set_only_and_list_semantics():
    good = np.float16([1.0, -2.0, 0.5])
    bad = np.float16([1.0, np.inf, 3.0])
    nan = np.float16([np.nan])
    empty = np.zeros(0, np.float16)
    assert oracle.unscale_check([good, empty, good], 1024.0)[1] == 0
    assert oracle.unscale_check([good, empty, bad], 1024.0)[1] == 1
    assert oracle.unscale_check([nan], 1024.0)[1] == 1
    # a flag raised by an earlier call in the same step is never cleared
    assert oracle.unscale_check([good], 1024.0, found_inf=1)[1] == 1
    # an empty list leaves the flag as it was
    assert oracle.unscale_check([], 1024.0)[1] == 0
    # overflow of the product itself (S tiny) counts as non-finite
    assert oracle.unscale_check([np.float16([60000.0])], 1e-38)[1] == 1
    outs, _ = oracle.unscale_check([good, empty, good], 2.0)
    assert outs[1].size == 0 and outs[2].tolist() == [0.5, -1.0, 0.25]


# ------------------------------------------------------------------ state machine
def _run(init, growth, interval, inf_steps, n_steps):
    st = oracle.ScalerState(init)
    hist = []
    for step in range(1, n_steps + 1):
        grads = [np.float16([1.0, -0.5])]
        if step in inf_steps:
            grads.append(np.float16([np.inf]))
        _, st.found_inf.value = oracle.unscale_check(grads, float(st.S), st.found_inf.value)
        skipped = bool(st.found_inf.value)
        oracle.update_scale(st, growth, 0.5, interval)
        hist.append((float(st.S), "skipped" if skipped else "applied"))
    return st, hist


def test_page_trace_interval3_inf_at_step4():
    """'Loss scaling, FP8, and the failure that never crashes': the printed
    5-step trace of SimpleGradScaler."""
    g = load_golden("scaler_trace.txt")
    st, hist = _run(float(g["init_scale"]), float(g["growth_factor"]),
                    int(g["growth_interval"]), {int(g["inf_steps"])}, 5)
    assert [h[0] for h in hist] == _floats(g["scale_after_step"])
    assert [h[1] for h in hist] == [s.strip() for s in g["status"].split(",")]


def test_tiny_case_trajectory_closed_form():
    """65536 start, default policy, overflow at steps 3, 7 and 20 of 50:
    three halvings, no growth (the longest clean run, 30 steps, is far below
    2000), tracker = steps since the last skip."""
    st, hist = _run(65536.0, 2.0, 2000, {3, 7, 20}, 50)
    assert float(st.S) == 65536.0 / 8 and st.tracker.value == 30 and st.skips.value == 3
    assert [h[0] for h in hist][:8] == [65536.0] * 2 + [32768.0] * 4 + [16384.0] * 2


def test_collapse_reaches_zero_at_step_166():
    """Overflow every step from 2^16: S = 2^(16-k) after k steps; the
    smallest FP32 subnormal 2^-149 is reached at k = 165 and the next
    halving rounds 2^-150 to 0 (a tie, to even).  A flush-to-zero model
    would reach 0 at k = 143."""
    st = oracle.ScalerState(65536.0)
    k_zero = None
    for k in range(1, 200):
        st.found_inf.value = 1
        oracle.update_scale(st)
        if float(st.S) == 0.0 and k_zero is None:
            k_zero = k
        if k == 165:
            assert float(st.S) == 2.0 ** -149
    assert k_zero == 166 and st.skips.value == 199
    # a stuck S = 0 flags every later step: 1/S = Inf, 0 * Inf = NaN
    assert oracle.unscale_check([np.float16([0.0, 1.0])], float(st.S))[1] == 1


def test_growth_overflows_to_inf_at_step_112():
    """Never an overflow, interval 1: S = 2^(16+k); 2^127 at k = 111 and the
    112th doubling rounds to +Inf (no clamp in the policy)."""
    st = oracle.ScalerState(65536.0)
    for k in range(1, 113):
        oracle.update_scale(st, 2.0, 0.5, 1)
        if k == 111:
            assert float(st.S) == 2.0 ** 127
    assert float(st.S) == np.inf
    # S = Inf makes every output 0 (1/Inf = 0) and the check stays clean
    outs, found = oracle.unscale_check([np.float16([5.0])], float(st.S))
    assert found == 0 and outs[0][0] == 0.0


def test_random_injection_10000_steps_closed_form():
    """'Try it yourself', intermediate exercise: 10,000 steps with a 0.1%
    random Inf rate.  Closed form: every clean run of length L contributes
    floor(L / interval) doublings, every Inf one halving, so
    log2(S_final) = 16 + sum(floor(L_i / 2000)) - (#Inf steps), and the
    tracker ends at (length of the last clean run) mod 2000."""
    rng = np.random.default_rng(2024)
    inf = rng.random(10000) < 0.001
    st = oracle.ScalerState(65536.0)
    for flag in inf:
        st.found_inf.value = int(flag)
        oracle.update_scale(st)
    # clean run lengths between Inf steps
    runs, cur = [], 0
    for flag in inf:
        if flag:
            runs.append(cur)
            cur = 0
        else:
            cur += 1
    runs.append(cur)
    expect_log2 = 16 + sum(L // 2000 for L in runs) - int(inf.sum())
    assert float(st.S) == 2.0 ** expect_log2
    assert st.tracker.value == runs[-1] % 2000
    assert st.skips.value == int(inf.sum())


def test_checkpoint_restore_identical_trajectory():
    rng = np.random.default_rng(5)
    flags = rng.random(3000) < 0.01
    a = oracle.ScalerState(65536.0)
    for f in flags[:1000]:
        a.found_inf.value = int(f)
        oracle.update_scale(a, 2.0, 0.5, 50)
    saved = (float(a.S), a.tracker.value)
    for f in flags[1000:]:
        a.found_inf.value = int(f)
        oracle.update_scale(a, 2.0, 0.5, 50)
    b = oracle.ScalerState(saved[0], saved[1])
    for f in flags[1000:]:
        b.found_inf.value = int(f)
        oracle.update_scale(b, 2.0, 0.5, 50)
    assert (float(a.S), a.tracker.value) == (float(b.S), b.tracker.value)
