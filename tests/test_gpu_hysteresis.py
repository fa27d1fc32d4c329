"""GPU parity: the loss-scale update with hysteresis, floor and growth
window (gs_update_scale_hysteresis) through the C ABI against the oracle,
state for state (S bits, tracker, hysteresis budget, skip count, flag)."""
import numpy as np
import pytest
import torch

import loss_scaling_fp8_amd as gs
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


class Dev:
    def __init__(self, S, H, dev):
        self.S = torch.tensor([S], dtype=torch.float32, device=dev)
        self.t = torch.zeros(1, dtype=torch.int32, device=dev)
        self.h = torch.tensor([H], dtype=torch.int32, device=dev)
        self.f = torch.zeros(1, dtype=torch.int32, device=dev)
        self.k = torch.zeros(1, dtype=torch.int64, device=dev)

    def state(self):
        torch.cuda.synchronize()
        return (int(self.S.view(torch.int32).item()), int(self.t.item()), int(self.h.item()),
                int(self.k.item()), int(self.f.item()))


def _ref_state(st):
    return (int(np.float32(st.S).view(np.int32)), st.tracker.value, st.h.value, st.skips.value,
            st.found_inf.value)


CONFIGS = [
    # (S0, growth, backoff, window, H, consecutive, min_scale, p_overflow, steps)
    (65536.0, 2.0, 0.5, 1000, 2, False, 1.0, 0.001, 10000),    # the page's constants
    (65536.0, 2.0, 0.5, 1000, 2, True, 1.0, 0.01, 10000),
    (1024.0, 2.0, 0.5, 7, 3, False, 0.25, 0.3, 5000),
    (1024.0, 2.0, 0.5, 7, 3, True, 0.25, 0.6, 5000),
    (3.0, 4.0, 0.25, 2, 1, False, 0.0, 0.5, 3000),             # non-power-of-two S, other factors
    (2.0 ** 100, 2.0, 0.5, 5, 4, False, 2.0 ** 90, 0.95, 3000),
]


@pytest.mark.parametrize("cfg", CONFIGS, ids=[str(i) for i in range(len(CONFIGS))])
def test_random_sequences_match_oracle(dev, cfg):
    S0, g, b, w, H, c, m, p, n = cfg
    flags = np.random.default_rng(int(p * 1e4) + w).random(n) < p
    D = Dev(S0, H, dev)
    R = oracle.HysteresisState(S0, h=H)
    fl = torch.from_numpy(flags.astype(np.int32)).to(dev)
    for i in range(n):
        D.f.copy_(fl[i:i + 1])
        gs.gs_update_scale_hysteresis(D.S, D.t, D.h, D.f, g, b, w, H, c, m, D.k)
        R.found_inf.value = int(flags[i])
        oracle.update_scale_hysteresis(R, g, b, w, H, c, m)
        if i % 97 == 0:
            assert D.state() == _ref_state(R), (cfg, i)
    assert D.state() == _ref_state(R), cfg


def test_collapse_to_floor_and_reduction_on_device(dev):
    """Every step overflows: S holds for one step (budget), halves 16 times
    to the floor 1 and stays; with hysteresis 1 and no floor the update is
    gs_update_scale's, step for step."""
    D = Dev(65536.0, 2, dev)
    seen = []
    for _ in range(40):
        D.f.fill_(1)
        gs.gs_update_scale_hysteresis(D.S, D.t, D.h, D.f, skip_count=D.k)
        seen.append(float(D.S.item()))
    assert seen[0] == 65536.0 and seen[1:17] == [2.0 ** (15 - k) for k in range(16)]
    assert set(seen[16:]) == {1.0} and D.state()[3] == 40
    rng = np.random.default_rng(3)
    A, B = Dev(65536.0, 1, dev), Dev(65536.0, 1, dev)
    for i in range(3000):
        v = int(rng.random() < 0.05)
        A.f.fill_(v)
        B.f.fill_(v)
        gs.gs_update_scale_hysteresis(A.S, A.t, A.h, A.f, 2.0, 0.5, 50, 1, False, 0.0, A.k)
        gs.gs_update_scale(B.S, B.t, B.f, 2.0, 0.5, 50, B.k)
    a, b = A.state(), B.state()
    assert (a[0], a[1], a[3]) == (b[0], b[1], b[3])


def test_errors_leave_no_side_effects(dev):
    D = Dev(8.0, 2, dev)
    D.f.fill_(1)
    for kw in (dict(hysteresis=0), dict(min_scale=-1.0), dict(growth_interval=0),
               dict(backoff_factor=float("nan"))):
        with pytest.raises(gs.GSError):
            gs.gs_update_scale_hysteresis(D.S, D.t, D.h, D.f, **kw)
    assert D.state() == (int(np.float32(8.0).view(np.int32)), 0, 2, 0, 1)
