"""Checkpoint and resume of the device-resident state, bit for bit.

The scaler state is part of a training run's state: a run that saves it after
k steps and resumes from the saved values must continue exactly as the
uninterrupted run.  For each state machine -- the GradScaler update (S,
tracker, skip count), the hysteresis policy (S, tracker, budget, skip count)
and delayed FP8 scaling (next scale, amax history ring, position) -- the
device run is interrupted after k steps, its state copied to the host, and a
fresh set of device buffers restored from the copy replays the remaining
steps.  Both continuations and the oracle's uninterrupted run agree bit for
bit (the delayed case also compares every step's codes and scale)."""
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


def _bits(t):
    a = t.detach().cpu().numpy()
    return a.view(np.uint32 if a.dtype.itemsize == 4 else np.uint64).tolist()


def _snapshot(tensors):
    torch.cuda.synchronize()
    return [t.detach().cpu().clone() for t in tensors]


def _restore(snap, dev):
    return [t.to(dev) for t in snap]


def test_gradscaler_state_resume(dev):
    rng = np.random.default_rng(601)
    flags = rng.random(3000) < 0.01
    k, interval = 1200, 50
    S = torch.tensor([65536.0], dtype=torch.float32, device=dev)
    tr = torch.zeros(1, dtype=torch.int32, device=dev)
    sk = torch.zeros(1, dtype=torch.int64, device=dev)
    fi = torch.zeros(1, dtype=torch.int32, device=dev)

    def run(state, fl):
        s_, t_, k_ = state
        for f in fl:
            if f:
                fi.fill_(1)
            gs.gs_update_scale(s_, t_, fi, 2.0, 0.5, interval, k_)

    run((S, tr, sk), flags[:k])
    snap = _snapshot([S, tr, sk])
    run((S, tr, sk), flags[k:])
    restored = _restore(snap, dev)
    run(restored, flags[k:])
    torch.cuda.synchronize()
    ref = oracle.ScalerState(65536.0)
    for f in flags:
        ref.found_inf.value = int(f)
        oracle.update_scale(ref, 2.0, 0.5, interval)
    a = (_bits(S), _bits(tr), _bits(sk))
    b = tuple(_bits(t) for t in restored)
    assert a == b
    assert np.float32(S.item()).view(np.uint32) == ref.S.view(np.uint32)
    assert (int(tr.item()), int(sk.item())) == (ref.tracker.value, ref.skips.value)
    assert int(fi.item()) == 0


@pytest.mark.parametrize("consecutive", [False, True])
def test_hysteresis_state_resume(dev, consecutive):
    rng = np.random.default_rng(602 + int(consecutive))
    flags = rng.random(4000) < 0.05
    k, window, H, floor = 1700, 40, 3, 1.0
    S = torch.tensor([65536.0], dtype=torch.float32, device=dev)
    tr = torch.zeros(1, dtype=torch.int32, device=dev)
    h = torch.full((1,), H, dtype=torch.int32, device=dev)
    sk = torch.zeros(1, dtype=torch.int64, device=dev)
    fi = torch.zeros(1, dtype=torch.int32, device=dev)

    def run(state, fl):
        s_, t_, h_, k_ = state
        for f in fl:
            if f:
                fi.fill_(1)
            gs.gs_update_scale_hysteresis(s_, t_, h_, fi, 2.0, 0.5, window, H, consecutive,
                                          floor, k_)

    run((S, tr, h, sk), flags[:k])
    snap = _snapshot([S, tr, h, sk])
    run((S, tr, h, sk), flags[k:])
    restored = _restore(snap, dev)
    run(restored, flags[k:])
    torch.cuda.synchronize()
    ref = oracle.HysteresisState(65536.0, 0, H)
    for f in flags:
        ref.found_inf.value = int(f)
        oracle.update_scale_hysteresis(ref, 2.0, 0.5, window, H, consecutive, floor)
    assert (_bits(S), _bits(tr), _bits(h), _bits(sk)) == tuple(_bits(t) for t in restored)
    assert np.float32(S.item()).view(np.uint32) == ref.S.view(np.uint32)
    assert (int(tr.item()), int(h.item()), int(sk.item())) == \
        (ref.tracker.value, ref.h.value, ref.skips.value)


def test_delayed_scaling_state_resume(dev):
    rng = np.random.default_rng(603)
    steps, k, hlen = 12, 5, 4
    xs = []
    for t in range(steps):
        x = rng.standard_normal((256, 512)).astype(np.float32) * np.float32(2.0 ** (t % 5 - 2))
        if t == 6:
            x[17, 33] = 3.0e4                       # a spike after steady steps
        xs.append(((x.view(np.uint32) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16))
    st = torch.ones(1, dtype=torch.float32, device=dev)
    hist = torch.zeros(hlen, dtype=torch.float32, device=dev)
    pos = torch.zeros(1, dtype=torch.int32, device=dev)

    def run(state, xs_):
        s_, h_, p_ = state
        out = []
        for xh in xs_:
            x = torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16).to(dev)
            codes, used = gs.fp8_quantize_delayed(x, gs.FP8_E4M3, s_, h_, p_)
            out.append((codes.cpu().numpy(), np.float32(used.item()).view(np.uint32)))
        return out

    run((st, hist, pos), xs[:k])
    snap = _snapshot([st, hist, pos])
    a = run((st, hist, pos), xs[k:])
    restored = _restore(snap, dev)
    b = run(restored, xs[k:])
    ref = oracle.DelayedState(hlen, 1.0)
    r = [oracle.quantize_delayed(xh, gs.FP8_E4M3, ref) for xh in xs]
    for j, ((ca, ua), (cb, ub)) in enumerate(zip(a, b)):
        rc, ru, _ = r[k + j]
        assert np.array_equal(ca, cb) and ua == ub, j
        assert np.array_equal(ca, rc) and ua == np.float32(ru).view(np.uint32), j
    assert (_bits(st), _bits(hist), _bits(pos)) == tuple(_bits(t) for t in restored)
    assert _bits(st) == ref.scale.view(np.uint32).tolist()
    assert _bits(hist) == ref.history.view(np.uint32).tolist()
    assert int(pos.item()) == int(ref.pos[0])
