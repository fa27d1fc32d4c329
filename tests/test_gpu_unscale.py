"""GPU parity: fused multi-tensor unscale + non-finite check and the device
scale update, through the C ABI, bit for bit against the oracle."""
import numpy as np
import pytest
import torch

import loss_scaling_fp8_amd as gs
import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _to_dev(h: np.ndarray, dev):
    return torch.from_numpy(np.ascontiguousarray(h).view(np.int16)).view(torch.float16).to(dev)


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint32)


class DevScaler:
    def __init__(self, S, dev):
        self.S = torch.tensor([S], dtype=torch.float32, device=dev)
        self.tracker = torch.zeros(1, dtype=torch.int32, device=dev)
        self.found = torch.zeros(1, dtype=torch.int32, device=dev)
        self.skips = torch.zeros(1, dtype=torch.int64, device=dev)

    def state(self):
        torch.cuda.synchronize()
        return (float(self.S.item()), int(self.tracker.item()), int(self.found.item()),
                int(self.skips.item()))


def test_tiny_gradset_50_step_trajectory(dev):
    """16 tensors, 2^20 elements, S = 65536; Inf at steps 3, 7 and NaN at 20:
    every output, the flag after every unscale and S / tracker / skips after
    every update equal the oracle's."""
    g = synth.tiny_gradset()
    host = [synth.as_u16_numpy(synth.to_f16_tensor(g.gen(t, torch.arange(sp.numel))))
            for t, sp in enumerate(g.tensors)]
    grads = [_to_dev(h, dev) for h in host]
    outs = [torch.empty(h.size, dtype=torch.float32, device=dev) for h in host]
    D = DevScaler(g.scale, dev)
    R = oracle.ScalerState(g.scale)
    for step in range(1, g.steps + 1):
        saved = []
        for (t, i, bits) in g.injections.get(step, []):
            saved.append((t, i, host[t][i]))
            host[t][i] = bits
            grads[t][i:i + 1] = _to_dev(np.array([bits], np.uint16), dev)
        gs.gs_unscale_check(grads, outs, D.S, D.found)
        ref, R.found_inf.value = oracle.unscale_check(host, float(R.S), R.found_inf.value)
        torch.cuda.synchronize()
        for t, (o, r) in enumerate(zip(outs, ref)):
            assert np.array_equal(_bits(o), r.view(np.uint32)), "step %d tensor %d" % (step, t)
        assert int(D.found.item()) == R.found_inf.value, step
        gs.gs_update_scale(D.S, D.tracker, D.found, 2.0, 0.5, 2000, D.skips)
        oracle.update_scale(R, 2.0, 0.5, 2000)
        assert D.state() == (float(R.S), R.tracker.value, 0, R.skips.value), step
        for (t, i, old) in saved:
            host[t][i] = old
            grads[t][i:i + 1] = _to_dev(np.array([old], np.uint16), dev)
    assert D.state() == (8192.0, 30, 0, 3)


SCALES = [2.0 ** k for k in range(-20, 41, 3)] + [3.0, 1000.0, 1e-30, 7e-39, 1e-45, 3.0e38,
                                                  float("inf"), 0.0, float("nan"),
                                                  float("-inf"), -0.0, -2.0, -3.0e38]


def test_every_fp16_pattern_times_scales(dev):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    g = _to_dev(h, dev)
    o = torch.empty(65536, dtype=torch.float32, device=dev)
    for S in SCALES:
        Sd = torch.tensor([S], dtype=torch.float32, device=dev)
        f = torch.zeros(1, dtype=torch.int32, device=dev)
        gs.gs_unscale_check([g], [o], Sd, f)
        ref, rf = oracle.unscale_check([h], S)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(o), ref[0].view(np.uint32)), S
        assert int(f.item()) == rf, S


def test_ragged_misaligned_and_empty(dev):
    """Sizes around the 8192-element chunk and the 8-element vector, bases
    offset by 0..7 elements (the scalar path), empty tensors in the list."""
    rng = np.random.default_rng(9)
    sizes = [0, 1, 7, 8, 9, 8191, 8192, 8193, 3 * 8192 + 5, 0, 100000]
    host, grads, outs = [], [], []
    pool = torch.empty(1 << 20, dtype=torch.float16, device=dev)
    opool = torch.empty(1 << 20, dtype=torch.float32, device=dev)
    off = 0
    for k, n in enumerate(sizes):
        h = rng.integers(0, 0x7C00, size=n, dtype=np.uint32).astype(np.uint16)
        h |= (rng.integers(0, 2, size=n).astype(np.uint16) << 15)
        shift = k % 8
        host.append(h)
        g = pool[off + shift: off + shift + n]
        g.copy_(_to_dev(h, dev) if n else g)
        o = opool[off + (7 - shift): off + (7 - shift) + n]
        grads.append(g)
        outs.append(o)
        off += n + 16
    for S in (1024.0, 3.0):
        Sd = torch.tensor([S], dtype=torch.float32, device=dev)
        f = torch.zeros(1, dtype=torch.int32, device=dev)
        gs.gs_unscale_check(grads, outs, Sd, f)
        ref, rf = oracle.unscale_check(host, S)
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert np.array_equal(_bits(o), r.view(np.uint32))
        assert int(f.item()) == rf == 0


def test_flag_is_set_only_and_empty_list(dev):
    g = _to_dev(np.float16([1.0, 2.0]).view(np.uint16), dev)
    o = torch.empty(2, dtype=torch.float32, device=dev)
    S = torch.tensor([2.0], dtype=torch.float32, device=dev)
    f = torch.ones(1, dtype=torch.int32, device=dev)
    gs.gs_unscale_check([g], [o], S, f)          # clean data never clears the flag
    gs.gs_unscale_check([], [], S, f)            # an empty list launches nothing
    torch.cuda.synchronize()
    assert int(f.item()) == 1 and o.tolist() == [0.5, 1.0]
    tr = torch.zeros(1, dtype=torch.int32, device=dev)
    gs.gs_update_scale(S, tr, f)                 # the update consumes the flag
    torch.cuda.synchronize()
    assert int(f.item()) == 0 and float(S.item()) == 1.0 and int(tr.item()) == 0


def test_page_trace_on_device(dev):
    """'Loss scaling, FP8, and the failure that never crashes': init 1024,
    interval 3, Inf at step 4 -> 1024, 1024, 2048, 1024, 1024."""
    good = _to_dev(np.float16([0.25, -4.0]).view(np.uint16), dev)
    bad = _to_dev(np.float16([np.inf]).view(np.uint16), dev)
    og, ob = torch.empty(2, device=dev), torch.empty(1, device=dev)
    D = DevScaler(1024.0, dev)
    seen = []
    for step in range(1, 6):
        lst = [good, bad] if step == 4 else [good]
        gs.gs_unscale_check(lst, [og, ob][:len(lst)], D.S, D.found)
        gs.gs_update_scale(D.S, D.tracker, D.found, 2.0, 0.5, 3, D.skips)
        seen.append(D.state()[0])
    assert seen == [1024.0, 1024.0, 2048.0, 1024.0, 1024.0]


def test_collapse_and_overflow_on_device(dev):
    D = DevScaler(65536.0, dev)
    for k in range(1, 167):
        D.found.fill_(1)
        gs.gs_update_scale(D.S, D.tracker, D.found, 2.0, 0.5, 2000, D.skips)
        if k == 165:
            assert D.state()[0] == 2.0 ** -149      # FP32 subnormals are honoured
    assert D.state()[0] == 0.0 and D.state()[3] == 166
    U = DevScaler(65536.0, dev)
    for k in range(1, 113):
        gs.gs_update_scale(U.S, U.tracker, U.found, 2.0, 0.5, 1, U.skips)
    assert U.state()[0] == float("inf")


def test_random_injection_10000_steps_matches_oracle(dev):
    rng = np.random.default_rng(2024)
    flags = rng.random(10000) < 0.001
    D = DevScaler(65536.0, dev)
    R = oracle.ScalerState(65536.0)
    fl = torch.from_numpy(flags.astype(np.int32)).to(dev)
    for i in range(10000):
        D.found.copy_(fl[i:i + 1])
        gs.gs_update_scale(D.S, D.tracker, D.found, 2.0, 0.5, 2000, D.skips)
        R.found_inf.value = int(flags[i])
        oracle.update_scale(R)
        if i % 997 == 0:
            assert D.state() == (float(R.S), R.tracker.value, 0, R.skips.value), i
    assert D.state() == (float(R.S), R.tracker.value, 0, R.skips.value)


def test_abi_errors_leave_no_side_effects(dev):
    g = torch.zeros(4, dtype=torch.float16, device=dev)
    o = torch.zeros(4, dtype=torch.float32, device=dev)
    S = torch.tensor([1.0], device=dev)
    f = torch.zeros(1, dtype=torch.int32, device=dev)
    with pytest.raises(gs.GSError):
        gs.gs_update_scale(S, f, f, 2.0, 0.5, 0)           # interval 0
    with pytest.raises(gs.GSError):
        gs.gs_update_scale(S, f, f, float("nan"), 0.5, 10)
    with pytest.raises(TypeError):
        gs.gs_unscale_check([g.float()], [o], S, f)
    torch.cuda.synchronize()
    assert float(S.item()) == 1.0 and int(f.item()) == 0


@pytest.mark.parametrize("S0", [0.0, float("inf"), float("-inf"), float("nan"), -0.0, -4.0,
                                3.0e38, 1e-45])
def test_forced_scale_states_step_by_step(dev, S0):
    """The loop forced into a degenerate state: S = 0, +-Inf, NaN, -0, a
    negative or a huge or a subnormal value, then 6 steps of unscale + update
    (one clean gradient list, growth interval 2).  Every step's outputs, flag
    and state match the oracle bit for bit."""
    rng = np.random.default_rng(77)
    host = [rng.integers(0, 0x7C00, size=n, dtype=np.uint32).astype(np.uint16) for n in (5, 3000)]
    grads = [_to_dev(h, dev) for h in host]
    outs = [torch.empty(h.size, dtype=torch.float32, device=dev) for h in host]
    D = DevScaler(S0, dev)
    R = oracle.ScalerState(S0)
    for step in range(6):
        gs.gs_unscale_check(grads, outs, D.S, D.found)
        ref, R.found_inf.value = oracle.unscale_check(host, float(R.S), R.found_inf.value)
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert np.array_equal(_bits(o), r.view(np.uint32)), (S0, step)
        assert int(D.found.item()) == R.found_inf.value, (S0, step)
        gs.gs_update_scale(D.S, D.tracker, D.found, 2.0, 0.5, 2, D.skips)
        oracle.update_scale(R, 2.0, 0.5, 2)
        S, t, f, k = D.state()
        assert np.float32(S).view(np.uint32) == R.S.view(np.uint32), (S0, step)
        assert (t, f, k) == (R.tracker.value, 0, R.skips.value), (S0, step)
