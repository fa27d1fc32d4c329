"""CPU oracle for the loss-scaling + FP8 scaled-cast path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does, and
this package imports nothing from the product package: the two share no code.

The arithmetic lives in ``oracle.c`` (plain scalar C, built with gcc
``-O2 -fno-fast-math -ffp-contract=off``, no FTZ/DAZ).  This module only
builds it, loads it with ctypes and marshals numpy arrays.  The functions
follow the pages cited in ``oracle.c``:

* ``unscale_check``  -- recovered gradient g_scaled/S in FP32 as a multiply
  by fl32(1/S), plus the Inf/NaN check ("Loss scaling, FP8, and the failure
  that never crashes", chain-rule section and the SimpleGradScaler listing).
* ``update_scale``   -- grow/backoff/skip ("SimpleGradScaler" listing; the
  GradScaler defaults paragraph of "Numerical Precision, Mixed Precision,
  and Loss Scaling").
* ``quantize`` / ``dequantize`` -- quant/per_tensor/per_block of the
  fp8_scaling.py listing ("Mixed precision and FP8 training", section
  "FP8 training"), after an exact widening to FP32.

Parity status of each function is listed in the module-level ``PINS`` dict.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liboracle.so")
_CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
           "-fPIC", "-shared", "-Wall", "-Wextra"]

F16, BF16, F32 = 1, 2, 3
E4M3, E5M2 = 0, 1
PER_TENSOR, BLOCK_1x128, BLOCK_128x128, BLOCK_1x32 = 0, 1, 2, 3
FROM_AMAX, GIVEN = 0, 1
FMT_MAX = {E4M3: 448.0, E5M2: 57344.0}
CANONICAL_NAN_BITS = 0x7FC00000

# What pins each function (see tests/test_oracle_*.py).  None is unpinned.
PINS = {
    "fp8_decode": "closed form of the OCP formats; torch CPU float8 view, all 256 codes",
    "fp8_encode": "torch CPU clamp+cast over every FP32 bit pattern (exhaustive)",
    "f16_to_f32": "numpy float16 widening, all 65536 patterns",
    "unscale_check": "page worked examples (1e-8 via 1024; 1e-8/1e-6/2e-5 via 2^16); "
                     "numpy f32 multiply over all FP16 patterns x scales",
    "unscale_check_sumsq": "exact integer sum of squares against Python integers; "
                           "norm_sq against numpy float64 sums within 1e-12",
    "update_scale": "page 5-step trace; closed-form trajectories (collapse, overflow, C1)",
    "update_scale_hysteresis": "reduces to the pinned GradScaler policy (hysteresis 1, no "
                               "floor) on random flag sequences; closed-form trajectories "
                               "(floor, budget spent and refilled, growth every window); the "
                               "page's comparison of the two policies (growth twice as eager, "
                               "different skip rate from the same start); the knob semantics "
                               "are a reading of their names",
    "quantize": "page fp8_scaling.py listing run by torch CPU; page error table; "
                "outlier exercise; scale-invariance and error-bound properties",
    "dequantize": "page quant() listing run by torch CPU",
    "quantize_mx": "the page's listing with 1x32 blocks run by torch CPU, its scale rounded "
                   "up to a power of two by torch.frexp (the E8M0 reading); the scale is the "
                   "exponent field; no saturation; power-of-two invariance",
    "dequantize_mx": "torch float8 decode times torch.ldexp of the byte, NaN byte",
    "quantize_delayed": "reduces to the pinned per-tensor quantizer (history 1, same "
                        "tensor twice); window max closed form; the pages' spike failure "
                        "shape (saturation); otherwise parity unpinned",
}

_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile oracle.c into oracle/_build/liboracle.so (always, when forced)."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            # ORACLE_LIB lets the mutation test load a deliberately broken copy
            path = os.environ.get("ORACLE_LIB") or build(force=False)
            L = ctypes.CDLL(path)
            P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
            L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
            L.orc_f16_to_f32.restype = F
            L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
            L.orc_bf16_to_f32.restype = F
            L.orc_fp8_decode.argtypes = [ctypes.c_uint8, ctypes.c_int]
            L.orc_fp8_decode.restype = ctypes.c_double
            L.orc_fp8_encode.argtypes = [F, ctypes.c_int]
            L.orc_fp8_encode.restype = ctypes.c_uint8
            L.orc_unscale_check.argtypes = [I32, P, P, P, F, P]
            L.orc_unscale_check.restype = None
            L.orc_unscale_check_sumsq.argtypes = [I32, P, P, P, F, P, P, P]
            L.orc_unscale_check_sumsq.restype = None
            L.orc_update_scale.argtypes = [P, P, P, F, F, I32, P]
            L.orc_update_scale.restype = None
            L.orc_update_scale_hysteresis.argtypes = [P, P, P, P, F, F, I32, I32, I32, F, P]
            L.orc_update_scale_hysteresis.restype = None
            L.orc_block_amax.argtypes = [P, ctypes.c_int, I64, I64, I64, I64, I64]
            L.orc_block_amax.restype = F
            L.orc_scale_from_amax.argtypes = [F, ctypes.c_int]
            L.orc_scale_from_amax.restype = F
            L.orc_cast.argtypes = [F, F, ctypes.c_int]
            L.orc_cast.restype = ctypes.c_uint8
            L.orc_quantize.argtypes = [P, ctypes.c_int, I64, I64, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, P, P, P]
            L.orc_quantize.restype = ctypes.c_int
            L.orc_quantize_delayed.argtypes = [P, ctypes.c_int, I64, I64, ctypes.c_int, P, P,
                                               I32, P, P, P, P]
            L.orc_quantize_delayed.restype = ctypes.c_int
            L.orc_dequantize.argtypes = [P, I64, I64, ctypes.c_int, ctypes.c_int, P, P]
            L.orc_quantize_mx.argtypes = [P, ctypes.c_int, I64, I64, ctypes.c_int, P, P, P]
            L.orc_quantize_mx.restype = ctypes.c_int
            L.orc_dequantize_mx.argtypes = [P, I64, I64, ctypes.c_int, P, P]
            L.orc_dequantize_mx.restype = ctypes.c_int
            L.orc_dequantize.restype = ctypes.c_int
            L.orc_dequantize_bf16.argtypes = [P, I64, I64, ctypes.c_int, ctypes.c_int, P, P]
            L.orc_dequantize_bf16.restype = ctypes.c_int
            L.orc_fp8_encode_array.argtypes = [P, I64, ctypes.c_int, P]
            L.orc_fp8_encode_array.restype = None
            L.orc_cast_array.argtypes = [P, I64, F, ctypes.c_int, P]
            L.orc_cast_array.restype = None
            L.orc_fp8_decode_table.argtypes = [ctypes.c_int, P]
            L.orc_fp8_decode_table.restype = None
            L.orc_f16_to_f32_array.argtypes = [P, I64, P]
            L.orc_f16_to_f32_array.restype = None
            L.orc_canonical_nan_bits.argtypes = []
            L.orc_canonical_nan_bits.restype = ctypes.c_uint32
            _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _parallel(fn, n: int, chunk: int, threads: int | None):
    """Run fn(lo, hi) over [0, n) in chunks; ctypes calls release the GIL."""
    if threads is None:
        threads = min(8, os.cpu_count() or 1)
    spans = [(lo, min(n, lo + chunk)) for lo in range(0, n, chunk)]
    if threads <= 1 or len(spans) <= 1:
        for lo, hi in spans:
            fn(lo, hi)
        return
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda sp: fn(*sp), spans))


# ---------------------------------------------------------------- codecs
def fp8_decode_table(fmt: int) -> np.ndarray:
    out = np.empty(256, np.float64)
    lib().orc_fp8_decode_table(fmt, _ptr(out))
    return out


def fp8_encode(y: np.ndarray, fmt: int, threads: int | None = None) -> np.ndarray:
    """Saturating RNE encode of FP32 values (NaN -> sign|0x7F)."""
    y = np.ascontiguousarray(y, np.float32).reshape(-1)
    out = np.empty(y.size, np.uint8)
    L = lib()
    _parallel(lambda lo, hi: L.orc_fp8_encode_array(
        y.ctypes.data + 4 * lo, hi - lo, fmt, out.ctypes.data + lo), y.size, 1 << 22, threads)
    return out


def cast(f: np.ndarray, s: float, fmt: int, threads: int | None = None) -> np.ndarray:
    """Per-element quant() of FP32 values with one given scale s."""
    f = np.ascontiguousarray(f, np.float32).reshape(-1)
    out = np.empty(f.size, np.uint8)
    L = lib()
    _parallel(lambda lo, hi: L.orc_cast_array(
        f.ctypes.data + 4 * lo, hi - lo, float(s), fmt, out.ctypes.data + lo), f.size, 1 << 22, threads)
    return out


def f16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, np.uint16).reshape(-1)
    out = np.empty(h.size, np.float32)
    lib().orc_f16_to_f32_array(_ptr(h), h.size, _ptr(out))
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    L = lib()
    b = np.ascontiguousarray(b, np.uint16).reshape(-1)
    return np.array([L.orc_bf16_to_f32(int(v)) for v in b], np.float32)


def scale_from_amax(amax: float, fmt: int) -> np.float32:
    return np.float32(lib().orc_scale_from_amax(float(np.float32(amax)), fmt))


# ---------------------------------------------------------------- unscale + update
def unscale_check(grads: list[np.ndarray], S: float, found_inf: int = 0):
    """Returns (list of FP32 outputs, found_inf).  grads are FP16 bit arrays
    (uint16) or float16 arrays; S is the current loss scale (FP32)."""
    gs = [np.ascontiguousarray(g).view(np.uint16).reshape(-1) for g in grads]
    outs = [np.empty(g.size, np.float32) for g in gs]
    n = len(gs)
    gp = (ctypes.c_void_p * max(n, 1))(*[g.ctypes.data for g in gs])
    op = (ctypes.c_void_p * max(n, 1))(*[o.ctypes.data for o in outs])
    ne = (ctypes.c_int64 * max(n, 1))(*[g.size for g in gs])
    flag = ctypes.c_int32(found_inf)
    lib().orc_unscale_check(n, gp, op, ne, float(np.float32(S)), ctypes.byref(flag))
    return outs, flag.value


def unscale_check_sumsq(grads: list[np.ndarray], S: float, found_inf: int = 0,
                        sumsq: tuple = (0, 0)):
    """unscale_check plus the exact sum of squares: returns (outputs,
    found_inf, (sumsq_lo, sumsq_hi) running total, norm_sq)."""
    gs = [np.ascontiguousarray(g).view(np.uint16).reshape(-1) for g in grads]
    outs = [np.empty(g.size, np.float32) for g in gs]
    n = len(gs)
    gp = (ctypes.c_void_p * max(n, 1))(*[g.ctypes.data for g in gs])
    op = (ctypes.c_void_p * max(n, 1))(*[o.ctypes.data for o in outs])
    ne = (ctypes.c_int64 * max(n, 1))(*[g.size for g in gs])
    flag = ctypes.c_int32(found_inf)
    acc = (ctypes.c_uint64 * 2)(*sumsq)
    nsq = ctypes.c_double(0.0)
    lib().orc_unscale_check_sumsq(n, gp, op, ne, float(np.float32(S)), ctypes.byref(flag),
                                  acc, ctypes.byref(nsq))
    return outs, flag.value, (acc[0], acc[1]), nsq.value


class ScalerState:
    """Device-state mirror: S (FP32), growth tracker, found_inf, skip count."""

    def __init__(self, scale: float = 65536.0, tracker: int = 0):
        self.scale = ctypes.c_float(scale)
        self.tracker = ctypes.c_int32(tracker)
        self.found_inf = ctypes.c_int32(0)
        self.skips = ctypes.c_int64(0)

    @property
    def S(self) -> np.float32:
        return np.float32(self.scale.value)


def update_scale(st: ScalerState, growth: float = 2.0, backoff: float = 0.5,
                 interval: int = 2000) -> None:
    lib().orc_update_scale(ctypes.byref(st.scale), ctypes.byref(st.tracker),
                           ctypes.byref(st.found_inf), float(growth), float(backoff),
                           int(interval), ctypes.byref(st.skips))


class HysteresisState(ScalerState):
    """ScalerState plus the hysteresis budget h (start it at H)."""

    def __init__(self, scale: float = 65536.0, tracker: int = 0, h: int = 2):
        super().__init__(scale, tracker)
        self.h = ctypes.c_int32(h)


def update_scale_hysteresis(st: HysteresisState, growth: float = 2.0, backoff: float = 0.5,
                            window: int = 1000, hysteresis: int = 2, consecutive: bool = False,
                            min_scale: float = 1.0) -> None:
    lib().orc_update_scale_hysteresis(ctypes.byref(st.scale), ctypes.byref(st.tracker),
                                      ctypes.byref(st.h), ctypes.byref(st.found_inf),
                                      float(growth), float(backoff), int(window), int(hysteresis),
                                      int(bool(consecutive)), float(min_scale),
                                      ctypes.byref(st.skips))


# ---------------------------------------------------------------- quantize
def _as_input(x: np.ndarray):
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), F32
    if x.dtype == np.uint16:          # BF16 bit patterns
        return np.ascontiguousarray(x), BF16
    raise TypeError("oracle quantize takes float32 or uint16 (BF16 bits)")


def n_scales(rows: int, cols: int, gran: int) -> int:
    if gran == PER_TENSOR:
        return 1
    if gran == BLOCK_1x128:
        return rows * (cols // 128)
    if gran == BLOCK_1x32:
        return rows * (cols // 32)
    return (rows // 128) * (cols // 128)


def quantize(x: np.ndarray, fmt: int, gran: int, mode: int = FROM_AMAX,
             scales: np.ndarray | None = None):
    """x: [rows, cols] float32 or uint16 (BF16 bits).  Returns
    (codes uint8 [rows, cols], scales float32 [n_blocks], nonfinite int)."""
    x, dt = _as_input(x)
    rows, cols = x.shape
    codes = np.empty((rows, cols), np.uint8)
    if mode == GIVEN:
        sc = np.ascontiguousarray(scales, np.float32).reshape(-1).copy()
    else:
        sc = np.empty(max(n_scales(rows, cols, gran), 1), np.float32)
    nf = ctypes.c_int32(0)
    rc = lib().orc_quantize(_ptr(x), dt, rows, cols, fmt, gran, mode,
                            _ptr(codes), _ptr(sc), ctypes.byref(nf))
    if rc != 0:
        raise ValueError("shape %dx%d not divisible into blocks" % (rows, cols))
    return codes, sc[:n_scales(rows, cols, gran)] if gran != PER_TENSOR else sc[:1], nf.value


def block_amax(x: np.ndarray, r0: int, nr: int, c0: int, nc: int) -> np.float32:
    x, dt = _as_input(x)
    return np.float32(lib().orc_block_amax(_ptr(x), dt, x.shape[1], r0, nr, c0, nc))


class DelayedState:
    """Delayed per-tensor scaling state: the scale for the next step, the
    amax history ring and its position."""

    def __init__(self, history_len: int, init_scale: float = 1.0):
        self.scale = np.float32([init_scale])
        self.history = np.zeros(history_len, np.float32)
        self.pos = np.int32([0])


def quantize_delayed(x: np.ndarray, fmt: int, st: DelayedState):
    """One delayed-scaling step; returns (codes, scale used, nonfinite) and
    updates st (history, position, next scale)."""
    x, dt = _as_input(x)
    rows, cols = x.shape
    codes = np.empty((rows, cols), np.uint8)
    used = np.zeros(1, np.float32)
    nf = ctypes.c_int32(0)
    rc = lib().orc_quantize_delayed(_ptr(x), dt, rows, cols, fmt, _ptr(st.scale),
                                    _ptr(st.history), st.history.size, _ptr(st.pos),
                                    _ptr(codes), _ptr(used), ctypes.byref(nf))
    if rc != 0:
        raise ValueError("bad delayed-scaling state")
    return codes, used[0], nf.value


def quantize_mx(x: np.ndarray, fmt: int):
    """MX-style 1x32 blocks with E8M0 power-of-two scales: returns (codes
    uint8 [rows, cols], scales uint8 [rows, cols/32], nonfinite)."""
    x, dt = _as_input(x)
    rows, cols = x.shape
    codes = np.empty((rows, cols), np.uint8)
    sc = np.empty((rows, max(cols // 32, 1)), np.uint8)
    nf = ctypes.c_int32(0)
    if lib().orc_quantize_mx(_ptr(x), dt, rows, cols, fmt, _ptr(codes), _ptr(sc),
                             ctypes.byref(nf)) != 0:
        raise ValueError("cols must be a multiple of 32")
    return codes, sc[:, :cols // 32], nf.value


def dequantize_mx(codes: np.ndarray, fmt: int, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    rows, cols = codes.shape
    sc = np.ascontiguousarray(scales, np.uint8)
    out = np.empty((rows, cols), np.float32)
    if lib().orc_dequantize_mx(_ptr(codes), rows, cols, fmt, _ptr(sc), _ptr(out)) != 0:
        raise ValueError("cols must be a multiple of 32")
    return out


def dequantize(codes: np.ndarray, fmt: int, gran: int, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    rows, cols = codes.shape
    sc = np.ascontiguousarray(scales, np.float32).reshape(-1)
    out = np.empty((rows, cols), np.float32)
    rc = lib().orc_dequantize(_ptr(codes), rows, cols, fmt, gran, _ptr(sc), _ptr(out))
    if rc != 0:
        raise ValueError("shape %dx%d not divisible into blocks" % (rows, cols))
    return out


def dequantize_bf16(codes: np.ndarray, fmt: int, gran: int, scales: np.ndarray) -> np.ndarray:
    """dequantize() rounded once more to BF16 (nearest, ties to even; NaN ->
    0x7FC0).  Returns BF16 bit patterns, uint16 [rows, cols]."""
    codes = np.ascontiguousarray(codes, np.uint8)
    rows, cols = codes.shape
    sc = np.ascontiguousarray(scales, np.float32).reshape(-1)
    out = np.empty((rows, cols), np.uint16)
    rc = lib().orc_dequantize_bf16(_ptr(codes), rows, cols, fmt, gran, _ptr(sc), _ptr(out))
    if rc == -2:
        raise MemoryError("oracle scratch allocation failed")
    if rc != 0:
        raise ValueError("shape %dx%d not divisible into blocks" % (rows, cols))
    return out
