"""loss_scaling_fp8_amd -- dynamic loss scaling and FP8 scaled casting on
AMD MI355X (gfx950).

A thin ctypes binding over libgsfp8.so, whose C ABI is include/gs.h.  The
functions here carry the same names as the C entry points and only marshal
arguments (tensor data pointers, sizes, the current HIP stream); every step
of the computation runs in the library's HIP kernels.  PyTorch is used for
device memory and streams only.  There is no fallback: if the library is not
built, or no GPU is present, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgsfp8.so")

GS_OK = 0
GS_F16, GS_BF16, GS_F32 = 1, 2, 3
FP8_E4M3, FP8_E5M2 = 0, 1
FP8_PER_TENSOR, FP8_BLOCK_1x128, FP8_BLOCK_128x128, FP8_BLOCK_1x32 = 0, 1, 2, 3
FP8_SCALE_FROM_AMAX, FP8_SCALE_GIVEN = 0, 1

EXPORTS = ("gs_unscale_check", "gs_unscale_list_descriptors",
           "gs_unscale_check_sumsq_workspace_size", "gs_unscale_check_sumsq",
           "gs_update_scale", "gs_update_scale_hysteresis", "fp8_quantize_workspace_size",
           "fp8_quantize", "fp8_quantize_no_workspace", "fp8_quantize_delayed", "fp8_dequantize", "fp8_dequantize_bf16",
           "fp8_quantize_mx", "fp8_dequantize_mx", "gs_status_string")

_lib = None


class GSError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s returned %d (%s)" % (where, status, status_string(status)))
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libgsfp8.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgsfp8.so is not built; run "
                               "`python -m loss_scaling_fp8_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        L.gs_unscale_check.argtypes = [I32, P, P, P, ctypes.c_int, P, P, P]
        L.gs_unscale_check.restype = I32
        L.gs_unscale_list_descriptors.argtypes = [I32, P, P, P, P, I64]
        L.gs_unscale_list_descriptors.restype = I64
        L.gs_unscale_check_sumsq_workspace_size.argtypes = [I32, P]
        L.gs_unscale_check_sumsq_workspace_size.restype = ctypes.c_size_t
        L.gs_unscale_check_sumsq.argtypes = [I32, P, P, P, ctypes.c_int, P, P, P, P, P,
                                             ctypes.c_size_t, P]
        L.gs_unscale_check_sumsq.restype = I32
        L.gs_update_scale.argtypes = [P, P, P, F, F, I32, P, P]
        L.gs_update_scale.restype = I32
        L.gs_update_scale_hysteresis.argtypes = [P, P, P, P, F, F, I32, I32, I32, F, P, P]
        L.gs_update_scale_hysteresis.restype = I32
        L.fp8_quantize_workspace_size.argtypes = [I64, I64, ctypes.c_int]
        L.fp8_quantize_workspace_size.restype = ctypes.c_size_t
        L.fp8_quantize.argtypes = [P, ctypes.c_int, I64, I64, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, P, P, P, P, ctypes.c_size_t, P]
        L.fp8_quantize.restype = I32
        L.fp8_quantize_no_workspace.argtypes = [P, ctypes.c_int, I64, I64, ctypes.c_int,
                                                ctypes.c_int, ctypes.c_int, P, P, P, P]
        L.fp8_quantize_no_workspace.restype = I32
        L.fp8_quantize_delayed.argtypes = [P, ctypes.c_int, I64, I64, ctypes.c_int, P, P, I32,
                                           P, P, P, P, P, ctypes.c_size_t, P]
        L.fp8_quantize_delayed.restype = I32
        L.fp8_dequantize.argtypes = [P, I64, I64, ctypes.c_int, ctypes.c_int, P, P, P]
        L.fp8_dequantize.restype = I32
        L.fp8_dequantize_bf16.argtypes = [P, I64, I64, ctypes.c_int, ctypes.c_int, P, P, P]
        L.fp8_dequantize_bf16.restype = I32
        L.fp8_quantize_mx.argtypes = [P, ctypes.c_int, I64, I64, ctypes.c_int, P, P, P, P]
        L.fp8_quantize_mx.restype = I32
        L.fp8_dequantize_mx.argtypes = [P, I64, I64, ctypes.c_int, P, P, P]
        L.fp8_dequantize_mx.restype = I32
        L.gs_status_string.argtypes = [I32]
        L.gs_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().gs_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != GS_OK:
        raise GSError(status, where)


def _gpu(t, name: str, dtypes, dev=None, numel: int | None = None, exact: bool = False,
         optional: bool = False):
    """Checks that t is a contiguous GPU tensor of one of `dtypes`, on `dev`
    when given, holding at least (or, with exact, exactly) `numel` elements;
    returns its device.  The C ABI takes bare device pointers and cannot see
    any of this: a host tensor or a short buffer would reach a kernel."""
    import torch
    if t is None:
        if optional:
            return dev
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU, not on %s" % (name, t.device))
    if dev is not None and t.get_device() != dev.index:
        raise ValueError("%s is on %s, the other arguments on %s" % (name, t.device, dev))
    if t.dtype not in dtypes:
        raise TypeError("%s must be %s, not %s" % (name, " or ".join(map(str, dtypes)), t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if numel is not None and (t.numel() != numel if exact else t.numel() < numel):
        raise ValueError("%s holds %d elements, %s%d needed" %
                         (name, t.numel(), "" if exact else "at least ", numel))
    return t.device


def _bytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream, dev) -> int | None:
    """The HIP stream handle: torch's current stream on dev by default (read
    as a raw handle where torch offers that, without building a Stream
    object); a torch stream must belong to dev; an integer is passed as is."""
    import torch
    if stream is None:
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return raw(dev.index)
        return torch.cuda.current_stream(dev).cuda_stream
    if hasattr(stream, "cuda_stream"):
        if stream.device != dev:
            raise ValueError("the stream is on %s, the tensors on %s" % (stream.device, dev))
        return stream.cuda_stream
    return stream


def _call(dev, where: str, fn, *args) -> None:
    """Calls a C entry point with the tensors' device current (the unscale's
    descriptor cache allocates on the current device) and raises on error."""
    import torch
    if dev.index == torch.cuda.current_device():
        status = fn(*args)
    else:
        with torch.cuda.device(dev):
            status = fn(*args)
    _check(status, where)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _input_dtype(x) -> int:
    import torch
    if x.dtype == torch.bfloat16:
        return GS_BF16
    if x.dtype == torch.float32:
        return GS_F32
    raise TypeError("x must be bfloat16 or float32, not %s" % x.dtype)


def _matrix(x, name: str, dtypes):
    """A contiguous 2-D GPU tensor: returns (rows, cols, device)."""
    dev = _gpu(x, name, dtypes)
    if x.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    return x.shape[0], x.shape[1], dev


def n_scales(rows: int, cols: int, gran: int) -> int:
    if gran == FP8_PER_TENSOR:
        return 1
    if gran == FP8_BLOCK_1x128:
        return rows * (cols // 128)
    if gran == FP8_BLOCK_1x32:
        return rows * (cols // 32)
    return (rows // 128) * (cols // 128)


def scale_shape(rows: int, cols: int, gran: int) -> tuple:
    if gran == FP8_PER_TENSOR:
        return (1,)
    if gran == FP8_BLOCK_1x128:
        return (rows, cols // 128)
    if gran == FP8_BLOCK_1x32:
        return (rows, cols // 32)
    return (rows // 128, cols // 128)


# ------------------------------------------------------------------ unscale
def _scalars(dev, **kw):
    """The device-resident scalars of the scaler state: name -> (tensor,
    dtypes, elements needed, optional)."""
    for name, (t, dtypes, k, opt) in kw.items():
        _gpu(t, name, dtypes, dev, k, optional=opt)


def gs_unscale_check(grads: Sequence, outs: Sequence, scale, found_inf, stream=None) -> None:
    """FP16 gradients -> FP32 outputs multiplied by fl32(1/S); found_inf set to
    1 on any non-finite output.  One kernel launch for the whole list."""
    import torch
    dev = _gpu(scale, "scale", (torch.float32,), None, 1)
    _gpu(found_inf, "found_inf", (torch.int32,), dev, 1)
    n, arr_g, arr_o, arr_n = _grad_lists(grads, outs, dev)
    _call(dev, "gs_unscale_check", lib().gs_unscale_check, n, arr_g, arr_o, arr_n, GS_F16,
          _ptr(scale), _ptr(found_inf), _stream(stream, dev))


def _grad_lists(grads, outs, dev):
    import torch
    n = len(grads)
    if len(outs) != n:
        raise ValueError("grads and outs differ in length")
    di = dev.index
    for g, o in zip(grads, outs):
        if not isinstance(g, torch.Tensor) or not isinstance(o, torch.Tensor):
            raise TypeError("grads and outs must be torch tensors")
        if g.dtype != torch.float16 or o.dtype != torch.float32:
            raise TypeError("grads must be float16 and outs float32")
        if not (g.is_cuda and o.is_cuda) or g.get_device() != di or o.get_device() != di:
            raise ValueError("every gradient and output must be on %s (the scale's device)" % dev)
        if o.numel() != g.numel() or not g.is_contiguous() or not o.is_contiguous():
            raise ValueError("each out must be a contiguous float32 tensor of its grad's size")
    arr_g = (ctypes.c_void_p * max(n, 1))(*[g.data_ptr() for g in grads])
    arr_o = (ctypes.c_void_p * max(n, 1))(*[o.data_ptr() for o in outs])
    arr_n = (ctypes.c_int64 * max(n, 1))(*[g.numel() for g in grads])
    return n, arr_g, arr_o, arr_n


def gs_unscale_check_sumsq_workspace_size(numels: Sequence[int]) -> int:
    n = len(numels)
    arr_n = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in numels])
    return int(lib().gs_unscale_check_sumsq_workspace_size(n, arr_n))


def gs_unscale_check_sumsq(grads: Sequence, outs: Sequence, scale, found_inf, sumsq, norm_sq,
                           workspace=None, stream=None) -> None:
    """gs_unscale_check plus the exact 128-bit sum of squares of the finite
    gradients, added to sumsq (int64 [2], low and high words), and the
    recovered-gradient norm squared written to norm_sq (float64 [1])."""
    import torch
    dev = _gpu(scale, "scale", (torch.float32,), None, 1)
    _gpu(found_inf, "found_inf", (torch.int32,), dev, 1)
    _gpu(sumsq, "sumsq", (torch.int64, torch.uint64), dev, 2, exact=True)
    _gpu(norm_sq, "norm_sq", (torch.float64,), dev, 1)
    n, arr_g, arr_o, arr_n = _grad_lists(grads, outs, dev)
    ws_bytes = gs_unscale_check_sumsq_workspace_size([g.numel() for g in grads])
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _gpu(workspace, "workspace", (torch.uint8,), dev, ws_bytes)
    _call(dev, "gs_unscale_check_sumsq", lib().gs_unscale_check_sumsq, n, arr_g, arr_o, arr_n,
          GS_F16, _ptr(scale), _ptr(found_inf), _ptr(sumsq), _ptr(norm_sq), _ptr(workspace),
          _bytes(workspace), _stream(stream, dev))


def gs_update_scale(scale, growth_tracker, found_inf, growth_factor: float = 2.0,
                    backoff_factor: float = 0.5, growth_interval: int = 2000,
                    skip_count=None, stream=None) -> None:
    """Grow/backoff/skip update of the device-resident loss scale."""
    import torch
    dev = _gpu(scale, "scale", (torch.float32,), None, 1)
    _scalars(dev, growth_tracker=(growth_tracker, (torch.int32,), 1, False),
             found_inf=(found_inf, (torch.int32,), 1, False),
             skip_count=(skip_count, (torch.int64,), 1, True))
    _call(dev, "gs_update_scale", lib().gs_update_scale, _ptr(scale), _ptr(growth_tracker),
          _ptr(found_inf), float(growth_factor), float(backoff_factor), int(growth_interval),
          _ptr(skip_count), _stream(stream, dev))


def gs_update_scale_hysteresis(scale, growth_tracker, hysteresis_left, found_inf,
                               growth_factor: float = 2.0, backoff_factor: float = 0.5,
                               growth_interval: int = 1000, hysteresis: int = 2,
                               consecutive_hysteresis: bool = False, min_scale: float = 1.0,
                               skip_count=None, stream=None) -> None:
    """Update with a hysteresis budget, a floor and a growth window (defaults:
    the DeepSpeed fp16 block's 1000 / 2 / false / 1)."""
    import torch
    dev = _gpu(scale, "scale", (torch.float32,), None, 1)
    _scalars(dev, growth_tracker=(growth_tracker, (torch.int32,), 1, False),
             hysteresis_left=(hysteresis_left, (torch.int32,), 1, False),
             found_inf=(found_inf, (torch.int32,), 1, False),
             skip_count=(skip_count, (torch.int64,), 1, True))
    _call(dev, "gs_update_scale_hysteresis", lib().gs_update_scale_hysteresis, _ptr(scale),
          _ptr(growth_tracker), _ptr(hysteresis_left), _ptr(found_inf), float(growth_factor),
          float(backoff_factor), int(growth_interval), int(hysteresis),
          int(bool(consecutive_hysteresis)), float(min_scale), _ptr(skip_count),
          _stream(stream, dev))


# ------------------------------------------------------------------ FP8
def fp8_quantize_workspace_size(rows: int, cols: int, gran: int) -> int:
    return int(lib().fp8_quantize_workspace_size(int(rows), int(cols), int(gran)))


def fp8_quantize(x, fmt: int, gran: int, mode: int = FP8_SCALE_FROM_AMAX, codes=None,
                 scales=None, nonfinite=None, workspace=None, stream=None):
    """Quantize a 2-D bfloat16/float32 CUDA tensor; returns (codes, scales).
    codes is uint8 [rows, cols]; scales float32 in the block layout.  In
    given-scale mode `scales` must be supplied."""
    import torch
    rows, cols, dev = _matrix(x, "x", (torch.bfloat16, torch.float32))
    dt = _input_dtype(x)
    if codes is None:
        codes = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if scales is None:
        if mode == FP8_SCALE_GIVEN:
            raise ValueError("given-scale mode needs scales")
        scales = torch.empty(scale_shape(rows, cols, gran), dtype=torch.float32, device=dev)
    _gpu(codes, "codes", (torch.uint8,), dev, rows * cols, exact=True)
    _gpu(scales, "scales", (torch.float32,), dev, n_scales(rows, cols, gran))
    _gpu(nonfinite, "nonfinite", (torch.int32,), dev, 1, optional=True)
    ws_bytes = fp8_quantize_workspace_size(rows, cols, gran)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _gpu(workspace, "workspace", (torch.uint8,), dev, ws_bytes, optional=True)
    _call(dev, "fp8_quantize", lib().fp8_quantize, _ptr(x), dt, rows, cols, int(fmt), int(gran),
          int(mode), _ptr(codes), _ptr(scales), _ptr(nonfinite), _ptr(workspace),
          _bytes(workspace), _stream(stream, dev))
    return codes, scales


def fp8_quantize_no_workspace(x, fmt: int, gran: int, codes, scales,
                              mode: int = FP8_SCALE_FROM_AMAX, nonfinite=None, stream=None):
    """fp8_quantize without a workspace: the per-tensor partial maxima live
    in the library's static device array.  codes and scales must be given
    (nothing is allocated); same results as fp8_quantize."""
    import torch
    rows, cols, dev = _matrix(x, "x", (torch.bfloat16, torch.float32))
    dt = _input_dtype(x)
    _gpu(codes, "codes", (torch.uint8,), dev, rows * cols, exact=True)
    _gpu(scales, "scales", (torch.float32,), dev, n_scales(rows, cols, gran))
    _gpu(nonfinite, "nonfinite", (torch.int32,), dev, 1, optional=True)
    _call(dev, "fp8_quantize_no_workspace", lib().fp8_quantize_no_workspace, _ptr(x), dt, rows,
          cols, int(fmt), int(gran), int(mode), _ptr(codes), _ptr(scales), _ptr(nonfinite),
          _stream(stream, dev))
    return codes, scales


def fp8_quantize_delayed(x, fmt: int, scale_state, amax_history, history_pos, codes=None,
                         scale_used=None, nonfinite=None, workspace=None, stream=None):
    """One delayed-scaling step on a 2-D bfloat16/float32 CUDA tensor: cast
    with the scale in scale_state, record this step's amax in the history
    ring, write the next step's scale.  Returns (codes, scale_used)."""
    import torch
    rows, cols, dev = _matrix(x, "x", (torch.bfloat16, torch.float32))
    dt = _input_dtype(x)
    _gpu(scale_state, "scale_state", (torch.float32,), dev, 1)
    _gpu(amax_history, "amax_history", (torch.float32,), dev)
    _gpu(history_pos, "history_pos", (torch.int32,), dev, 1)
    if codes is None:
        codes = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if scale_used is None:
        scale_used = torch.empty(1, dtype=torch.float32, device=dev)
    _gpu(codes, "codes", (torch.uint8,), dev, rows * cols, exact=True)
    _gpu(scale_used, "scale_used", (torch.float32,), dev, 1)
    _gpu(nonfinite, "nonfinite", (torch.int32,), dev, 1, optional=True)
    ws_bytes = fp8_quantize_workspace_size(rows, cols, FP8_PER_TENSOR)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _gpu(workspace, "workspace", (torch.uint8,), dev, ws_bytes)
    _call(dev, "fp8_quantize_delayed", lib().fp8_quantize_delayed, _ptr(x), dt, rows, cols,
          int(fmt), _ptr(scale_state), _ptr(amax_history), amax_history.numel(),
          _ptr(history_pos), _ptr(codes), _ptr(scale_used), _ptr(nonfinite), _ptr(workspace),
          _bytes(workspace), _stream(stream, dev))
    return codes, scale_used


def _dequantize(entry, out_dtype, codes, fmt, gran, scales, out, stream):
    import torch
    rows, cols, dev = _matrix(codes, "codes", (torch.uint8,))
    _gpu(scales, "scales", (torch.float32,), dev, n_scales(rows, cols, gran))
    if out is None:
        out = torch.empty((rows, cols), dtype=out_dtype, device=dev)
    _gpu(out, "out", (out_dtype,), dev, rows * cols, exact=True)
    _call(dev, entry, getattr(lib(), entry), _ptr(codes), rows, cols, int(fmt), int(gran),
          _ptr(scales), _ptr(out), _stream(stream, dev))
    return out


def fp8_dequantize(codes, fmt: int, gran: int, scales, out=None, stream=None):
    """decode(code) * s in float32; returns out [rows, cols]."""
    import torch
    return _dequantize("fp8_dequantize", torch.float32, codes, fmt, gran, scales, out, stream)


def fp8_dequantize_bf16(codes, fmt: int, gran: int, scales, out=None, stream=None):
    """decode(code) * s in float32, rounded to bfloat16 (nearest, ties to
    even); returns out [rows, cols] (torch.bfloat16)."""
    import torch
    return _dequantize("fp8_dequantize_bf16", torch.bfloat16, codes, fmt, gran, scales, out,
                       stream)


def fp8_quantize_mx(x, fmt: int, codes=None, scales=None, nonfinite=None, stream=None):
    """MX-style 1x32 blocks with E8M0 power-of-two scales on a 2-D
    bfloat16/float32 CUDA tensor; returns (codes uint8 [rows, cols], scales
    uint8 [rows, cols/32])."""
    import torch
    rows, cols, dev = _matrix(x, "x", (torch.bfloat16, torch.float32))
    dt = _input_dtype(x)
    if codes is None:
        codes = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
    _gpu(codes, "codes", (torch.uint8,), dev, rows * cols, exact=True)
    _gpu(scales, "scales", (torch.uint8,), dev, rows * (cols // 32))
    _gpu(nonfinite, "nonfinite", (torch.int32,), dev, 1, optional=True)
    _call(dev, "fp8_quantize_mx", lib().fp8_quantize_mx, _ptr(x), dt, rows, cols, int(fmt),
          _ptr(codes), _ptr(scales), _ptr(nonfinite), _stream(stream, dev))
    return codes, scales


def fp8_dequantize_mx(codes, fmt: int, scales, out=None, stream=None):
    """decode(code) * 2^(byte - 127) in float32; returns out [rows, cols]."""
    import torch
    rows, cols, dev = _matrix(codes, "codes", (torch.uint8,))
    _gpu(scales, "scales", (torch.uint8,), dev, rows * (cols // 32))
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    _gpu(out, "out", (torch.float32,), dev, rows * cols, exact=True)
    _call(dev, "fp8_dequantize_mx", lib().fp8_dequantize_mx, _ptr(codes), rows, cols, int(fmt),
          _ptr(scales), _ptr(out), _stream(stream, dev))
    return out
