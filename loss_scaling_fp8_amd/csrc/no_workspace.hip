// no_workspace.hip -- fp8_quantize_no_workspace: fp8_quantize for callers
// that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Per-tensor scaling from the amax is the
// one fp8_quantize mode that needs scratch memory (a partial maximum per
// workgroup of the first pass); here those partials live in a static device
// array instead of a caller workspace.  Every other mode needs none and is
// passed straight through.
#include <hip/hip_runtime.h>

#include <mutex>
#include <unordered_map>

#include "gs.h"
#include "gs_internal.hpp"

namespace {

// The partial maxima of per-tensor scaling: kPartialSlots words (32 KiB).
// Every GPU the library runs on holds its own copy until the process ends,
// and every call on that GPU shares it.  Nothing in it needs to start at
// zero: each pass writes the partials it later reads.  In host code
// `scratch` names a host-side stand-in, not a device address, so kernels
// receive the address hipGetSymbolAddress returns for the current device,
// looked up once per device (with that device current) and kept.
constexpr size_t kScratchBytes = size_t(gsk::kPartialSlots) * sizeof(uint32_t);
static __device__ __align__(256) uint32_t scratch[gsk::kPartialSlots];

gs_status scratch_address(void **out) {
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return GS_ERR_HIP;
    static std::mutex mu;
    static auto *addr = new std::unordered_map<int, void *>();   // never destroyed
    std::lock_guard<std::mutex> lock(mu);
    auto it = addr->find(device);
    if (it != addr->end()) {
        *out = it->second;
        return GS_OK;
    }
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GS_ERR_HIP;
    addr->emplace(device, p);
    *out = p;
    return GS_OK;
}

}  // namespace

extern "C" gs_status fp8_quantize_no_workspace(const void *x, gs_dtype x_dtype, int64_t rows,
                                               int64_t cols, fp8_format fmt, fp8_granularity g,
                                               fp8_scale_mode mode, uint8_t *codes,
                                               float *scales, int32_t *nonfinite, void *stream) {
    gs_status st = gsk::check_quantize(x, x_dtype, rows, cols, fmt, g, mode, codes, scales,
                                       nonfinite);
    if (st != GS_OK) return st;
    void *ws = nullptr;
    if (g == FP8_PER_TENSOR && mode == FP8_SCALE_FROM_AMAX) {
        if (fp8_quantize_workspace_size(rows, cols, g) > kScratchBytes) return GS_ERR_WORKSPACE;
        st = scratch_address(&ws);
        if (st != GS_OK) return st;
    }
    const hipError_t e = gsk::launch_quantize(x, x_dtype, rows, cols, fmt, g, mode, codes, scales,
                                              nonfinite, static_cast<uint32_t *>(ws),
                                              static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GS_OK : GS_ERR_HIP;
}
