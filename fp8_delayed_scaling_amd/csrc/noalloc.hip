// noalloc.hip -- the dbias + cast + transpose of dy for callers that cannot allocate device
// memory (code under graph capture, tight serving loops, harnesses that forbid allocation).
//
// fp8_dbias_cast_transpose needs scratch for its fixed-order partial column sums, which the
// caller normally passes in.  This variant keeps that scratch in a file-scope device array of
// kNoallocScratchBytes instead, so the caller passes only inputs and outputs.  Each GPU the
// library runs on holds its own copy of the array until the process ends.  Every call on a GPU
// uses that GPU's one array: calls that overlap in time on one GPU (two streams, or two host
// threads) race on it.  The partials are fully written before they are read within a call; the
// strip counters at the start of the array are zero when the library is loaded (static storage)
// and every call leaves them zero, so nothing needs clearing between calls.
//
// The array's name is only a host-side stand-in in host code; its device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and is what the kernels
// receive.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/fp8ds.h"
#include "launch.h"

namespace {

constexpr size_t kNoallocScratchBytes = size_t(8) << 20;   // FP8DS_NOALLOC_SCRATCH_BYTES
static_assert(kNoallocScratchBytes == FP8DS_NOALLOC_SCRATCH_BYTES, "header and library agree");

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// Device address of this device's scratch array, looked up on the first call per device.
int scratch_ptr(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8DS_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FP8DS_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FP8DS_OK;
}

}  // namespace

extern "C" int fp8_dbias_cast_transpose_noalloc(const uint16_t *dy, int64_t rows, int64_t cols, const float *scale,
                                                int fmt, uint8_t *out, uint8_t *out_t, float *scale_inv_out,
                                                float *amax_slot, float *dbias, hipStream_t stream) {
    if (rows < 0 || cols < 0) return FP8DS_ERR_SHAPE;
    const size_t need = fp8_dbias_workspace_bytes(rows, cols);
    if (need > kNoallocScratchBytes) return FP8DS_ERR_SCRATCH;
    void *ws = nullptr;
    if (need > 0) {
        const int st = scratch_ptr(&ws);
        if (st != FP8DS_OK) return st;
    }
    // the regular entry point validates everything else and launches the same kernels
    return fp8_dbias_cast_transpose(dy, rows, cols, scale, fmt, out, out_t, scale_inv_out, amax_slot, dbias, ws,
                                    need > 0 ? kNoallocScratchBytes : 0, stream);
}
