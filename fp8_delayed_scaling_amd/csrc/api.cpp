// api.cpp -- the extern "C" boundary of libfp8ds.so (declared in include/fp8ds.h).
//
// Host-side argument checks, then kernel launches on the caller's stream.  Nothing here
// allocates device memory, copies between host and device or synchronises; a rejected call
// launches nothing.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <mutex>

#include "../../include/fp8ds.h"
#include "launch.h"

namespace {

using fp8ds::kMaxScaleTensors;

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline bool valid_fmt(int f) { return f == FP8DS_E4M3 || f == FP8DS_E5M2; }
inline bool valid_out(int d) { return d == FP8DS_OUT_BF16 || d == FP8DS_OUT_FP32; }
// Output codes of the GEMM launcher: the two public dtypes, then FP8 output in each format.
constexpr int kOutE4M3 = 2, kOutE5M2 = 3;
inline int64_t out_esize(int d) { return d == FP8DS_OUT_BF16 ? 2 : d == FP8DS_OUT_FP32 ? 4 : 1; }
inline int hip_status(hipError_t e) { return e == hipSuccess ? FP8DS_OK : FP8DS_ERR_HIP; }

// rows * cols fits comfortably in int64 (and in the kernels' index arithmetic)
inline bool size_ok(int64_t rows, int64_t cols) {
    if (rows < 0 || cols < 0) return false;
    if (rows == 0 || cols == 0) return true;
    return rows <= (INT64_C(1) << 40) / cols;
}

// The cast kernels take one 256 x 256 tile per workgroup, numbered in 32 bits; a launch holds at
// most two tensors.
inline bool ct_tiles_ok(int64_t rows, int64_t cols) {
    return ((rows + 255) / 256) * ((cols + 255) / 256) <= INT_MAX / 2;
}

int check_cast_common(const uint16_t *x, const float *scale, int fmt, const uint8_t *out, const float *sinv,
                      const float *amax, const float *noop) {
    if (!valid_fmt(fmt)) return FP8DS_ERR_FORMAT;
    if (x == nullptr || scale == nullptr || out == nullptr) return FP8DS_ERR_NULL;
    if (!aligned16(x) || !aligned16(out) || !aligned4(scale)) return FP8DS_ERR_ALIGN;
    if ((sinv && !aligned4(sinv)) || (amax && !aligned4(amax)) || (noop && !aligned4(noop))) return FP8DS_ERR_ALIGN;
    return FP8DS_OK;
}

int check_gemm(const uint8_t *A, int fa, const float *a_sinv, int64_t lda, const uint8_t *B, int fb,
               const float *b_sinv, int64_t ldb, const uint16_t *bias, const void *D, int64_t ldd, int out_dtype,
               int64_t M, int64_t N, int64_t K) {
    if (!valid_fmt(fa) || !valid_fmt(fb) || out_dtype < 0 || out_dtype > kOutE5M2) return FP8DS_ERR_FORMAT;
    if (M < 0 || N < 0 || K < 0 || M > INT_MAX || N > INT_MAX || K > INT_MAX) return FP8DS_ERR_SHAPE;
    if (K % 16 != 0) return FP8DS_ERR_SHAPE;
    if (((M + 255) / 256) * ((N + 255) / 256) > INT_MAX) return FP8DS_ERR_SHAPE;
    if (M == 0 || N == 0) return FP8DS_OK;
    if (D == nullptr) return FP8DS_ERR_NULL;
    if (K > 0 && (A == nullptr || B == nullptr || a_sinv == nullptr || b_sinv == nullptr)) return FP8DS_ERR_NULL;
    if (K > 0 && (lda < K || ldb < K)) return FP8DS_ERR_SHAPE;
    if (ldd < N) return FP8DS_ERR_SHAPE;
    const uintptr_t esize = (uintptr_t)out_esize(out_dtype);
    if ((reinterpret_cast<uintptr_t>(D) & (esize - 1)) != 0) return FP8DS_ERR_ALIGN;
    if (K > 0 && (lda % 16 != 0 || ldb % 16 != 0 || !aligned16(A) || !aligned16(B))) return FP8DS_ERR_ALIGN;
    if ((a_sinv && !aligned4(a_sinv)) || (b_sinv && !aligned4(b_sinv))) return FP8DS_ERR_ALIGN;
    if (bias != nullptr && (reinterpret_cast<uintptr_t>(bias) & 1u)) return FP8DS_ERR_ALIGN;
    if (!size_ok(M, ldd) || !size_ok(M, lda) || !size_ok(N, ldb)) return FP8DS_ERR_SHAPE;
    return FP8DS_OK;
}

// Events for the chunked GEMM's fork / join, created once per device on first use and kept
// for the life of the process (event objects, not device memory).  A stream waits on the
// event's most recent record at the time of the wait call, so one call's whole record / wait
// sequence is enqueued under the device's lock: concurrent host threads cannot interleave
// their records with another call's waits.
constexpr int kMaxChunks = 16;
constexpr int kMaxDevices = 64;
struct ChunkEvents {
    hipEvent_t fork = nullptr;
    hipEvent_t join[kMaxChunks] = {};
    bool ready = false;
    std::mutex mu;   // held while a chunked call enqueues its records, waits and launches
};
ChunkEvents g_events[kMaxDevices];
std::mutex g_events_mu;

int chunk_events(ChunkEvents **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8DS_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_events_mu);
    ChunkEvents &ev = g_events[dev];
    if (!ev.ready) {
        if (hipEventCreateWithFlags(&ev.fork, hipEventDisableTiming) != hipSuccess) return FP8DS_ERR_HIP;
        for (int i = 0; i < kMaxChunks; ++i)
            if (hipEventCreateWithFlags(&ev.join[i], hipEventDisableTiming) != hipSuccess) return FP8DS_ERR_HIP;
        ev.ready = true;
    }
    *out = &ev;
    return FP8DS_OK;
}

}  // namespace

extern "C" {

const char *fp8ds_status_string(int status) {
    switch (status) {
        case FP8DS_OK: return "FP8DS_OK";
        case FP8DS_ERR_NULL: return "FP8DS_ERR_NULL: a required pointer is NULL";
        case FP8DS_ERR_SHAPE: return "FP8DS_ERR_SHAPE: invalid size";
        case FP8DS_ERR_ALIGN: return "FP8DS_ERR_ALIGN: misaligned pointer or leading dimension";
        case FP8DS_ERR_FORMAT: return "FP8DS_ERR_FORMAT: unknown FP8 format or output dtype";
        case FP8DS_ERR_WORKSPACE: return "FP8DS_ERR_WORKSPACE: workspace missing or too small";
        case FP8DS_ERR_HIP: return "FP8DS_ERR_HIP: the HIP runtime reported an error";
        case FP8DS_ERR_ARG: return "FP8DS_ERR_ARG: argument out of range";
        case FP8DS_ERR_SCRATCH: return "FP8DS_ERR_SCRATCH: problem larger than the library's static scratch";
        default: return "FP8DS: unknown status";
    }
}

int fp8ds_version(void) { return 100; }

int fp8_cast_amax(const uint16_t *x, int64_t numel, const float *scale, int fmt, uint8_t *out,
                  float *scale_inv_out, float *amax_slot, const float *noop, hipStream_t stream) {
    if (numel < 0 || numel > (INT64_C(1) << 40)) return FP8DS_ERR_SHAPE;
    if (!valid_fmt(fmt)) return FP8DS_ERR_FORMAT;
    if (numel == 0) return FP8DS_OK;
    int st = check_cast_common(x, scale, fmt, out, scale_inv_out, amax_slot, noop);
    if (st != FP8DS_OK) return st;
    return hip_status(fp8ds::launch_cast_amax(x, numel, scale, fmt, out, scale_inv_out, amax_slot, noop, stream));
}

int fp8_cast_transpose(const uint16_t *x, int64_t rows, int64_t cols, const float *scale, int fmt, uint8_t *out,
                       uint8_t *out_t, float *scale_inv_out, float *amax_slot, const float *noop,
                       hipStream_t stream) {
    if (!size_ok(rows, cols) || !ct_tiles_ok(rows, cols)) return FP8DS_ERR_SHAPE;
    if (!valid_fmt(fmt)) return FP8DS_ERR_FORMAT;
    if (rows == 0 || cols == 0) return FP8DS_OK;
    int st = check_cast_common(x, scale, fmt, out, scale_inv_out, amax_slot, noop);
    if (st != FP8DS_OK) return st;
    if (out_t == nullptr) return FP8DS_ERR_NULL;
    if (!aligned16(out_t)) return FP8DS_ERR_ALIGN;
    return hip_status(fp8ds::launch_cast_transpose(x, rows, cols, scale, fmt, out, out_t, scale_inv_out, amax_slot,
                                                   noop, stream));
}

size_t fp8_dbias_workspace_bytes(int64_t rows, int64_t cols) {
    if (!size_ok(rows, cols)) return 0;
    return fp8ds::dbias_workspace_bytes(rows, cols);
}

int fp8_dbias_cast_transpose(const uint16_t *dy, int64_t rows, int64_t cols, const float *scale, int fmt,
                             uint8_t *out, uint8_t *out_t, float *scale_inv_out, float *amax_slot, float *dbias,
                             void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!size_ok(rows, cols) || !ct_tiles_ok(rows, cols)) return FP8DS_ERR_SHAPE;
    if (!valid_fmt(fmt)) return FP8DS_ERR_FORMAT;
    if (cols == 0) return FP8DS_OK;
    if (dbias == nullptr) return FP8DS_ERR_NULL;
    if (!aligned4(dbias)) return FP8DS_ERR_ALIGN;
    if (rows > 0) {
        int st = check_cast_common(dy, scale, fmt, out, scale_inv_out, amax_slot, nullptr);
        if (st != FP8DS_OK) return st;
        if (out_t == nullptr) return FP8DS_ERR_NULL;
        if (!aligned16(out_t)) return FP8DS_ERR_ALIGN;
        const size_t need = fp8ds::dbias_workspace_bytes(rows, cols);
        if (workspace == nullptr || workspace_bytes < need) return FP8DS_ERR_WORKSPACE;
        if (!aligned4(workspace)) return FP8DS_ERR_ALIGN;
    }
    return hip_status(fp8ds::launch_dbias_cast_transpose(dy, rows, cols, scale, fmt, out, out_t, scale_inv_out,
                                                         amax_slot, dbias, workspace, stream));
}

int fp8_scale_update(float *amax_history, int64_t L, int64_t T, float *scale, float *scale_inv,
                     const int32_t *fmts, int32_t margin, hipStream_t stream) {
    if (L < 1 || T < 1 || T > kMaxScaleTensors || !size_ok(L, T)) return FP8DS_ERR_SHAPE;
    if (margin < -126 || margin > 126) return FP8DS_ERR_ARG;
    if (amax_history == nullptr || scale == nullptr || scale_inv == nullptr || fmts == nullptr)
        return FP8DS_ERR_NULL;
    if (!aligned4(amax_history) || !aligned4(scale) || !aligned4(scale_inv)) return FP8DS_ERR_ALIGN;
    for (int64_t t = 0; t < T; ++t)
        if (!valid_fmt(fmts[t])) return FP8DS_ERR_FORMAT;
    return hip_status(fp8ds::launch_scale_update(amax_history, L, T, scale, scale_inv, fmts, margin, stream));
}

int fp8_gemm_bias(const uint8_t *A, int fa, const float *a_scale_inv, int64_t lda, const uint8_t *B, int fb,
                  const float *b_scale_inv, int64_t ldb, const uint16_t *bias, void *D, int64_t ldd, int out_dtype,
                  int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    if (!valid_out(out_dtype)) return FP8DS_ERR_FORMAT;
    int st = check_gemm(A, fa, a_scale_inv, lda, B, fb, b_scale_inv, ldb, bias, D, ldd, out_dtype, M, N, K);
    if (st != FP8DS_OK) return st;
    return hip_status(fp8ds::launch_gemm_bias(A, fa, a_scale_inv, lda, B, fb, b_scale_inv, ldb, bias, D, ldd,
                                              out_dtype, M, N, K, nullptr, nullptr, nullptr, stream));
}

int fp8_gemm_bias_fp8(const uint8_t *A, int fa, const float *a_scale_inv, int64_t lda, const uint8_t *B, int fb,
                      const float *b_scale_inv, int64_t ldb, const uint16_t *bias, uint8_t *D, int64_t ldd,
                      int d_fmt, const float *d_scale, float *d_scale_inv_out, float *d_amax_slot, int64_t M,
                      int64_t N, int64_t K, hipStream_t stream) {
    if (!valid_fmt(d_fmt)) return FP8DS_ERR_FORMAT;
    if (d_scale == nullptr) return FP8DS_ERR_NULL;
    if (!aligned4(d_scale) || (d_scale_inv_out && !aligned4(d_scale_inv_out)) || (d_amax_slot && !aligned4(d_amax_slot)))
        return FP8DS_ERR_ALIGN;
    const int out = d_fmt == FP8DS_E4M3 ? kOutE4M3 : kOutE5M2;
    int st = check_gemm(A, fa, a_scale_inv, lda, B, fb, b_scale_inv, ldb, bias, D, ldd, out, M, N, K);
    if (st != FP8DS_OK) return st;
    return hip_status(fp8ds::launch_gemm_bias(A, fa, a_scale_inv, lda, B, fb, b_scale_inv, ldb, bias, D, ldd, out,
                                              M, N, K, d_scale, d_scale_inv_out, d_amax_slot, stream));
}

int fp8_transpose(const uint8_t *in, int64_t rows, int64_t cols, uint8_t *out_t, const float *noop,
                  hipStream_t stream) {
    if (!size_ok(rows, cols)) return FP8DS_ERR_SHAPE;
    if (rows == 0 || cols == 0) return FP8DS_OK;
    if (((rows + 255) / 256) * ((cols + 255) / 256) > INT_MAX) return FP8DS_ERR_SHAPE;
    if (in == nullptr || out_t == nullptr) return FP8DS_ERR_NULL;
    if (noop && !aligned4(noop)) return FP8DS_ERR_ALIGN;
    return hip_status(fp8ds::launch_fp8_transpose(in, rows, cols, out_t, noop, stream));
}

int fp8_gemm_bias_chunked(const uint8_t *A, int fa, const float *a_scale_inv, int64_t lda, const uint8_t *B, int fb,
                          const float *b_scale_inv, int64_t ldb, const uint16_t *bias, void *D, int64_t ldd,
                          int out_dtype, int64_t M, int64_t N, int64_t K, int n_chunks,
                          const hipStream_t *chunk_streams, hipStream_t stream) {
    if (n_chunks < 1 || n_chunks > kMaxChunks) return FP8DS_ERR_ARG;
    if (!valid_out(out_dtype)) return FP8DS_ERR_FORMAT;
    int st = check_gemm(A, fa, a_scale_inv, lda, B, fb, b_scale_inv, ldb, bias, D, ldd, out_dtype, M, N, K);
    if (st != FP8DS_OK) return st;
    if (M == 0 || N == 0) return FP8DS_OK;
    const int64_t esize = out_dtype == FP8DS_OUT_BF16 ? 2 : 4;
    int64_t nc = (N + n_chunks - 1) / n_chunks;
    nc = (nc + 15) / 16 * 16;   // chunk starts stay 16-byte aligned in D for both dtypes
    ChunkEvents *ev = nullptr;
    std::unique_lock<std::mutex> seq;
    if (chunk_streams != nullptr) {
        st = chunk_events(&ev);
        if (st != FP8DS_OK) return st;
        seq = std::unique_lock<std::mutex>(ev->mu);
        if (hipEventRecord(ev->fork, stream) != hipSuccess) return FP8DS_ERR_HIP;
    }
    for (int c = 0; c < n_chunks; ++c) {
        const int64_t c0 = c * nc;
        if (c0 >= N) break;
        const int64_t cn = (N - c0 < nc) ? N - c0 : nc;
        hipStream_t s = chunk_streams != nullptr ? chunk_streams[c] : stream;
        if (chunk_streams != nullptr && hipStreamWaitEvent(s, ev->fork, 0) != hipSuccess) return FP8DS_ERR_HIP;
        hipError_t e = fp8ds::launch_gemm_bias(A, fa, a_scale_inv, lda, B + c0 * ldb, fb, b_scale_inv, ldb,
                                               bias != nullptr ? bias + c0 : nullptr,
                                               static_cast<uint8_t *>(D) + c0 * esize, ldd, out_dtype, M, cn, K,
                                               nullptr, nullptr, nullptr, s);
        if (e != hipSuccess) return FP8DS_ERR_HIP;
        if (chunk_streams != nullptr) {
            if (hipEventRecord(ev->join[c], s) != hipSuccess) return FP8DS_ERR_HIP;
            if (hipStreamWaitEvent(stream, ev->join[c], 0) != hipSuccess) return FP8DS_ERR_HIP;
        }
    }
    return FP8DS_OK;
}

int fp8_linear_fwd(const uint16_t *x, const uint16_t *w, const uint16_t *bias, int64_t M, int64_t N, int64_t K,
                   const float *x_scale, float *x_amax, uint8_t *x8, uint8_t *x8_t, float *x_scale_inv,
                   const float *w_scale, float *w_amax, uint8_t *w8, uint8_t *w8_t, float *w_scale_inv,
                   const float *w_noop, uint16_t *y, hipStream_t stream) {
    if (M < 0 || N < 0 || K < 0 || !size_ok(M, K) || !size_ok(N, K) || !size_ok(M, N)) return FP8DS_ERR_SHAPE;
    if (!ct_tiles_ok(M, K) || !ct_tiles_ok(N, K)) return FP8DS_ERR_SHAPE;
    if (K % 16 != 0) return FP8DS_ERR_SHAPE;
    if (M == 0 || N == 0) return FP8DS_OK;
    if (y == nullptr || x_scale_inv == nullptr || w_scale_inv == nullptr) return FP8DS_ERR_NULL;
    if (w8_t == nullptr && K > 0) return FP8DS_ERR_NULL;
    int st;
    if (K > 0) {
        st = check_cast_common(x, x_scale, FP8DS_E4M3, x8, x_scale_inv, x_amax, nullptr);
        if (st != FP8DS_OK) return st;
        st = check_cast_common(w, w_scale, FP8DS_E4M3, w8, w_scale_inv, w_amax, w_noop);
        if (st != FP8DS_OK) return st;
        if ((x8_t && !aligned16(x8_t)) || !aligned16(w8_t)) return FP8DS_ERR_ALIGN;
    }
    st = check_gemm(x8, FP8DS_E4M3, x_scale_inv, K, w8, FP8DS_E4M3, w_scale_inv, K, bias, y, N, FP8DS_OUT_BF16, M,
                    N, K);
    if (st != FP8DS_OK) return st;
    if (fp8ds::linear_fwd_small_ok(M, N, K, x8_t))
        return hip_status(fp8ds::launch_linear_fwd_small(x, w, bias, M, N, K, x_scale, x_amax, x8, x_scale_inv,
                                                         w_scale, w_amax, w8, w8_t, w_scale_inv, w_noop, y, stream));
    if (K > 0) {
        // x (with or without its transpose) and W in one launch
        hipError_t e = fp8ds::launch_cast_transpose_pair(x, M, K, x_scale, x8, x8_t, x_scale_inv, x_amax, nullptr,
                                                         w, N, K, w_scale, w8, w8_t, w_scale_inv, w_amax, w_noop,
                                                         FP8DS_E4M3, stream);
        if (e != hipSuccess) return FP8DS_ERR_HIP;
    }
    return hip_status(fp8ds::launch_gemm_bias(x8, FP8DS_E4M3, x_scale_inv, K, w8, FP8DS_E4M3, w_scale_inv, K, bias,
                                              y, N, FP8DS_OUT_BF16, M, N, K, nullptr, nullptr, nullptr, stream));
}

int fp8_linear_bwd(const uint16_t *dy, int64_t M, int64_t N, int64_t K, const float *dy_scale, float *dy_amax,
                   uint8_t *dy8, uint8_t *dy8_t, float *dy_scale_inv, float *dbias, void *workspace,
                   size_t workspace_bytes, const uint8_t *x8_t, const float *x_scale_inv, const uint8_t *w8_t,
                   const float *w_scale_inv, uint16_t *dx, void *dw, int dw_dtype, hipStream_t stream) {
    if (M < 0 || N < 0 || K < 0 || !size_ok(M, N) || !size_ok(M, K) || !size_ok(N, K)) return FP8DS_ERR_SHAPE;
    if (!ct_tiles_ok(M, N)) return FP8DS_ERR_SHAPE;
    if (M % 16 != 0 || N % 16 != 0) return FP8DS_ERR_SHAPE;
    if (!valid_out(dw_dtype)) return FP8DS_ERR_FORMAT;
    if (M == 0 || N == 0 || K == 0) return FP8DS_ERR_SHAPE;
    int st = check_cast_common(dy, dy_scale, FP8DS_E5M2, dy8, dy_scale_inv, dy_amax, nullptr);
    if (st != FP8DS_OK) return st;
    if (dy8_t == nullptr || dy_scale_inv == nullptr) return FP8DS_ERR_NULL;
    if (!aligned16(dy8_t)) return FP8DS_ERR_ALIGN;
    if (dbias != nullptr) {
        if (!aligned4(dbias)) return FP8DS_ERR_ALIGN;
        if (workspace == nullptr || workspace_bytes < fp8ds::dbias_workspace_bytes(M, N)) return FP8DS_ERR_WORKSPACE;
        if (!aligned4(workspace)) return FP8DS_ERR_ALIGN;
    }
    // dgrad: A = dy8 [M, N] (E5M2), B = w8_t [K, N] (E4M3) -> dx [M, K]
    st = check_gemm(dy8, FP8DS_E5M2, dy_scale_inv, N, w8_t, FP8DS_E4M3, w_scale_inv, N, nullptr, dx, K,
                    FP8DS_OUT_BF16, M, K, N);
    if (st != FP8DS_OK) return st;
    // wgrad: A = dy8_t [N, M] (E5M2), B = x8_t [K, M] (E4M3) -> dW [N, K]
    st = check_gemm(dy8_t, FP8DS_E5M2, dy_scale_inv, M, x8_t, FP8DS_E4M3, x_scale_inv, M, nullptr, dw, K, dw_dtype, N,
                    K, M);
    if (st != FP8DS_OK) return st;
    hipError_t e = dbias != nullptr
                       ? fp8ds::launch_dbias_cast_transpose(dy, M, N, dy_scale, FP8DS_E5M2, dy8, dy8_t, dy_scale_inv,
                                                            dy_amax, dbias, workspace, stream)
                       : fp8ds::launch_cast_transpose(dy, M, N, dy_scale, FP8DS_E5M2, dy8, dy8_t, dy_scale_inv,
                                                      dy_amax, nullptr, stream);
    if (e != hipSuccess) return FP8DS_ERR_HIP;
    e = fp8ds::launch_gemm_bias(dy8, FP8DS_E5M2, dy_scale_inv, N, w8_t, FP8DS_E4M3, w_scale_inv, N, nullptr, dx, K,
                                FP8DS_OUT_BF16, M, K, N, nullptr, nullptr, nullptr, stream);
    if (e != hipSuccess) return FP8DS_ERR_HIP;
    return hip_status(fp8ds::launch_gemm_bias(dy8_t, FP8DS_E5M2, dy_scale_inv, M, x8_t, FP8DS_E4M3, x_scale_inv, M,
                                              nullptr, dw, K, dw_dtype, N, K, M, nullptr, nullptr, nullptr, stream));
}

}  // extern "C"
