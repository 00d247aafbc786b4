// launch.h -- internal launchers behind the C ABI (host side; arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8ds {

hipError_t launch_cast_amax(const uint16_t *x, int64_t n, const float *scale, int fmt, uint8_t *out,
                            float *sinv_out, float *amax_slot, const float *noop, hipStream_t st);
hipError_t launch_cast_transpose(const uint16_t *x, int64_t rows, int64_t cols, const float *scale, int fmt,
                                 uint8_t *out, uint8_t *out_t, float *sinv_out, float *amax_slot,
                                 const float *noop, hipStream_t st);
// x0 and x1 cast+transposed (out_t may be nullptr: codes only) by one launch when both take the
// same code path, else by two; one FP8 format for both.
hipError_t launch_cast_transpose_pair(const uint16_t *x0, int64_t rows0, int64_t cols0, const float *scale0,
                                      uint8_t *out0, uint8_t *out_t0, float *sinv0, float *amax0, const float *noop0,
                                      const uint16_t *x1, int64_t rows1, int64_t cols1, const float *scale1,
                                      uint8_t *out1, uint8_t *out_t1, float *sinv1, float *amax1, const float *noop1,
                                      int fmt, hipStream_t st);
size_t dbias_workspace_bytes(int64_t rows, int64_t cols);
hipError_t launch_dbias_cast_transpose(const uint16_t *dy, int64_t rows, int64_t cols, const float *scale,
                                       int fmt, uint8_t *out, uint8_t *out_t, float *sinv_out,
                                       float *amax_slot, float *dbias, void *ws, hipStream_t st);

hipError_t launch_fp8_transpose(const uint8_t *in, int64_t rows, int64_t cols, uint8_t *out_t, const float *noop,
                                hipStream_t st);

constexpr int kMaxScaleTensors = 4096;
hipError_t launch_scale_update(float *hist, int64_t L, int64_t T, float *scale, float *scale_inv,
                               const int32_t *fmts_host, int32_t margin, hipStream_t st);

// out_dtype: 0 bfloat16, 1 float32, 2 E4M3, 3 E5M2 (the last two use d_scale, d_sinv_out, d_amax).
hipError_t launch_gemm_bias(const uint8_t *A, int fa, const float *a_sinv, int64_t lda, const uint8_t *B, int fb,
                            const float *b_sinv, int64_t ldb, const uint16_t *bias, void *D, int64_t ldd,
                            int out_dtype, int64_t M, int64_t N, int64_t K, const float *d_scale,
                            float *d_sinv_out, float *d_amax, hipStream_t st);

// The forward of a small layer (casts of x and W, GEMM + bias, bfloat16 y) in one launch, with
// the results of the cast-pair launch + GEMM launch; linear_fwd_small_ok says when it applies.
bool linear_fwd_small_ok(int64_t M, int64_t N, int64_t K, const uint8_t *x8_t);
hipError_t launch_linear_fwd_small(const uint16_t *x, const uint16_t *w, const uint16_t *bias, int64_t M, int64_t N,
                                   int64_t K, const float *x_scale, float *x_amax, uint8_t *x8, float *x_scale_inv,
                                   const float *w_scale, float *w_amax, uint8_t *w8, uint8_t *w8_t,
                                   float *w_scale_inv, const float *w_noop, uint16_t *y, hipStream_t st);

}  // namespace fp8ds
