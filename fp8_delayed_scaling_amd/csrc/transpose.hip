// transpose.hip -- FP8 -> FP8 transpose of a tensor that already exists: the lazy fill of a
// Float8Tensor's transpose cache ("[PyTorch] Refactor FP8 workspaces in linear modules",
// "grown in scope" first bullet: transpose_2d(cache=True) and lazy transpose caching;
// "[PyTorch] cuda graph support", transpose-cache thread: the transpose of an FP8 dy that
// carries no cache, and the noop flag in transpose that keeps a cached weight transpose across
// microbatches).  Codes are moved, never re-encoded.
//
// HBM-bound: 1 byte read + 1 byte written per element.  A block of 256 threads owns a 256 x 256
// byte tile and each thread one 16 x 16 byte block: 16 loads of 16 bytes (one row segment
// each), a register transpose made of sixteen 4 x 4 byte transposes, and 16 stores of 16 bytes
// (one segment of each of 16 output rows).  Lane l of wave w takes row block (w / 2) * 8 + l % 8
// and column block (w % 2) * 8 + l / 8, so one load instruction of a wave reads 8 rows x 128
// contiguous bytes and one store instruction writes 8 output rows x 128 contiguous bytes.  No
// LDS.  Tiles go row tiles fastest: the blocks resident at one time then cover many 256-byte
// column ranges of out_t, whose rows are `rows` bytes apart, instead of the few that column tiles
// fastest gives (measured on the same buffers: +7.7% at [8192, 12288], +8.8% at [18432, 12288],
// +18-22% at [16384, 12288], [8192, 18432] and [12288, 49152], +2-7% on [65536, 2048] and
// [2048, 65536], -0.8% at [49152, 12288], launch-bound sizes unchanged).  The vector path needs rows and cols multiples of 16 and 16-byte aligned buffers;
// otherwise each thread moves its block byte by byte with bounds checks.  Tensors of whole
// 512 x 256 tiles take k_fp8_transpose512 instead (below), which writes 512-byte output
// segments through LDS.
#include "device_common.h"
#include "launch.h"

namespace fp8ds {

namespace {
constexpr int kTT = 256;   // tile edge (bytes)
}  // namespace

template <bool VEC>
__global__ __launch_bounds__(256) void k_fp8_transpose(const uint8_t *__restrict__ in, int64_t rows, int64_t cols,
                                                       uint8_t *__restrict__ out_t, const float *__restrict__ noop,
                                                       int64_t tiles_r) {
    if (noop != nullptr && *noop == 1.0f) return;
    const int64_t tile = blockIdx.x;
    const int64_t r0 = (tile % tiles_r) * kTT, c0 = (tile / tiles_r) * kTT;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t rb = r0 + (int64_t)((wave >> 1) * 8 + (lane & 7)) * 16;
    const int64_t cb = c0 + (int64_t)((wave & 1) * 8 + (lane >> 3)) * 16;
    if (rb >= rows || cb >= cols) return;
    if constexpr (VEC) {
        // rows and cols are multiples of 16, so the whole 16 x 16 block is in range
        uint32_t R[16][4];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(in + (rb + j) * cols + cb));
            R[j][0] = v.x; R[j][1] = v.y; R[j][2] = v.z; R[j][3] = v.w;
        }
        uint32_t O[16][4];
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
            for (int d = 0; d < 4; ++d)
                tr4(R[4 * d][w], R[4 * d + 1][w], R[4 * d + 2][w], R[4 * d + 3][w], O[4 * w][d], O[4 * w + 1][d],
                    O[4 * w + 2][d], O[4 * w + 3][d]);
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const u32x4 v = {O[c][0], O[c][1], O[c][2], O[c][3]};
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(out_t + (cb + c) * rows + rb));
        }
    } else {
        for (int j = 0; j < 16 && rb + j < rows; ++j)
            for (int c = 0; c < 16 && cb + c < cols; ++c) out_t[(cb + c) * rows + rb + j] = in[(rb + j) * cols + cb + c];
    }
}

// Tensors of whole 512 x 256 byte tiles (rows % 512 == 0, cols % 256 == 0, 16-byte aligned):
// a 512-thread block per tile, each thread one 16 x 16 byte block (row block t / 16, column
// block t % 16) transposed in registers as above, then written to a 128 KB LDS tile
// T[256 output rows][512 bytes] (16-byte chunk k of output row o stored at chunk k ^ (o / 16), so
// the 16 column blocks of a wave's stores fall in distinct banks), read back as whole output
// rows: each output row of the tile leaves as one 512-byte segment (32 lanes).  Measured in one
// process on the same buffers against k_fp8_transpose: +6.7% at [8192, 12288], +1.9% at
// [8192, 18432], +0.3% at [18432, 12288].
constexpr int kTR512 = 512;
__global__ __launch_bounds__(512) void k_fp8_transpose512(const uint8_t *__restrict__ in, int64_t rows, int64_t cols,
                                                          uint8_t *__restrict__ out_t, const float *__restrict__ noop,
                                                          int64_t tiles_r) {
    __shared__ __align__(16) uint8_t T[kTT * kTR512];
    if (noop != nullptr && *noop == 1.0f) return;   // block-uniform: the whole block leaves
    const int64_t tile = blockIdx.x;
    const int64_t r0 = (tile % tiles_r) * kTR512, c0 = (tile / tiles_r) * kTT;
    const int t = threadIdx.x;
    const int cb = t & 15, rb = t >> 4;   // column block 0..15, row block 0..31
    const uint8_t *src = in + (r0 + rb * 16) * cols + c0 + cb * 16;
    uint32_t R[16][4];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + j * cols));
        R[j][0] = v.x; R[j][1] = v.y; R[j][2] = v.z; R[j][3] = v.w;
    }
    uint32_t O[16][4];
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int d = 0; d < 4; ++d)
            tr4(R[4 * d][w], R[4 * d + 1][w], R[4 * d + 2][w], R[4 * d + 3][w], O[4 * w][d], O[4 * w + 1][d],
                O[4 * w + 2][d], O[4 * w + 3][d]);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const int orow = cb * 16 + c;
        *reinterpret_cast<u32x4 *>(&T[orow * kTR512 + ((rb ^ cb) << 4)]) = u32x4{O[c][0], O[c][1], O[c][2], O[c][3]};
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int q = t + 512 * i;
        const int orow = q >> 5, p = q & 31;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(&T[orow * kTR512 + ((p ^ (orow >> 4)) << 4)]);
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(out_t + (c0 + orow) * rows + r0 + p * 16));
    }
}

hipError_t launch_fp8_transpose(const uint8_t *in, int64_t rows, int64_t cols, uint8_t *out_t, const float *noop,
                                hipStream_t st) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const int64_t tr = (rows + kTT - 1) / kTT, tc = (cols + kTT - 1) / kTT;
    const bool vec = rows % 16 == 0 && cols % 16 == 0 && (reinterpret_cast<uintptr_t>(in) & 15u) == 0 &&
                     (reinterpret_cast<uintptr_t>(out_t) & 15u) == 0;
    if (vec && rows % kTR512 == 0 && cols % kTT == 0) {
        const int64_t tr5 = rows / kTR512;
        k_fp8_transpose512<<<dim3((unsigned)(tr5 * tc)), dim3(512), 0, st>>>(in, rows, cols, out_t, noop, tr5);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)(tr * tc));
    if (vec)
        k_fp8_transpose<true><<<grid, dim3(256), 0, st>>>(in, rows, cols, out_t, noop, tr);
    else
        k_fp8_transpose<false><<<grid, dim3(256), 0, st>>>(in, rows, cols, out_t, noop, tr);
    return hipGetLastError();
}

}  // namespace fp8ds
