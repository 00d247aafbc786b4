// cast.hip -- the cast family of the FP8 delayed-scaling path on gfx950:
//   cast + amax                  (Float8Tensor.to_float8 in "[PyTorch] cuda graph support",
//                                 transpose-cache thread)
//   cast + transpose + amax      (the transpose cache of "[PyTorch] Refactor FP8 workspaces in
//                                 linear modules", "grown in scope" first bullet)
//   dbias + cast + transpose     (DbiasCastTranspose in "[PyTorch] cuda graph support")
//
// All three are HBM-streaming kernels.  Reads are 16-byte per lane and coalesced along rows;
// the FP8 codes are produced by the hardware converter after a v_med3 clamp (saturation);
// each row's codes are converted once, and the transposed copy is made from them by 4 x 4 byte
// transposes in registers (v_perm_b32) staged through an LDS tile, so both outputs leave in
// coalesced stores.  dbias + cast + transpose has two forms: the tile kernel writing per-tile
// column sums plus a reduction launch, and a one-launch strip form for tensors of few whole
// tiles.  The amax is a packed 16-bit integer max of the bfloat16 magnitudes, reduced per wave
// and per block, with one atomic per block.
#include <algorithm>

#include "../../include/fp8ds.h"
#include "device_common.h"
#include "launch.h"

namespace fp8ds {

// ------------------------------------------------------------------------------------------
// 1-D cast + amax.  A thread converts one 16-element group (two 16-byte loads, one 16-byte
// store), one block of 256 threads per 4096 elements, so a launch of any size up to 2^32
// elements takes its groups in one pass (a grid-stride loop covers larger ones); a remainder of
// up to 15 elements is converted element by element.  Measured on the same buffers at
// [8192, 12288] (cold): 50.2 us (75% of 8 TB/s) against 56.3 us for a grid-stride loop over 2048
// blocks with two groups per thread per step, 53-56 us with 4096-8192 blocks.
// ------------------------------------------------------------------------------------------
template <int FMT>
__device__ __forceinline__ u32x4 cast16(const u32x4 &p, const u32x4 &q, float s, bool fast) {
    const uint32_t w[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
    uint32_t o[4];
    if (fast) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = pack4<FMT>(clamp_fmt<FMT>(bf16_lo(w[2 * i]) * s), clamp_fmt<FMT>(bf16_hi(w[2 * i]) * s),
                              clamp_fmt<FMT>(bf16_lo(w[2 * i + 1]) * s), clamp_fmt<FMT>(bf16_hi(w[2 * i + 1]) * s));
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = encode_exact<FMT>(bf16_lo(w[2 * i]) * s) | (encode_exact<FMT>(bf16_hi(w[2 * i]) * s) << 8) |
                   (encode_exact<FMT>(bf16_lo(w[2 * i + 1]) * s) << 16) |
                   (encode_exact<FMT>(bf16_hi(w[2 * i + 1]) * s) << 24);
    }
    return u32x4{o[0], o[1], o[2], o[3]};
}

__device__ __forceinline__ uint32_t amax_vec(uint32_t acc, const u32x4 &v) {
    acc = amax_pk(acc, v.x);
    acc = amax_pk(acc, v.y);
    acc = amax_pk(acc, v.z);
    return amax_pk(acc, v.w);
}

constexpr int64_t kCastMaxBlocks = INT64_C(1) << 20;

template <int FMT>
__global__ __launch_bounds__(256) void k_cast_amax(const uint16_t *__restrict__ x, int64_t n,
                                                   const float *__restrict__ scale_p,
                                                   uint8_t *__restrict__ out,
                                                   float *__restrict__ sinv_out, float *amax_slot,
                                                   const float *__restrict__ noop) {
    __shared__ uint32_t red[4];
    if (noop != nullptr && *noop == 1.0f) return;
    const float s = *scale_p;
    const bool plain = scale_is_plain(s);
    uint32_t am = 0;
    const int64_t nvec = n >> 4;                       // 16-element groups
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(x + (v << 4));
        const u32x4 p = __builtin_nontemporal_load(src), q = __builtin_nontemporal_load(src + 1);
        const uint32_t tam = amax_vec(amax_vec(0u, p), q);
        const bool fast = plain && amax_unpack(tam) < 0x7F80u;
        am = amax_pk(am, tam);
        __builtin_nontemporal_store(cast16<FMT>(p, q, s, fast), reinterpret_cast<u32x4 *>(out + (v << 4)));
    }
    // remainder
    for (int64_t i = (nvec << 4) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        uint32_t w = x[i];
        am = amax_pk(am, w);
        out[i] = (uint8_t)encode_exact<FMT>(bf16_lo(w) * s);
    }
    uint32_t bm = block_max_u32<256>(amax_unpack(am), red);
    if (threadIdx.x == 0) {
        fold_amax(amax_slot, bm);
        if (blockIdx.x == 0 && sinv_out != nullptr) *sinv_out = 1.0f / s;
    }
}

// ------------------------------------------------------------------------------------------
// 2-D cast + transpose (+ dbias partials).  A 1024-thread block owns a 256 x 256 tile; thread
// (rb = t / 32, cb = t % 32) owns the 8 x 8 micro-tile at rows 8rb.., columns 8cb...
//   loads   : eight 16-byte row segments (32 lanes = 512 B of one row; a wave reads 2 rows);
//   out     : each row's eight codes converted once (clamp + hardware conversion, four values
//             per dword) -> one 8-byte store per row (32 lanes = 256 B per row);
//   out_t   : the 8 x 8 byte block of codes transposed in registers (4 x 4 byte transposes,
//             v_perm_b32) -> one 8-byte fragment per column into the LDS tile T[col][row] ->
//             after a barrier 16-byte row chunks of the transposed tile (16 lanes = 256 B per
//             transposed row);
//   dbias   : per-column sums of the micro-tile, reduced over the 32 row blocks through LDS in
//             a fixed order, one partial per (256-row tile, column) into the workspace.
// With 256 rows per tile every transposed row segment is 256 contiguous bytes.  Measured on the
// same buffers against 128-row x 256-column tiles of 512 threads: +5.3% at [8192, 12288],
// +1.3% for the [8192, 18432] gradient, +10% at [8192, 4096], +18% at [4096, 4096] (one block
// wave instead of two), -0.6% for the [18432, 12288] weight; 256-row tiles of 512 threads, or
// 1024-thread blocks held to 64 registers (two blocks per CU, with spills), were slower, and
// 512-byte transposed segments (two stacked tiles per block) gained nothing.
// VEC: cols % 8 == 0 and rows % 16 == 0, so every 16-byte load, 8-byte store and 16-byte
// transposed store is either wholly inside the tensor or wholly outside.  Otherwise each element
// is loaded and stored on its own with bounds checks (same tile structure).
// ------------------------------------------------------------------------------------------
constexpr int kTile = 256;                // tile rows (also the dbias partial granularity)
constexpr int kTileC = 256;               // tile columns
constexpr int kCtThreads = (kTile / 8) * (kTileC / 8);   // 1024
constexpr int kRowBlocks = kTile / 8;                    // 32
// The transposed tile lives in LDS as T[col][row] (256 x 256 bytes, no padding).  The 8-byte
// fragment of row block rb in transposed row `col` sits at slot rb ^ ((col >> 3) & 31): the
// lanes that write one row block all hit different 8-byte slots, and a 16-byte read of chunk p
// finds its two halves at slots 2p ^ g and (2p + 1) ^ g, i.e. in 16-byte chunk p ^ (g >> 1),
// swapped when g is odd.
__device__ __forceinline__ int t_swz(int col) { return (col >> 3) & (kRowBlocks - 1); }

// One tensor of a cast launch.  out_t == nullptr: row-major codes only (no transpose cache).
struct CtTensor {
    const uint16_t *x;
    int64_t rows, cols;
    const float *scale;
    uint8_t *out, *out_t;
    float *sinv_out, *amax_slot;
    const float *noop;
};
// Up to two tensors cast by one launch (the forward pass casts x and W together): blocks
// [0, first1) take tiles of t[0], blocks [first1, ...) tiles of t[1].
struct CtBatch {
    CtTensor t[2];
    int64_t first1;
};

// Tile order.  With column tiles fastest, the ~256 blocks resident at once cover only about
// 256 / tiles_c row tiles, so their transposed stores all fall in the same few 256-byte column
// ranges of out_t, rows of out_t being `rows` bytes apart.  When that stride is a multiple of
// 4 KB the stores crowd onto few HBM channels.  Such tensors (rows % 4096 == 0, at least two
// bands of 16 row tiles, and at least 32 column tiles) take their tiles in bands of 16 row
// tiles (4096 rows), row tiles fastest inside a band.  Measured on the same buffers against
// column tiles fastest: +2% at [8192, 12288], +11% for the [8192, 18432] gradient, +5% at
// [12288, 12288], +9% at [16384, 12288]; against bands of 8 or 32 row tiles: 3-13% and 6-12%
// faster at those shapes; against a band order that alternates blocks between two bands, or a
// pseudo-random order, 4-10% faster.  The [18432, 12288] weight (stride not a multiple of 4 KB)
// and the 16-column-tile [8192, 4096] gradient are faster in the default order.
constexpr int kRowBand = 16;
// (32-bit arithmetic: the host rejects tensors of 2^31 tiles or more.)
__device__ __forceinline__ void ct_tile_of(uint32_t block, int64_t rows, uint32_t tiles_c, uint32_t &tile_r,
                                           uint32_t &tile_c) {
    if (rows % 4096 == 0 && rows >= 2 * kRowBand * kTile && tiles_c >= 32) {
        // rows is a multiple of 16 tiles, so every band is full
        const uint32_t per = kRowBand * tiles_c, g = block / per, local = block - g * per;
        tile_r = g * kRowBand + local % kRowBand;
        tile_c = local / kRowBand;
    } else {
        tile_r = block / tiles_c;
        tile_c = block - tile_r * tiles_c;
    }
}

// Sum of 16 values as a balanced tree (adjacent pairs first), so that a column sum's rounding
// depth grows by 4 per 16 partials instead of by 16.
__device__ __forceinline__ float sum16_pairwise(const float (&v)[16]) {
    float a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = v[2 * u] + v[2 * u + 1];
#pragma unroll
    for (int u = 0; u < 4; ++u) a[u] = a[2 * u] + a[2 * u + 1];
    return (a[0] + a[1]) + (a[2] + a[3]);
}

template <int FMT, bool VEC, bool DBIAS, int TS = kTile>
__global__ __launch_bounds__((TS / 8) * (TS / 8)) void k_cast_transpose(const CtBatch batch, float *__restrict__ partial) {
    // TS x TS tiles: 256 (1024 threads) in general, 64 (64 threads) for tensors of few tiles
    constexpr int NRB = TS / 8, NT = NRB * NRB, CH = TS / 16;
    static_assert(!DBIAS || TS == kTile, "the dbias partials are per 256-row tile");
    __shared__ __align__(16) uint8_t tT[TS * TS];
    __shared__ float csum[DBIAS ? kRowBlocks * kTileC : 1];
    __shared__ uint32_t red[NT / 64];
    // Both tensors' fields are kernel arguments: selecting values (not a pointer to one tensor)
    // lets every argument load go out in one round, and the first input loads follow it.
    const bool second = (int64_t)blockIdx.x >= batch.first1;
    const uint16_t *__restrict__ x = second ? batch.t[1].x : batch.t[0].x;
    const int64_t rows = second ? batch.t[1].rows : batch.t[0].rows;
    const int64_t cols = second ? batch.t[1].cols : batch.t[0].cols;
    uint8_t *__restrict__ out = second ? batch.t[1].out : batch.t[0].out;
    uint8_t *__restrict__ out_t = second ? batch.t[1].out_t : batch.t[0].out_t;
    const float *noop = second ? batch.t[1].noop : batch.t[0].noop;
    const float *scale_p = second ? batch.t[1].scale : batch.t[0].scale;
    float *amax_slot = second ? batch.t[1].amax_slot : batch.t[0].amax_slot;
    float *sinv_out = second ? batch.t[1].sinv_out : batch.t[0].sinv_out;
    const float s = *scale_p;
    const float skip_flag = noop != nullptr ? *noop : 0.0f;

    const int t = threadIdx.x;
    const int rb = t / NRB, cb = t % NRB;
    const uint32_t block = blockIdx.x - (second ? (uint32_t)batch.first1 : 0u);
    const uint32_t tiles_c = (uint32_t)((cols + TS - 1) / TS);
    uint32_t tile_r, tile_c;
    if (TS == kTile) {
        ct_tile_of(block, rows, tiles_c, tile_r, tile_c);
    } else {
        tile_r = block / tiles_c;
        tile_c = block - tile_r * tiles_c;
    }
    const int64_t r0 = (int64_t)tile_r * TS;
    const int64_t c0 = (int64_t)tile_c * TS;
    const int64_t row = r0 + rb * 8;   // first row of the micro-tile
    const int64_t col = c0 + cb * 8;   // first column of the micro-tile
    // Interior tile (block-uniform): every access of the 16-byte path is in bounds, so loads and
    // stores go out unconditionally (per-access checks put each one in a branch of its own).
    const bool full = VEC && r0 + TS <= rows && c0 + TS <= cols;

    // ---- load 8 rows x 8 columns (bfloat16 pairs in dwords: w[r][0..3])
    uint32_t w[8][4];
    if (full) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x + (row + r) * cols + col));
            w[r][0] = v.x; w[r][1] = v.y; w[r][2] = v.z; w[r][3] = v.w;
        }
    } else if constexpr (VEC) {
        const bool cin = col < cols;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if (cin && row + r < rows) {
                u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x + (row + r) * cols + col));
                w[r][0] = v.x; w[r][1] = v.y; w[r][2] = v.z; w[r][3] = v.w;
            } else {
                w[r][0] = w[r][1] = w[r][2] = w[r][3] = 0u;
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                uint32_t lo = 0, hi = 0;
                if (row + r < rows) {
                    if (col + 2 * c < cols) lo = x[(row + r) * cols + col + 2 * c];
                    if (col + 2 * c + 1 < cols) hi = x[(row + r) * cols + col + 2 * c + 1];
                }
                w[r][c] = lo | (hi << 16);
            }
        }
    }

    // The noop flag is tested only now, so the input loads do not wait behind its round trip
    // (the compiler would otherwise sink them below the early exit); a skipped cast drains its
    // loads before it ends and writes nothing.
    __asm__ volatile("" ::: "memory");
    if (skip_flag == 1.0f) {
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }

    // ---- amax of the micro-tile (out-of-range elements are zero)
    uint32_t tam = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) tam = amax_pk(tam, w[r][c]);
    const uint32_t mag = amax_unpack(tam);

    // ---- dbias: column sums of the micro-tile in row order
    if constexpr (DBIAS) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float slo = 0.f, shi = 0.f;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                slo += bf16_lo(w[r][c]);
                shi += bf16_hi(w[r][c]);
            }
            csum[rb * kTileC + cb * 8 + 2 * c] = slo;
            csum[rb * kTileC + cb * 8 + 2 * c + 1] = shi;
        }
    }

    // ---- row codes: orow[r][h] = the four codes of row r, columns 4h .. 4h+3
    uint32_t orow[8][2];
    if (scale_is_plain(s) && mag < 0x7F80u) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                orow[r][h] = pack4<FMT>(clamp_fmt<FMT>(bf16_lo(w[r][2 * h]) * s), clamp_fmt<FMT>(bf16_hi(w[r][2 * h]) * s),
                                        clamp_fmt<FMT>(bf16_lo(w[r][2 * h + 1]) * s),
                                        clamp_fmt<FMT>(bf16_hi(w[r][2 * h + 1]) * s));
    } else {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                orow[r][h] = encode_exact<FMT>(bf16_lo(w[r][2 * h]) * s) |
                             (encode_exact<FMT>(bf16_hi(w[r][2 * h]) * s) << 8) |
                             (encode_exact<FMT>(bf16_lo(w[r][2 * h + 1]) * s) << 16) |
                             (encode_exact<FMT>(bf16_hi(w[r][2 * h + 1]) * s) << 24);
    }

    // ---- row-major codes straight to global memory
    if (full) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            u32x2 v = {orow[r][0], orow[r][1]};
            __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(out + (row + r) * cols + col));
        }
    } else if constexpr (VEC) {
        if (col < cols) {
#pragma unroll
            for (int r = 0; r < 8; ++r)
                if (row + r < rows) {
                    u32x2 v = {orow[r][0], orow[r][1]};
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(out + (row + r) * cols + col));
                }
        }
    } else {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c)
                if (row + r < rows && col + c < cols)
                    out[(row + r) * cols + col + c] = (uint8_t)(orow[r][c >> 2] >> (8 * (c & 3)));
    }

    const bool want_t = out_t != nullptr;   // block-uniform
    // ---- column codes by byte transposes: ocol[c][h] = rows 4h .. 4h+3 of column c; then the
    // transposed fragments into LDS: T[cb*8 + c][rb*8 .. rb*8+7]
    if (want_t) {
        uint32_t ocol[8][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            tr4(orow[0][h], orow[1][h], orow[2][h], orow[3][h], ocol[4 * h][0], ocol[4 * h + 1][0], ocol[4 * h + 2][0],
                ocol[4 * h + 3][0]);
            tr4(orow[4][h], orow[5][h], orow[6][h], orow[7][h], ocol[4 * h][1], ocol[4 * h + 1][1], ocol[4 * h + 2][1],
                ocol[4 * h + 3][1]);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int tc = cb * 8 + c;
            u32x2 v = {ocol[c][0], ocol[c][1]};
            *reinterpret_cast<u32x2 *>(&tT[tc * TS + ((rb ^ ((tc >> 3) & (NRB - 1))) << 3)]) = v;
        }
    }

    __syncthreads();

    // ---- transposed tile out: 256 transposed rows x 256 bytes, 16-byte chunks
    if (want_t)
#pragma unroll
    for (int i = 0; i < (TS * TS / 16) / NT; ++i) {
        const int q = t + NT * i;
        const int tr = q / CH, part = q % CH;          // transposed row (= tile column), chunk
        const int64_t orow_g = c0 + tr;                 // row of out_t
        const int64_t ocol_g = r0 + part * 16;          // first column of out_t in this chunk
        const int g = (tr >> 3) & (NRB - 1);
        u32x4 v = *reinterpret_cast<const u32x4 *>(&tT[tr * TS + ((part ^ (g >> 1)) << 4)]);
        if (g & 1) v = v.zwxy;
        if (full) {
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(out_t + orow_g * rows + ocol_g));
        } else if constexpr (VEC) {
            if (orow_g < cols && ocol_g < rows)
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(out_t + orow_g * rows + ocol_g));
        } else {
            if (orow_g < cols) {
                const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int b = 0; b < 16; ++b)
                    if (ocol_g + b < rows) out_t[orow_g * rows + ocol_g + b] = (uint8_t)(d[b >> 2] >> (8 * (b & 3)));
            }
        }
    }

    // ---- dbias partial of this row tile: fixed-order sum over the 32 row blocks
    if constexpr (DBIAS) {
        if (t < kTileC) {
            float acc = 0.f;
#pragma unroll
            for (int b = 0; b < kRowBlocks; ++b) acc += csum[b * kTileC + t];
            if (c0 + t < cols) partial[(int64_t)tile_r * cols + c0 + t] = acc;
        }
    }

    // ---- amax: one atomic per block; inverse scale from block (0, 0)
    uint32_t bm = block_max_u32<NT>(mag, red);
    if (t == 0) {
        fold_amax(amax_slot, bm);
        if (block == 0 && sinv_out != nullptr) *sinv_out = 1.0f / s;
    }
}

// dbias[j] = sum over row tiles of partial[tile][j], in a fixed order: a 256-thread block owns
// 64 columns; thread (g = t / 64, c = t % 64) takes tiles g, g + 4, g + 8, ... in batches of 16
// (the last batch's missing tiles count as zero), sums each batch as a balanced tree and the
// batch sums in increasing order; then (g0 + g1) + (g2 + g3).  The order depends only on the
// number of tiles, so the result is the same run to run.  A thread's 16 loads go out before
// their sums, so it waits for one memory round trip per 16 tiles instead of one per tile.
__global__ __launch_bounds__(256) void k_dbias_reduce(const float *__restrict__ partial, int64_t ntiles,
                                                      int64_t cols, float *__restrict__ dbias) {
    __shared__ float part[4][64];
    const int g = threadIdx.x >> 6, c = threadIdx.x & 63;
    const int64_t j = (int64_t)blockIdx.x * 64 + c;
    float acc = 0.f;
    if (j < cols) {
        const float *__restrict__ p = partial + j;
        for (int64_t i = g; i < ntiles; i += 64) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = i + 4 * u < ntiles ? p[(i + 4 * u) * cols] : 0.f;
            acc += sum16_pairwise(v);
        }
    }
    part[g][c] = acc;
    __syncthreads();
    if (g == 0 && j < cols) dbias[j] = (part[0][c] + part[1][c]) + (part[2][c] + part[3][c]);
}

// ------------------------------------------------------------------------------------------
// dbias + cast + transpose in one launch, for tensors of whole 256 x 256 tiles that take at
// most two tiles per CU, or three or four evenly (the bias gradient of a narrow layer, e.g. dy
// [8192, 4096]: 512 tiles; [8192, 8192]: 1024).
// With that few tiles the two-kernel form above pays twice for ramp-up and drain (two waves of
// blocks, then the reduction launch); here one block per CU works through the row tiles of one
// 256-column strip, and the column sums are finished inside the same launch:
//   * block b owns strip b % tiles_c and the row tiles slot, slot + nslots, ... (slot = b /
//     tiles_c); each tile's eight rows per thread are converted row by row as they are consumed
//     (the column sums folded in), and the next tile's rows are loaded before the current one
//     is converted, so its reads overlap this tile's conversion and stores;
//   * column sums: per thread over its 8 rows in row order and over its tiles in tile order;
//     then row blocks 2w and 2w + 1 (lanes l and l + 32 of wave w), the even one first; then the
//     16 waves in order: one partial per block and column, partial[slot][column];
//   * before its last tile's stores, a block publishes its partials (agent-scope atomic stores,
//     coherent across the XCDs' L2 caches, complete before the next step) and adds one to its
//     strip's counter (a relaxed agent-scope atomic add); the block that brings the count to
//     nslots sums the strip's nslots partials into dbias (agent-scope atomic loads; batches of
//     16 slots, each a balanced tree, the batch sums in slot order) and sets the counter back
//     to zero.
// The result does not depend on which block comes last, so it is the same run to run.  The
// counters live at the start of the workspace: zero before the first call, and every call
// leaves them zero.  Measured on the same buffers at [8192, 4096], cold: 24.7 us (68% of
// 8 TB/s) against 29.1 us for the tile kernel + reduction, 27.2 us for this kernel with the
// reduction as a second launch, 27.5 us for one-tile blocks at two blocks per CU.
// ------------------------------------------------------------------------------------------
constexpr int kStripBlocks = 256;                      // one 1024-thread block per CU
constexpr int64_t kStripCounterBytes = 1024;           // counters for up to 256 strips
constexpr int kMaxStrips = (int)(kStripCounterBytes / 4);
static_assert(kStripCounterBytes == (int64_t)FP8DS_DBIAS_COUNTER_BYTES, "header and library agree");

// Slots per strip for the one-launch form, or 0 when the tensor takes the two-kernel form.
// Up to two tiles per block always; three or four only when every block gets the same number
// (tiles_r a multiple of the slots) and there are at least 16 strips.  Measured on the same
// buffers, cold, against the two-kernel form: [8192, 8192] 54.5 against 64.2 us (four tiles per
// block), [12288, 4096] 37.9 against 41.4 us (three); with blocks of unequal work ([8192, 6144],
// [4096, 12288]) or few wide strips ([32768, 2048]) the two-kernel form is 1-4% faster.
constexpr int64_t kStripMinStripsDeep = 16;
static int dbias_strip_slots(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0 || rows % kTile != 0 || cols % kTileC != 0) return 0;
    const int64_t tiles_r = rows / kTile, tiles_c = cols / kTileC;
    if (tiles_c > kMaxStrips || tiles_r * tiles_c > 4 * kStripBlocks) return 0;
    const int64_t ns = std::min<int64_t>(tiles_r, kStripBlocks / tiles_c);
    if (ns < 1 || 4 * ns < tiles_r) return 0;                   // at most four tiles per block
    if (2 * ns < tiles_r && (tiles_r % ns != 0 || tiles_c < kStripMinStripsDeep)) return 0;
    return (int)ns;
}

// Row-by-row conversion of a thread's 8 x 8 micro-tile: amax, column sums and codes.  The sums
// are pinned row by row (left to itself the compiler sinks them past the loop and keeps all 64
// unpacked values live).  The rare exact path (a non-finite input, or a zero / non-finite
// scale) reads the rows again.
template <int FMT>
__device__ __forceinline__ void strip_convert(const uint32_t (&w)[8][4], float s, const uint16_t *__restrict__ xr,
                                              int64_t cols, uint32_t &mag, float (&cs)[8], uint32_t (&orow)[8][2]) {
    uint32_t tam = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
#pragma unroll
        for (int c = 0; c < 4; ++c) tam = amax_pk(tam, w[r][c]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            cs[2 * c] += bf16_lo(w[r][c]);
            cs[2 * c + 1] += bf16_hi(w[r][c]);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) __asm__ volatile("" : "+v"(cs[k]));
#pragma unroll
        for (int h = 0; h < 2; ++h)
            orow[r][h] = pack4<FMT>(clamp_fmt<FMT>(bf16_lo(w[r][2 * h]) * s), clamp_fmt<FMT>(bf16_hi(w[r][2 * h]) * s),
                                    clamp_fmt<FMT>(bf16_lo(w[r][2 * h + 1]) * s),
                                    clamp_fmt<FMT>(bf16_hi(w[r][2 * h + 1]) * s));
        __builtin_amdgcn_sched_barrier(0);
    }
    const uint32_t m = amax_unpack(tam);
    mag = max(mag, m);
    if (!(scale_is_plain(s) && m < 0x7F80u)) {
#pragma unroll 1
        for (int r = 0; r < 8; ++r) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(xr + r * cols);
            const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int h = 0; h < 2; ++h)
                orow[r][h] = encode_exact<FMT>(bf16_lo(q[2 * h]) * s) | (encode_exact<FMT>(bf16_hi(q[2 * h]) * s) << 8) |
                             (encode_exact<FMT>(bf16_lo(q[2 * h + 1]) * s) << 16) |
                             (encode_exact<FMT>(bf16_hi(q[2 * h + 1]) * s) << 24);
        }
    }
}

// Codes of one whole tile to out (row-major) and, through the LDS tile T[col][row], to out_t.
__device__ __forceinline__ void strip_store(const uint32_t (&orow)[8][2], int64_t rows, int64_t cols, int64_t r0,
                                            int64_t c0, int rb, int cb, int t, uint8_t *tT,
                                            uint8_t *__restrict__ out, uint8_t *__restrict__ out_t) {
    const int64_t row = r0 + rb * 8, col = c0 + cb * 8;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        u32x2 v = {orow[r][0], orow[r][1]};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(out + (row + r) * cols + col));
    }
    uint32_t ocol[8][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        tr4(orow[0][h], orow[1][h], orow[2][h], orow[3][h], ocol[4 * h][0], ocol[4 * h + 1][0], ocol[4 * h + 2][0],
            ocol[4 * h + 3][0]);
        tr4(orow[4][h], orow[5][h], orow[6][h], orow[7][h], ocol[4 * h][1], ocol[4 * h + 1][1], ocol[4 * h + 2][1],
            ocol[4 * h + 3][1]);
    }
    __syncthreads();   // the previous tile's transposed reads are done
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int tc = cb * 8 + c;
        u32x2 v = {ocol[c][0], ocol[c][1]};
        *reinterpret_cast<u32x2 *>(&tT[tc * kTile + ((rb ^ t_swz(tc)) << 3)]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < (kTileC * kTile / 16) / kCtThreads; ++i) {
        const int q = t + kCtThreads * i;
        const int tr = q >> 4, part = q & 15;
        const int g = t_swz(tr);
        u32x4 v = *reinterpret_cast<const u32x4 *>(&tT[tr * kTile + ((part ^ (g >> 1)) << 4)]);
        if (g & 1) v = v.zwxy;
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(out_t + (c0 + tr) * rows + r0 + part * 16));
    }
}

template <int FMT>
__global__ __launch_bounds__(kCtThreads) void k_dbias_strips(const uint16_t *__restrict__ x, int64_t rows,
                                                             int64_t cols, const float *__restrict__ scale_p,
                                                             uint8_t *__restrict__ out, uint8_t *__restrict__ out_t,
                                                             float *sinv_out, float *amax_slot, float *partial,
                                                             uint32_t *counters, float *__restrict__ dbias,
                                                             int nslots) {
    __shared__ __align__(16) uint8_t tT[kTileC * kTile];
    __shared__ __align__(16) float csl[(kCtThreads / 64) * kTileC];
    __shared__ uint32_t red[kCtThreads / 64];
    __shared__ int last;
    const float s = *scale_p;
    const int t = threadIdx.x, rb = t >> 5, cb = t & 31, lane = t & 63, wave = t >> 6;
    const int tiles_r = (int)(rows / kTile), tiles_c = (int)(cols / kTileC);
    const int strip = (int)blockIdx.x % tiles_c, slot = (int)blockIdx.x / tiles_c;
    const int64_t c0 = (int64_t)strip * kTileC, col = c0 + cb * 8;
    uint32_t mag = 0;
    float cs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    uint32_t w[8][4];
    {
        const uint16_t *xr = x + ((int64_t)slot * kTile + rb * 8) * cols + col;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xr + r * cols));
            w[r][0] = v.x; w[r][1] = v.y; w[r][2] = v.z; w[r][3] = v.w;
        }
    }
    for (int tr = slot; tr < tiles_r; tr += nslots) {
        const int nx = tr + nslots;   // block-uniform
        const uint16_t *xr = x + ((int64_t)tr * kTile + rb * 8) * cols + col;
        uint32_t cur[8][4];
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) cur[r][c] = w[r][c];
        if (nx < tiles_r) {
            const uint16_t *xn = x + ((int64_t)nx * kTile + rb * 8) * cols + col;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xn + r * cols));
                w[r][0] = v.x; w[r][1] = v.y; w[r][2] = v.z; w[r][3] = v.w;
            }
        }
        uint32_t orow[8][2];
        strip_convert<FMT>(cur, s, xr, cols, mag, cs, orow);
        if (nx >= tiles_r) {
            // last tile of this block: publish the block's column sums and arrive on the strip
            float o[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) o[k] = __shfl_xor(cs[k], 32);
#pragma unroll
            for (int k = 0; k < 8; ++k) cs[k] = lane < 32 ? cs[k] + o[k] : o[k] + cs[k];
            if (lane < 32) {
                *reinterpret_cast<float4 *>(&csl[wave * kTileC + cb * 8]) = float4{cs[0], cs[1], cs[2], cs[3]};
                *reinterpret_cast<float4 *>(&csl[wave * kTileC + cb * 8 + 4]) = float4{cs[4], cs[5], cs[6], cs[7]};
            }
            __syncthreads();
            if (t < kTileC) {
                float acc = 0.f;
#pragma unroll
                for (int wv = 0; wv < kCtThreads / 64; ++wv) acc += csl[wv * kTileC + t];
                __hip_atomic_store(&partial[(int64_t)slot * cols + c0 + t], acc, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                // the partial has reached the coherent level before the arrival below
                __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            __syncthreads();
            if (t == 0) {
                const uint32_t before =
                    __hip_atomic_fetch_add(&counters[strip], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                last = before == (uint32_t)(nslots - 1);
            }
        }
        strip_store(orow, rows, cols, (int64_t)tr * kTile, c0, rb, cb, t, tT, out, out_t);
    }
    __syncthreads();   // `last` is visible to every wave
    if (last) {
        if (t < kTileC) {
            const float *p = partial + c0 + t;
            float acc = 0.f;
            for (int i = 0; i < nslots; i += 16) {
                float v[16];
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    v[u] = i + u < nslots ? __hip_atomic_load(p + (int64_t)(i + u) * cols, __ATOMIC_RELAXED,
                                                              __HIP_MEMORY_SCOPE_AGENT)
                                          : 0.f;
                acc += sum16_pairwise(v);
            }
            dbias[c0 + t] = acc;
        }
        if (t == 0) __hip_atomic_store(&counters[strip], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const uint32_t bm = block_max_u32<kCtThreads>(mag, red);
    if (t == 0) {
        fold_amax(amax_slot, bm);
        if (blockIdx.x == 0 && sinv_out != nullptr) *sinv_out = 1.0f / s;
    }
}

// ------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------
hipError_t launch_cast_amax(const uint16_t *x, int64_t n, const float *scale, int fmt, uint8_t *out,
                            float *sinv_out, float *amax_slot, const float *noop, hipStream_t st) {
    if (n == 0) return hipSuccess;
    int64_t nvec = n >> 4;
    int64_t blocks = (nvec + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > kCastMaxBlocks) blocks = kCastMaxBlocks;  // grid-stride beyond that
    if (fmt == kE4M3)
        k_cast_amax<kE4M3><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(x, n, scale, out, sinv_out, amax_slot, noop);
    else
        k_cast_amax<kE5M2><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(x, n, scale, out, sinv_out, amax_slot, noop);
    return hipGetLastError();
}

static int64_t ct_tiles(int64_t rows, int64_t cols, int ts = kTile) {
    return ((cols + ts - 1) / ts) * ((rows + ts - 1) / ts);
}
static bool ct_vec(int64_t rows, int64_t cols) { return (cols % 8 == 0) && (rows % 16 == 0); }

// Launches that would have fewer 256 x 256 tiles than this take 64 x 64 tiles of 64 threads:
// with few tiles the 1024-thread blocks leave most CUs idle and each tile is a long chain of
// dependent steps.  Measured on the same buffers (E4M3, cold): [1024, 1024] 3.9 us against
// 7.3 us, [2048, 2048] 5.1 against 7.8 us; at [4096, 4096] (256 tiles) the 256 x 256 tile is
// faster, 13.3 against 18.4 us.
constexpr int kSmallTs = 64;
constexpr int64_t kSmallCastTiles = 128;

template <bool DBIAS>
static hipError_t launch_batch(const CtBatch &b, int64_t blocks, bool vec, bool small, int fmt, float *partial,
                               hipStream_t st) {
    dim3 grid((unsigned)blocks);
#define FP8DS_CT(F, V, TS_) k_cast_transpose<F, V, DBIAS, TS_><<<grid, dim3((TS_ / 8) * (TS_ / 8)), 0, st>>>(b, partial)
#define FP8DS_CT_FMT(TS_)                                                                                  \
    do {                                                                                                   \
        if (fmt == kE4M3) {                                                                                \
            if (vec) FP8DS_CT(kE4M3, true, TS_); else FP8DS_CT(kE4M3, false, TS_);                         \
        } else {                                                                                           \
            if (vec) FP8DS_CT(kE5M2, true, TS_); else FP8DS_CT(kE5M2, false, TS_);                         \
        }                                                                                                  \
    } while (0)
    if constexpr (!DBIAS) {
        if (small) {
            FP8DS_CT_FMT(kSmallTs);
            return hipGetLastError();
        }
    }
    FP8DS_CT_FMT(kTile);
#undef FP8DS_CT_FMT
#undef FP8DS_CT
    return hipGetLastError();
}

template <bool DBIAS>
static hipError_t launch_ct(const uint16_t *x, int64_t rows, int64_t cols, const float *scale, int fmt,
                            uint8_t *out, uint8_t *out_t, float *sinv_out, float *amax_slot,
                            const float *noop, float *partial, hipStream_t st) {
    CtBatch b{};
    b.t[0] = CtTensor{x, rows, cols, scale, out, out_t, sinv_out, amax_slot, noop};
    b.t[1] = b.t[0];
    const bool small = !DBIAS && ct_tiles(rows, cols) < kSmallCastTiles;
    const int64_t n = ct_tiles(rows, cols, small ? kSmallTs : kTile);
    b.first1 = n;
    return launch_batch<DBIAS>(b, n, ct_vec(rows, cols), small, fmt, partial, st);
}

hipError_t launch_cast_transpose(const uint16_t *x, int64_t rows, int64_t cols, const float *scale, int fmt,
                                 uint8_t *out, uint8_t *out_t, float *sinv_out, float *amax_slot,
                                 const float *noop, hipStream_t st) {
    if (rows == 0 || cols == 0) return hipSuccess;
    return launch_ct<false>(x, rows, cols, scale, fmt, out, out_t, sinv_out, amax_slot, noop, nullptr, st);
}

hipError_t launch_cast_transpose_pair(const uint16_t *x0, int64_t rows0, int64_t cols0, const float *scale0,
                                      uint8_t *out0, uint8_t *out_t0, float *sinv0, float *amax0, const float *noop0,
                                      const uint16_t *x1, int64_t rows1, int64_t cols1, const float *scale1,
                                      uint8_t *out1, uint8_t *out_t1, float *sinv1, float *amax1, const float *noop1,
                                      int fmt, hipStream_t st) {
    const bool v0 = ct_vec(rows0, cols0), v1 = ct_vec(rows1, cols1);
    const bool e0 = rows0 == 0 || cols0 == 0, e1 = rows1 == 0 || cols1 == 0;
    if (v0 != v1 || e0 || e1) {
        // the two tensors need different code paths (or one is empty): one launch each
        hipError_t e = hipSuccess;
        if (!e0) e = launch_ct<false>(x0, rows0, cols0, scale0, fmt, out0, out_t0, sinv0, amax0, noop0, nullptr, st);
        if (e == hipSuccess && !e1)
            e = launch_ct<false>(x1, rows1, cols1, scale1, fmt, out1, out_t1, sinv1, amax1, noop1, nullptr, st);
        return e;
    }
    // one tile size for both: the small one when the pair together has few tiles
    const bool small = ct_tiles(rows0, cols0) + ct_tiles(rows1, cols1) < kSmallCastTiles;
    const int ts = small ? kSmallTs : kTile;
    const int64_t n0 = ct_tiles(rows0, cols0, ts), n1 = ct_tiles(rows1, cols1, ts);
    CtBatch b{};
    b.t[0] = CtTensor{x0, rows0, cols0, scale0, out0, out_t0, sinv0, amax0, noop0};
    b.t[1] = CtTensor{x1, rows1, cols1, scale1, out1, out_t1, sinv1, amax1, noop1};
    b.first1 = n0;
    return launch_batch<false>(b, n0 + n1, v0, small, fmt, nullptr, st);
}

// Workspace: the strip counters of the one-launch form (kStripCounterBytes, zero between
// calls), then the partial column sums, one row of cols floats per 256-row tile.
size_t dbias_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    return (size_t)kStripCounterBytes + (size_t)((rows + kTile - 1) / kTile) * (size_t)cols * sizeof(float);
}

hipError_t launch_dbias_cast_transpose(const uint16_t *dy, int64_t rows, int64_t cols, const float *scale,
                                       int fmt, uint8_t *out, uint8_t *out_t, float *sinv_out,
                                       float *amax_slot, float *dbias, void *ws, hipStream_t st) {
    if (cols == 0) return hipSuccess;
    if (rows == 0) {
        // no rows: the column sums are zero; nothing else to write (a fill kernel, not a
        // memset node, so the call stays safe to capture into a graph)
        k_dbias_reduce<<<dim3((unsigned)((cols + 63) / 64)), dim3(256), 0, st>>>(nullptr, 0, cols, dbias);
        return hipGetLastError();
    }
    uint32_t *counters = static_cast<uint32_t *>(ws);
    float *partial = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + kStripCounterBytes);
    if (const int nslots = dbias_strip_slots(rows, cols)) {
        const unsigned grid = (unsigned)(nslots * (cols / kTileC));
        if (fmt == kE4M3)
            k_dbias_strips<kE4M3><<<dim3(grid), dim3(kCtThreads), 0, st>>>(dy, rows, cols, scale, out, out_t, sinv_out,
                                                                          amax_slot, partial, counters, dbias, nslots);
        else
            k_dbias_strips<kE5M2><<<dim3(grid), dim3(kCtThreads), 0, st>>>(dy, rows, cols, scale, out, out_t, sinv_out,
                                                                          amax_slot, partial, counters, dbias, nslots);
        return hipGetLastError();
    }
    hipError_t e = launch_ct<true>(dy, rows, cols, scale, fmt, out, out_t, sinv_out, amax_slot, nullptr, partial, st);
    if (e != hipSuccess) return e;
    const int64_t ntiles = (rows + kTile - 1) / kTile;
    k_dbias_reduce<<<dim3((unsigned)((cols + 63) / 64)), dim3(256), 0, st>>>(partial, ntiles, cols, dbias);
    return hipGetLastError();
}

}  // namespace fp8ds
