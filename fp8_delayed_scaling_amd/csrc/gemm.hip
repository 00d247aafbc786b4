// gemm.hip -- FP8 GEMM with inverse-scale dequantisation and bias on gfx950 matrix cores.
//
//   D[m, n] = (sum_k A[m, k] * B[n, k]) * a_scale_inv * b_scale_inv + bias[n]
//
// The fp8_gemm of "[PyTorch] cuda graph support" (transpose-cache thread, FP8Linear.backward)
// and the per-chunk bias of "[PyTorch] Userbuffers support in operation-based API" (bias-offset
// fix).  Both operands are K-contiguous ("TN"); the transposes the backward needs come from
// the cast+transpose kernels, so the GEMM never transposes.
//
// Both kernels: block tile 256 x 256, 256 threads = 4 waves in a 2 x 2 grid, each wave a 128 x 128
// sub-tile made of 4 x 4 v_mfma_f32_32x32x64_f8f6f4 tiles (float32 accumulate; the A / B formats
// are the instruction's cbsz / blgp selectors, so every format pair shares one template).
// Blocks are remapped so that each XCD (blocks are dealt round-robin to the 8 XCDs) works on a
// contiguous range of tiles, walked in groups of kGroupM tile-rows for L2 reuse.  Epilogue:
// acc * a_scale_inv * b_scale_inv + bias in float32, rounded to bfloat16 (nearest even) or stored
// as float32 (the pipelined kernel stages it through LDS and writes 16-byte row segments).  Ragged M / N are handled by clamping the rows that are loaded and masking the
// stores.  No split-K: every output element is one fixed sequence of MFMAs over K in the same
// K order in both kernels, whatever tile it falls in.
//
// k_gemm_bias_pipe (K % 64 == 0 and row strides below 8 MiB, the hot path): a 4-stage pipeline
// of 64-byte K slices (4 x 32 KB of LDS).  Global memory goes straight into LDS with
// buffer_load_dwordx4 ... lds (no staging registers; per-tile descriptors, 32-bit per-lane
// offsets, the K slice in the scalar offset), three slices ahead of the MFMAs; each wave prefetches the next slice's
// operand fragments from LDS while its MFMAs run on the current ones (double-buffered
// fragments), and the instruction scheduler is told to place the fragment reads and global loads
// among the first 12 of the slice's 16 MFMAs.  The four stages are four distinct LDS arrays so the
// compiler can tell the in-flight loads of one stage from the reads of another, and the
// per-slice barrier is a bare s_barrier after an explicit vmcnt wait (a fenced barrier would
// drain every load in flight).  LDS rows are 64 bytes; 16-byte chunk c of row r sits at chunk
// c ^ ((r >> 2) & 3), which measured bank-conflict free for the MFMA operand reads.
//
// k_gemm_bias (any K % 16 == 0): global -> registers -> LDS with double-buffered 128-byte K
// slices, the K tail zero-filled.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace fp8ds {

namespace {
constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kThreads = 256;
constexpr int kGroupM = 4;
constexpr int kLdsA = BM * BK;             // bytes per A buffer
constexpr int kLdsB = BN * BK;
constexpr int kLdsBytes = 2 * (kLdsA + kLdsB);

__device__ __forceinline__ int lds_chunk(int row, int c) { return c ^ (row & 7) ^ ((row >> 3) & 1); }

// Tile of this block: XCD-contiguous ranges, walked in groups of kGroupM tile-rows.
__device__ __forceinline__ void block_tile(int tiles_m, int tiles_n, int &tm, int &tn) {
    const int nwg = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, local = bid >> 3;
    const int q8 = nwg >> 3, r8 = nwg & 7;
    const int tile = (xcd < r8) ? xcd * (q8 + 1) + local : r8 * (q8 + 1) + (xcd - r8) * q8 + local;
    const int group = tile / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    const int in_group = tile - group * kGroupM * tiles_n;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}
}  // namespace

// FP8 output (OUT 2 = E4M3, 3 = E5M2): D is encoded with its own scale, max |D| (float32, before
// the scale) is folded into an amax slot, and block 0 records 1/scale as the output's private
// inverse scale.  Ignored for bfloat16 / float32 output.
struct OutQuant {
    const float *scale;
    float *scale_inv_out;
    float *amax;
};

// Epilogue of one wave's 128 x 128 sub-tile at (row0, col0).  Accumulator element e of lane l in
// a 32 x 32 MFMA tile is row (e / 4) * 8 + (l / 32) * 4 + e % 4, column l % 32.
template <int OUT>
__device__ __forceinline__ void epilogue(const f32x16 (&acc)[4][4], const float *__restrict__ a_sinv,
                                         const float *__restrict__ b_sinv, const uint16_t *__restrict__ bias,
                                         void *__restrict__ D, int64_t ldd, int M, int N, int row0, int col0,
                                         int lane, OutQuant oq) {
    const int frow = lane & 31, fhalf = lane >> 5;
    const float sa = *a_sinv, sb = *b_sinv;
    float ds = 0.f;
    if constexpr (OUT >= 2) ds = *oq.scale;
    uint32_t amag = 0;
    // the four bias columns, loaded together (unconditional loads: without a bias they read the
    // first two bytes of a_sinv) before any is used
    const bool has_bias = bias != nullptr;
    const uint16_t *bsrc = has_bias ? bias : reinterpret_cast<const uint16_t *>(a_sinv);
    uint32_t braw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) braw[j] = bsrc[has_bias ? min(col0 + j * 32 + frow, N - 1) : 0];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = col0 + j * 32 + frow;
        if (col >= N) continue;
        const float bv = has_bias ? __uint_as_float(braw[j] << 16) : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = row0 + i * 32 + (e >> 2) * 8 + fhalf * 4 + (e & 3);
                if (row < M) {
                    const float v = dequant_bias(acc[i][j][e], sa, sb, bv);
                    if constexpr (OUT == 0) {
                        reinterpret_cast<uint16_t *>(D)[(int64_t)row * ldd + col] = f32_to_bf16_rne(v);
                    } else if constexpr (OUT == 1) {
                        reinterpret_cast<float *>(D)[(int64_t)row * ldd + col] = v;
                    } else {
                        amag = max(amag, __float_as_uint(v) & 0x7FFFFFFFu);
                        reinterpret_cast<uint8_t *>(D)[(int64_t)row * ldd + col] =
                            (uint8_t)encode_exact<OUT - 2>(v * ds);
                    }
                }
            }
        }
    }
    if constexpr (OUT >= 2) {
        amag = wave_max_u32(amag);
        if (lane == 0) fold_amax_bits(oq.amax, amag);
    }
}

// Epilogue of the pipelined kernel, whose MFMAs take B as the first operand: there lane l holds
// D[row0 + 32 i + l % 32][col0 + 32 j + 8 (e / 4) + 4 (l / 32) + e % 4] in element e of acc[i][j]
// (the products and their summation order are the same as with A first).  Each wave scales, adds
// the bias and rounds its 128 x 128 sub-tile into its own 32 KB of LDS, then writes whole rows
// with 16-byte streaming (nontemporal) stores.  bf16: one pass, row r at r * 256, 8-byte slot s
// (columns 4 s .. 4 s + 3) stored at slot s ^ (r & 31).  float32: two passes of 64 rows, row r at
// r * 512, 16-byte slot s at s ^ (r & 31).  Where D or ldd is not 16-byte aligned, or at the
// ragged right edge, the elements are stored one by one.
template <int OUT>
__device__ __forceinline__ void epilogue_staged(const f32x16 (&acc)[4][4], float sa, float sb, float ds,
                                                bool has_bias, const us2 (&braw)[4][4][2],
                                                void *__restrict__ D, int64_t ldd, int M, int N, int row0,
                                                int col0, int lane, uint8_t *wlds, OutQuant oq) {
    const int frow = lane & 31, fhalf = lane >> 5;
    constexpr int kElemsPer16 = OUT == 0 ? 8 : OUT == 1 ? 4 : 16;
    const bool vec_ok = ((reinterpret_cast<uintptr_t>(D) & 15u) == 0) && (ldd % kElemsPer16 == 0);
    // bias of the 16 columns this lane holds in column block j, from the raw bits the caller
    // loaded (braw[j][q][u / 2][u % 2] = bias[min(col0 + 32 j + 8 q + 4 (lane / 32) + u, N - 1)]).
    // Columns past N take bias[N - 1]: their operand rows are clamped to row N - 1 of B, so every
    // value a lane holds outside the output (rows past M read row M - 1 of A) is bit-identical to
    // an element inside it.  Such values are never stored, and the FP8 output's amax can take the
    // max over the whole sub-tile without masking.
    auto load_bias = [&](int j, float (&bv)[4][4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                bv[q][u] = has_bias ? __uint_as_float((uint32_t)braw[j][q][u >> 1][u & 1] << 16) : 0.f;
    };
    if constexpr (OUT == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float bv[4][4];
            load_bias(j, bv);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = i * 32 + frow, sl = j * 8 + q * 2 + fhalf;
                    float v[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) v[u] = dequant_bias(acc[i][j][q * 4 + u], sa, sb, bv[q][u]);
                    const u32x2 pk = {f32x2_to_bf16x2_rne(v[0], v[1]), f32x2_to_bf16x2_rne(v[2], v[3])};
                    *reinterpret_cast<u32x2 *>(wlds + r * 256 + ((sl ^ (r & 31)) << 3)) = pk;
                }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        // 16-byte chunk ch of row r = slots 2 ch, 2 ch + 1, stored at (2 ch) ^ x and (2 ch + 1) ^ x
        // with x = r & 31: one aligned 16-byte read at (2 ch) ^ (x & ~1), halves swapped if x is odd.
#pragma unroll
        for (int pq = 0; pq < 32; ++pq) {
            const int r = pq * 4 + (lane >> 4), ch = lane & 15;
            const int x = r & 31;
            u32x4 v = *reinterpret_cast<const u32x4 *>(wlds + r * 256 + (((2 * ch) ^ (x & ~1)) << 3));
            if (x & 1) v = v.zwxy;
            const int row = row0 + r, col = col0 + ch * 8;
            if (row < M && col < N) {
                uint16_t *dst = reinterpret_cast<uint16_t *>(D) + (int64_t)row * ldd + col;
                if (vec_ok && col + 7 < N) {
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst));
                } else {
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        if (col + u < N) dst[u] = (uint16_t)(w[u >> 1] >> (16 * (u & 1)));
                }
            }
        }
    } else if constexpr (OUT == 1) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float bv[4][4];
                load_bias(j, bv);
#pragma unroll
                for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int i = h * 2 + ii;
                        const int r = ii * 32 + frow, sl = j * 8 + q * 2 + fhalf;
                        u32x4 pk;
                        pk.x = __float_as_uint(dequant_bias(acc[i][j][q * 4 + 0], sa, sb, bv[q][0]));
                        pk.y = __float_as_uint(dequant_bias(acc[i][j][q * 4 + 1], sa, sb, bv[q][1]));
                        pk.z = __float_as_uint(dequant_bias(acc[i][j][q * 4 + 2], sa, sb, bv[q][2]));
                        pk.w = __float_as_uint(dequant_bias(acc[i][j][q * 4 + 3], sa, sb, bv[q][3]));
                        *reinterpret_cast<u32x4 *>(wlds + r * 512 + ((sl ^ (r & 31)) << 4)) = pk;
                    }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int pq = 0; pq < 32; ++pq) {
                const int r = pq * 2 + (lane >> 5), ch = lane & 31;
                const u32x4 v = *reinterpret_cast<const u32x4 *>(wlds + r * 512 + ((ch ^ (r & 31)) << 4));
                const int row = row0 + h * 64 + r, col = col0 + ch * 4;
                if (row < M && col < N) {
                    float *dst = reinterpret_cast<float *>(D) + (int64_t)row * ldd + col;
                    if (vec_ok && col + 3 < N) {
                        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst));
                    } else {
                        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (col + u < N) dst[u] = __uint_as_float(w[u]);
                    }
                }
            }
            // the second pass overwrites what this pass read
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
        }
    } else {
        // FP8: 128 rows x 128 bytes = 16 KB; row r at r * 128, 4-byte slot s (columns 4 s ..
        // 4 s + 3) stored at slot s ^ (r & 31).
        // Pass 1: the amax.  Unsigned order of magnitude bit patterns is numeric order with NaN
        // above inf, so the wave's amax also says whether any value is NaN.  Pass 2 recomputes
        // the values and, unless a NaN or a non-plain scale makes a scaled value NaN, encodes
        // them with the clamp + hardware conversion alone (one wave-uniform branch).
        constexpr int F = OUT - 2;
        uint32_t amag = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float bv[4][4];
            load_bias(j, bv);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        amag = max(amag, __float_as_uint(dequant_bias(acc[i][j][q * 4 + u], sa, sb, bv[q][u])) &
                                             0x7FFFFFFFu);
        }
        amag = __builtin_amdgcn_readfirstlane(wave_max_u32(amag));   // wave-uniform
        if (lane == 0) fold_amax_bits(oq.amax, amag);
        auto stage = [&](auto fast_tag) {
            constexpr bool kFast = decltype(fast_tag)::value;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float bv[4][4];
                load_bias(j, bv);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r = i * 32 + frow, sl = j * 8 + q * 2 + fhalf;
                        float y[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) y[u] = dequant_bias(acc[i][j][q * 4 + u], sa, sb, bv[q][u]) * ds;
                        uint32_t w;
                        if constexpr (kFast)
                            w = pack4<F>(clamp_fmt<F>(y[0]), clamp_fmt<F>(y[1]), clamp_fmt<F>(y[2]), clamp_fmt<F>(y[3]));
                        else
                            w = encode_exact<F>(y[0]) | (encode_exact<F>(y[1]) << 8) | (encode_exact<F>(y[2]) << 16) |
                                (encode_exact<F>(y[3]) << 24);
                        *reinterpret_cast<uint32_t *>(wlds + r * 128 + ((sl ^ (r & 31)) << 2)) = w;
                    }
            }
        };
        if (scale_is_plain(ds) && amag <= 0x7F800000u)
            stage(std::true_type{});
        else
            stage(std::false_type{});
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
        // 16-byte chunk ch of row r = slots 4 ch .. 4 ch + 3, stored in the aligned group
        // (4 ch) ^ (x & ~3), x = r & 31, with slot 4 ch + k at position k ^ (x & 3).
#pragma unroll
        for (int pq = 0; pq < 16; ++pq) {
            const int r = pq * 8 + (lane >> 3), ch = lane & 7;
            const int x = r & 31;
            u32x4 v = *reinterpret_cast<const u32x4 *>(wlds + r * 128 + (((4 * ch) ^ (x & ~3)) << 2));
            if (x & 1) v = v.yxwz;
            if (x & 2) v = v.zwxy;
            const int row = row0 + r, col = col0 + ch * 16;
            if (row < M && col < N) {
                uint8_t *dst = reinterpret_cast<uint8_t *>(D) + (int64_t)row * ldd + col;
                if (vec_ok && col + 15 < N) {
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst));
                } else {
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int u = 0; u < 16; ++u)
                        if (col + u < N) dst[u] = (uint8_t)(w[u >> 2] >> (8 * (u & 3)));
                }
            }
        }
    }
}

template <int FA, int FB, int OUT>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_bias(const uint8_t *__restrict__ A, int64_t lda,
                                                           const uint8_t *__restrict__ B, int64_t ldb,
                                                           const float *__restrict__ a_sinv,
                                                           const float *__restrict__ b_sinv,
                                                           const uint16_t *__restrict__ bias,
                                                           void *__restrict__ D, int64_t ldd, int M, int N,
                                                           int K, int tiles_m, int tiles_n, OutQuant oq) {
    if constexpr (OUT >= 2)
        if (blockIdx.x == 0 && threadIdx.x == 0 && oq.scale_inv_out != nullptr) *oq.scale_inv_out = 1.0f / *oq.scale;
    __shared__ __align__(16) uint8_t smem[kLdsBytes];

    int tm, tn;
    block_tile(tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- global load assignment: 8 chunks of 16 bytes per operand per K step
    //      chunk i: tile row (tid >> 3) + 32 i, 16-byte column part (tid & 7)
    const int lrow = tid >> 3, part = tid & 7;
    const uint8_t *pa[8];
    const uint8_t *pb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int ra = min(m0 + lrow + 32 * i, M - 1);
        const int rb = min(n0 + lrow + 32 * i, N - 1);
        pa[i] = A + (int64_t)ra * lda + part * 16;
        pb[i] = B + (int64_t)rb * ldb + part * 16;
    }
    int lds_off[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = lrow + 32 * i;
        lds_off[i] = r * BK + lds_chunk(r, part) * 16;
    }

    u32x4 ra_[8], rb_[8];
    auto gload = [&](int kt) {
        const int kofs = kt * BK;
        const bool ok = kofs + part * 16 < K;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (ok) {
                ra_[i] = *reinterpret_cast<const u32x4 *>(pa[i] + kofs);
                rb_[i] = *reinterpret_cast<const u32x4 *>(pb[i] + kofs);
            } else {
                ra_[i] = u32x4{0u, 0u, 0u, 0u};
                rb_[i] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto lstore = [&](int buf) {
        uint8_t *as = smem + buf * kLdsA;
        uint8_t *bs = smem + 2 * kLdsA + buf * kLdsB;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            *reinterpret_cast<u32x4 *>(as + lds_off[i]) = ra_[i];
            *reinterpret_cast<u32x4 *>(bs + lds_off[i]) = rb_[i];
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // operand read positions: lane supplies row (lane & 31) of a 32-row MFMA tile and the 32
    // bytes [32 * (lane >> 5), +32) of each 64-byte K sub-step (the same K bytes for A and B,
    // so the K order inside the instruction is the same on both sides)
    const int frow = lane & 31, fhalf = lane >> 5;
    auto frag = [&](const uint8_t *base, int row, int ks) -> i32x8 {
        const int c0 = ks * 4 + fhalf * 2;
        u32x4 lo = *reinterpret_cast<const u32x4 *>(base + row * BK + lds_chunk(row, c0) * 16);
        u32x4 hi = *reinterpret_cast<const u32x4 *>(base + row * BK + lds_chunk(row, c0 + 1) * 16);
        i32x8 r;
        r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
        r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
        return r;
    };

    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
        gload(0);
        lstore(0);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const uint8_t *as = smem + buf * kLdsA;
        const uint8_t *bs = smem + 2 * kLdsA + buf * kLdsB;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            i32x8 af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                af[i] = frag(as, wm * 128 + i * 32 + frow, ks);
                bf[i] = frag(bs, wn * 128 + i * 32 + frow, ks);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], FA, FB,
                                                                                 0, 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    epilogue<OUT>(acc, a_sinv, b_sinv, bias, D, ldd, M, N, m0 + wm * 128, n0 + wn * 128, lane, oq);
}


// ------------------------------------------------------------------------------------------
// k_gemm_bias_pipe: the 4-stage direct-to-LDS pipeline (K % 64 == 0).
// ------------------------------------------------------------------------------------------
namespace {
constexpr int kPK = 64;                          // K bytes per pipeline slice
// Word 3 of a raw buffer descriptor (no format conversion, bounds checked against the byte
// count in word 2).
constexpr int kBufDesc3 = 0x00020000;
// Row strides below this keep a 256-row tile's extent, the buffer bound, under 2^31 bytes.
constexpr int64_t kPipeMaxLd = INT64_C(1) << 23;
constexpr int kPStage = (BM + BN) * kPK;         // 32 KB: A rows then B rows, 64 bytes each
__device__ __forceinline__ int pswz(int r) { return (r >> 2) & 3; }
}  // namespace

// vmcnt-only wait: expcnt and lgkmcnt fields left at their maxima (no wait on them).
#define FP8DS_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0xF70 | ((n) & 0xF) | (((n) >> 4) << 14))
// Workgroup barrier without a memory fence: the caller has already waited for the loads it
// needs (a fenced barrier would also wait for the later slices still in flight).  The empty
// asm statements keep the compiler from moving LDS accesses across it.
#define FP8DS_BARRIER()                          \
    do {                                         \
        asm volatile("" ::: "memory");           \
        __builtin_amdgcn_s_barrier();            \
        asm volatile("" ::: "memory");           \
    } while (0)

template <int FA, int FB, int OUT>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_bias_pipe(const uint8_t *__restrict__ A, int64_t lda,
                                                                const uint8_t *__restrict__ B, int64_t ldb,
                                                                const float *__restrict__ a_sinv,
                                                                const float *__restrict__ b_sinv,
                                                                const uint16_t *__restrict__ bias,
                                                                void *__restrict__ D, int64_t ldd, int M, int N,
                                                                int K, int tiles_m, int tiles_n, OutQuant oq) {
    if constexpr (OUT >= 2)
        if (blockIdx.x == 0 && threadIdx.x == 0 && oq.scale_inv_out != nullptr) *oq.scale_inv_out = 1.0f / *oq.scale;
    // scalars the epilogue needs, read before the K loop (uniform: scalar registers)
    const float sa = *a_sinv, sb = *b_sinv;
    float ds = 0.f;
    if constexpr (OUT >= 2) ds = *oq.scale;
    __shared__ __align__(16) uint8_t st0[kPStage];
    __shared__ __align__(16) uint8_t st1[kPStage];
    __shared__ __align__(16) uint8_t st2[kPStage];
    __shared__ __align__(16) uint8_t st3[kPStage];

    int tm, tn;
    block_tile(tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // Direct loads: a slice is 2048 chunks of 16 bytes; load i of wave w writes the 1 KB of the
    // stage at (i * 4 + w) * 1024, lane l at + 16 l.  Position p holds row p / 64 (A rows 0-255,
    // then B rows) and stored chunk (p / 16) % 4, i.e. source chunk stored ^ pswz(row).
    // The loads are buffer loads into LDS: one descriptor per operand whose base is the tile's
    // first row and whose bound is the tile's extent (256 rows x lda bytes, below 2^31 as the
    // launcher requires), a 32-bit offset per lane and the K slice in the scalar offset.  Against
    // 64-bit per-lane addresses this saves the per-slice address arithmetic and lets the compiler
    // count the LDS reads in flight exactly; an offset past the bound would read zeros.
    const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(A + (int64_t)m0 * lda), (short)0, (int)(rows_a * lda), kBufDesc3);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(B + (int64_t)n0 * ldb), (short)0, (int)(rows_b * ldb), kBufDesc3);
    uint32_t voff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int p = (i * 4 + wave) * 1024 + lane * 16;
        const int row = p >> 6, slot = (p >> 4) & 3;
        const int r = row & 255;
        const int c = slot ^ pswz(r);
        voff[i] = row < 256 ? (uint32_t)(min(r, rows_a - 1) * lda + c * 16)
                            : (uint32_t)(min(r, rows_b - 1) * ldb + c * 16);
    }
    const int nk = K / kPK;
#define FP8DS_ISSUE(ST, kt)                                                                               \
    _Pragma("unroll") for (int i = 0; i < 8; ++i)                                                         \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(i < 4 ? rs_a : rs_b,                                      \
                                                 (__attribute__((address_space(3))) void *)((ST) + (i * 4 + wave) * 1024), \
                                                 16, voff[i], (uint32_t)((kt) * kPK), 0, 0);

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // Operand fragments: lane l supplies row l % 32 of a 32-row MFMA tile and the 32 bytes
    // [32 (l / 32), +32) of the 64-byte slice, two 16-byte reads.
    const int frow = lane & 31, fhalf = lane >> 5;
    int oa0[4], oa1[4], ob0[4], ob1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ra = wm * 128 + i * 32 + frow, rb = wn * 128 + i * 32 + frow;
        oa0[i] = ra * kPK + (((fhalf * 2) ^ pswz(ra)) << 4);
        oa1[i] = ra * kPK + (((fhalf * 2 + 1) ^ pswz(ra)) << 4);
        ob0[i] = BM * kPK + rb * kPK + (((fhalf * 2) ^ pswz(rb)) << 4);
        ob1[i] = BM * kPK + rb * kPK + (((fhalf * 2 + 1) ^ pswz(rb)) << 4);
    }
    auto ld = [&](const uint8_t *st, int o0, int o1) -> i32x8 {
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(st + o0);
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(st + o1);
        i32x8 r;
        r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
        r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
        return r;
    };
#define FP8DS_FRAGS(ST, FA_, FB_)                                                                          \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                                       \
        FA_[i] = ld((ST), oa0[i], oa1[i]);                                                                \
        FB_[i] = ld((ST), ob0[i], ob1[i]);                                                                \
    }
#define FP8DS_MFMA(CA, CB)                                                                                \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                         \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                         \
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(CB[j], CA[i], acc[i][j], FB, FA, 0, 0, 0, 0);
    // One slice: wait for slice kt+1, barrier, issue slice kt+3 into the stage slice kt-1 used,
    // prefetch slice kt+1's fragments, run slice kt's 16 MFMAs.  The scheduler places the 16
    // fragment reads and the 8 loads among the first 12 MFMAs (per three MFMAs: four reads, two
    // loads) and leaves the last four MFMAs free, so the reads have landed before the next
    // slice's wait (3% faster on the three QKV GEMM shapes than one read per MFMA throughout).
#define FP8DS_STEP(kt, NXT1, ISS, CA, CB, NA, NB)                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                                    \
    FP8DS_WAIT_VM(8);                                                                                     \
    FP8DS_BARRIER();                                                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                                    \
    FP8DS_ISSUE(ISS, (kt) + 3)                                                                            \
    FP8DS_FRAGS(NXT1, NA, NB)                                                                             \
    FP8DS_MFMA(CA, CB)                                                                                    \
    _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                                       \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                \
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                                                \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                                \
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);                                                \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                                \
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);                                                \
    }                                                                                                     \
    _Pragma("unroll") for (int q = 0; q < 4; ++q) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      \
    __builtin_amdgcn_sched_barrier(0);

    i32x8 fa0[4], fb0[4], fa1[4], fb1[4];
    // prologue: slices 0..2 in flight, wait for slice 0, fetch its fragments
    FP8DS_ISSUE(st0, 0)
    if (nk > 1) { FP8DS_ISSUE(st1, 1) }
    if (nk > 2) { FP8DS_ISSUE(st2, 2) }
    if (nk > 2) FP8DS_WAIT_VM(16);
    else if (nk > 1) FP8DS_WAIT_VM(8);
    else FP8DS_WAIT_VM(0);
    FP8DS_BARRIER();
    FP8DS_FRAGS(st0, fa0, fb0)
    int kt = 0;
    // steady state: four slices per trip, every slice issues slice kt+3 (< nk)
    for (; kt + 6 < nk; kt += 4) {
        FP8DS_STEP(kt + 0, st1, st3, fa0, fb0, fa1, fb1)
        FP8DS_STEP(kt + 1, st2, st0, fa1, fb1, fa0, fb0)
        FP8DS_STEP(kt + 2, st3, st1, fa0, fb0, fa1, fb1)
        FP8DS_STEP(kt + 3, st0, st2, fa1, fb1, fa0, fb0)
    }
    // The last slices (fewer than 7; the steady loop leaves kt % 4 == 0, so the stages keep the
    // same rotation): the steady step without the issues that would pass the end of K, waiting
    // only for the next slice (8 loads, of the slice after it, may stay in flight); the last
    // slice needs no wait, fragments or barrier.  Every condition is uniform across the block.
#define FP8DS_TSTEP(kt, NXT1, ISS, CA, CB, NA, NB)                                                        \
    if ((kt) < nk) {                                                                                      \
        if ((kt) + 1 < nk) {                                                                              \
            __builtin_amdgcn_sched_barrier(0);                                                            \
            if ((kt) + 2 < nk) FP8DS_WAIT_VM(8);                                                          \
            else FP8DS_WAIT_VM(0);                                                                        \
            FP8DS_BARRIER();                                                                              \
            __builtin_amdgcn_sched_barrier(0);                                                            \
            if ((kt) + 3 < nk) { FP8DS_ISSUE(ISS, (kt) + 3) }                                             \
            FP8DS_FRAGS(NXT1, NA, NB)                                                                     \
        }                                                                                                 \
        FP8DS_MFMA(CA, CB)                                                                                \
        __builtin_amdgcn_sched_barrier(0);                                                                \
    }
    FP8DS_TSTEP(kt + 0, st1, st3, fa0, fb0, fa1, fb1)
    FP8DS_TSTEP(kt + 1, st2, st0, fa1, fb1, fa0, fb0)
    FP8DS_TSTEP(kt + 2, st3, st1, fa0, fb0, fa1, fb1)
    FP8DS_TSTEP(kt + 3, st0, st2, fa1, fb1, fa0, fb0)
    FP8DS_TSTEP(kt + 4, st1, st3, fa0, fb0, fa1, fb1)
    FP8DS_TSTEP(kt + 5, st2, st0, fa1, fb1, fa0, fb0)
#undef FP8DS_TSTEP
#undef FP8DS_ISSUE
#undef FP8DS_FRAGS
#undef FP8DS_MFMA
#undef FP8DS_STEP
    __syncthreads();   // every wave is done reading the operand stages
    uint8_t *wl = wave == 0 ? st0 : wave == 1 ? st1 : wave == 2 ? st2 : st3;
    // The bias of the 64 columns this lane holds, two values per register, loaded together before
    // the epilogue uses them: a load guarded by the null check (or a select right after it) would
    // be waited for on its own, one memory round trip per column.  Without a bias the loads read
    // the first two bytes of a_sinv.
    const bool has_bias = bias != nullptr;
    const uint16_t *bsrc = has_bias ? bias : reinterpret_cast<const uint16_t *>(a_sinv);
    const int col0 = n0 + wn * 128, bhalf = lane >> 5;
    us2 braw[4][4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                braw[j][q][u >> 1][u & 1] = bsrc[has_bias ? min(col0 + j * 32 + q * 8 + bhalf * 4 + u, N - 1) : 0];
    epilogue_staged<OUT>(acc, sa, sb, ds, has_bias, braw, D, ldd, M, N, m0 + wm * 128, col0, lane, wl, oq);
}

// ------------------------------------------------------------------------------------------
// k_gemm_small: problems with fewer than kSmallTiles 256 x 256 tiles (K % 64 == 0).  One wave
// per 64 x 64 tile, so small outputs still spread over many CUs; each lane loads its own operand
// fragments straight from global memory into registers, four 64-byte K slices ahead (no LDS,
// no barriers).  The MFMAs, their operand order and their K order are those of
// k_gemm_bias_pipe, and so is the epilogue arithmetic, so both kernels give the same bits for
// every element.
// ------------------------------------------------------------------------------------------
constexpr int kSmallTile = 64;
// Below this many 256 x 256 tiles the small kernel is used: measured crossover on MI355X
// (M x N x K = 1024 x 2048 x 4096, 32 tiles: small 38 us vs 44 us; 2048 x 2048 x 4096, 64 tiles:
// small 72 us vs 44 us).
constexpr int kSmallTiles = 40;

template <int FA, int FB, int OUT>
__global__ __launch_bounds__(64) void k_gemm_small(const uint8_t *__restrict__ A, int64_t lda,
                                                   const uint8_t *__restrict__ B, int64_t ldb,
                                                   const float *__restrict__ a_sinv, const float *__restrict__ b_sinv,
                                                   const uint16_t *__restrict__ bias, void *__restrict__ D, int64_t ldd,
                                                   int M, int N, int K, int tiles_n, OutQuant oq) {
    if constexpr (OUT >= 2)
        if (blockIdx.x == 0 && threadIdx.x == 0 && oq.scale_inv_out != nullptr) *oq.scale_inv_out = 1.0f / *oq.scale;
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - (blockIdx.x / tiles_n) * tiles_n;
    const int m0 = tm * kSmallTile, n0 = tn * kSmallTile;
    const int lane = threadIdx.x, frow = lane & 31, fhalf = lane >> 5;
    // lane l supplies row l % 32 of each 32-row operand tile and bytes [32 (l / 32), +32) of the
    // slice; rows past M / N read the last row (their values are never stored or counted)
    const uint8_t *pa[2], *pb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        pa[i] = A + (int64_t)min(m0 + i * 32 + frow, M - 1) * lda + fhalf * 32;
        pb[i] = B + (int64_t)min(n0 + i * 32 + frow, N - 1) * ldb + fhalf * 32;
    }
    auto ld32 = [](const uint8_t *p) -> i32x8 {
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(p);
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(p + 16);
        i32x8 r;
        r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
        r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
        return r;
    };
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    // the inverse scales, output scale and bias are read before the K loop, so their latency
    // overlaps the operand loads; bias columns past N read bias[N - 1] (never stored).  The bias
    // loads are unconditional (without a bias they read the first two bytes of a_sinv) and the
    // raw bits are kept: a load inside a branch, or a select right after it, would wait for each
    // load in turn; the bias itself is chosen where it is used.
    const float sa = *a_sinv, sb = *b_sinv;
    float ds = 0.f;
    if constexpr (OUT >= 2) ds = *oq.scale;
    const bool has_bias = bias != nullptr;
    const uint16_t *bsrc = has_bias ? bias : reinterpret_cast<const uint16_t *>(a_sinv);
    uint32_t braw[2][4][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int col = min(n0 + j * 32 + q * 8 + fhalf * 4 + u, N - 1);
                braw[j][q][u] = bsrc[has_bias ? col : 0];
            }
    const int nk = K / kPK;
#define FP8DS_SLOAD(FA_, FB_, kt)                                                                          \
    _Pragma("unroll") for (int i = 0; i < 2; ++i) {                                                       \
        FA_[i] = ld32(pa[i] + (int64_t)(kt) * kPK);                                                       \
        FB_[i] = ld32(pb[i] + (int64_t)(kt) * kPK);                                                       \
    }
#define FP8DS_SMFMA(FA_, FB_)                                                                              \
    _Pragma("unroll") for (int i = 0; i < 2; ++i)                                                         \
    _Pragma("unroll") for (int j = 0; j < 2; ++j)                                                         \
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(FB_[j], FA_[i], acc[i][j], FB, FA, 0, 0, 0, 0);
    // The loads are unconditional (slice indices clamped to the last slice; the extra loads at
    // the end stay in bounds and are never used): a load behind a branch leaves the compiler
    // unable to count what is in flight, and it then waits for every outstanding load.
    i32x8 a0[2], b0[2], a1[2], b1[2], a2[2], b2[2], a3[2], b3[2];
    FP8DS_SLOAD(a0, b0, 0)
    FP8DS_SLOAD(a1, b1, min(1, nk - 1))
    FP8DS_SLOAD(a2, b2, min(2, nk - 1))
    FP8DS_SLOAD(a3, b3, min(3, nk - 1))
    int kt = 0;
    for (; kt + 4 <= nk; kt += 4) {
        FP8DS_SMFMA(a0, b0)
        FP8DS_SLOAD(a0, b0, min(kt + 4, nk - 1))
        FP8DS_SMFMA(a1, b1)
        FP8DS_SLOAD(a1, b1, min(kt + 5, nk - 1))
        FP8DS_SMFMA(a2, b2)
        FP8DS_SLOAD(a2, b2, min(kt + 6, nk - 1))
        FP8DS_SMFMA(a3, b3)
        FP8DS_SLOAD(a3, b3, min(kt + 7, nk - 1))
    }
    // the last nk % 4 slices, already in a0, a1, a2 in K order
    if (kt < nk) { FP8DS_SMFMA(a0, b0) }
    if (kt + 1 < nk) { FP8DS_SMFMA(a1, b1) }
    if (kt + 2 < nk) { FP8DS_SMFMA(a2, b2) }
#undef FP8DS_SLOAD
#undef FP8DS_SMFMA
    // epilogue, element by element: lane l holds D[m0 + 32 i + l % 32][n0 + 32 j + 8 (e / 4) +
    // 4 (l / 32) + e % 4] in element e of acc[i][j]
    uint32_t amag = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = m0 + i * 32 + frow;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int col = n0 + j * 32 + (e >> 2) * 8 + fhalf * 4 + (e & 3);
                const float b = has_bias ? __uint_as_float(braw[j][e >> 2][e & 3] << 16) : 0.f;
                const float v = dequant_bias(acc[i][j][e], sa, sb, b);
                if (row < M && col < N) {
                    const int64_t o = (int64_t)row * ldd + col;
                    if constexpr (OUT == 0) {
                        reinterpret_cast<uint16_t *>(D)[o] = f32_to_bf16_rne(v);
                    } else if constexpr (OUT == 1) {
                        reinterpret_cast<float *>(D)[o] = v;
                    } else {
                        amag = max(amag, __float_as_uint(v) & 0x7FFFFFFFu);
                        reinterpret_cast<uint8_t *>(D)[o] = (uint8_t)encode_exact<OUT - 2>(v * ds);
                    }
                }
            }
    }
    if constexpr (OUT >= 2) {
        amag = wave_max_u32(amag);
        if (lane == 0) fold_amax_bits(oq.amax, amag);
    }
}

// D = bias broadcast (K == 0): no products at all.
template <int OUT>
__global__ __launch_bounds__(256) void k_bias_only(const uint16_t *__restrict__ bias, void *__restrict__ D,
                                                   int64_t ldd, int M, int N, OutQuant oq) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t amag = 0;
    if (idx < (int64_t)M * N) {
        const int64_t m = idx / N, n = idx % N;
        // 0 + bias, as for K > 0 with a zero sum (a -0 bias gives +0)
        const float v = (bias != nullptr ? __uint_as_float((uint32_t)bias[n] << 16) : 0.f) + 0.0f;
        if constexpr (OUT == 0) {
            reinterpret_cast<uint16_t *>(D)[m * ldd + n] = f32_to_bf16_rne(v);
        } else if constexpr (OUT == 1) {
            reinterpret_cast<float *>(D)[m * ldd + n] = v;
        } else {
            amag = __float_as_uint(v) & 0x7FFFFFFFu;
            reinterpret_cast<uint8_t *>(D)[m * ldd + n] = (uint8_t)encode_exact<OUT - 2>(v * *oq.scale);
        }
    }
    if constexpr (OUT >= 2) {
        if (blockIdx.x == 0 && threadIdx.x == 0 && oq.scale_inv_out != nullptr) *oq.scale_inv_out = 1.0f / *oq.scale;
        amag = wave_max_u32(amag);
        if ((threadIdx.x & 63) == 0) fold_amax_bits(oq.amax, amag);
    }
}

hipError_t launch_gemm_bias(const uint8_t *A, int fa, const float *a_sinv, int64_t lda, const uint8_t *B, int fb,
                            const float *b_sinv, int64_t ldb, const uint16_t *bias, void *D, int64_t ldd,
                            int out_dtype, int64_t M, int64_t N, int64_t K, const float *d_scale,
                            float *d_sinv_out, float *d_amax, hipStream_t st) {
    const OutQuant oq{d_scale, d_sinv_out, d_amax};
    if (M == 0 || N == 0) {
        // nothing to write but the output's inverse scale
        if (out_dtype >= 2 && d_sinv_out != nullptr) {
            if (out_dtype == 2) k_bias_only<2><<<1, 64, 0, st>>>(bias, D, ldd, 0, 0, oq);
            else k_bias_only<3><<<1, 64, 0, st>>>(bias, D, ldd, 0, 0, oq);
            return hipGetLastError();
        }
        return hipSuccess;
    }
    if (K == 0) {
        const int64_t total = M * N;
        dim3 grid((unsigned)((total + 255) / 256));
        switch (out_dtype) {
            case 0: k_bias_only<0><<<grid, 256, 0, st>>>(bias, D, ldd, (int)M, (int)N, oq); break;
            case 1: k_bias_only<1><<<grid, 256, 0, st>>>(bias, D, ldd, (int)M, (int)N, oq); break;
            case 2: k_bias_only<2><<<grid, 256, 0, st>>>(bias, D, ldd, (int)M, (int)N, oq); break;
            default: k_bias_only<3><<<grid, 256, 0, st>>>(bias, D, ldd, (int)M, (int)N, oq); break;
        }
        return hipGetLastError();
    }
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    dim3 grid((unsigned)(tiles_m * tiles_n));
    const bool k64 = (K % kPK) == 0;
    const bool pipe = k64 && lda < kPipeMaxLd && ldb < kPipeMaxLd;
    const bool small = k64 && (int64_t)tiles_m * tiles_n < kSmallTiles;
    const int stiles_n = (int)((N + kSmallTile - 1) / kSmallTile);
    dim3 sgrid((unsigned)(((M + kSmallTile - 1) / kSmallTile) * stiles_n));
#define FP8DS_GEMM(FA_, FB_, O_)                                                                           \
    do {                                                                                                   \
        if (small)                                                                                         \
            k_gemm_small<FA_, FB_, O_><<<sgrid, dim3(64), 0, st>>>(                                        \
                A, lda, B, ldb, a_sinv, b_sinv, bias, D, ldd, (int)M, (int)N, (int)K, stiles_n, oq);       \
        else if (pipe)                                                                                     \
            k_gemm_bias_pipe<FA_, FB_, O_><<<grid, dim3(kThreads), 0, st>>>(                               \
                A, lda, B, ldb, a_sinv, b_sinv, bias, D, ldd, (int)M, (int)N, (int)K, tiles_m, tiles_n, oq); \
        else                                                                                               \
            k_gemm_bias<FA_, FB_, O_><<<grid, dim3(kThreads), 0, st>>>(                                    \
                A, lda, B, ldb, a_sinv, b_sinv, bias, D, ldd, (int)M, (int)N, (int)K, tiles_m, tiles_n, oq); \
    } while (0)
#define FP8DS_GEMM_OUT(FA_, FB_)                                                                           \
    switch (out_dtype) {                                                                                   \
        case 0: FP8DS_GEMM(FA_, FB_, 0); break;                                                            \
        case 1: FP8DS_GEMM(FA_, FB_, 1); break;                                                            \
        case 2: FP8DS_GEMM(FA_, FB_, 2); break;                                                            \
        default: FP8DS_GEMM(FA_, FB_, 3); break;                                                           \
    }
    switch (fa * 2 + fb) {
        case 0: FP8DS_GEMM_OUT(kE4M3, kE4M3) break;
        case 1: FP8DS_GEMM_OUT(kE4M3, kE5M2) break;
        case 2: FP8DS_GEMM_OUT(kE5M2, kE4M3) break;
        default: FP8DS_GEMM_OUT(kE5M2, kE5M2) break;
    }
#undef FP8DS_GEMM_OUT
#undef FP8DS_GEMM
    return hipGetLastError();
}

}  // namespace fp8ds
