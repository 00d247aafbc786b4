// gemm.hip -- FP8 GEMM with inverse-scale dequantisation and bias on gfx950 matrix cores.
//
//   D[m, n] = (sum_k A[m, k] * B[n, k]) * a_scale_inv * b_scale_inv + bias[n]
//
// The fp8_gemm of "[PyTorch] cuda graph support" (transpose-cache thread, FP8Linear.backward)
// and the per-chunk bias of "[PyTorch] Userbuffers support in operation-based API" (bias-offset
// fix).  Both operands are K-contiguous ("TN"); the transposes the backward needs come from
// the cast+transpose kernels, so the GEMM never transposes.
//
// Two kernel families, chosen from K and the row strides alone (never from M or N, so every
// N-chunk of a GEMM takes the same family as the whole):
//   * the 16 x 16 x 128 family (K % 256 == 0, row strides below 8 MiB; the hot path):
//     k_gemm_pipe16 (256 x 256 tiles, 2 x 2 waves of 128 x 128 made of 8 x 8
//     v_mfma_f32_16x16x128_f8f6f4 tiles) and k_gemm_small16 (one wave per 64 x 64 tile, for
//     problems of few large tiles: up to 32, 48 with K <= 1024, 64 with K == 256);
//   * the 32 x 32 x 64 family (every other K % 16 == 0): k_gemm_bias_pipe (K % 64 == 0, strides
//     below 8 MiB), k_gemm_small (K % 64 == 0, under 45 large tiles) and k_gemm_bias (general
//     K, tail zero-filled), waves of 4 x 4 v_mfma_f32_32x32x64_f8f6f4 tiles.
// Inside a family every output element is one fixed sequence of MFMAs over K in the same K
// order, whatever kernel or tile it falls in, so the kernels of a family give identical bits
// (no split-K).  The two families differ in the last bits now and then: the 16 x 16 x 128 MFMA
// sums 128 products per instruction, the 32 x 32 x 64 one 64.  Float32 accumulate; the A / B
// formats are the instruction's cbsz / blgp selectors, so every format pair shares one template.
// Blocks of the 256 x 256 kernels are remapped so that each XCD (blocks are dealt round-robin to
// the 8 XCDs) works on a contiguous range of tiles, walked in groups of kGroupM tile-rows for L2
// reuse.  Epilogue: acc * a_scale_inv * b_scale_inv + bias in float32, rounded to bfloat16
// (nearest even), stored as float32, or encoded to FP8 with amax capture (the pipelined kernels
// stage bfloat16 and FP8 outputs through LDS and write 16-byte row segments; interior float32
// sub-tiles go straight from the accumulators as whole 128-byte lines).  Ragged M / N are
// handled by clamping the rows that are loaded and masking the stores.
//
// k_gemm_bias_pipe: a 4-stage pipeline of 64-byte K slices (4 x 32 KB of LDS).  Global memory goes
// straight into LDS with buffer_load_dwordx4 ... lds (no staging registers; per-tile descriptors,
// 32-bit per-lane offsets, the K slice in the scalar offset), three slices ahead of the MFMAs;
// each wave prefetches the next slice's operand fragments from LDS while its MFMAs run on the
// current ones (double-buffered fragments), and the instruction scheduler is told to place the
// fragment reads and global loads among the first 12 of the slice's 16 MFMAs.  The four stages
// are four distinct LDS arrays so the compiler can tell the in-flight loads of one stage from the
// reads of another, and the per-slice barrier is a bare s_barrier after an explicit vmcnt wait (a
// fenced barrier would drain every load in flight).  LDS rows are 64 bytes; 16-byte chunk c of
// row r sits at chunk c ^ ((r >> 2) & 3), which measured bank-conflict free for the MFMA operand
// reads.  k_gemm_pipe16 (further down) keeps these techniques with 128-byte K steps.
//
// k_gemm_bias (any K % 16 == 0): global -> registers -> LDS with double-buffered 128-byte K
// slices, the K tail zero-filled.
//
// k_linear_fwd_small (further down): the whole forward of a small layer (casts of x and W, GEMM +
// bias) in one launch, with the MFMAs of k_gemm_small16.
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

// Tile of this block.  The tile-rows are taken in bands of band_rows (all of them when the
// operands fit in the chip's 256 MB Infinity Cache), one band after the other in block order;
// inside a band each XCD (blocks are dealt round-robin to the 8 XCDs) works on a contiguous range
// of tiles, walked in groups of kGroupM tile-rows for L2 reuse.  When A and B together exceed the
// Infinity Cache, finishing a band of A rows against all of B before the next keeps the A rows
// every XCD re-reads cache-resident while B streams through (measured on the QKV forward GEMM,
// 327 MB of operands: 5% faster with bands of 8 tile-rows, no change where the operands fit).
__device__ __forceinline__ void block_tile(int tiles_m, int tiles_n, int band_rows, int &tm, int &tn) {
    const int per = band_rows * tiles_n;
    const int band = (int)blockIdx.x / per;
    const int rows0 = band * band_rows;
    const int rows = min(band_rows, tiles_m - rows0);
    const int bid = (int)blockIdx.x - band * per;
    const int nwg = rows * tiles_n;
    const int xcd = bid & 7, local = bid >> 3;
    const int q8 = nwg >> 3, r8 = nwg & 7;
    const int tile = (xcd < r8) ? xcd * (q8 + 1) + local : r8 * (q8 + 1) + (xcd - r8) * q8 + local;
    const int group = tile / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gm = min(rows - first_m, kGroupM);
    const int in_group = tile - group * kGroupM * tiles_n;
    tm = rows0 + first_m + in_group % gm;
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

// A wave's 128 x 128 accumulator sub-tile seen as 64 "quads" of four consecutive columns of one
// row, in one of the two MFMA layouts the pipelined kernels use (both take B as the MFMA's first
// operand; the products and their summation order are the same as with A first).  visit<RLO, RHI>
// calls f(r, sl, v) for every quad whose sub-tile row r lies in [RLO, RHI), with sl the 4-column
// slot (columns 4 sl .. 4 sl + 3) and v the four values after acc * a_scale_inv * b_scale_inv +
// bias.  The bias comes from raw bits the kernel loaded before its epilogue; columns past N take
// bias[N - 1]: their operand rows are clamped to row N - 1 of B, so every value a lane holds
// outside the output (rows past M read row M - 1 of A) is bit-identical to an element inside it.
// Such values are never stored, and the FP8 output's amax can take the max over the whole
// sub-tile without masking.
//
// 32 x 32 x 64 MFMAs: lane l holds D[row0 + 32 i + l % 32][col0 + 32 j + 8 q + 4 (l / 32) + u] in
// element 4 q + u of acc[i][j]; braw[j][q][u / 2][u % 2] = bias[col0 + 32 j + 8 q + 4 (l / 32) + u].
struct Quads32 {
    const f32x16 (&acc)[4][4];
    const us2 (&braw)[4][4][2];
    bool has_bias;
    float sa, sb;
    int lane;
    template <int RLO, int RHI, class F>
    __device__ __forceinline__ void visit(F &&f) const {
        const int frow = lane & 31, fhalf = lane >> 5;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i * 32 < RLO || i * 32 >= RHI) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float v[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        v[u] = dequant_bias(acc[i][j][q * 4 + u], sa, sb,
                                            has_bias ? __uint_as_float((uint32_t)braw[j][q][u >> 1][u & 1] << 16) : 0.f);
                    f(i * 32 + frow, j * 8 + q * 2 + fhalf, v);
                }
            }
    }
};

// 16 x 16 x 128 MFMAs: lane l holds D[row0 + 16 i + l % 16][col0 + 16 j + 4 (l / 16) + u] in
// element u of acc[i][j]; braw[j][u / 2][u % 2] = bias[col0 + 16 j + 4 (l / 16) + u].
struct Quads16 {
    const f32x4 (&acc)[8][8];
    const us2 (&braw)[8][2];
    bool has_bias;
    float sa, sb;
    int lane;
    template <int RLO, int RHI, class F>
    __device__ __forceinline__ void visit(F &&f) const {
        const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i * 16 < RLO || i * 16 >= RHI) continue;
                float v[4];
                values(i, j, v);
                f(i * 16 + r16, j * 4 + g, v);
            }
    }
    // the four values of MFMA tile (i, j) this lane holds
    __device__ __forceinline__ void values(int i, int j, float (&v)[4]) const {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            v[u] = dequant_bias(acc[i][j][u], sa, sb,
                                has_bias ? __uint_as_float((uint32_t)braw[j][u >> 1][u & 1] << 16) : 0.f);
    }
};

// float32 output of a wave's 128 x 128 sub-tile straight from the 16 x 16 x 128 accumulators.
// In MFMA tiles (i, j) and (i, j + 1), row r of the pair is 128 contiguous bytes: 64 from the four
// lanes (r, g) of tile j and 64 from the same lanes of tile j + 1.  Lanes r and r ^ 8 (the same
// 16-lane DPP row) swap one of their two 16-byte quads (lanes r < 8 send tile j + 1, lanes r >= 8
// send tile j), so each store instruction writes eight rows as whole 128-byte lines: the first
// rows 0-7 of the pair (lanes r < 8 the left halves, lanes r >= 8 the right halves of rows r - 8),
// the second rows 8-15.  Interior sub-tiles with 16-byte aligned rows only.
__device__ __forceinline__ float dpp_swap8(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, true));   // row_ror:8
}
__device__ __forceinline__ void store_f32_direct(const Quads16 &q, float *__restrict__ D, int64_t ldd, int row0,
                                                 int col0) {
    const int r16 = q.lane & 15, g = q.lane >> 4;
    const bool hi = r16 >= 8;
    const int rr = r16 & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jp = 0; jp < 4; ++jp) {
            float t0[4], t1[4], x[4];
            q.values(i, 2 * jp, t0);
            q.values(i, 2 * jp + 1, t1);
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] = dpp_swap8(hi ? t0[u] : t1[u]);
            const int col = col0 + 16 * (2 * jp + (hi ? 1 : 0)) + 4 * g;
            float *pa = D + (int64_t)(row0 + i * 16 + rr) * ldd + col;
            float *pb = pa + 8 * ldd;
            const f32x4 va = hi ? f32x4{x[0], x[1], x[2], x[3]} : f32x4{t0[0], t0[1], t0[2], t0[3]};
            const f32x4 vb = hi ? f32x4{t1[0], t1[1], t1[2], t1[3]} : f32x4{x[0], x[1], x[2], x[3]};
            __builtin_nontemporal_store(va, reinterpret_cast<f32x4 *>(pa));
            __builtin_nontemporal_store(vb, reinterpret_cast<f32x4 *>(pb));
        }
}

// Epilogue of the pipelined kernels.  Each wave scales, adds the bias and rounds its 128 x 128
// sub-tile into its own 32 KB of LDS, then writes whole rows with 16-byte streaming
// (nontemporal) stores.  bf16: one pass, row r at r * 256, 8-byte slot s (columns 4 s .. 4 s + 3)
// stored at slot s ^ (r & 31).  float32: two passes of 64 rows, row r at r * 512, 16-byte slot s
// at s ^ (r & 31).  Where D or ldd is not 16-byte aligned, or at the ragged right edge, the
// elements are stored one by one.
template <int OUT, class Q>
__device__ __forceinline__ void epilogue_staged(const Q &quads, float ds, void *__restrict__ D, int64_t ldd,
                                                int M, int N, int row0, int col0, int lane, uint8_t *wlds,
                                                OutQuant oq) {
    constexpr int kElemsPer16 = OUT == 0 ? 8 : OUT == 1 ? 4 : 16;
    const bool vec_ok = ((reinterpret_cast<uintptr_t>(D) & 15u) == 0) && (ldd % kElemsPer16 == 0);
    if constexpr (OUT == 0) {
        quads.template visit<0, 128>([&](int r, int sl, const float (&v)[4]) {
            const u32x2 pk = {f32x2_to_bf16x2_rne(v[0], v[1]), f32x2_to_bf16x2_rne(v[2], v[3])};
            *reinterpret_cast<u32x2 *>(wlds + r * 256 + ((sl ^ (r & 31)) << 3)) = pk;
        });
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
        // interior 16 x 16 x 128 sub-tiles: straight from the accumulators (same-process A/B on
        // the wgrad shape: +0.5% against the staged passes below, identical bits)
        if constexpr (std::is_same_v<Q, Quads16>) {
            if (vec_ok && row0 + 128 <= M && col0 + 128 <= N) {
                store_f32_direct(quads, reinterpret_cast<float *>(D), ldd, row0, col0);
                return;
            }
        }
        auto pass = [&](auto hc) {
            constexpr int h = decltype(hc)::value;
            quads.template visit<h * 64, h * 64 + 64>([&](int r, int sl, const float (&v)[4]) {
                const int rr = r - h * 64;
                const u32x4 pk = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                  __float_as_uint(v[3])};
                *reinterpret_cast<u32x4 *>(wlds + rr * 512 + ((sl ^ (rr & 31)) << 4)) = pk;
            });
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
        };
        pass(std::integral_constant<int, 0>{});
        pass(std::integral_constant<int, 1>{});
    } else {
        // FP8: 128 rows x 128 bytes = 16 KB; row r at r * 128, 4-byte slot s (columns 4 s ..
        // 4 s + 3) stored at slot s ^ (r & 31).
        // Pass 1: the amax.  Unsigned order of magnitude bit patterns is numeric order with NaN
        // above inf, so the wave's amax also says whether any value is NaN.  Pass 2 recomputes
        // the values and, unless a NaN or a non-plain scale makes a scaled value NaN, encodes
        // them with the clamp + hardware conversion alone (one wave-uniform branch).
        constexpr int F = OUT - 2;
        uint32_t amag = 0;
        quads.template visit<0, 128>([&](int, int, const float (&v)[4]) {
#pragma unroll
            for (int u = 0; u < 4; ++u) amag = max(amag, __float_as_uint(v[u]) & 0x7FFFFFFFu);
        });
        amag = __builtin_amdgcn_readfirstlane(wave_max_u32(amag));   // wave-uniform
        if (lane == 0) fold_amax_bits(oq.amax, amag);
        auto stage = [&](auto fast_tag) {
            constexpr bool kFast = decltype(fast_tag)::value;
            quads.template visit<0, 128>([&](int r, int sl, const float (&v)[4]) {
                float y[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) y[u] = v[u] * ds;
                uint32_t w;
                if constexpr (kFast)
                    w = pack4<F>(clamp_fmt<F>(y[0]), clamp_fmt<F>(y[1]), clamp_fmt<F>(y[2]), clamp_fmt<F>(y[3]));
                else
                    w = encode_exact<F>(y[0]) | (encode_exact<F>(y[1]) << 8) | (encode_exact<F>(y[2]) << 16) |
                        (encode_exact<F>(y[3]) << 24);
                *reinterpret_cast<uint32_t *>(wlds + r * 128 + ((sl ^ (r & 31)) << 2)) = w;
            });
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
                                                           int K, int tiles_m, int tiles_n, int band_rows,
                                                             OutQuant oq) {
    if constexpr (OUT >= 2)
        if (blockIdx.x == 0 && threadIdx.x == 0 && oq.scale_inv_out != nullptr) *oq.scale_inv_out = 1.0f / *oq.scale;
    __shared__ __align__(16) uint8_t smem[kLdsBytes];

    int tm, tn;
    block_tile(tiles_m, tiles_n, band_rows, tm, tn);
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
                                                                int K, int tiles_m, int tiles_n, int band_rows,
                                                             OutQuant oq) {
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
    block_tile(tiles_m, tiles_n, band_rows, tm, tn);
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
    epilogue_staged<OUT>(Quads32{acc, braw, has_bias, sa, sb, lane}, ds, D, ldd, M, N, m0 + wm * 128, col0, lane, wl, oq);
}

// ------------------------------------------------------------------------------------------
// k_gemm_pipe16: the hot-path kernel for K % 256 == 0.  Same 256 x 256 block tile and 2 x 2 waves
// of 128 x 128, but built on v_mfma_f32_16x16x128_f8f6f4 (8 x 8 MFMA tiles per wave), which under
// the chip's power limit sustains more FP8 throughput than the 32 x 32 x 64 form.  One K step is
// 128 bytes; A and B have separate 32 KB LDS slots (256 rows x 128 bytes), two of each:
//   step j computes with A_j (its fragments read one 16-row block ahead of the MFMAs) and B_j
//   (whose fragments were read into registers during step j-1), while reading the fragments of
//   B_{j+1} and, last, A_{j+1}'s first block.  B_j's slot is free once its fragments are in
//   registers, so B runs a step further ahead than A: the loads of step j are B_{j+2} (into B_j's
//   slot) and A_{j+1} (into the slot A_{j-1} used), 16 per wave, B's first, issued four after the
//   previous step's barrier and three in each of the first four 16-row blocks; step j waits for
//   them once, before its last block, with one barrier (which also frees A_j's and B_{j+1}'s
//   slots).
// Loads into LDS are buffer loads (per-tile descriptors, 32-bit lane offsets, the K step in the
// scalar offset); a load index past the last K step is clamped to it (the extra loads at the end
// refill free slots and are never read).  LDS rows are 128 bytes; 16-byte chunk c of row r sits
// at c ^ (r % 8) ^ ((r / 8) % 2): the 16 lanes of a fragment read that share a chunk then hit
// distinct banks both as two groups of 8 rows and as one group of 16 (the bank-conflict counter
// reads 0; c ^ ((r / 2) % 8), distinct only for 16, counted 7.6e7 conflict cycles per launch).  The epilogue is
// the staged one above.  k_gemm_small16 does the same MFMAs in the same K order, so the two give
// identical bits; they do not match the 32 x 32 x 64 kernels bit for bit (the MFMA sums 128
// products per instruction), so a GEMM takes all its tiles from one family: the launcher picks
// the family from K and the row strides alone, never from M or N.
// ------------------------------------------------------------------------------------------
namespace {
constexpr int kQK = 128;                          // K bytes per step
constexpr int kQSlice = 256 * kQK;                // one operand slot: 256 rows x 128 bytes
constexpr int kFam16K = 2 * kQK;                  // K multiple for the 16 x 16 x 128 family
__device__ __forceinline__ int qswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
}  // namespace

// vmcnt(0) and lgkmcnt(0): every load into LDS and every LDS read of this wave has completed
#define FP8DS_WAIT_ALL() __builtin_amdgcn_s_waitcnt(0x0070)

template <int FA, int FB, int OUT>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_pipe16(const uint8_t *__restrict__ A, int64_t lda,
                                                             const uint8_t *__restrict__ B, int64_t ldb,
                                                             const float *__restrict__ a_sinv,
                                                             const float *__restrict__ b_sinv,
                                                             const uint16_t *__restrict__ bias,
                                                             void *__restrict__ D, int64_t ldd, int M, int N,
                                                             int K, int tiles_m, int tiles_n, int band_rows,
                                                             OutQuant oq) {
    if constexpr (OUT >= 2)
        if (blockIdx.x == 0 && threadIdx.x == 0 && oq.scale_inv_out != nullptr) *oq.scale_inv_out = 1.0f / *oq.scale;
    const float sa = *a_sinv, sb = *b_sinv;
    float ds = 0.f;
    if constexpr (OUT >= 2) ds = *oq.scale;
    __shared__ __align__(16) uint8_t sa0[kQSlice];
    __shared__ __align__(16) uint8_t sa1[kQSlice];
    __shared__ __align__(16) uint8_t sb0[kQSlice];
    __shared__ __align__(16) uint8_t sb1[kQSlice];

    int tm, tn;
    block_tile(tiles_m, tiles_n, band_rows, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // Load i (0-7) of wave w fills the slot's 1 KB block 4 i + w = rows 8 (4 i + w) .. +7: lane l
    // takes row 32 i + 8 w + l / 8, stored chunk l % 8, i.e. source chunk (l % 8) ^ qswz(row),
    // where qswz(row) = (l / 8) ^ (w % 2) for every i.
    const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(A + (int64_t)m0 * lda), (short)0, (int)(rows_a * lda), kBufDesc3);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(B + (int64_t)n0 * ldb), (short)0, (int)(rows_b * ldb), kBufDesc3);
    const int lrow = wave * 8 + (lane >> 3);
    const int lsc = (lane & 7) ^ ((lane >> 3) ^ (wave & 1));
    uint32_t va[8], vb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = i * 32 + lrow;
        va[i] = (uint32_t)(min(r, rows_a - 1) * lda + lsc * 16);
        vb[i] = (uint32_t)(min(r, rows_b - 1) * ldb + lsc * 16);
    }
    const int nk = K / kQK;   // even
#define FP8DS_LD_A(SA_, j, i)                                                                              \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, (__attribute__((address_space(3))) void *)((SA_) + ((i) * 4 + wave) * 1024), \
                                             16, va[i], (uint32_t)(min((j), nk - 1) * kQK), 0, 0);
#define FP8DS_LD_B(SB_, j, i)                                                                              \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, (__attribute__((address_space(3))) void *)((SB_) + ((i) * 4 + wave) * 1024), \
                                             16, vb[i], (uint32_t)(min((j), nk - 1) * kQK), 0, 0);
    // loads n0 .. n1-1 of a step's 16, B's eight first, then A's (A step jA, B step jB): each
    // operand's loads issued as a group measured 2.5-4.3% faster on the two QKV shapes whose
    // operands exceed the Infinity Cache than A and B alternating (A first: 1.7-3.1%)
#define FP8DS_LDS(n0, n1, SA_, SB_, jA, jB)                                                                \
    _Pragma("unroll") for (int n = (n0); n < (n1); ++n) {                                                 \
        if (n < 8) { FP8DS_LD_B(SB_, jB, n) } else { FP8DS_LD_A(SA_, jA, n - 8) }                          \
    }

    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Operand fragment of a 16-row MFMA tile: lane l supplies row l % 16 and K bytes
    // [32 (l / 16), +32) of the step, two 16-byte reads.
    const int r16 = lane & 15, g = lane >> 4;
    const int oc0 = r16 * kQK + (((2 * g) ^ qswz(r16)) << 4);
    const int oc1 = r16 * kQK + (((2 * g + 1) ^ qswz(r16)) << 4);
    const int offa = wm * 128 * kQK, offb = wn * 128 * kQK;
    auto ld = [&](const uint8_t *p) -> i32x8 {
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(p + oc0);
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(p + oc1);
        i32x8 r;
        r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
        r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
        return r;
    };
    i32x8 fb0[8], fb1[8], fa0, fa1;
#define FP8DS_MF(FBC, FA_, i)                                                                              \
    _Pragma("unroll") for (int j = 0; j < 8; ++j)                                                         \
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(FBC[j], FA_, acc[i][j], FB, FA, 0, 0, 0, 0);
    // scheduling of one 16-row block: its 8 MFMAs, with NRD fragment reads and NLD loads placed
    // one (loads: up to two) after each MFMA from the first on
#define FP8DS_SG(NRD, NLD)                                                                                 \
    _Pragma("unroll") for (int q = 0; q < 8; ++q) {                                                       \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                \
        if (q < (NRD)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                 \
        if (q < (NLD)) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);                                 \
        if (q + 8 < (NLD)) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);                             \
    }
    // 16-row block i (0-6) of step j: read A frag i+1 and the next step's B frag i+1 (block 0 also
    // B frag 0); issue loads N0 .. N1-1 of step j; MFMAs with A frag i
#define FP8DS_BLK(i, j, SA_CUR, SA_NXT, SB_NXT, SB_FREE, FBC, FBN, FA_C, FA_N, N0, N1)                     \
    {                                                                                                     \
        FA_N = ld((SA_CUR) + offa + ((i) + 1) * 16 * kQK);                                                \
        if ((i) == 0) FBN[0] = ld((SB_NXT) + offb);                                                       \
        FBN[(i) + 1] = ld((SB_NXT) + offb + ((i) + 1) * 16 * kQK);                                        \
        FP8DS_LDS(N0, N1, SA_NXT, SB_FREE, (j) + 1, (j) + 2)                                              \
        FP8DS_MF(FBC, FA_C, i)                                                                            \
        FP8DS_SG(((i) == 0 ? 6 : 4), ((N1) - (N0)))                                                        \
        __builtin_amdgcn_sched_barrier(0);                                                                \
    }
    // Step j: A_j in SA_CUR, A_{j+1} in SA_NXT, B_{j+1} in SB_NXT, B_j's slot SB_FREE, B_j's
    // fragments in FBC.  Loads 4-15 of step j in blocks 0-3 (three each); wait + barrier; then
    // block 7 reads the next step's A frag 0 and issues loads 0-3 of step j+1 (the first four of
    // B_{j+3}, into SB_NXT, which the barrier freed; A_{j+2} follows into SA_CUR in blocks 1-3).
#define FP8DS_STEP16(j, SA_CUR, SA_NXT, SB_NXT, SB_FREE, FBC, FBN)                                         \
    {                                                                                                     \
        __builtin_amdgcn_sched_barrier(0);                                                                \
        FP8DS_BLK(0, j, SA_CUR, SA_NXT, SB_NXT, SB_FREE, FBC, FBN, fa0, fa1, 4, 7)                         \
        FP8DS_BLK(1, j, SA_CUR, SA_NXT, SB_NXT, SB_FREE, FBC, FBN, fa1, fa0, 7, 10)                        \
        FP8DS_BLK(2, j, SA_CUR, SA_NXT, SB_NXT, SB_FREE, FBC, FBN, fa0, fa1, 10, 13)                       \
        FP8DS_BLK(3, j, SA_CUR, SA_NXT, SB_NXT, SB_FREE, FBC, FBN, fa1, fa0, 13, 16)                       \
        FP8DS_BLK(4, j, SA_CUR, SA_NXT, SB_NXT, SB_FREE, FBC, FBN, fa0, fa1, 16, 16)                       \
        FP8DS_BLK(5, j, SA_CUR, SA_NXT, SB_NXT, SB_FREE, FBC, FBN, fa1, fa0, 16, 16)                       \
        FP8DS_BLK(6, j, SA_CUR, SA_NXT, SB_NXT, SB_FREE, FBC, FBN, fa0, fa1, 16, 16)                       \
        FP8DS_WAIT_ALL();                                                                                 \
        FP8DS_BARRIER();                                                                                  \
        __builtin_amdgcn_sched_barrier(0);                                                                \
        fa0 = ld((SA_NXT) + offa);                                                                        \
        FP8DS_LDS(0, 4, SA_CUR, SB_NXT, (j) + 2, (j) + 3)                                                 \
        FP8DS_MF(FBC, fa1, 7)                                                                             \
        FP8DS_SG(2, 4)                                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                                \
    }
    // prologue: A_0 and B_0, then B_1; wait for step 0, read B_0's fragments and A frag 0; wait
    // for B_1 and for every wave's reads of B_0's slot; issue loads 0-3 of step 0
    FP8DS_LDS(0, 16, sa0, sb0, 0, 0)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 8; ++i) { FP8DS_LD_B(sb1, 1, i) }
    __builtin_amdgcn_sched_barrier(0);
    FP8DS_WAIT_VM(8);
    FP8DS_BARRIER();
#pragma unroll
    for (int j = 0; j < 8; ++j) fb0[j] = ld(sb0 + offb + j * 16 * kQK);
    fa0 = ld(sa0 + offa);
    FP8DS_WAIT_ALL();
    FP8DS_BARRIER();
    __builtin_amdgcn_sched_barrier(0);
    FP8DS_LDS(0, 4, sa1, sb0, 1, 2)
    __builtin_amdgcn_sched_barrier(0);
    // A_j and B_j in slot j % 2, B_j's fragments in fb[j % 2]
    for (int j = 0; j < nk; j += 2) {
        FP8DS_STEP16(j, sa0, sa1, sb1, sb0, fb0, fb1)
        FP8DS_STEP16(j + 1, sa1, sa0, sb0, sb1, fb1, fb0)
    }
#undef FP8DS_STEP16
#undef FP8DS_BLK
#undef FP8DS_SG
#undef FP8DS_MF
#undef FP8DS_LDS
#undef FP8DS_LD_A
#undef FP8DS_LD_B
    __syncthreads();   // every load has landed and every wave is done reading the slots
    uint8_t *wl = wave == 0 ? sa0 : wave == 1 ? sa1 : wave == 2 ? sb0 : sb1;
    // the bias of the 32 columns this lane holds, two values per register, loaded together
    // (unconditional loads: without a bias they read the first two bytes of a_sinv)
    const bool has_bias = bias != nullptr;
    const uint16_t *bsrc = has_bias ? bias : reinterpret_cast<const uint16_t *>(a_sinv);
    const int col0 = n0 + wn * 128;
    us2 braw[8][2];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int u = 0; u < 4; ++u)
            braw[j][u >> 1][u & 1] = bsrc[has_bias ? min(col0 + j * 16 + g * 4 + u, N - 1) : 0];
    epilogue_staged<OUT>(Quads16{acc, braw, has_bias, sa, sb, lane}, ds, D, ldd, M, N, m0 + wm * 128, col0, lane, wl, oq);
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
// The 32 x 32 x 64 family takes its small kernel below this many 256 x 256 tiles (kernel time
// per launch on MI355X, small against pipelined: 36 tiles 24.5 vs 25.9 us at K = 2112, 40 tiles
// 15.9 vs 19.1 us at K = 1088, 48 tiles 15.3 vs 14.2 us at K = 320, 64 tiles 20.0 vs 16.3 us at
// K = 576).
constexpr int kSmallTiles = 45;
// The 16 x 16 x 128 family's choice also weighs K: k_gemm_small16 keeps one wave per 64 x 64
// tile, so it wins while its waves are few or short.  Kernel time per launch (graph of 20
// launches, MI355X), small16 against pipe16: 25-32 tiles 33 vs 40 us at K = 4096; 36-48 tiles
// 16.0-16.4 vs 17.5-17.8 us at K = 1024 but 27.7 vs 24.4 us at K = 2048; 64 tiles 8.7 vs
// 12.7 us at K = 256 but 15.3 vs 14.8 us at K = 512; 80 tiles 12.5 vs 12.9 us at K = 256.
__host__ __device__ constexpr bool small16_preferred(int64_t tiles, int64_t K) {
    return tiles <= 32 || (tiles <= 48 && K <= 1024) || (tiles <= 64 && K <= 256);
}

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

// k_gemm_small16: the small-problem kernel of the 16 x 16 x 128 family (K % 256 == 0).  One wave
// per 64 x 64 tile, 4 x 4 MFMA tiles of 16 x 16; each lane loads its operand fragments straight
// into registers, three 128-byte K steps ahead.  The MFMAs, their operand order and K order and
// the epilogue arithmetic are those of k_gemm_pipe16, so the two give the same bits.
template <int FA, int FB, int OUT>
__global__ __launch_bounds__(64) void k_gemm_small16(const uint8_t *__restrict__ A, int64_t lda,
                                                     const uint8_t *__restrict__ B, int64_t ldb,
                                                     const float *__restrict__ a_sinv, const float *__restrict__ b_sinv,
                                                     const uint16_t *__restrict__ bias, void *__restrict__ D,
                                                     int64_t ldd, int M, int N, int K, int tiles_n, OutQuant oq) {
    if constexpr (OUT >= 2)
        if (blockIdx.x == 0 && threadIdx.x == 0 && oq.scale_inv_out != nullptr) *oq.scale_inv_out = 1.0f / *oq.scale;
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - (blockIdx.x / tiles_n) * tiles_n;
    const int m0 = tm * kSmallTile, n0 = tn * kSmallTile;
    const int lane = threadIdx.x, r16 = lane & 15, g = lane >> 4;
    // lane l supplies row l % 16 of each 16-row operand tile and bytes [32 (l / 16), +32) of the
    // step; rows past M / N read the last row (their values are never stored or counted)
    const uint8_t *pa[4], *pb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        pa[i] = A + (int64_t)min(m0 + i * 16 + r16, M - 1) * lda + g * 32;
        pb[i] = B + (int64_t)min(n0 + i * 16 + r16, N - 1) * ldb + g * 32;
    }
    auto ld32 = [](const uint8_t *p) -> i32x8 {
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(p);
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(p + 16);
        i32x8 r;
        r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
        r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
        return r;
    };
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // scales, output scale and bias before the K loop; bias loads unconditional (see k_gemm_small)
    const float sa = *a_sinv, sb = *b_sinv;
    float ds = 0.f;
    if constexpr (OUT >= 2) ds = *oq.scale;
    const bool has_bias = bias != nullptr;
    const uint16_t *bsrc = has_bias ? bias : reinterpret_cast<const uint16_t *>(a_sinv);
    uint32_t braw[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int u = 0; u < 4; ++u) braw[j][u] = bsrc[has_bias ? min(n0 + j * 16 + g * 4 + u, N - 1) : 0];
    const int nk = K / kQK;
#define FP8DS_SLOAD(FA_, FB_, kt)                                                                          \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                                       \
        FA_[i] = ld32(pa[i] + (int64_t)(kt) * kQK);                                                       \
        FB_[i] = ld32(pb[i] + (int64_t)(kt) * kQK);                                                       \
    }
#define FP8DS_SMFMA(FA_, FB_)                                                                              \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                         \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                         \
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(FB_[j], FA_[i], acc[i][j], FB, FA, 0, 0, 0, 0);
    // unconditional loads, step index clamped (see k_gemm_small)
    i32x8 a0[4], b0[4], a1[4], b1[4], a2[4], b2[4];
    FP8DS_SLOAD(a0, b0, 0)
    FP8DS_SLOAD(a1, b1, min(1, nk - 1))
    FP8DS_SLOAD(a2, b2, min(2, nk - 1))
    int kt = 0;
    for (; kt + 3 <= nk; kt += 3) {
        FP8DS_SMFMA(a0, b0)
        FP8DS_SLOAD(a0, b0, min(kt + 3, nk - 1))
        FP8DS_SMFMA(a1, b1)
        FP8DS_SLOAD(a1, b1, min(kt + 4, nk - 1))
        FP8DS_SMFMA(a2, b2)
        FP8DS_SLOAD(a2, b2, min(kt + 5, nk - 1))
    }
    // the last nk % 3 steps, already in a0, a1 in K order
    if (kt < nk) { FP8DS_SMFMA(a0, b0) }
    if (kt + 1 < nk) { FP8DS_SMFMA(a1, b1) }
#undef FP8DS_SLOAD
#undef FP8DS_SMFMA
    // epilogue: lane l holds D[m0 + 16 i + l % 16][n0 + 16 j + 4 (l / 16) + u] in element u of
    // acc[i][j]; the four columns go out in one store when they are inside D and the store is
    // aligned (4 x the element size), else element by element
    constexpr int kEsz = OUT == 0 ? 2 : OUT == 1 ? 4 : 1;
    const bool vec4 = ((reinterpret_cast<uintptr_t>(D) & (uintptr_t)(4 * kEsz - 1)) == 0) && (ldd % 4 == 0);
    uint32_t amag = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = m0 + i * 16 + r16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + j * 16 + g * 4;
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float b = has_bias ? __uint_as_float(braw[j][u] << 16) : 0.f;
                v[u] = dequant_bias(acc[i][j][u], sa, sb, b);
            }
            if (row >= M) continue;
            const int64_t o = (int64_t)row * ldd + col;
            if constexpr (OUT >= 2) {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (col + u < N) amag = max(amag, __float_as_uint(v[u]) & 0x7FFFFFFFu);
            }
            if (vec4 && col + 3 < N) {
                if constexpr (OUT == 0) {
                    *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(D) + o) =
                        u32x2{f32x2_to_bf16x2_rne(v[0], v[1]), f32x2_to_bf16x2_rne(v[2], v[3])};
                } else if constexpr (OUT == 1) {
                    *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(D) + o) = f32x4{v[0], v[1], v[2], v[3]};
                } else {
                    *reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(D) + o) =
                        encode_exact<OUT - 2>(v[0] * ds) | (encode_exact<OUT - 2>(v[1] * ds) << 8) |
                        (encode_exact<OUT - 2>(v[2] * ds) << 16) | (encode_exact<OUT - 2>(v[3] * ds) << 24);
                }
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (col + u >= N) continue;
                    if constexpr (OUT == 0) {
                        reinterpret_cast<uint16_t *>(D)[o + u] = f32_to_bf16_rne(v[u]);
                    } else if constexpr (OUT == 1) {
                        reinterpret_cast<float *>(D)[o + u] = v[u];
                    } else {
                        reinterpret_cast<uint8_t *>(D)[o + u] = (uint8_t)encode_exact<OUT - 2>(v[u] * ds);
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

// ------------------------------------------------------------------------------------------
// k_linear_fwd_small<TILE, K>: the forward of a small FP8 linear layer in one launch.  At the
// size of a [128, 256] x [256, 256] layer both kernels of the two-launch form are pure latency (a
// cast launch of two tiles, then eight waves of GEMM), so here each TILE x TILE output tile's
// block (TILE 32 or 64, 8 TILE threads) casts the bfloat16 rows it multiplies itself.  K is 256,
// 512 or 1024, so a block casts every row it needs in one pass: the first 4 TILE threads the
// tile's x rows, the others its W rows, each thread K / 4 consecutive K values (four threads per
// row); the codes go to two TILE x K-byte LDS tiles (16-byte chunk c of row r at chunk
// c ^ (r % 16)).  After one barrier each wave multiplies TILE / 32 of the 16 x 16 output tiles
// (one x slice, TILE / 32 adjacent W slices) with the K / 128 steps of k_gemm_small16 in its
// order, on the same fragments, so y is identical.  The casts' outputs are written by the blocks that own them: tile column 0
// writes x8 and folds x's amax; tile row 0 writes w8, folds W's amax and writes w8_t from the W
// tile with 4 x 4 byte register transposes.  A cached weight (*w_noop == 1) is read as codes
// from w8 and nothing of W is written.  Every code equals the cast kernels' (same clamp +
// hardware conversion, the exact encoder for a group holding an inf / NaN or under a zero /
// non-finite scale), and 1/scale is formed as the cast kernels form it.  Every load that depends
// on nothing else (bias, bfloat16 rows, the four scalars) is issued first and without branches;
// each wave folds its amax with one atomic (no read first: a few hundred blocks at most).
// ------------------------------------------------------------------------------------------
struct SmallFwdArgs {
    const uint16_t *x, *w, *bias;
    const float *x_scale, *w_scale, *w_noop;
    float *x_amax, *w_amax, *x_scale_inv, *w_scale_inv;
    uint8_t *x8, *w8, *w8_t;
    uint16_t *y;
    int M, N, K, tiles_n;
};

// 32 bfloat16 values (16 dwords, element 2q in the low half of dword q) -> 32 E4M3 codes
// (8 dwords, element 4d in byte 0 of dword d); *tam receives the packed magnitudes' max.
__device__ __forceinline__ i32x8 cast32_e4m3(const uint32_t (&v)[16], float s, bool plain, uint32_t *tam) {
    uint32_t m = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) m = amax_pk(m, v[q]);
    *tam = m;
    i32x8 r;
    if (plain && amax_unpack(m) < 0x7F80u) {
#pragma unroll
        for (int d = 0; d < 8; ++d)
            r[d] = (int)pack4<kE4M3>(clamp_fmt<kE4M3>(bf16_lo(v[2 * d]) * s), clamp_fmt<kE4M3>(bf16_hi(v[2 * d]) * s),
                                     clamp_fmt<kE4M3>(bf16_lo(v[2 * d + 1]) * s),
                                     clamp_fmt<kE4M3>(bf16_hi(v[2 * d + 1]) * s));
    } else {
#pragma unroll
        for (int d = 0; d < 8; ++d)
            r[d] = (int)(encode_exact<kE4M3>(bf16_lo(v[2 * d]) * s) | (encode_exact<kE4M3>(bf16_hi(v[2 * d]) * s) << 8) |
                         (encode_exact<kE4M3>(bf16_lo(v[2 * d + 1]) * s) << 16) |
                         (encode_exact<kE4M3>(bf16_hi(v[2 * d + 1]) * s) << 24));
    }
    return r;
}

__device__ __forceinline__ void load32_bf16(const uint16_t *p, uint32_t (&v)[16]) {
    const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const u32x4 t = q[c];
        v[4 * c] = t.x; v[4 * c + 1] = t.y; v[4 * c + 2] = t.z; v[4 * c + 3] = t.w;
    }
}

__device__ __forceinline__ void store32_codes(uint8_t *p, const i32x8 &c) {
    reinterpret_cast<u32x4 *>(p)[0] = u32x4{(uint32_t)c[0], (uint32_t)c[1], (uint32_t)c[2], (uint32_t)c[3]};
    reinterpret_cast<u32x4 *>(p)[1] = u32x4{(uint32_t)c[4], (uint32_t)c[5], (uint32_t)c[6], (uint32_t)c[7]};
}

template <int TILE, int KK>
__global__ __launch_bounds__(8 * TILE) void k_linear_fwd_small(const SmallFwdArgs a) {
    constexpr int kRowsT = 4 * TILE;                  // threads casting one operand (four per row)
    constexpr int kT16 = TILE / 16;                   // 16 x 16 output tiles per tile edge
    constexpr int kPerWave = TILE / 32;               // 16 x 16 output tiles per wave
    constexpr int kVpt = KK / 4;                      // K values (code bytes) per casting thread
    constexpr int kG = kVpt / 32;                     // groups of 32 values per thread
    __shared__ __align__(16) uint8_t sx[TILE * KK];
    __shared__ __align__(16) uint8_t sw[TILE * KK];
    const int tm = blockIdx.y, tn = blockIdx.x;   // a 2-D grid: no division by the tile count
    const int m0 = tm * TILE, n0 = tn * TILE;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int M = a.M, N = a.N;
    // thread t casts operand t / (4 TILE) (x, W), row (t / 4) % TILE, K values kVpt (t % 4) ..
    const bool is_w = t >= kRowsT;                              // wave-uniform
    const int row = (t >> 2) & (TILE - 1), q = t & 3;
    const int grow = (is_w ? n0 : m0) + row, lim = is_w ? N : M;
    const int64_t srow = min(grow, lim - 1);                    // rows past M / N repeat the last
    // every load that depends on nothing else goes out first: the bias of this lane's output
    // columns and the bfloat16 rows (W's also when the weight turns out to be cached: unused then)
    // (unconditional loads, so they issue together: without a bias they read x_scale's first bytes)
    const int r16 = lane & 15, g = lane >> 4;
    const int t0 = wave * kPerWave;                             // this wave's first output tile
    const int tm16 = t0 / kT16, tn16 = t0 % kT16;               // its tiles: (tm16, tn16 + j)
    const int xrow = m0 + tm16 * 16 + r16;
    const bool has_bias = a.bias != nullptr;
    const uint16_t *bsrc = has_bias ? a.bias : reinterpret_cast<const uint16_t *>(a.x_scale);
    uint16_t braw[kPerWave][4];
#pragma unroll
    for (int j = 0; j < kPerWave; ++j)
#pragma unroll
        for (int u = 0; u < 4; ++u)
            braw[j][u] = bsrc[has_bias ? min(n0 + (tn16 + j) * 16 + g * 4 + u, N - 1) : 0];
    uint32_t v[kG][16];
    {
        const uint16_t *src = (is_w ? a.w : a.x) + srow * KK + q * kVpt;
#pragma unroll
        for (int c = 0; c < kG; ++c) load32_bf16(src + 32 * c, v[c]);
    }
    // the four scalars in one round (the flag read from x_scale when there is none; w_scale_inv
    // is used only for a cached weight, which no block rewrites)
    const float flag = *(a.w_noop != nullptr ? a.w_noop : a.x_scale);
    const float xs = *a.x_scale, ws = *a.w_scale, wsi = *a.w_scale_inv;
    const bool wcached = a.w_noop != nullptr && flag == 1.0f;
    const float sa = 1.0f / xs;
    const float sb = wcached ? wsi : 1.0f / ws;
    if (blockIdx.x == 0 && blockIdx.y == 0 && t == 0) {
        *a.x_scale_inv = sa;
        if (!wcached) *a.w_scale_inv = sb;
    }
    const bool own_x = tn == 0, own_w = tm == 0 && !wcached;   // block-uniform
    uint8_t *lds = is_w ? sw : sx;
    i32x8 cd[kG];
    uint32_t mag = 0;
    if (is_w && wcached) {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(a.w8 + srow * KK + q * kVpt);
#pragma unroll
        for (int c = 0; c < kG; ++c) {
            const u32x4 p0 = p[2 * c], p1 = p[2 * c + 1];
            cd[c] = i32x8{(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w, (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w};
        }
    } else {
        const float s = is_w ? ws : xs;
        const bool plain = scale_is_plain(s);
        uint32_t mp = 0;
#pragma unroll
        for (int c = 0; c < kG; ++c) {
            uint32_t mc;
            cd[c] = cast32_e4m3(v[c], s, plain, &mc);
            mp = amax_pk(mp, mc);
        }
        mag = amax_unpack(mp);
    }
    {
        // 16-byte chunk h of this thread's codes is chunk (kVpt / 16) q + h of the row
        const int sw4 = row & 15;
        u32x4 *l = reinterpret_cast<u32x4 *>(lds + row * KK);
#pragma unroll
        for (int c = 0; c < kG; ++c) {
            const int h = (kVpt / 16) * q + 2 * c;
            l[h ^ sw4] = u32x4{(uint32_t)cd[c][0], (uint32_t)cd[c][1], (uint32_t)cd[c][2], (uint32_t)cd[c][3]};
            l[(h + 1) ^ sw4] = u32x4{(uint32_t)cd[c][4], (uint32_t)cd[c][5], (uint32_t)cd[c][6], (uint32_t)cd[c][7]};
        }
    }
    const bool own = is_w ? own_w : own_x;
    if (own && grow < lim) {
        uint8_t *dst = (is_w ? a.w8 : a.x8) + (int64_t)grow * KK + q * kVpt;
#pragma unroll
        for (int c = 0; c < kG; ++c) store32_codes(dst + 32 * c, cd[c]);
    }
    float *amax_slot = is_w ? a.w_amax : a.x_amax;
    if (own && amax_slot != nullptr) {
        const uint32_t m = wave_max_u32(mag);
        if (lane == 0 && m != 0u) atomicMax(reinterpret_cast<unsigned int *>(amax_slot), m << 16);
    }
    __syncthreads();
    // ---- w8_t rows k, columns n0 .. n0 + TILE - 1 from the W tile: 4 x 8 byte blocks, block b
    // = t + 8 TILE i covering k = 4 (b / (TILE / 8)) .., n = 8 (b % (TILE / 8)) ..
    if (own_w) {
#pragma unroll
        for (int i = 0; i < KK / 256; ++i) {
            const int b = t + 8 * TILE * i;
            const int n8 = (b % (TILE / 8)) * 8, k4 = (b / (TILE / 8)) * 4;
            uint32_t d[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int n = n8 + e;
                d[e] = *reinterpret_cast<const uint32_t *>(sw + n * KK + (((k4 >> 4) ^ (n & 15)) << 4) + (k4 & 15));
            }
            uint32_t o[4], p[4];
            tr4(d[0], d[1], d[2], d[3], o[0], o[1], o[2], o[3]);
            tr4(d[4], d[5], d[6], d[7], p[0], p[1], p[2], p[3]);
            if (n0 + n8 < N) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<u32x2 *>(a.w8_t + (int64_t)(k4 + j) * N + n0 + n8) = u32x2{o[j], p[j]};
            }
        }
    }
    // ---- the K steps of 128 bytes: lane l supplies row l % 16 of the 16-row x and W slices and
    // K bytes [32 (l / 16), +32) of each step
    f32x4 acc[kPerWave];
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < KK / kQK; ++st) {
        const int ch = 8 * st + 2 * g;
        const int ra = tm16 * 16 + r16;
        const u32x4 a0 = *reinterpret_cast<const u32x4 *>(sx + ra * KK + ((ch ^ r16) << 4));
        const u32x4 a1 = *reinterpret_cast<const u32x4 *>(sx + ra * KK + (((ch + 1) ^ r16) << 4));
        const i32x8 fa = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
#pragma unroll
        for (int j = 0; j < kPerWave; ++j) {
            const int rb = (tn16 + j) * 16 + r16;
            const u32x4 b0 = *reinterpret_cast<const u32x4 *>(sw + rb * KK + ((ch ^ r16) << 4));
            const u32x4 b1 = *reinterpret_cast<const u32x4 *>(sw + rb * KK + (((ch + 1) ^ r16) << 4));
            const i32x8 fb = i32x8{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
            acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb, fa, acc[j], kE4M3, kE4M3, 0, 0, 0, 0);
        }
    }
    // ---- y: lane l holds y[xrow][col + u] of tile j in element u (N % 16 == 0: the four
    // columns are all inside or all outside)
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
        const int col = n0 + (tn16 + j) * 16 + g * 4;
        if (xrow < M && col < N) {
            float val[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                val[u] = dequant_bias(acc[j][u], sa, sb, has_bias ? __uint_as_float((uint32_t)braw[j][u] << 16) : 0.f);
            uint16_t *dst = a.y + (int64_t)xrow * N + col;
            if ((reinterpret_cast<uintptr_t>(a.y) & 7u) == 0) {
                *reinterpret_cast<u32x2 *>(dst) =
                    u32x2{f32x2_to_bf16x2_rne(val[0], val[1]), f32x2_to_bf16x2_rne(val[2], val[3])};
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) dst[u] = f32_to_bf16_rne(val[u]);
            }
        }
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
    // the 16 x 16 x 128 family (k_gemm_pipe16 / k_gemm_small16, identical bits) for K % 256 == 0;
    // the choice depends on K and the strides only, so every N-chunk of a GEMM takes the same one
    const bool fam16 = (K % kFam16K) == 0 && pipe;
    const bool small16 = fam16 && small16_preferred((int64_t)tiles_m * tiles_n, K);
    const int stiles_n = (int)((N + kSmallTile - 1) / kSmallTile);
    // bands of 8 tile-rows when the operands exceed the 256 MB Infinity Cache (block_tile)
    constexpr int64_t kInfinityCache = INT64_C(256) << 20;
    const int band_rows = (M * lda + N * ldb > kInfinityCache) ? 8 : tiles_m;
    dim3 sgrid((unsigned)(((M + kSmallTile - 1) / kSmallTile) * stiles_n));
#define FP8DS_GEMM(FA_, FB_, O_)                                                                           \
    do {                                                                                                   \
        if (fam16 && small16)                                                                              \
            k_gemm_small16<FA_, FB_, O_><<<sgrid, dim3(64), 0, st>>>(                                      \
                A, lda, B, ldb, a_sinv, b_sinv, bias, D, ldd, (int)M, (int)N, (int)K, stiles_n, oq);       \
        else if (fam16)                                                                                    \
            k_gemm_pipe16<FA_, FB_, O_><<<grid, dim3(kThreads), 0, st>>>(                                  \
                A, lda, B, ldb, a_sinv, b_sinv, bias, D, ldd, (int)M, (int)N, (int)K, tiles_m, tiles_n, band_rows, oq); \
        else if (small)                                                                                    \
            k_gemm_small<FA_, FB_, O_><<<sgrid, dim3(64), 0, st>>>(                                        \
                A, lda, B, ldb, a_sinv, b_sinv, bias, D, ldd, (int)M, (int)N, (int)K, stiles_n, oq);       \
        else if (pipe)                                                                                     \
            k_gemm_bias_pipe<FA_, FB_, O_><<<grid, dim3(kThreads), 0, st>>>(                               \
                A, lda, B, ldb, a_sinv, b_sinv, bias, D, ldd, (int)M, (int)N, (int)K, tiles_m, tiles_n, band_rows, oq); \
        else                                                                                               \
            k_gemm_bias<FA_, FB_, O_><<<grid, dim3(kThreads), 0, st>>>(                                    \
                A, lda, B, ldb, a_sinv, b_sinv, bias, D, ldd, (int)M, (int)N, (int)K, tiles_m, tiles_n, band_rows, oq); \
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

// The one-launch small forward takes K = 256, 512 or 1024 (a block casts a row's K values in one
// pass), no x transpose, N % 16 == 0 (whole 8-byte groups of w8_t rows), at most 256 x 256 / K
// blocks of 64 x 64 and fewer than 40 tiles of 256 x 256 (the GEMM of the two-launch form is
// then k_gemm_small16, whose bits it reproduces).  Measured through the C ABI, back to back,
// against the cast-pair launch + GEMM launch: [1024, 1024, 256] 6.2 against 8.5 us, beyond 256
// blocks close ([768, 1536, 256] 9.1 against 9.4 us), then the two launches win ([1024, 2048,
// 256] 10.1 against 9.7 us); K = 512: [128, 256, 512] 6.2 against 9.7 us, [512, 1024, 512]
// (128 blocks) 8.6 against 9.9 us, [1024, 1024, 512] 10.7 against 10.5 us; K = 1024: [512, 512,
// 1024] (64 blocks) 10.5 against 11.8 us, [1024, 1024, 1024] 19.5 against 13.2 us.  Up to 128
// blocks of 64 x 64 the 32 x 32 tiles are faster ([128, 256, 256] 4.2 against 5.7 us,
// [512, 1024, 256] 5.3 against 6.0 us), beyond it the 64 x 64 tiles ([768, 768, 256] 6.0 against
// 6.4 us, [1024, 1024, 256] 6.2 against 8.3 us).
constexpr int64_t kSmallFwdMaxBlocks = 256;
constexpr int64_t kTinyMaxBlocks64 = 128;
constexpr int64_t kSmallFwdMaxTiles = 39;
bool linear_fwd_small_ok(int64_t M, int64_t N, int64_t K, const uint8_t *x8_t) {
    if (x8_t != nullptr || M <= 0 || N <= 0 || N % 16 != 0) return false;
    if (K != 256 && K != 512 && K != 1024) return false;
    const int64_t blocks64 = ((M + kSmallTile - 1) / kSmallTile) * ((N + kSmallTile - 1) / kSmallTile);
    if (blocks64 * K > kSmallFwdMaxBlocks * 256) return false;   // 256, 128, 64 blocks for K = 256, 512, 1024
    return ((M + BM - 1) / BM) * ((N + BN - 1) / BN) <= kSmallFwdMaxTiles;
}

hipError_t launch_linear_fwd_small(const uint16_t *x, const uint16_t *w, const uint16_t *bias, int64_t M, int64_t N,
                                   int64_t K, const float *x_scale, float *x_amax, uint8_t *x8, float *x_scale_inv,
                                   const float *w_scale, float *w_amax, uint8_t *w8, uint8_t *w8_t,
                                   float *w_scale_inv, const float *w_noop, uint16_t *y, hipStream_t st) {
    SmallFwdArgs a{};
    a.x = x; a.w = w; a.bias = bias;
    a.x_scale = x_scale; a.w_scale = w_scale; a.w_noop = w_noop;
    a.x_amax = x_amax; a.w_amax = w_amax; a.x_scale_inv = x_scale_inv; a.w_scale_inv = w_scale_inv;
    a.x8 = x8; a.w8 = w8; a.w8_t = w8_t; a.y = y;
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    const int64_t blocks64 = ((M + kSmallTile - 1) / kSmallTile) * ((N + kSmallTile - 1) / kSmallTile);
#define FP8DS_SMALL_FWD(TILE_, KK_)                                                                        \
    do {                                                                                                   \
        a.tiles_n = (int)((N + TILE_ - 1) / TILE_);                                                        \
        const dim3 grid((unsigned)a.tiles_n, (unsigned)((M + TILE_ - 1) / TILE_));                         \
        k_linear_fwd_small<TILE_, KK_><<<grid, dim3(8 * TILE_), 0, st>>>(a);                               \
    } while (0)
    // (K = 512 and 1024 stay within 128 blocks of 64 x 64 by the rule, so they take 32 x 32 tiles)
    if (K == 256 && blocks64 > kTinyMaxBlocks64) FP8DS_SMALL_FWD(64, 256);
    else if (K == 256) FP8DS_SMALL_FWD(32, 256);
    else if (K == 512) FP8DS_SMALL_FWD(32, 512);
    else FP8DS_SMALL_FWD(32, 1024);
#undef FP8DS_SMALL_FWD
    return hipGetLastError();
}

}  // namespace fp8ds
