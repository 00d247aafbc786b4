// device_common.h -- device helpers shared by the HIP kernels of the FP8 delayed-scaling path
// (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8ds {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));   // two 16-bit values in one register
typedef int i32x8 __attribute__((ext_vector_type(8)));        // one lane's 32 FP8 MFMA operand bytes
typedef float f32x16 __attribute__((ext_vector_type(16)));    // one lane's 32 x 32 MFMA accumulators
typedef float f32x4 __attribute__((ext_vector_type(4)));      // one lane's 16 x 16 MFMA accumulators

constexpr int kE4M3 = 0;
constexpr int kE5M2 = 1;

// Largest finite magnitude of each OCP format: E4M3 S.1111.110 = 1.75 * 2^8, E5M2
// S.11110.11 = 1.75 * 2^15.
template <int FMT> struct FmtTraits;
template <> struct FmtTraits<kE4M3> { static constexpr float kMax = 448.0f; };
template <> struct FmtTraits<kE5M2> { static constexpr float kMax = 57344.0f; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Saturating clamp of a finite or infinite value into the format's range.  v_med3_f32 returns
// the middle of the three operands, which is the clamp for every non-NaN input.
template <int FMT>
__device__ __forceinline__ float clamp_fmt(float y) {
    return __builtin_amdgcn_fmed3f(y, -FmtTraits<FMT>::kMax, FmtTraits<FMT>::kMax);
}

// Hardware conversion of two float32 values (already inside the format's range) into two FP8
// codes: v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 round to nearest even and produce the OCP
// subnormals; `old` keeps the other 16-bit half.  byte 0 of the half takes `a`, byte 1 takes `b`.
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t cvt_pk(float a, float b, uint32_t old) {
    if constexpr (FMT == kE4M3)
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
    else
        return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, HI);
}

// Four clamped values -> one dword of four codes (bytes in argument order).
template <int FMT>
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
    uint32_t w = cvt_pk<FMT, false>(a, b, 0u);
    return cvt_pk<FMT, true>(c, d, w);
}

// Exact single-element encoder for the rare inputs the fast path does not cover (a NaN
// scaled value): every NaN gives the one code 0x7F (the sign of a NaN made by an invalid
// operation is not meaningful); anything else is clamped and converted like the fast path.
template <int FMT>
__device__ __forceinline__ uint32_t encode_exact(float y) {
    if (y != y) return 0x7Fu;
    return cvt_pk<FMT, false>(clamp_fmt<FMT>(y), 0.0f, 0u) & 0xFFu;
}

// A scaled value x * s can be NaN only when x is NaN, or when s is NaN, infinite or zero
// (inf * 0).  With a finite non-zero scale and inputs whose |bf16| bit patterns stay below
// 0x7F80 (no inf / NaN) the fast clamp-and-convert path is exact.
__device__ __forceinline__ bool scale_is_plain(float s) {
    return (__float_as_uint(s) & 0x7FFFFFFFu) - 1u < 0x7F7FFFFFu;  // 0 < |s| < inf
}

// Packed 16-bit max of the magnitudes of two bfloat16 values in a dword.
__device__ __forceinline__ uint32_t amax_pk(uint32_t acc, uint32_t w) {
    w &= 0x7FFF7FFFu;
    uint32_t lo = max(acc & 0xFFFFu, w & 0xFFFFu);
    uint32_t hi = max(acc >> 16, w >> 16);
    return lo | (hi << 16);
}
__device__ __forceinline__ uint32_t amax_unpack(uint32_t acc) { return max(acc & 0xFFFFu, acc >> 16); }

// Wave-wide max (64 lanes) of an unsigned value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    return v;
}

// Block-wide max of an unsigned value; result valid in thread 0.  `red` needs one slot per wave.
template <int NT>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t *red) {
    v = wave_max_u32(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    uint32_t r = 0;
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 0; i < NT / 64; ++i) r = max(r, red[i]);
    }
    return r;
}

// Fold a bfloat16 magnitude bit pattern (0..0xFFFF without sign) into a float32 amax slot.
// The slot holds a non-negative float or NaN; for those, unsigned order of the bit patterns is
// the numeric order (with NaN above +inf), so an integer atomic max is exact and order free.
// The slot only grows while casts run, so a plain read that already shows a value at least as
// large proves the atomic would change nothing: skipping it keeps thousands of blocks from
// serialising on one address.
__device__ __forceinline__ void fold_amax_bits(float *slot, uint32_t f32_mag) {
    if (slot == nullptr || f32_mag == 0u) return;
    unsigned int *u = reinterpret_cast<unsigned int *>(slot);
    if (__hip_atomic_load(u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= f32_mag) return;
    atomicMax(u, f32_mag);
}
__device__ __forceinline__ void fold_amax(float *slot, uint32_t bf16_mag) { fold_amax_bits(slot, bf16_mag << 16); }

// Four float32 values already multiplied by the scale -> one dword of four codes.  The clamp +
// hardware conversion is exact for everything but NaN, which takes the exact encoder.
template <int FMT>
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d) {
    if (a == a && b == b && c == c && d == d)
        return pack4<FMT>(clamp_fmt<FMT>(a), clamp_fmt<FMT>(b), clamp_fmt<FMT>(c), clamp_fmt<FMT>(d));
    return encode_exact<FMT>(a) | (encode_exact<FMT>(b) << 8) | (encode_exact<FMT>(c) << 16) |
           (encode_exact<FMT>(d) << 24);
}

// float32 -> bfloat16, round to nearest even, by the hardware conversion (gfx950 converts two
// values per instruction).  A NaN stays a NaN; its payload is not specified.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float lo, float hi) {
    const bf16x2_t p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

// GEMM epilogue arithmetic, acc * a_scale_inv * b_scale_inv + bias: one product, then one fused
// multiply-add.  Every GEMM kernel and output dtype uses exactly this sequence, so they all see
// the same float32 value.
__device__ __forceinline__ float dequant_bias(float acc, float sa, float sb, float b) {
    return __builtin_fmaf(acc * sa, sb, b);
}

// 4 x 4 byte transpose: byte k of a, b, c, d is element (row 0..3, column k); o_k receives
// column k in row order (byte 0 from a).  Two rounds of two-source byte selects.
__device__ __forceinline__ void tr4(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t &o0, uint32_t &o1,
                                    uint32_t &o2, uint32_t &o3) {
    const uint32_t ab_lo = __builtin_amdgcn_perm(b, a, 0x05010400u);   // a0 b0 a1 b1
    const uint32_t ab_hi = __builtin_amdgcn_perm(b, a, 0x07030602u);   // a2 b2 a3 b3
    const uint32_t cd_lo = __builtin_amdgcn_perm(d, c, 0x05010400u);
    const uint32_t cd_hi = __builtin_amdgcn_perm(d, c, 0x07030602u);
    o0 = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u);             // a0 b0 c0 d0
    o1 = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u);             // a1 b1 c1 d1
    o2 = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u);
    o3 = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u);
}

}  // namespace fp8ds
