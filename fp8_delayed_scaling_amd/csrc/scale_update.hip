// scale_update.hip -- fused delayed-scaling update of T tensors in one launch: history max,
// guarded scale recompute and history roll.  The scale-update kernel, and a fix for amaxes small
// enough to drive the scale to infinity, are named in "[PyTorch] Refactor FP8 workspaces in
// linear modules" (Motivations, first bullet); amaxes are reduced within the current iteration
// ("[PyTorch] cuda graph support", feature list).
//
// One 256-thread block per tensor.  The history is [L][T] float32 (row 0 = current amaxes), so
// a tensor's column is strided by T; at the sizes this runs at (L up to a few thousand, T up to
// a few thousand) the kernel is latency bound, not bandwidth bound.  A window of up to
// kSuLdsRows rows is staged whole in LDS by direct loads (one memory round trip); the max and
// the roll then read LDS.  Longer windows take the max and the roll in 256-row chunks.
#include "device_common.h"
#include "launch.h"

namespace fp8ds {

struct FmtMask {
    uint32_t bits[kMaxScaleTensors / 32];  // bit t set: tensor t is E5M2, else E4M3
};

constexpr int kSuLdsRows = 8192;

__global__ __launch_bounds__(256) void k_scale_update(float *__restrict__ hist, int64_t L, int64_t T,
                                                      float *__restrict__ scale, float *__restrict__ scale_inv,
                                                      FmtMask fm, float pow2_neg_margin) {
    __shared__ float red[4];
    __shared__ int nanw[4];   // per wave: any NaN in the rows it read (written once, no init)
    __shared__ __align__(16) float col[kSuLdsRows];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool staged = L <= kSuLdsRows;   // uniform

    // pass 1: max over the window (all L rows), NaN tracked on its own
    float a = 0.f, row0, prev_scale;
    bool nan = false;
    if (staged) {
        // col[i] = hist[i][t] for every row: lane l of wave w loads row base + 64 w + l into that
        // LDS slot (rows past the end re-read row L - 1; their slots, < 256 rounded-up rows, are
        // never read).  No register depends on these loads, so all of them are in flight at once.
        for (int64_t base = 0; base < L; base += 256) {
            const int64_t i = min(base + tid, L - 1);
            __builtin_amdgcn_global_load_lds((const void *)(hist + i * T + t),
                                             (__attribute__((address_space(3))) void *)(col + base + wave * 64),
                                             4, 0, 0);
        }
        prev_scale = scale[t];                // issued behind the history loads, overlapping them
        __builtin_amdgcn_s_waitcnt(0xF70);   // vmcnt(0): this wave's rows have landed in LDS
        __syncthreads();
        for (int64_t i = tid; i < L; i += 256) {
            const float h = col[i];
            nan |= (h != h);
            a = fmaxf(a, h);
        }
        row0 = col[0];
    } else {
        prev_scale = scale[t];
        for (int64_t i = tid; i < L; i += 256) {
            const float h = hist[i * T + t];
            nan |= (h != h);
            a = fmaxf(a, h);
        }
        row0 = hist[t];   // old row 0, read before any write below
    }
    const bool wave_nan = __ballot(nan) != 0;   // every lane of the wave takes part
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    if ((tid & 63) == 0) {
        red[tid >> 6] = a;
        nanw[tid >> 6] = wave_nan ? 1 : 0;
    }
    __syncthreads();

    if (tid == 0) {
        float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        if (nanw[0] | nanw[1] | nanw[2] | nanw[3]) amax = __uint_as_float(0x7FC00000u);
        const bool e5 = (fm.bits[t >> 5] >> (t & 31)) & 1u;
        const float fmax = e5 ? FmtTraits<kE5M2>::kMax : FmtTraits<kE4M3>::kMax;
        float s = (fmax / amax) * pow2_neg_margin;
        // a zero scale, or one below 2^-128, has an inverse that overflows float32
        const float inf = __uint_as_float(0x7F800000u);
        const bool bad = !(amax > 0.f) || !(amax < inf) || !(fabsf(s) < inf) || !(fabsf(1.0f / s) < inf);
        if (bad) s = prev_scale;
        scale[t] = s;
        scale_inv[t] = 1.0f / s;
    }

    // pass 2: roll towards row 0 (new row i = old row i + 1 for i < L - 1)
    if (staged) {
        for (int64_t i = tid; i < L - 1; i += 256) hist[i * T + t] = col[i + 1];
    } else {
        // in chunks of 256 rows: read row i + 1, barrier, write row i
        for (int64_t base = 0; base < L - 1; base += 256) {
            const int64_t i = base + tid;
            float v = 0.f;
            if (i < L - 1) v = hist[(i + 1) * T + t];
            __syncthreads();
            if (i < L - 1) hist[i * T + t] = v;
            __syncthreads();
        }
    }
    if (tid == 0) {
        hist[(L - 1) * T + t] = row0;   // the amax just used becomes the newest past entry
        hist[t] = 0.f;                  // row 0 cleared for the next iteration
    }
}

hipError_t launch_scale_update(float *hist, int64_t L, int64_t T, float *scale, float *scale_inv,
                               const int32_t *fmts_host, int32_t margin, hipStream_t st) {
    FmtMask fm;
    for (int i = 0; i < kMaxScaleTensors / 32; ++i) fm.bits[i] = 0u;
    for (int64_t t = 0; t < T; ++t)
        if (fmts_host[t] == kE5M2) fm.bits[t >> 5] |= 1u << (t & 31);
    const float p = ldexpf(1.0f, -margin);   // exact power of two for |margin| <= 126
    k_scale_update<<<dim3((unsigned)T), dim3(256), 0, st>>>(hist, L, T, scale, scale_inv, fm, p);
    return hipGetLastError();
}

}  // namespace fp8ds
