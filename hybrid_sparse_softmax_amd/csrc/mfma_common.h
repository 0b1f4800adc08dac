// gfx950 matrix-core helpers for the STILL kernels (wave64, bf16 MFMA).
//
// v_mfma_f32_32x32x16_bf16 lane layouts (checked on the device):
//   A (32 x 16):  lane l holds A[l % 32][8 * (l / 32) + j],   j = 0..7
//   B (16 x 32):  lane l holds B[8 * (l / 32) + j][l % 32],   j = 0..7
//   D (32 x 32):  lane l, element v holds D[acc_row(v, l / 32)][l % 32]
//
// An accumulator can feed the next product directly when its rows become
// that product's contraction index: element v = 8 * s2 + j of a lane is then
// operand element j of k-step s2, which stands for row
//   16 * s2 + 8 * (j / 4) + 4 * (l / 32) + j % 4.
// The other operand of such a product must supply the same rows, so tensors
// that meet an accumulator this way are stored with bits 2 and 3 of their
// contraction index swapped (kperm): the eight rows a lane needs are then
// contiguous.
#pragma once
#include "device_common.h"

namespace still {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// row of accumulator element v in a lane of half hf (0: lanes 0-31, 1: 32-63)
__host__ __device__ constexpr int acc_row(int v, int hf) { return 8 * (v >> 2) + 4 * hf + (v & 3); }

// storage position of contraction index k (bits 2 and 3 swapped; an involution)
__host__ __device__ constexpr int kperm(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

__device__ __forceinline__ bf16x8 zero_bf8() {
    bf16x8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.f;
    return z;
}

__device__ __forceinline__ bf16x8 ld_bf8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void st_bf8(__bf16* p, bf16x8 x) { *reinterpret_cast<bf16x8*>(p) = x; }

// 8 fp32 (two 16-byte loads) split into bf16 high and low parts: x = hi + lo
// up to the rounding of lo (relative 2^-16).
__device__ __forceinline__ void ld_split8(const float* p, bf16x8& hi, bf16x8& lo) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const __bf16 ha = (__bf16)a[j], hb = (__bf16)b[j];
        hi[j] = ha;
        hi[4 + j] = hb;
        lo[j] = (__bf16)(a[j] - (float)ha);
        lo[4 + j] = (__bf16)(b[j] - (float)hb);
    }
}

// the same for the sum of two fp32 arrays (a + b, then split)
__device__ __forceinline__ void ld_split8_sum(const float* a, const float* b, bf16x8& hi, bf16x8& lo) {
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(a), a1 = *reinterpret_cast<const f32x4*>(a + 4);
    const f32x4 b0 = *reinterpret_cast<const f32x4*>(b), b1 = *reinterpret_cast<const f32x4*>(b + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float x0 = a0[j] + b0[j], x1 = a1[j] + b1[j];
        const __bf16 h0 = (__bf16)x0, h1 = (__bf16)x1;
        hi[j] = h0;
        hi[4 + j] = h1;
        lo[j] = (__bf16)(x0 - (float)h0);
        lo[4 + j] = (__bf16)(x1 - (float)h1);
    }
}

// elements 8*s2 .. 8*s2+7 of an accumulator as a bf16 operand
__device__ __forceinline__ bf16x8 pack_acc(const f32x16& x, int s2) {
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (__bf16)x[8 * s2 + j];
    return r;
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, kWave); }

// IEEE 754-2019 maximum / minimum (a NaN operand gives NaN).  On gfx950 these
// become v_maximum3_f32 / v_minimum3_f32 with no canonicalising of the
// operands, which fmaxf needs after matrix-core results.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmin(float a, float b) { return __builtin_elementwise_minimum(a, b); }

// max of x over lanes l and l ^ 32 (the two halves of a query's accumulator
// column).  A lane-half swap (v_permlane32_swap) would do it without the
// LDS crossbar, but the compiler folds the maximum of the swap's two
// results into its first result alone, which keeps only the lower half's
// value; the cross-lane read below has no such fold.
__device__ __forceinline__ float half_pair_max(float x) { return vmax(x, xor32(x)); }

}  // namespace still
