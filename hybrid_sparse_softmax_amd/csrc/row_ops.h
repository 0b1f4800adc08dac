// Row-at-a-time helpers of the general fp32 kernels (backward pass,
// future-KV-utility diagnostic): 16-byte row loads, dots of one row with
// several LDS vectors, and an XCD-aware order of 1-D launches.
#pragma once
#include "device_common.h"

namespace still {

// 8 consecutive elements of a row as fp32 (16-byte loads; rows are 16-byte
// aligned: every row starts at a multiple of d elements of an aligned tensor)
__device__ __forceinline__ void load8(const __bf16* p, float* x) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float* p, float* x) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// a . r for an LDS vector a (read by the whole wave) and a row r
template <int DD, typename T1>
__device__ __forceinline__ float dot_row(const float* a, const T1* r) {
    float x0 = 0.f, x1 = 0.f;
#pragma unroll 4
    for (int i = 0; i < DD; i += 8) {
        float xr[8];
        load8(r + i, xr);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            x0 = fmaf(a[i + e], xr[e], x0);
            x1 = fmaf(a[i + e + 1], xr[e + 1], x1);
        }
    }
    return x0 + x1;
}

// dots of one row r (DD elements) with G LDS vectors a[h], h < G <= GM
template <int DD, int GM, typename T1>
__device__ __forceinline__ void dot_multi(const float (*a)[DD], const T1* r, int G, float* out) {
#pragma unroll
    for (int h = 0; h < GM; ++h) out[h] = 0.f;
#pragma unroll 2
    for (int i = 0; i < DD; i += 8) {
        float xr[8];
        load8(r + i, xr);
#pragma unroll
        for (int h = 0; h < GM; ++h)
            if (h < G) {
#pragma unroll
                for (int e = 0; e < 8; ++e) out[h] = fmaf(a[h][i + e], xr[e], out[h]);
            }
    }
}

// 8 consecutive elements at an address that is the same in every lane,
// read as constant memory (through the scalar cache; such rows are not
// written while the kernel runs)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) u32x4* const_u4_ptr;
__device__ __forceinline__ void load8_u(const __bf16* p, float* x) {
    const u32x4 u = *reinterpret_cast<const_u4_ptr>(reinterpret_cast<uintptr_t>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(u[i] << 16);
        x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8_u(const float* p, float* x) {
    const const_u4_ptr q = reinterpret_cast<const_u4_ptr>(reinterpret_cast<uintptr_t>(p));
    const u32x4 a = q[0], b = q[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = __uint_as_float(a[i]);
        x[4 + i] = __uint_as_float(b[i]);
    }
}

// dots of one row r (DD elements) with the rows a[i], i < R, whose
// addresses are the same in every lane (rows with use[i] false are skipped)
template <int DD, int R, typename TA, typename T1>
__device__ __forceinline__ void dot_rows_u(const TA* const* a, const bool* use, const T1* r, float* out) {
#pragma unroll
    for (int h = 0; h < R; ++h) out[h] = 0.f;
#pragma unroll 2
    for (int i = 0; i < DD; i += 8) {
        float xr[8];
        load8(r + i, xr);
#pragma unroll
        for (int h = 0; h < R; ++h)
            if (use[h]) {
                float xa[8];
                load8_u(a[h] + i, xa);
#pragma unroll
                for (int e = 0; e < 8; ++e) out[h] = fmaf(xa[e], xr[e], out[h]);
            }
    }
}

// Work item of a 1-D launch of nx * ny * nz blocks, laid out so that the
// blocks of one (y, z) pair -- one (sequence, KV head), whose waves read the
// same query and key rows -- run on one XCD and share its L2: the hardware
// hands block L to XCD L mod 8, so block L takes item (L mod 8) * per + L / 8.
struct Item {
    int x, y, z;
};
__device__ __forceinline__ Item xcd_item(int nx, int ny) {
    const int L = blockIdx.x, total = gridDim.x, per = total / 8;
    const int w = L < per * 8 ? (L % 8) * per + L / 8 : L;
    return Item{w % nx, (w / nx) % ny, w / (nx * ny)};
}

}  // namespace still
