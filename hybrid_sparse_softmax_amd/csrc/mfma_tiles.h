// Tile constants and plain LDS tile loaders shared by the gfx950 matrix-core
// kernels of the STILL operator (forward and backward).
#pragma once
#include "mfma_common.h"

namespace still {
namespace mt {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kC = 64;          // chunk (and key / query tile) rows
constexpr int kD = 128;         // head_dim = NP-Map feature dim
constexpr int kKS = kD + 8;     // LDS row stride (elements) of a row-major tile
constexpr int kVS = kC + 8;     // LDS row stride (elements) of a transposed tile
constexpr float kLog2e = 1.4426950408889634f;

// 64 rows of a row-major bf16 matrix (row stride ld) into LDS, row-major with
// stride kKS; rows >= nvalid are zero.
__device__ __forceinline__ void load_k_tile(const bf16* __restrict__ src, size_t ld, int nvalid,
                                            bf16* __restrict__ dst, int tid, int nthr) {
    for (int x = tid; x < kC * 16; x += nthr) {
        const int row = x >> 4, piece = x & 15;
        const bf16x8 val = row < nvalid ? ld_bf8(src + (size_t)row * ld + 8 * piece) : zero_bf8();
        st_bf8(dst + row * kKS + 8 * piece, val);
    }
}

// 64 rows x 128 columns of a row-major bf16 matrix into LDS transposed:
// dst[col * kVS + kperm(row)]; rows >= nvalid are zero.
__device__ __forceinline__ void load_vt_tile(const bf16* __restrict__ src, size_t ld, int nvalid,
                                             bf16* __restrict__ dst, int tid, int nthr) {
    for (int x = tid; x < 16 * 16; x += nthr) {
        // rows 4kq..4kq+3, columns 8oct..8oct+7; consecutive threads fill one
        // LDS row (no bank conflicts on the transposed stores)
        const int kq = x & 15, oct = x >> 4;
        bf16x8 r[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int row = 4 * kq + rr;
            r[rr] = row < nvalid ? ld_bf8(src + (size_t)row * ld + 8 * oct) : zero_bf8();
        }
        const int pos = kperm(4 * kq);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16x4 t4;
            t4[0] = r[0][e];
            t4[1] = r[1][e];
            t4[2] = r[2][e];
            t4[3] = r[3][e];
            *reinterpret_cast<bf16x4*>(dst + (8 * oct + e) * kVS + pos) = t4;
        }
    }
}

// The same for 64 rows x 64 columns: dst[col * kVS + kperm(row)].
__device__ __forceinline__ void load_vt_tile64(const bf16* __restrict__ src, size_t ld, int nvalid,
                                               bf16* __restrict__ dst, int tid, int nthr) {
    for (int x = tid; x < 16 * 8; x += nthr) {
        const int kq = x & 15, oct = x >> 4;
        bf16x8 r[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int row = 4 * kq + rr;
            r[rr] = row < nvalid ? ld_bf8(src + (size_t)row * ld + 8 * oct) : zero_bf8();
        }
        const int pos = kperm(4 * kq);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16x4 t4;
            t4[0] = r[0][e];
            t4[1] = r[1][e];
            t4[2] = r[2][e];
            t4[3] = r[3][e];
            *reinterpret_cast<bf16x4*>(dst + (8 * oct + e) * kVS + pos) = t4;
        }
    }
}

// 64 rows x 128 columns of a row-major bf16 matrix into LDS twice, in one
// round trip per thread: row-major (dst[row * kKS + col]) and transposed
// (dst_t[col * kVS + kperm(row)]); rows >= nvalid are zero.  Each task loads
// rows 4 kq .. 4 kq + 3, columns 8 oct .. 8 oct + 7 and stores them both
// ways; the loads of all a thread's tasks are issued before any store.
template <int NTHR>
__device__ __forceinline__ void load_tile_both(const bf16* __restrict__ src, size_t ld, int nvalid,
                                               bf16* __restrict__ dst, bf16* __restrict__ dst_t, int tid) {
    constexpr int NT = 256 / NTHR;  // tasks per thread
    bf16x8 r[NT][4];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        const int x = tid + NTHR * u, kq = x & 15, oct = x >> 4;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int row = 4 * kq + rr;
            r[u][rr] = row < nvalid ? ld_bf8(src + (size_t)row * ld + 8 * oct) : zero_bf8();
        }
    }
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        const int x = tid + NTHR * u, kq = x & 15, oct = x >> 4;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) st_bf8(dst + (4 * kq + rr) * kKS + 8 * oct, r[u][rr]);
        const int pos = kperm(4 * kq);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16x4 t4;
            t4[0] = r[u][0][e];
            t4[1] = r[u][1][e];
            t4[2] = r[u][2][e];
            t4[3] = r[u][3][e];
            *reinterpret_cast<bf16x4*>(dst_t + (8 * oct + e) * kVS + pos) = t4;
        }
    }
}

// 64 rows x 128 columns row-major into LDS (stride kKS), loads first
template <int NTHR>
__device__ __forceinline__ void load_rows(const bf16* __restrict__ src, size_t ld, int nvalid,
                                          bf16* __restrict__ dst, int tid) {
    constexpr int NT = kC * 16 / NTHR;
    bf16x8 r[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        const int x = tid + NTHR * u, row = x >> 4, piece = x & 15;
        r[u] = row < nvalid ? ld_bf8(src + (size_t)row * ld + 8 * piece) : zero_bf8();
    }
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        const int x = tid + NTHR * u, row = x >> 4, piece = x & 15;
        st_bf8(dst + row * kKS + 8 * piece, r[u]);
    }
}

// NP-Map (Sec. 3.2, Hedgehog form of Sec. 2) of NT*32 tokens by one wave.
//   u = P x (P: [64][128] fp32, given as bf16 high and low parts Ph, Pl with
//   P = Ph + Pl up to the rounding of Pl; both go through the MFMA),
//   z = ||x|| u / ||u|| (0 if u = 0),  phi = [softmax(z); softmax(-z)].
// The softmax exps are exp2 of (z - max) log2(e), one fma each.
// xb[tt][s]: token 32tt + l%32, dims 16s + 8(l/32) .. +7.
// phi[tt][sgn][ft]: accumulator layout, rows = feature 64 sgn + 32 ft +
// acc_row(v, l/32), column = token.
template <int NT>
__device__ __forceinline__ void np_map_mfma(const bf16x8 (&xb)[NT][8], const bf16* __restrict__ Ph,
                                            const bf16* __restrict__ Pl, int ldp, f32x16 (&phi)[NT][2][2]) {
    const int lane = threadIdx.x & 63, hf = lane >> 5, col = lane & 31;
    f32x16 u[NT][2];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        u[tt][0] = zero16();
        u[tt][1] = zero16();
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
        for (int ft = 0; ft < 2; ++ft) {
            const bf16x8 hi = ld_bf8(Ph + (32 * ft + col) * ldp + 16 * s + 8 * hf);
            const bf16x8 lo = ld_bf8(Pl + (32 * ft + col) * ldp + 16 * s + 8 * hf);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                u[tt][ft] = mfma32(hi, xb[tt][s], u[tt][ft]);
                u[tt][ft] = mfma32(lo, xb[tt][s], u[tt][ft]);
            }
        }
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        float nx = 0.f, nu = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x2 x2 = {xb[tt][s][2 * j], xb[tt][s][2 * j + 1]};
                nx = __builtin_amdgcn_fdot2_f32_bf16(x2, x2, nx, false);
            }
        float umax = -__builtin_inff(), umin = __builtin_inff();
#pragma unroll
        for (int ft = 0; ft < 2; ++ft)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                nu = fmaf(u[tt][ft][v], u[tt][ft][v], nu);
                umax = vmax(umax, u[tt][ft][v]);
                umin = vmin(umin, u[tt][ft][v]);
            }
        nx += xor32(nx);
        nu += xor32(nu);
        umax = vmax(umax, xor32(umax));
        umin = vmin(umin, xor32(umin));
        // z = sc u with sc >= 0, so max z = sc umax and max(-z) = -sc umin
        const float scl = (nu > 0.f ? sqrtf(nx) / sqrtf(nu) : 0.f) * kLog2e;
        const float mp = scl * umax, mn = -scl * umin;
        float sp = 0.f, sn = 0.f;
#pragma unroll
        for (int ft = 0; ft < 2; ++ft)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float uu = u[tt][ft][v];
                const float ep = __builtin_amdgcn_exp2f(fmaf(uu, scl, -mp));
                const float en = __builtin_amdgcn_exp2f(fmaf(uu, -scl, -mn));
                phi[tt][0][ft][v] = ep;
                phi[tt][1][ft][v] = en;
                sp += ep;
                sn += en;
            }
        sp += xor32(sp);
        sn += xor32(sn);
        const float ip = 1.f / sp, in = 1.f / sn;
#pragma unroll
        for (int ft = 0; ft < 2; ++ft)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                phi[tt][0][ft][v] *= ip;
                phi[tt][1][ft][v] *= in;
            }
    }
}

}  // namespace mt
}  // namespace still
