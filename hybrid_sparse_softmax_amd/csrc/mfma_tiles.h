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

// Tile staging (the forward's window-score and output kernels, the backward's
// query kernel): global memory straight into LDS
// (global_load_lds, 16 bytes per lane; lane l of one instruction lands at
// byte 16 l of that instruction's 1 KB).  Rows at or beyond a tile's valid
// count nv (>= 1) repeat row nv-1, so every address stays in bounds; those
// keys are masked out of every sum.
//   K tile: 64 rows of kKS elements (17 slots of 16 bytes, the last one
//     padding); 17 instructions cover its 1088 slots, padding slots load a
//     slot of the same row.  The logits read a K row per lane at a fixed slot:
//     the 17-slot stride spreads 16 rows over all banks.
//   V tile: 64 unpadded rows of 128 elements; slot x of row r is stored at
//     x ^ vswz(r); 16 instructions.  The value product reads it transposed.
typedef __attribute__((address_space(3))) void lds_void;
constexpr int kKTile = kC * kKS;  // elements of a staged K tile
constexpr int kVTile = kC * kD;   // elements of a staged V tile
constexpr int kKPieces = kKTile / 512;  // 17 staging instructions
constexpr int kVPieces = kVTile / 512;  // 16

__device__ __forceinline__ int vswz(int r) { return 4 * (r & 3) + 2 * ((r >> 2) & 1); }

__device__ __forceinline__ void dma16(const bf16* g, bf16* lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}

// The same load written out, for the lock-step loop: the compiler does not
// track it, so it places no wait for it before later LDS reads of other
// buffers; its users wait for it (vmcnt) explicitly.  M0 holds the LDS
// destination (wave-uniform); one wait state separates the M0 write from the
// load that reads it.
__device__ __forceinline__ void dma16_untracked(const bf16* g, unsigned lds_byte) {
    const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_byte);
    __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     :
                     : "v"(g), "s"(m0)
                     : "memory", "m0");
}

// staging instruction j (0..16) of a K tile
__device__ __forceinline__ void stage_k_piece(int j, const bf16* __restrict__ src, size_t ld, int nv,
                                              bf16* __restrict__ dst) {
    const int p = 64 * j + (threadIdx.x & 63), row = p / 17, slot = min(p - 17 * row, 15);
    dma16(src + (size_t)min(row, nv - 1) * ld + 8 * slot, dst + 512 * j);
}

// The same, issued only when en != 0 (wave-uniform); the test and skip sit
// inside the asm statement, so the surrounding code stays one basic block.
__device__ __forceinline__ void dma16_untracked_if(const bf16* g, unsigned lds_byte, int en) {
    const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_byte);
    const int e = __builtin_amdgcn_readfirstlane(en);
    __asm__ volatile("s_cmp_eq_u32 %2, 0\n\ts_cbranch_scc1 1f\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                     "global_load_lds_dwordx4 %0, off\n1:"
                     :
                     : "v"(g), "s"(m0), "s"(e)
                     : "memory", "m0", "scc");
}

// staging instruction j (0..16) of a K tile, untracked load; dst = LDS
// byte address of the tile; ld (elements) and row offsets fit 24 bits
__device__ __forceinline__ void stage_k_piece_u(int j, const bf16* __restrict__ src, int ld, int nv,
                                                unsigned dst) {
    const int p = 64 * j + (threadIdx.x & 63), row = p / 17, slot = min(p - 17 * row, 15);
    dma16_untracked(src + (__umul24(min(row, nv - 1), ld) + 8 * slot), dst + 1024u * j);
}

// staging instruction j of a K tile when j < 17 (no branch around it)
__device__ __forceinline__ void stage_k_piece_if(int j, const bf16* __restrict__ src, int ld, int nv,
                                                 unsigned dst) {
    const int jj = min(j, kKPieces - 1);
    const int p = 64 * jj + (threadIdx.x & 63), row = p / 17, slot = min(p - 17 * row, 15);
    dma16_untracked_if(src + (__umul24(min(row, nv - 1), ld) + 8 * slot), dst + 1024u * jj, j < kKPieces);
}

// Untracked load in the scalar-base form: the address is base (wave-uniform,
// 64-bit) plus the lane's unsigned 32-bit byte offset, so no per-lane 64-bit
// arithmetic is needed.  Issued only when en != 0 (wave-uniform), the test
// and skip inside the asm statement as above.
__device__ __forceinline__ void dma16_sbase_if(const bf16* base, unsigned off, unsigned lds_byte, int en) {
    const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_byte);
    const int e = __builtin_amdgcn_readfirstlane(en);
    __asm__ volatile("s_cmp_eq_u32 %3, 0\n\ts_cbranch_scc1 1f\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                     "global_load_lds_dwordx4 %0, %1\n1:"
                     :
                     : "v"(off), "s"(base), "s"(m0), "s"(e)
                     : "memory", "m0", "scc");
}

// Byte offset, from a tile's first row, of the lane's 16 bytes in staging
// instruction j of a K or V tile whose 64 rows are all readable and ld2
// bytes apart (the same for every tile of the output kernel's loop).
__device__ __forceinline__ unsigned k_piece_off(int j, unsigned ld2) {
    const int p = 64 * j + (threadIdx.x & 63), row = p / 17;
    return (unsigned)row * ld2 + 16u * (unsigned)min(p - 17 * row, 15);
}
__device__ __forceinline__ unsigned v_piece_off(int j, unsigned ld2) {
    const int l = threadIdx.x & 63, row = 4 * j + (l >> 4);
    return (unsigned)row * ld2 + 16u * (unsigned)((l & 15) ^ vswz(row));
}

// staging instruction j (0..15) of a V tile, untracked load
__device__ __forceinline__ void stage_v_piece_u(int j, const bf16* __restrict__ src, int ld, int nv,
                                                unsigned dst) {
    const int l = threadIdx.x & 63, row = 4 * j + (l >> 4), slot = (l & 15) ^ vswz(row);
    dma16_untracked(src + (__umul24(min(row, nv - 1), ld) + 8 * slot), dst + 1024u * j);
}

// staging instruction j (0..15) of a V tile
__device__ __forceinline__ void stage_v_piece(int j, const bf16* __restrict__ src, size_t ld, int nv,
                                              bf16* __restrict__ dst) {
    const int l = threadIdx.x & 63, row = 4 * j + (l >> 4), slot = (l & 15) ^ vswz(row);
    dma16(src + (size_t)min(row, nv - 1) * ld + 8 * slot, dst + 512 * j);
}

// Transposed reads of a staged V tile: the value product's A operand for dims
// 32 dt + l%32 and key storage positions 16 ks + 8 hf .. +7 (key kperm(pos)).
// ds_read_b64_tr_b16 hands lane d of each 16-lane group element j of the
// 8-byte read of lane 4j + d/4 of the group (element d%4); lane s of group
// G = l/16 therefore reads row K0 + s/4, dims 32 dt + 16 (G&1) + 4 (s&3) ..+3,
// and receives keys K0 .. K0+3 of dim 32 dt + l%32.  K0 = 16 ks + 4 hf for
// operand elements 0-3 and K0 + 8 for elements 4-7, which are exactly the
// keys kperm assigns to those elements.  voff[dt] holds the lane's part of
// the element offset.
__device__ __forceinline__ void vt_lane_offsets(int (&voff)[4]) {
    const int l = threadIdx.x & 63, s = l & 15, grp = l >> 4, hf = grp >> 1, gc = grp & 1, m = s >> 2;
    const int c = (4 * hf + m) * kD + 8 * ((2 * gc + ((s & 3) >> 1)) ^ (2 * hf)) + 4 * (s & 1);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) voff[dt] = c + 32 * (dt ^ m);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 vt_frag(const bf16* vtile, const int (&voff)[4], int dt, int ks) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const bf16* p = vtile + voff[dt] + 16 * ks * kD;
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    const i16x4 b2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8 * kD));
    const i16x8 r = __builtin_shufflevector(a, b2, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, r);
}

// Transposed reads of a staged K tile (64 rows of kKS elements, the padded
// layout): the same operand as vt_frag, dims 32 dt + l%32 and row storage
// positions 16 ks + 8 hf .. +7 (row kperm(pos)), from the padded rows (the
// four rows of one read sit 272 bytes apart, so some reads share banks).
__device__ __forceinline__ void kt_pad_lane_offsets(int (&poff)[4]) {
    const int l = threadIdx.x & 63, s16 = l & 15, grp = l >> 4;
    const int c0 = (4 * (grp >> 1) + (s16 >> 2)) * kKS + 16 * (grp & 1) + 4 * (s16 & 3);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) poff[dt] = c0 + 32 * dt;
}

__device__ __forceinline__ bf16x8 kt_pad_frag(const bf16* ktile, const int (&poff)[4], int dt, int ks) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const bf16* p = ktile + poff[dt] + 16 * ks * kKS;
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    const i16x4 b2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8 * kKS));
    const i16x8 r = __builtin_shufflevector(a, b2, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, r);
}

}  // namespace mt
}  // namespace still
