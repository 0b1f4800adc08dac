// STILL chunk-parallel forward on gfx950 matrix cores (bf16 storage, fp32
// accumulation) for head_dim = feature dim = 128 and window = chunk = 64.
//
// Sec. 3.3 "Chunk-Wise Parallel Form" of the STILL paper, one chunk of 64
// tokens per block, the query heads of one KV head (GQA) sharing every K/V
// tile a block stages in LDS:
//   win_select_kernel   window logits (MFMA), Self-Saliency (Sec. 3.1,
//                       Appendix A.3), group mean, per-chunk top-k, route
//                       flags, gather of the selected K/V rows into a
//                       compact per-KV-head list
//   la_state_kernel     NP-Map of the chunk's keys (Sec. 3.2, MFMA
//                       projection), phi_k rows for the read-out, and the
//                       chunk's linear-attention sums over its unselected
//                       tokens (MFMA; Appendix A.2 state)
//   la_scan_t_kernel    inclusive prefix of those sums over chunks
//   hybrid_main_kernel  per query chunk: linear prefix read-out, chunk c-1
//                       (window, routed selected and routed linear tokens),
//                       chunk c (causal window), then every selected token of
//                       chunks <= c-2 from the compact list; one online
//                       normaliser shared by both branches (Fig. 2)
//
// Routing: token j is routed for query t once j <= t - 64, so for a query of
// chunk c the tokens of chunk c-1 at an offset <= its own are routed (their
// chunk's decision is final), later ones are still in its window.
#include <type_traits>

#include "launch.h"
#include "mfma_common.h"

namespace still {

namespace {
typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr int kC = 64;          // chunk = window
constexpr int kD = 128;         // head_dim = NP-Map feature dim
constexpr int kKS = kD + 8;     // LDS row stride (elements) of a K tile
constexpr int kVS = kC + 8;     // LDS row stride (elements) of a transposed V tile
constexpr int kFS = kC + 4;     // LDS row stride (floats) of transposed phi_k
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;   // rescale only when the running max grows by more (log2 units)

enum { kModePrev = 0, kModeDiag = 1, kModeSparse = 2 };

// Q operand of one wave: tokens t0 .. t0+63 of head h; qf[qt][s] holds
// token t0 + 32 qt + l%32, dims 16 s + 8 (l/32) .. +7 (zero beyond N).
__device__ __forceinline__ void load_q(const bf16* __restrict__ q, const Dims& D, int b, int t0,
                                       int h, bf16x8 (&qf)[2][8]) {
    const int lane = threadIdx.x & 63, hf = lane >> 5, col = lane & 31;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int t = t0 + 32 * qt + col;
        const bf16* row = q + (((size_t)b * D.N + t) * D.Hq + h) * kD + 8 * hf;
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[qt][s] = t < D.N ? ld_bf8(row + 16 * s) : zero_bf8();
    }
}

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
        const int kq = x >> 4, oct = x & 15;  // rows 4kq..4kq+3, columns 8oct..8oct+7
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

// NP-Map (Sec. 3.2, Hedgehog form of Sec. 2) of NT*32 tokens by one wave.
//   u = P x (P: [64][128] fp32 as bf16 high + low parts on MFMA),
//   z = ||x|| u / ||u|| (0 if u = 0),  phi = [softmax(z); softmax(-z)].
// xb[tt][s]: token 32tt + l%32, dims 16s + 8(l/32) .. +7.
// phi[tt][sgn][ft]: accumulator layout, rows = feature 64 sgn + 32 ft +
// acc_row(v, l/32), column = token.
template <int NT>
__device__ __forceinline__ void np_map_mfma(const bf16x8 (&xb)[NT][8], const float* __restrict__ P,
                                            f32x16 (&phi)[NT][2][2]) {
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
            bf16x8 hi, lo;
            ld_split8(P + (32 * ft + col) * kD + 16 * s + 8 * hf, hi, lo);
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
            for (int j = 0; j < 8; ++j) {
                const float x = (float)xb[tt][s][j];
                nx = fmaf(x, x, nx);
            }
#pragma unroll
        for (int ft = 0; ft < 2; ++ft)
#pragma unroll
            for (int v = 0; v < 16; ++v) nu = fmaf(u[tt][ft][v], u[tt][ft][v], nu);
        nx += xor32(nx);
        nu += xor32(nu);
        const float sc = nu > 0.f ? sqrtf(nx) / sqrtf(nu) : 0.f;
        float mp = kNegInf, mn = kNegInf;
#pragma unroll
        for (int ft = 0; ft < 2; ++ft)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float z = u[tt][ft][v] * sc;
                u[tt][ft][v] = z;
                mp = fmaxf(mp, z);
                mn = fmaxf(mn, -z);
            }
        mp = fmaxf(mp, xor32(mp));
        mn = fmaxf(mn, xor32(mn));
        float sp = 0.f, sn = 0.f;
#pragma unroll
        for (int ft = 0; ft < 2; ++ft)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float z = u[tt][ft][v];
                const float ep = expf(z - mp), en = expf(-z - mn);
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

// ---------------------------------------------------------------------------
// window scores, selection, gather
// ---------------------------------------------------------------------------
template <int NW>
__global__ __launch_bounds__(NW * 64) void win_select_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    float* __restrict__ scores, int32_t* __restrict__ sel_idx, uint8_t* __restrict__ route,
    bf16* __restrict__ ksel, bf16* __restrict__ vsel, Dims D) {
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, col = lane & 31;
    const int t0 = c * kC;
    const size_t bg = (size_t)b * D.Hkv + g;
    __shared__ float hsc[8][kC];
    __shared__ float key_s[kC];
    __shared__ int flag_s[kC];
    __shared__ int src_s[kC];

    for (int hh = wave; hh < D.G; hh += NW) {
        const int h = g * D.G + hh;
#pragma unroll 1
        for (int qt = 0; qt < 2; ++qt) {
            bf16x8 qf[8];
            {
                const int t = t0 + 32 * qt + col;
                const bf16* row = q + (((size_t)b * D.N + t) * D.Hq + h) * kD + 8 * hf;
#pragma unroll
                for (int s = 0; s < 8; ++s) qf[s] = t < D.N ? ld_bf8(row + 16 * s) : zero_bf8();
            }
            // logits against keys t0-64 .. t0+63: key index kk = 32 kt + row
            f32x16 sc[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) sc[kt] = zero16();
#pragma unroll
            for (int s = 0; s < 8; ++s) {
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    const int key = t0 - kC + 32 * kt + col;
                    const bf16x8 a = (key >= 0 && key < D.N)
                                         ? ld_bf8(k + (((size_t)b * D.N + key) * D.Hkv + g) * kD + 16 * s + 8 * hf)
                                         : zero_bf8();
                    sc[kt] = mfma32(a, qf[s], sc[kt]);
                }
            }
            const int qo = 32 * qt + col;  // query offset in the chunk; its own key is kk = qo + 64
            float mx = kNegInf;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) {
                    const int kk = 32 * kt + acc_row(vv, hf);
                    const bool ok = kk >= qo + 1 && kk <= qo + kC && t0 - kC + kk >= 0;
                    const float x = ok ? D.tau * sc[kt][vv] : kNegInf;
                    sc[kt][vv] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, xor32(mx));
            float sa = 0.f, so = 0.f, et = 0.f;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) {
                    const int kk = 32 * kt + acc_row(vv, hf);
                    const float x = sc[kt][vv];
                    const float e = x == kNegInf ? 0.f : expf(x - mx);
                    sc[kt][vv] = e;
                    sa += e;
                    if (kk == qo + kC) et += e;
                    else so += e;
                }
            sa += xor32(sa);
            so += xor32(so);
            et += xor32(et);
            float term = 0.f;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) {
                    const int kk = 32 * kt + acc_row(vv, hf);
                    term += saliency_term(sc[kt][vv], kk == qo + kC, et, sa, so, D.eps);
                }
            term += xor32(term);
            if (hf == 0) hsc[hh][qo] = term;
        }
    }
    __syncthreads();
    const int nq = min(kC, D.N - t0);
    if (tid < nq) {
        float acc = 0.f;
        for (int hh = 0; hh < D.G; ++hh) acc += hsc[hh][tid];
        const float sig = acc / (float)D.G;
        scores[bg * D.N + t0 + tid] = sig;
        key_s[tid] = route_key(sig);
    }
    __syncthreads();
    uint8_t* rt = route + bg * D.N + t0;
    if (c >= D.n_full) {  // the open chunk: no decision yet
        if (tid < nq) rt[tid] = kPending;
        return;
    }
    if (tid < kC) {
        const float ki = key_s[tid];
        int rank = 0;
        for (int j = 0; j < kC; ++j) {
            const float kj = key_s[j];
            rank += (kj > ki) || (kj == ki && j < tid);
        }
        flag_s[tid] = rank < D.lam ? 1 : 0;
    }
    __syncthreads();
    const size_t base = (bg * D.n_full + c) * D.lam;
    if (tid < kC) {
        const int f = flag_s[tid];
        int before = 0;
        for (int j = 0; j < tid; ++j) before += flag_s[j];
        rt[tid] = f ? kRouteSA : kRouteLA;
        if (f) {
            sel_idx[base + before] = t0 + tid;
            src_s[before] = tid;
        }
    }
    __syncthreads();
    for (int x = tid; x < D.lam * 16; x += NW * 64) {
        const int p = x >> 4, piece = x & 15;
        const size_t src = (((size_t)b * D.N + t0 + src_s[p]) * D.Hkv + g) * kD + 8 * piece;
        st_bf8(ksel + (base + p) * kD + 8 * piece, ld_bf8(k + src));
        st_bf8(vsel + (base + p) * kD + 8 * piece, ld_bf8(v + src));
    }
}

// ---------------------------------------------------------------------------
// NP-Map of keys and per-chunk linear-attention sums (complete chunks only)
// ---------------------------------------------------------------------------
// lin block of chunk c: rows 0..127 = S^T[dim][kperm(f)] = sum over the
// chunk's LA tokens of v[dim] phi_k[f]; row 128 = z[kperm(f)] = sum phi_k[f].
__global__ __launch_bounds__(256) void la_state_kernel(const bf16* __restrict__ k,
                                                       const bf16* __restrict__ v,
                                                       const float* __restrict__ wk,
                                                       const uint8_t* __restrict__ route,
                                                       bf16* __restrict__ phik,
                                                       float* __restrict__ lin, Dims D) {
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, col = lane & 31;
    const int t0 = c * kC;
    const size_t bg = (size_t)b * D.Hkv + g;
    __shared__ __align__(16) bf16 vt[kD * kVS];
    __shared__ __align__(16) float ft[kD * kFS];

    if (wave < 2) {
        const int tt = wave;
        const int tok = t0 + 32 * tt + col;
        bf16x8 xb[1][8];
        const bf16* kr = k + (((size_t)b * D.N + tok) * D.Hkv + g) * kD + 8 * hf;
#pragma unroll
        for (int s = 0; s < 8; ++s) xb[0][s] = ld_bf8(kr + 16 * s);
        f32x16 phi[1][2][2];
        np_map_mfma<1>(xb, wk + (size_t)g * (kD / 2) * kD, phi);
        // phi_k row of the token, features in kperm order, for the read-out
        bf16* pr = phik + (bg * D.N + tok) * kD;
#pragma unroll
        for (int sgn = 0; sgn < 2; ++sgn)
#pragma unroll
            for (int f2 = 0; f2 < 2; ++f2)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    st_bf8(pr + 64 * sgn + 32 * f2 + 16 * s2 + 8 * hf, pack_acc(phi[0][sgn][f2], s2));
        const bool la = route[bg * D.N + tok] == kRouteLA;
        const int tp = kperm(32 * tt + col);
#pragma unroll
        for (int sgn = 0; sgn < 2; ++sgn)
#pragma unroll
            for (int f2 = 0; f2 < 2; ++f2)
#pragma unroll
                for (int vv = 0; vv < 16; ++vv)
                    ft[(64 * sgn + 32 * f2 + acc_row(vv, hf)) * kFS + tp] = la ? phi[0][sgn][f2][vv] : 0.f;
    } else {
        load_vt_tile(v + (((size_t)b * D.N + t0) * D.Hkv + g) * kD, (size_t)D.Hkv * kD, kC, vt,
                     tid - 128, 128);
    }
    __syncthreads();
    float* out = lin + (bg * D.n_full + c) * (size_t)((kD + 1) * kD);
    {
        const int dt = wave;  // dims 32 dt .. 32 dt + 31
#pragma unroll
        for (int f4 = 0; f4 < 4; ++f4) {
            f32x16 acc = zero16();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 a = ld_bf8(vt + (32 * dt + col) * kVS + 16 * ks + 8 * hf);
                bf16x8 hi, lo;
                ld_split8(ft + (32 * f4 + col) * kFS + 16 * ks + 8 * hf, hi, lo);
                acc = mfma32(a, hi, acc);
                acc = mfma32(a, lo, acc);
            }
            const int sp = kperm(32 * f4 + col);
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) out[(size_t)(32 * dt + acc_row(vv, hf)) * kD + sp] = acc[vv];
        }
    }
    if (tid < kD) {
        float z = 0.f;
        for (int t = 0; t < kC; ++t) z += ft[tid * kFS + t];
        out[(size_t)kD * kD + kperm(tid)] = z;
    }
}

// Inclusive prefix over complete chunks, in place; chunk cap_chunk is also
// copied into the decode cache's lin_S [f][dim] / lin_z [f].
__global__ __launch_bounds__(256) void la_scan_t_kernel(float* __restrict__ lin, int cap_chunk,
                                                        float* __restrict__ cap_S,
                                                        float* __restrict__ cap_z, Dims D) {
    constexpr int E1 = (kD + 1) * kD;
    const int e = blockIdx.x * 256 + threadIdx.x, g = blockIdx.y, b = blockIdx.z;
    if (e >= E1) return;
    const size_t bg = (size_t)b * D.Hkv + g;
    float* base = lin + bg * D.n_full * (size_t)E1 + e;
    float run = 0.f;
    for (int c = 0; c < D.n_full; ++c) {
        run += base[(size_t)c * E1];
        base[(size_t)c * E1] = run;
        if (c == cap_chunk && cap_S) {
            const int row = e / kD, f = kperm(e % kD);
            if (row < kD) cap_S[(bg * kD + f) * kD + row] = run;
            else cap_z[bg * kD + f] = run;
        }
    }
}

// ---------------------------------------------------------------------------
// hybrid output
// ---------------------------------------------------------------------------
// Block = NW query heads of KV head g (one wave each) x the 64 tokens of
// chunk c.  Blocks are issued longest first (largest c); consecutive blocks
// take different KV heads, so each XCD's L2 keeps few compact lists.
template <int NW>
__global__ __launch_bounds__(NW * 64) void hybrid_main_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ wq, const bf16* __restrict__ phik, const uint8_t* __restrict__ route,
    const bf16* __restrict__ ksel, const bf16* __restrict__ vsel, const float* __restrict__ lin,
    bf16* __restrict__ out, Dims D) {
    const int HG = D.G / NW;
    const int per_c = D.B * D.Hkv * HG;
    const int c = D.T - 1 - (int)(blockIdx.x / per_c);
    int r = (int)(blockIdx.x % per_c);
    const int hg = r % HG;
    r /= HG;
    const int g = r % D.Hkv, b = r / D.Hkv;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, col = lane & 31;
    const int h = g * D.G + hg * NW + wave;
    const int t0 = c * kC;
    const size_t bg = (size_t)b * D.Hkv + g;
    const float cl2 = D.tau * kLog2e;
    constexpr int NT = NW * 64;

    __shared__ __align__(16) bf16 ks_lds[kC * kKS];
    __shared__ __align__(16) bf16 vt_lds[kD * kVS];

    bf16x8 qf[2][8];
    load_q(q, D, b, t0, h, qf);

    // running state per query (lane column): reference point m2 (log2 units,
    // starts at 0, the linear terms' reference), partial normaliser ls of this
    // half's rows; O rows = queries, columns = dims
    f32x16 o[2][4];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[qt][dt] = zero16();
    float m2[2] = {0.f, 0.f}, ls[2] = {0.f, 0.f};

    f32x16 wla[2][2];  // linear weights of chunk c-1: rows = keys, column = query
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        wla[kt][0] = zero16();
        wla[kt][1] = zero16();
    }
    if (c >= 1) {
        f32x16 phi[2][2][2];
        np_map_mfma<2>(qf, wq + (size_t)g * (kD / 2) * kD, phi);
        const float* st = lin + (bg * D.n_full + (c >= 2 ? c - 2 : 0)) * (size_t)((kD + 1) * kD);
        if (c >= 2) {
            // normaliser of the linear prefix (chunks <= c-2): phi_q . z
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                float acc = 0.f;
#pragma unroll
                for (int sgn = 0; sgn < 2; ++sgn)
#pragma unroll
                    for (int f2 = 0; f2 < 2; ++f2)
#pragma unroll
                        for (int vv = 0; vv < 16; ++vv)
                            acc = fmaf(st[kD * kD + kperm(64 * sgn + 32 * f2 + acc_row(vv, hf))],
                                       phi[qt][sgn][f2][vv], acc);
                ls[qt] = acc;
            }
        }
        bf16x8 phb[2][2][2][2];  // [qt][sgn][ft][s2]
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int sgn = 0; sgn < 2; ++sgn)
#pragma unroll
                for (int f2 = 0; f2 < 2; ++f2) {
                    phb[qt][sgn][f2][0] = pack_acc(phi[qt][sgn][f2], 0);
                    phb[qt][sgn][f2][1] = pack_acc(phi[qt][sgn][f2], 1);
                }
        // phi_k(k_j) . phi_q(q_t) for the keys j of chunk c-1
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const bf16* pk = phik + (bg * D.N + (t0 - kC) + 32 * kt + col) * kD + 8 * hf;
#pragma unroll
            for (int sgn = 0; sgn < 2; ++sgn)
#pragma unroll
                for (int f2 = 0; f2 < 2; ++f2)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        const bf16x8 a = ld_bf8(pk + 64 * sgn + 32 * f2 + 16 * s2);
                        wla[kt][0] = mfma32(a, phb[0][sgn][f2][s2], wla[kt][0]);
                        wla[kt][1] = mfma32(a, phb[1][sgn][f2][s2], wla[kt][1]);
                    }
        }
        if (c >= 2) {
            // numerator of the linear prefix: O = phi_q S
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int sgn = 0; sgn < 2; ++sgn)
#pragma unroll
                    for (int f2 = 0; f2 < 2; ++f2)
#pragma unroll
                        for (int s2 = 0; s2 < 2; ++s2) {
                            bf16x8 hi, lo;
                            ld_split8(st + (size_t)(32 * dt + col) * kD + 64 * sgn + 32 * f2 + 16 * s2 + 8 * hf,
                                      hi, lo);
#pragma unroll
                            for (int qt = 0; qt < 2; ++qt) {
                                o[qt][dt] = mfma32(phb[qt][sgn][f2][s2], hi, o[qt][dt]);
                                o[qt][dt] = mfma32(phb[qt][sgn][f2][s2], lo, o[qt][dt]);
                            }
                        }
        }
    }

    // one 64-key tile staged in LDS (K rows, V transposed)
    auto run_tile = [&](auto mode_tag, int nvalid, uint64_t selmask) {
        constexpr int MODE = decltype(mode_tag)::value;
        f32x16 sc[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            sc[kt][0] = zero16();
            sc[kt][1] = zero16();
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const bf16x8 a = ld_bf8(ks_lds + (32 * kt + col) * kKS + 16 * s + 8 * hf);
                sc[kt][0] = mfma32(a, qf[0][s], sc[kt][0]);
                sc[kt][1] = mfma32(a, qf[1][s], sc[kt][1]);
            }
        }
        float tmax[2] = {kNegInf, kNegInf};
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) {
                    const int rk = 32 * kt + acc_row(vv, hf), oq = 32 * qt + col;
                    bool sa;
                    if constexpr (MODE == kModePrev) sa = rk > oq || ((selmask >> rk) & 1ull);
                    else if constexpr (MODE == kModeDiag) sa = rk <= oq;
                    else sa = rk < nvalid;
                    const float x = sa ? sc[kt][qt][vv] * cl2 : kNegInf;
                    sc[kt][qt][vv] = x;
                    tmax[qt] = fmaxf(tmax[qt], x);
                }
        tmax[0] = fmaxf(tmax[0], xor32(tmax[0]));
        tmax[1] = fmaxf(tmax[1], xor32(tmax[1]));
        const bool need = tmax[0] > m2[0] + kLazy || tmax[1] > m2[1] + kLazy;
        if (__any(need)) {
            float al[2];
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                const float mn = fmaxf(m2[qt], tmax[qt]);
                al[qt] = exp2f(m2[qt] - mn);
                m2[qt] = mn;
                ls[qt] *= al[qt];
            }
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) {
                    const float a = __shfl(al[qt], acc_row(vv, hf), kWave);
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) o[qt][dt][vv] *= a;
                }
        }
        float fla[2] = {0.f, 0.f};
        if constexpr (MODE == kModePrev) {
            fla[0] = exp2f(-m2[0]);
            fla[1] = exp2f(-m2[1]);
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) {
                    const float x = sc[kt][qt][vv];
                    float p = exp2f(x - m2[qt]);
                    if constexpr (MODE == kModePrev) {
                        if (x == kNegInf) p = wla[kt][qt][vv] * fla[qt];  // routed to linear attention
                    }
                    sc[kt][qt][vv] = p;
                    ls[qt] += p;
                }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int kt = ks >> 1, s2 = ks & 1;
            const bf16x8 pa0 = pack_acc(sc[kt][0], s2), pa1 = pack_acc(sc[kt][1], s2);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x8 bv = ld_bf8(vt_lds + (32 * dt + col) * kVS + 16 * ks + 8 * hf);
                o[0][dt] = mfma32(pa0, bv, o[0][dt]);
                o[1][dt] = mfma32(pa1, bv, o[1][dt]);
            }
        }
    };

    const size_t ldkv = (size_t)D.Hkv * kD;
    if (c >= 1) {
        const uint8_t rf = route[bg * D.N + (t0 - kC) + lane];
        const uint64_t selmask = __ballot(rf == kRouteSA);
        const size_t off = (((size_t)b * D.N + (t0 - kC)) * D.Hkv + g) * kD;
        load_k_tile(k + off, ldkv, kC, ks_lds, tid, NT);
        load_vt_tile(v + off, ldkv, kC, vt_lds, tid, NT);
        __syncthreads();
        run_tile(std::integral_constant<int, kModePrev>{}, kC, selmask);
        __syncthreads();
    }
    {
        const int nvalid = min(kC, D.N - t0);
        const size_t off = (((size_t)b * D.N + t0) * D.Hkv + g) * kD;
        load_k_tile(k + off, ldkv, nvalid, ks_lds, tid, NT);
        load_vt_tile(v + off, ldkv, nvalid, vt_lds, tid, NT);
        __syncthreads();
        run_tile(std::integral_constant<int, kModeDiag>{}, nvalid, 0ull);
    }
    if (c >= 2) {
        const int nrows = (c - 1) * D.lam;
        const bf16* kb = ksel + bg * (size_t)D.n_full * D.lam * kD;
        const bf16* vb = vsel + bg * (size_t)D.n_full * D.lam * kD;
        for (int r0 = 0; r0 < nrows; r0 += kC) {
            const int nv = min(kC, nrows - r0);
            __syncthreads();
            load_k_tile(kb + (size_t)r0 * kD, kD, nv, ks_lds, tid, NT);
            load_vt_tile(vb + (size_t)r0 * kD, kD, nv, vt_lds, tid, NT);
            __syncthreads();
            run_tile(std::integral_constant<int, kModeSparse>{}, nv, 0ull);
        }
    }

    float il[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) il[qt] = 1.f / (ls[qt] + xor32(ls[qt]));
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) {
            const float a = __shfl(il[qt], acc_row(vv, hf), kWave);
            const int t = t0 + 32 * qt + acc_row(vv, hf);
            if (t < D.N) {
                bf16* orow = out + (((size_t)b * D.N + t) * D.Hq + h) * kD + col;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) orow[32 * dt] = (bf16)(o[qt][dt][vv] * a);
            }
        }
}

}  // namespace

bool mfma_fwd_supported(const Dims& D) {
    return D.bf16 && D.d == kD && D.fd == kD && D.W == kC && D.C == kC && D.lam > 0 &&
           (D.G == 1 || D.G == 2 || D.G == 4 || D.G == 8);
}

hipError_t launch_win_select(const Dims& D, const void* q, const void* k, const void* v,
                             float* scores, int32_t* sel_idx, uint8_t* route, void* ksel,
                             void* vsel, hipStream_t s) {
    dim3 grid(D.T, D.Hkv, D.B);
    const bf16* qq = reinterpret_cast<const bf16*>(q);
    const bf16* kk = reinterpret_cast<const bf16*>(k);
    const bf16* vv = reinterpret_cast<const bf16*>(v);
    bf16* ks = reinterpret_cast<bf16*>(ksel);
    bf16* vs = reinterpret_cast<bf16*>(vsel);
    if (D.G >= 4)
        hipLaunchKernelGGL(win_select_kernel<4>, grid, dim3(256), 0, s, qq, kk, vv, scores, sel_idx, route, ks, vs, D);
    else if (D.G == 2)
        hipLaunchKernelGGL(win_select_kernel<2>, grid, dim3(128), 0, s, qq, kk, vv, scores, sel_idx, route, ks, vs, D);
    else
        hipLaunchKernelGGL(win_select_kernel<1>, grid, dim3(64), 0, s, qq, kk, vv, scores, sel_idx, route, ks, vs, D);
    return hipGetLastError();
}

hipError_t launch_la_state(const Dims& D, const void* k, const void* v, const float* wphi_k,
                           const uint8_t* route, void* phik, float* lin, hipStream_t s) {
    if (D.n_full == 0) return hipSuccess;
    dim3 grid(D.n_full, D.Hkv, D.B);
    hipLaunchKernelGGL(la_state_kernel, grid, dim3(256), 0, s, reinterpret_cast<const bf16*>(k),
                       reinterpret_cast<const bf16*>(v), wphi_k, route, reinterpret_cast<bf16*>(phik),
                       lin, D);
    return hipGetLastError();
}

hipError_t launch_la_scan_t(const Dims& D, float* lin, int cap_chunk, float* cap_S, float* cap_z,
                            hipStream_t s) {
    constexpr int E1 = (kD + 1) * kD;
    dim3 grid((E1 + 255) / 256, D.Hkv, D.B);
    hipLaunchKernelGGL(la_scan_t_kernel, grid, dim3(256), 0, s, lin, cap_chunk, cap_S, cap_z, D);
    return hipGetLastError();
}

hipError_t launch_hybrid_main(const Dims& D, const void* q, const void* k, const void* v,
                              const float* wphi_q, const void* phik, const uint8_t* route,
                              const void* ksel, const void* vsel, const float* lin, void* out,
                              hipStream_t s) {
    const int NW = D.G >= 4 ? 4 : D.G;
    const unsigned nblk = (unsigned)D.T * D.B * D.Hkv * (D.G / NW);
#define STILL_MAIN(W)                                                                            \
    hipLaunchKernelGGL(hybrid_main_kernel<W>, dim3(nblk), dim3(64 * W), 0, s,                   \
                       reinterpret_cast<const bf16*>(q), reinterpret_cast<const bf16*>(k),      \
                       reinterpret_cast<const bf16*>(v), wphi_q,                                \
                       reinterpret_cast<const bf16*>(phik), route,                              \
                       reinterpret_cast<const bf16*>(ksel), reinterpret_cast<const bf16*>(vsel), \
                       lin, reinterpret_cast<bf16*>(out), D)
    if (NW == 4) STILL_MAIN(4);
    else if (NW == 2) STILL_MAIN(2);
    else STILL_MAIN(1);
#undef STILL_MAIN
    return hipGetLastError();
}

}  // namespace still
