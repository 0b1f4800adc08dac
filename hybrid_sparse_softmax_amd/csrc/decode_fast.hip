// STILL decode step (Sec. 3.3 "Recurrent Form" of the STILL paper) for bf16
// storage, head_dim = feature dim = 128, window 1..256, GQA group 1/2/4/8.
//
// One launch of dec_stream_kernel does all per-step work; one launch of
// dec_combine_kernel merges it:
//   stream blocks  split-KV over the selected list: each wave streams 256
//                  rows, 16 lanes per 256-byte row (coalesced), bf16 dot2
//                  products reduced over the row with DPP, online softmax
//                  rescaled lazily, all query heads of the KV head sharing
//                  every row read
//   state blocks   one per (sequence, KV head): evict token t-W (to the
//                  selected list, or into the linear state S, z of
//                  Appendix A.2), write token t into the window ring,
//                  window softmax row + Self-Saliency of t (Sec. 3.1),
//                  window partial (with the evicted token when it was
//                  selected), linear read-out phi_q . S over one pass of S,
//                  and the chunk-end top-k
//   combine        one shared normaliser over the linear terms (reference
//                  point 0), the window partial and the stream partials
//                  (Fig. 2 "hybrid aggregation"); sel_count advances here,
//                  so stream blocks read the list length of the step start
#include "device_common.h"
#include "launch.h"

namespace still {

namespace {
typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kRowsPerWave = 256;
constexpr int kRowsPerBlock = 4 * kRowsPerWave;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;  // rescale only when the running max grows by more (log2 units)

__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
// the same for rows read once per step: non-temporal, so the stream does not
// displace cached data (and streams faster)
__device__ __forceinline__ bf16x8 ld8_stream(const bf16* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
}

// sum over the 16 lanes of a DPP row; every lane of the row gets the sum
__device__ __forceinline__ float row_sum16(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));   // lane ^ 1
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));   // lane ^ 2
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));  // half-row mirror
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));  // row mirror
    return x;
}

// 8-element bf16 dot product accumulated in fp32
__device__ __forceinline__ float dot8(bf16x8 a, bf16x8 b, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(b, b, 0, 1), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(b, b, 2, 3), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(b, b, 4, 5), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(b, b, 6, 7), acc, false);
    return acc;
}

// NP-Map of one 128-vector by one wave (Sec. 3.2): lane f < 64 forms
// u_f = P[f] . x from its projection row (float4 loads), z = ||x|| u / ||u||,
// phi = [softmax(z); softmax(-z)], times `scale` (a query's gate weight; 1
// for keys).  xs, out: LDS.
__device__ __forceinline__ void np_map_wave128(const float* xs, const float* __restrict__ P,
                                               float* out, int lane, float scale = 1.f) {
    float ss = xs[lane] * xs[lane] + xs[lane + 64] * xs[lane + 64];
    const float nx = sqrtf(wave_sum(ss));
    const f32x4* pr = reinterpret_cast<const f32x4*>(P + (size_t)lane * kD);
    float u = 0.f;
#pragma unroll 8
    for (int i = 0; i < kD / 4; ++i) {
        const f32x4 p = pr[i];
        u = fmaf(p[0], xs[4 * i], u);
        u = fmaf(p[1], xs[4 * i + 1], u);
        u = fmaf(p[2], xs[4 * i + 2], u);
        u = fmaf(p[3], xs[4 * i + 3], u);
    }
    const float nu = sqrtf(wave_sum(u * u));
    const float z = nu > 0.f ? nx * (u / nu) : 0.f;
    const float m1 = wave_max(z), m2 = wave_max(-z);
    const float e1 = expf(z - m1), e2 = expf(-z - m2);
    const float s1 = wave_sum(e1), s2 = wave_sum(e2);
    out[lane] = scale * (e1 / s1);
    out[64 + lane] = scale * (e2 / s2);
}

struct FastWork {
    float* la;      // [B, Hq, kD + 1]      linear numerator, denominator (reference 0)
    float* win;     // [B, Hq, kD + 2]      window partial: max (log2 units), sum, acc
    float* part;    // [B, Hkv, nsplit, G, kD + 2] stream partials
    int* appended;  // [B, Hkv]             1 when the evicted token joined the list
    int nsplit;
};

// --------------------------------------------------------------------------
// stream role: rows [split * 1024 + wave * 256, +256) of the selected list
// --------------------------------------------------------------------------
template <int G>
__device__ __forceinline__ void stream_role(const bf16* __restrict__ q, const CacheView& c,
                                            const FastWork& w, const Dims& D, int b, int g,
                                            int split) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 4, sub = lane & 15;
    const size_t bg = (size_t)b * D.Hkv + g;
    const int n = min(c.sel_count[bg], c.cap);
    const int lo = split * kRowsPerBlock + wave * kRowsPerWave;
    const int hi = min(n, lo + kRowsPerWave);
    const float cl2 = D.tau * kLog2e;

    bf16x8 qv[G];
#pragma unroll
    for (int h = 0; h < G; ++h) qv[h] = ld8(q + ((size_t)b * D.Hq + g * G + h) * kD + 8 * sub);
    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = kNegInf;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }
    const bf16* sk = reinterpret_cast<const bf16*>(c.sel_k) + bg * c.cap * kD + 8 * sub;
    const bf16* sv = reinterpret_cast<const bf16*>(c.sel_v) + bg * c.cap * kD + 8 * sub;
    // kRI rows per lane group and iteration (4 kRI rows per wave), all
    // requested before any is used
    constexpr int kRI = 8;
    for (int r0 = lo; r0 < hi; r0 += 4 * kRI) {
        bf16x8 kr[kRI], vr[kRI];
#pragma unroll
        for (int i = 0; i < kRI; ++i) {
            const int rc = min(r0 + 4 * i + grp, hi - 1);  // rows past the end repeat a valid row
            kr[i] = ld8_stream(sk + (size_t)rc * kD);
            vr[i] = ld8_stream(sv + (size_t)rc * kD);
        }
        float s[kRI][G];
#pragma unroll
        for (int i = 0; i < kRI; ++i) {
            const bool valid = r0 + 4 * i + grp < hi;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float d = row_sum16(dot8(kr[i], qv[h], 0.f));
                s[i][h] = valid ? d * cl2 : kNegInf;
            }
        }
        float tm[G];
        bool need = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float x = s[0][h];
#pragma unroll
            for (int i = 1; i < kRI; ++i) x = fmaxf(x, s[i][h]);
            x = fmaxf(x, __shfl_xor(x, 16, kWave));
            x = fmaxf(x, __shfl_xor(x, 32, kWave));
            tm[h] = x;
            need = need || x > m[h] + kLazy;
        }
        if (__any(need)) {
            __asm__ volatile("");
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float mn = fmaxf(m[h], tm[h]);
                const float al = __builtin_amdgcn_exp2f(m[h] - mn);
                m[h] = mn;
                l[h] *= al;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= al;
            }
        }
#pragma unroll
        for (int i = 0; i < kRI; ++i) {
            float vf[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) vf[e] = (float)vr[i][e];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float p = __builtin_amdgcn_exp2f(s[i][h] - m[h]);
                l[h] += p;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
            }
        }
    }
    // the wave's rows: sum over the four row groups (every lane of a group
    // holds the same l; the 16 lanes of a group hold different dims)
#pragma unroll
    for (int h = 0; h < G; ++h) {
        l[h] += __shfl_xor(l[h], 16, kWave);
        l[h] += __shfl_xor(l[h], 32, kWave);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[h][e] += __shfl_xor(acc[h][e], 16, kWave);
            acc[h][e] += __shfl_xor(acc[h][e], 32, kWave);
        }
    }
    __shared__ float wm[4][G], wl[4][G];
    __shared__ float wacc[4][G][kD];
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            wm[wave][h] = m[h];
            wl[wave][h] = l[h];
        }
    }
    if (grp == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) wacc[wave][h][8 * sub + e] = acc[h][e];
    }
    __syncthreads();
    for (int x = tid; x < G * kD; x += 256) {
        const int h = x / kD, dim = x % kD;
        float M = kNegInf;
#pragma unroll
        for (int v = 0; v < 4; ++v)
            if (wl[v][h] > 0.f) M = fmaxf(M, wm[v][h]);
        float L = 0.f, A = 0.f;
        if (M != kNegInf) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (wl[v][h] > 0.f) {
                    const float f = __builtin_amdgcn_exp2f(wm[v][h] - M);
                    L = fmaf(wl[v][h], f, L);
                    A = fmaf(wacc[v][h][dim], f, A);
                }
        }
        float* pp = w.part + ((bg * w.nsplit + split) * G + h) * (kD + 2);
        if (dim == 0) {
            pp[0] = M;
            pp[1] = L;
        }
        pp[2 + dim] = A;
    }
}

// --------------------------------------------------------------------------
// state role: one (sequence, KV head)
// --------------------------------------------------------------------------
// R: window keys per lane (the window holds up to 64 R tokens)
template <int R>
__device__ __forceinline__ void state_role(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                           const bf16* __restrict__ v, const float* __restrict__ wq,
                                           const float* __restrict__ wk,
                                           const float* __restrict__ gate, const CacheView& c,
                                           const FastWork& w, const Dims& D, int b, int g) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t bg = (size_t)b * D.Hkv + g;
    const int W = D.W, C = D.C, G = D.G;
    const int64_t t = c.pos_dev ? c.pos_dev[b] : c.pos;
    const int slot_t = (int)(t % W);
    bf16* ring_k = reinterpret_cast<bf16*>(c.win_k) + bg * W * kD;
    bf16* ring_v = reinterpret_cast<bf16*>(c.win_v) + bg * W * kD;
    uint8_t* flags = c.win_route + bg * W;
    const bf16* kt = k + bg * kD;
    const bf16* vt = v + bg * kD;

    __shared__ float qs[8][kD], phq[8][kD];
    __shared__ float xs[kD], vs[kD], ph[kD], zl[kD];
    __shared__ float numl[2][8][kD];
    __shared__ float hsc[8];

    // 1. the token at t - W leaves the window (ring slot t % W)
    uint8_t ev = 0;
    if (t >= W) {
        ev = D.lam == 0 ? kRouteLA : flags[slot_t];
        if (ev == kPending) ev = kRouteLA;  // unreachable for a consistent cache (W >= C)
    }
    for (int x = tid; x < G * kD; x += 256)
        qs[x / kD][x % kD] = (float)q[((size_t)b * D.Hq + g * G) * kD + x];
    if (ev != 0 && tid < kD) {
        xs[tid] = (float)ring_k[(size_t)slot_t * kD + tid];
        vs[tid] = (float)ring_v[(size_t)slot_t * kD + tid];
    }
    __syncthreads();
    // NP-Map of the query heads and, for a linear eviction, of the leaving key
    const int items = G + (ev == kRouteLA ? 1 : 0);
    for (int it = wave; it < items; it += 4) {
        if (it < G)  // the query's features carry its gate weight
            np_map_wave128(qs[it], wq + (size_t)g * (kD / 2) * kD, phq[it], lane,
                           gate_weight(gate, (size_t)b * D.Hq + g * G + it));
        else np_map_wave128(xs, wk + (size_t)g * (kD / 2) * kD, ph, lane);
    }
    int appended = 0;
    if (ev == kRouteSA) {
        const int n = c.sel_count[bg];
        if (n < c.cap) {
            appended = 1;
            if (tid < 32) {
                const int piece = tid & 15;
                const bf16* src = (tid < 16 ? ring_k : ring_v) + (size_t)slot_t * kD + 8 * piece;
                bf16* dst = reinterpret_cast<bf16*>(tid < 16 ? c.sel_k : c.sel_v) + (bg * c.cap + n) * kD + 8 * piece;
                *reinterpret_cast<bf16x8*>(dst) = ld8(src);
            }
        }
    }
    if (tid == 0) w.appended[bg] = appended;
    __syncthreads();
    // 2. token t enters the ring (the leaving row was read above)
    if (tid < 32) {
        const int piece = tid & 15;
        const bf16* src = (tid < 16 ? kt : vt) + 8 * piece;
        bf16* dst = (tid < 16 ? ring_k : ring_v) + (size_t)slot_t * kD + 8 * piece;
        *reinterpret_cast<bf16x8*>(dst) = ld8(src);
    }
    if (tid == 0) flags[slot_t] = kPending;
    // 3. one pass over S: fold in a linear eviction, read out phi_q . S
    {
        const int dim = tid & (kD - 1), half = tid >> 7;
        float num[8];
#pragma unroll
        for (int h = 0; h < 8; ++h) num[h] = 0.f;
        float* Sg = c.lin_S + bg * D.fd * kD;
        const bool la = ev == kRouteLA;
        const float vd = la ? vs[dim] : 0.f;
        // rows in batches of 32, each batch's loads issued before any is used
        // (the step's latency chain otherwise)
        for (int f0 = half * 64; f0 < half * 64 + 64; f0 += 32) {
            float sv[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) sv[u] = Sg[(size_t)(f0 + u) * kD + dim];
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                const int f = f0 + u;
                if (la) {
                    sv[u] = fmaf(ph[f], vd, sv[u]);
                    Sg[(size_t)f * kD + dim] = sv[u];
                }
#pragma unroll
                for (int h = 0; h < 8; ++h)
                    if (h < G) num[h] = fmaf(phq[h][f], sv[u], num[h]);
            }
        }
#pragma unroll
        for (int h = 0; h < 8; ++h)
            if (h < G) numl[half][h][dim] = num[h];
        if (tid < kD) {
            float z = c.lin_z[bg * D.fd + tid];
            if (la) {
                z += ph[tid];
                c.lin_z[bg * D.fd + tid] = z;
            }
            zl[tid] = z;
        }
    }
    __syncthreads();
    for (int x = tid; x < G * kD; x += 256) {
        const int h = x / kD, dim = x % kD;
        w.la[((size_t)b * D.Hq + g * G + h) * (kD + 1) + dim] = numl[0][h][dim] + numl[1][h][dim];
    }
    // 4. per query head: window row, Self-Saliency, window partial, denominator
    //    (window index i = lane + 64 r in register r; the own key is i = n_win - 1)
    const int n_win = (int)min<int64_t>(t + 1, W);
    for (int hh = wave; hh < G; hh += 4) {
        const float* qh = qs[hh];
        float sj[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = lane + 64 * r;
            sj[r] = kNegInf;
            if (i < n_win) {
                const int64_t pos = t - n_win + 1 + i;
                const bf16* kr = i == n_win - 1 ? kt : ring_k + (size_t)(pos % W) * kD;
                float d = 0.f;
#pragma unroll 8
                for (int x = 0; x < kD / 8; ++x) {
                    const bf16x8 kk = ld8(kr + 8 * x);
#pragma unroll
                    for (int e = 0; e < 8; ++e) d = fmaf(qh[8 * x + e], (float)kk[e], d);
                }
                sj[r] = D.tau * d;
            }
        }
        // Self-Saliency of t over its window
        float lmx = sj[0];
#pragma unroll
        for (int r = 1; r < R; ++r) lmx = fmaxf(lmx, sj[r]);
        const float mx = wave_max(lmx);
        float e[R], sal = 0.f, sol = 0.f, etl = 0.f, own = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = lane + 64 * r;
            e[r] = i < n_win ? expf(sj[r] - mx) : 0.f;
            sal += e[r];
            if (i == n_win - 1) {
                etl += e[r];
                own += sj[r];
            } else {
                sol += e[r];
            }
        }
        const float sa = wave_sum(sal), so = wave_sum(sol), et = wave_sum(etl);
        float term = 0.f;
        if (D.route == kRouteSaliency) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int i = lane + 64 * r;
                if (i < n_win && e[r] > 0.f) {
                    const float a = e[r] / sa;
                    if (i == n_win - 1) term += a * log1pf(a / D.eps);
                    else term += -a * log1p_fast(fast_div((et / so) * e[r], e[r] + D.eps * sa));
                }
            }
            term = wave_sum(term);
        } else if (D.route == kRouteDiagonal) {
            term = et / sa;  // the own weight a_tt
        } else {
            term = wave_sum(own);  // the own logit tau q_t.k_t (one lane holds it)
        }
        if (lane == 0) hsc[hh] = term;
        // the evicted token when it joined the selected list this step
        float sev = kNegInf;
        if (appended) {
            float dp = xs[lane] * qh[lane] + xs[lane + 64] * qh[lane + 64];
            sev = D.tau * wave_sum(dp);
        }
        const float mw = fmaxf(mx, sev);
        float p[R], pl = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            p[r] = lane + 64 * r < n_win ? expf(sj[r] - mw) : 0.f;
            pl += p[r];
        }
        const float pev = appended ? expf(sev - mw) : 0.f;
        float lw = wave_sum(pl) + pev;
        float a0 = pev * vs[2 * lane], a1 = pev * vs[2 * lane + 1];
        if (!appended) a0 = a1 = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int nb = min(64, n_win - 64 * r);
            // rows in batches of 16, loaded before use; a batch's rows past
            // the window repeat its last row and take no weight
            for (int j0 = 0; j0 < nb; j0 += 16) {
                bf16x2 v2[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int j = 64 * r + min(j0 + u, nb - 1);
                    const int64_t pos = t - n_win + 1 + j;
                    const bf16* vr = j == n_win - 1 ? vt : ring_v + (size_t)(pos % W) * kD;
                    v2[u] = *reinterpret_cast<const bf16x2*>(vr + 2 * lane);
                }
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const float pj = __shfl(p[r], min(j0 + u, 63), kWave);
                    if (j0 + u < nb) {
                        a0 = fmaf(pj, (float)v2[u][0], a0);
                        a1 = fmaf(pj, (float)v2[u][1], a1);
                    }
                }
            }
        }
        float* wp = w.win + ((size_t)b * D.Hq + g * G + hh) * (kD + 2);
        if (lane == 0) {
            wp[0] = mw * kLog2e;
            wp[1] = lw;
        }
        wp[2 + 2 * lane] = a0;
        wp[3 + 2 * lane] = a1;
        // linear denominator phi_q . z
        const float dz = phq[hh][lane] * zl[lane] + phq[hh][lane + 64] * zl[lane + 64];
        const float den = wave_sum(dz);
        if (lane == 0) w.la[((size_t)b * D.Hq + g * G + hh) * (kD + 1) + kD] = den;
    }
    __syncthreads();
    // 5. group-mean score of t; chunk end: top-k of the chunk's scores
    __shared__ float sig_s;
    if (tid == 0) {
        float sig;
        if (route_query_free(D.route)) {
            float kn = 0.f;
            if (D.route == kRouteKeyNorm)
                for (int e = 0; e < kD; ++e) kn = fmaf((float)kt[e], (float)kt[e], kn);
            sig = query_free_score(D.route, sqrtf(kn), t, b, g, D.Hkv, C, D.lam);
        } else {
            float acc = 0.f;
            for (int hh = 0; hh < G; ++hh) acc += hsc[hh];
            sig = acc / (float)G;
        }
        c.pend[bg * C + (int)(t % C)] = sig;
        sig_s = sig;
    }
    __syncthreads();
    if ((t % C) == C - 1) {
        const int64_t c0 = t - C + 1;
        const int own = (int)(t % C);
        const float* pend = c.pend + bg * C;
        if (D.lam == 0) {
            for (int i = tid; i < C; i += 256) flags[(int)((c0 + i) % W)] = kRouteLA;
        } else if (tid < 64) {
            // radix top-lam of the chunk's scores by one wave (C <= 256: four per lane)
            uint32_t kb[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 64 * r + lane;
                kb[r] = i < C ? key_bits(route_key(i == own ? sig_s : pend[i])) : 0u;
            }
            bool f[4];
            int at[4];
            wave_topk<4>(kb, C, D.lam, f, at);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 64 * r + lane;
                if (i < C) flags[(int)((c0 + i) % W)] = f[r] ? kRouteSA : kRouteLA;
            }
        }
    }
}

template <int G, int R>
__global__ __launch_bounds__(256) void dec_stream_kernel(const bf16* __restrict__ q,
                                                         const bf16* __restrict__ k,
                                                         const bf16* __restrict__ v,
                                                         const float* __restrict__ wq,
                                                         const float* __restrict__ wk,
                                                         const float* __restrict__ gate, CacheView c,
                                                         FastWork w, Dims D) {
    const int nstate = D.B * D.Hkv;
    const int bid = blockIdx.x;
    if (bid < nstate) {
        state_role<R>(q, k, v, wq, wk, gate, c, w, D, bid / D.Hkv, bid % D.Hkv);
    } else {
        const int x = bid - nstate;
        const int split = x % w.nsplit, bg = x / w.nsplit;
        stream_role<G>(q, c, w, D, bg / D.Hkv, bg % D.Hkv, split);
    }
}

__global__ __launch_bounds__(kD) void dec_combine_kernel(FastWork w, CacheView c, bf16* __restrict__ out,
                                                         Dims D) {
    const int h = blockIdx.x, b = blockIdx.y, dim = threadIdx.x;
    const int g = h / D.G, hh = h % D.G;
    // the last launch of the step: every read of this step's positions is done
    if (c.pos_dev && h == 0 && dim == 0) c.pos_dev[b] += 1;
    const size_t bh = (size_t)b * D.Hq + h, bg = (size_t)b * D.Hkv + g;
    const float* la = w.la + bh * (kD + 1);
    const float* wp = w.win + bh * (kD + 2);
    // Linear terms sit at reference 0 (log2 units), so with linear mass the
    // common reference is max(0, the partials' maxima); without it (no routed
    // linear token) it is the partials' maximum alone, which may be negative:
    // logits far below 0 would otherwise underflow every weight and leave 0 / 0.
    const bool has_la = la[kD] > 0.f;
    float M = has_la ? 0.f : -__builtin_inff();
    if (wp[1] > 0.f) M = fmaxf(M, wp[0]);
    for (int s = 0; s < w.nsplit; ++s) {
        const float* pp = w.part + ((bg * w.nsplit + s) * D.G + hh) * (kD + 2);
        if (pp[1] > 0.f) M = fmaxf(M, pp[0]);
    }
    const float fl = has_la ? __builtin_amdgcn_exp2f(-M) : 0.f;
    float num = la[dim] * fl, den = la[kD] * fl;
    if (wp[1] > 0.f) {
        const float f = __builtin_amdgcn_exp2f(wp[0] - M);
        num = fmaf(wp[2 + dim], f, num);
        den = fmaf(wp[1], f, den);
    }
    for (int s = 0; s < w.nsplit; ++s) {
        const float* pp = w.part + ((bg * w.nsplit + s) * D.G + hh) * (kD + 2);
        if (pp[1] > 0.f) {
            const float f = __builtin_amdgcn_exp2f(pp[0] - M);
            num = fmaf(pp[2 + dim], f, num);
            den = fmaf(pp[1], f, den);
        }
    }
    out[bh * kD + dim] = (bf16)(num / den);
    if (hh == 0 && dim == 0 && c.sel_count) c.sel_count[bg] += w.appended[bg];
}
}  // namespace

bool fast_decode_supported(const Dims& D) {
    return D.bf16 && D.d == kD && D.fd == kD && D.W >= 1 && D.W <= 256 && D.C <= 256 &&
           (D.G == 1 || D.G == 2 || D.G == 4 || D.G == 8);
}

int fast_decode_splits(int cap) { return cap <= 0 ? 0 : (cap + kRowsPerBlock - 1) / kRowsPerBlock; }

size_t fast_decode_floats(const Dims& D, int nsplit) {
    return (size_t)D.B * D.Hq * (kD + 1) + (size_t)D.B * D.Hq * (kD + 2) +
           (size_t)D.B * D.Hkv * (nsplit > 0 ? nsplit : 1) * D.G * (kD + 2) + (size_t)D.B * D.Hkv;
}

hipError_t launch_fast_decode(const Dims& D, const void* q, const void* k, const void* v,
                              const float* wq, const float* wk, const float* gate,
                              const CacheView& c, float* ws,
                              int nsplit, void* out, int phase, hipStream_t s) {
    FastWork w;
    w.nsplit = D.lam > 0 ? nsplit : 0;
    w.la = ws;
    w.win = w.la + (size_t)D.B * D.Hq * (kD + 1);
    w.part = w.win + (size_t)D.B * D.Hq * (kD + 2);
    w.appended = reinterpret_cast<int*>(w.part + (size_t)D.B * D.Hkv * (nsplit > 0 ? nsplit : 1) * D.G * (kD + 2));
    if (phase == 1) {
        hipLaunchKernelGGL(dec_combine_kernel, dim3(D.Hq, D.B), dim3(kD), 0, s, w, c,
                           reinterpret_cast<bf16*>(out), D);
        return hipGetLastError();
    }
    const unsigned nblk = (unsigned)(D.B * D.Hkv) * (1 + w.nsplit);
    const bf16* qq = reinterpret_cast<const bf16*>(q);
    const bf16* kk = reinterpret_cast<const bf16*>(k);
    const bf16* vv = reinterpret_cast<const bf16*>(v);
#define STILL_DEC2(GG, RR) \
    hipLaunchKernelGGL((dec_stream_kernel<GG, RR>), dim3(nblk), dim3(256), 0, s, qq, kk, vv, wq, wk, gate, c, w, D)
#define STILL_DEC(GG)                     \
    do {                                  \
        if (D.W <= 64) STILL_DEC2(GG, 1);  \
        else if (D.W <= 128) STILL_DEC2(GG, 2); \
        else STILL_DEC2(GG, 4);           \
    } while (0)
    if (D.G == 1) STILL_DEC(1);
    else if (D.G == 2) STILL_DEC(2);
    else if (D.G == 4) STILL_DEC(4);
    else STILL_DEC(8);
#undef STILL_DEC
#undef STILL_DEC2
    return hipGetLastError();
}

}  // namespace still
