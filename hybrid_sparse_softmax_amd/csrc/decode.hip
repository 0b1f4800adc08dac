// STILL decode step (Sec. 3.3 "Recurrent Form" of the STILL paper).
//
//   decode_prep_kernel     one block per (b, g): evict t-W (selected list or
//                          linear state, Appendix A.2), write t into the ring,
//                          window softmax row + Self-Saliency of t per head,
//                          window partial, linear read-out, chunk-end top-k
//   decode_sel_kernel      split-KV pass over the selected list, all heads of
//                          the group sharing each K/V row read
//   decode_combine_kernel  merge linear + window + split partials, one shared
//                          normaliser (Fig. 2 "hybrid aggregation")
#include "device_common.h"
#include "launch.h"
#include "np_map.h"

namespace still {

namespace {
constexpr float kNegInf = -__builtin_inff();
constexpr int kMaxG = 8;

// Chunk-end top-lam of the C pending scores (slot i = position c0 + i) by
// one wave: route flags of the chunk's ring slots.
template <int R>
__device__ __forceinline__ void decode_topk(const float* pend, int C, int lam, int64_t c0, int W,
                                            uint8_t* flags) {
    const int lane = threadIdx.x & 63;
    uint32_t kb[R];
#pragma unroll
    for (int r = 0; r < R; ++r) kb[r] = 64 * r + lane < C ? key_bits(route_key(pend[64 * r + lane])) : 0u;
    bool f[R];
    int at[R];
    wave_topk<R>(kb, C, lam, f, at);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = 64 * r + lane;
        if (i < C) flags[(int)((c0 + i) % W)] = f[r] ? kRouteSA : kRouteLA;
    }
}

template <typename T, int DD, int R>
__global__ __launch_bounds__(256) void decode_prep_kernel(const T* __restrict__ q,
                                                          const T* __restrict__ k,
                                                          const T* __restrict__ v,
                                                          const float* __restrict__ wq,
                                                          const float* __restrict__ wk,
                                                          const float* __restrict__ gate,
                                                          CacheView c, DecodeWork w, Dims D) {
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const size_t bg = (size_t)b * D.Hkv + g;
    const int W = D.W, C = D.C, G = D.G;
    const int64_t t = c.pos_dev ? c.pos_dev[b] : c.pos;
    const T* kt = k + bg * DD;
    const T* vt = v + bg * DD;
    T* ring_k = W > 0 ? reinterpret_cast<T*>(c.win_k) + bg * W * DD : nullptr;
    T* ring_v = W > 0 ? reinterpret_cast<T*>(c.win_v) + bg * W * DD : nullptr;
    uint8_t* flags = W > 0 ? c.win_route + bg * W : nullptr;
    float* S = c.lin_S + bg * D.fd * DD;
    float* z = c.lin_z + bg * D.fd;

    __shared__ float xs[DD], vs[DD], ph[DD];
    __shared__ float qs[4][DD], fq[4][DD];
    __shared__ float hscore[kMaxG];
    __shared__ int s_n;

    // 1. the token at t - W leaves the window
    uint8_t ev = 0;
    const T *ek = nullptr, *evv = nullptr;
    if (W == 0) {
        ev = kRouteLA; ek = kt; evv = vt;
    } else if (t >= W) {
        const int slot = (int)(t % W);
        ev = D.lam == 0 ? kRouteLA : flags[slot];
        if (ev == kPending) ev = kRouteLA;  // unreachable for a consistent cache (W >= C)
        ek = ring_k + (size_t)slot * DD;
        evv = ring_v + (size_t)slot * DD;
    }
    if (ev == kRouteSA) {
        if (tid == 0) s_n = c.sel_count[bg];
        __syncthreads();
        const int n = s_n;
        if (n < c.cap) {
            T* sk = reinterpret_cast<T*>(c.sel_k) + (bg * c.cap + n) * DD;
            T* sv = reinterpret_cast<T*>(c.sel_v) + (bg * c.cap + n) * DD;
            for (int i = tid; i < DD; i += 256) { sk[i] = ek[i]; sv[i] = evv[i]; }
            if (tid == 0) c.sel_count[bg] = n + 1;
        }
    } else if (ev == kRouteLA) {
        for (int i = tid; i < DD; i += 256) { xs[i] = to_f32(ek[i]); vs[i] = to_f32(evv[i]); }
        __syncthreads();
        if (wave == 0) np_map_wave(xs, wk + (size_t)g * (D.fd / 2) * DD, DD, D.fd, ph, lane);
        __syncthreads();
        for (int e = tid; e < D.fd * DD; e += 256) S[e] += ph[e / DD] * vs[e % DD];
        for (int e = tid; e < D.fd; e += 256) z[e] += ph[e];
    }
    __syncthreads();
    // 2. the new token enters the ring
    if (W > 0) {
        const int slot = (int)(t % W);
        for (int i = tid; i < DD; i += 256) {
            ring_k[(size_t)slot * DD + i] = kt[i];
            ring_v[(size_t)slot * DD + i] = vt[i];
        }
        if (tid == 0) flags[slot] = kPending;
    }
    __syncthreads();
    // 3, 4. per query head of the group: wave w takes head base + w of each
    // round of four; every wave reaches every barrier.
    const int n_win = W > 0 ? (int)min<int64_t>(t + 1, W) : 0;
    for (int base = 0; base < G; base += 4) {
        const int hh = base + wave;
        const bool act = hh < G;
        const int h = g * G + hh;
        if (act) {
            const T* qr = q + ((size_t)b * D.Hq + h) * DD;
            for (int i = lane; i < DD; i += kWave) qs[wave][i] = to_f32(qr[i]);
        }
        __syncthreads();
        if (act) {
            float* win_part = w.win + ((size_t)b * D.Hq + h) * (DD + 2);
            if (W > 0) {
                // window row: positions t-n_win+1 .. t; index n_win-1 is t itself
                float s[R];
                float mx = kNegInf;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int idx = r * kWave + lane;
                    s[r] = kNegInf;
                    if (idx < n_win) {
                        const int64_t pos = t - n_win + 1 + idx;
                        const T* kr = ring_k + (size_t)(pos % W) * DD;
                        float dot = 0.f;
                        for (int i = 0; i < DD; ++i) dot = fmaf(qs[wave][i], to_f32(kr[i]), dot);
                        s[r] = D.tau * dot;
                        mx = fmaxf(mx, s[r]);
                    }
                }
                mx = wave_max(mx);
                float e[R];
                float sa = 0.f, so = 0.f, et = 0.f;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int idx = r * kWave + lane;
                    e[r] = idx < n_win ? expf(s[r] - mx) : 0.f;
                    sa += e[r];
                    if (idx == n_win - 1) et = e[r]; else so += e[r];
                }
                sa = wave_sum(sa); so = wave_sum(so); et = wave_sum(et);
                float term = 0.f;
                if (D.route == kRouteSaliency) {
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const int idx = r * kWave + lane;
                        if (idx < n_win) term += saliency_term(e[r], idx == n_win - 1, et, sa, so, D.eps);
                    }
                    term = wave_sum(term);
                } else if (D.route == kRouteDiagonal) {
                    term = et / sa;  // the own weight a_tt
                } else {
                    // the own logit tau q_t.k_t (query-free criteria ignore it)
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        if (r * kWave + lane == n_win - 1) term = s[r];
                    term = wave_sum(term);
                }
                if (lane == 0) hscore[hh] = term;
                // window partial at reference mx: l = sum e_j, acc = sum e_j v_j
                float acc[DD / kWave];
#pragma unroll
                for (int p = 0; p < DD / kWave; ++p) acc[p] = 0.f;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int nb = min(kWave, n_win - r * kWave);
                    for (int jj = 0; jj < nb; ++jj) {
                        const float ej = __shfl(e[r], jj, kWave);
                        const int64_t pos = t - n_win + 1 + r * kWave + jj;
                        const T* vr = ring_v + (size_t)(pos % W) * DD;
#pragma unroll
                        for (int p = 0; p < DD / kWave; ++p)
                            acc[p] = fmaf(ej, to_f32(vr[lane + kWave * p]), acc[p]);
                    }
                }
                if (lane == 0) { win_part[0] = mx; win_part[1] = sa; }
#pragma unroll
                for (int p = 0; p < DD / kWave; ++p) win_part[2 + lane + kWave * p] = acc[p];
            } else {
                if (lane == 0) { win_part[0] = kNegInf; win_part[1] = 0.f; }
                for (int i = lane; i < DD; i += kWave) win_part[2 + i] = 0.f;
            }
            // the query's features carry its gate weight (the linear branch's weight)
            np_map_wave(qs[wave], wq + (size_t)g * (D.fd / 2) * DD, DD, D.fd, fq[wave], lane,
                        gate_weight(gate, (size_t)b * D.Hq + h));
        }
        __syncthreads();
        if (act) {
            // linear read-out with phi_q(q_t) and the updated state
            float* la = w.la + ((size_t)b * D.Hq + h) * (DD + 1);
            for (int dim = lane; dim < DD; dim += kWave) {
                float a = 0.f;
                for (int i = 0; i < D.fd; ++i) a = fmaf(fq[wave][i], S[(size_t)i * DD + dim], a);
                la[dim] = a;
            }
            float dp = 0.f;
            for (int i = lane; i < D.fd; i += kWave) dp = fmaf(fq[wave][i], z[i], dp);
            dp = wave_sum(dp);
            if (lane == 0) la[DD] = dp;
        }
        __syncthreads();
    }
    // group-mean score of t into the open chunk
    if (W > 0 && tid == 0) {
        if (route_query_free(D.route)) {
            float kn = 0.f;
            if (D.route == kRouteKeyNorm)
                for (int i = 0; i < DD; ++i) kn = fmaf(to_f32(kt[i]), to_f32(kt[i]), kn);
            c.pend[bg * C + (int)(t % C)] = query_free_score(D.route, sqrtf(kn), t, b, g, D.Hkv, C, D.lam);
        } else {
            float acc = 0.f;
            for (int hh = 0; hh < G; ++hh) acc += hscore[hh];
            c.pend[bg * C + (int)(t % C)] = acc / (float)G;
        }
    }
    __syncthreads();
    // 5. t closes its chunk: top-lam of the chunk's pending scores
    if (W > 0 && (t % C) == C - 1) {
        const int64_t c0 = t - C + 1;
        const float* pend = c.pend + bg * C;
        if (D.lam == 0) {
            for (int i = tid; i < C; i += 256) flags[(int)((c0 + i) % W)] = kRouteLA;
        } else if (tid < kWave) {  // radix top-lam of the chunk's pending scores by one wave
            if (C <= kWave) decode_topk<1>(pend, C, D.lam, c0, W, flags);
            else if (C <= 4 * kWave) decode_topk<4>(pend, C, D.lam, c0, W, flags);
            else decode_topk<16>(pend, C, D.lam, c0, W, flags);
        }
    }
}

// Split-KV pass over rows [split * rps, min(count, (split+1) * rps)) of the
// selected list; partial (m, l, acc) per query head of the group.
template <typename T, int DD>
__global__ __launch_bounds__(64) void decode_sel_kernel(const T* __restrict__ q, CacheView c,
                                                        DecodeWork w, Dims D) {
    constexpr int PL = DD / kWave;
    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const size_t bg = (size_t)b * D.Hkv + g;
    const int G = D.G;
    const int n = min(c.sel_count[bg], c.cap);  // never read past the buffer
    const int lo = split * w.rows_per_split, hi = min(n, lo + w.rows_per_split);
    __shared__ float qs[kMaxG][DD];
    for (int x = lane; x < G * DD; x += kWave)
        qs[x / DD][x % DD] = to_f32(q[((size_t)b * D.Hq + g * G) * DD + x]);
    __syncthreads();
    const T* sk = reinterpret_cast<const T*>(c.sel_k) + bg * c.cap * DD;
    const T* sv = reinterpret_cast<const T*>(c.sel_v) + bg * c.cap * DD;
    float m[kMaxG], l[kMaxG], acc[kMaxG][PL];
#pragma unroll
    for (int hh = 0; hh < kMaxG; ++hh) {
        m[hh] = kNegInf; l[hh] = 0.f;
#pragma unroll
        for (int p = 0; p < PL; ++p) acc[hh][p] = 0.f;
    }
    for (int j0 = lo; j0 < hi; j0 += kWave) {
        const int j = j0 + lane;
        const bool valid = j < hi;
        float s[kMaxG], pj[kMaxG];
#pragma unroll
        for (int hh = 0; hh < kMaxG; ++hh) s[hh] = 0.f;
        if (valid) {
            const T* kr = sk + (size_t)j * DD;
            for (int i = 0; i < DD; ++i) {
                const float kv = to_f32(kr[i]);
#pragma unroll
                for (int hh = 0; hh < kMaxG; ++hh)
                    if (hh < G) s[hh] = fmaf(qs[hh][i], kv, s[hh]);
            }
        }
#pragma unroll
        for (int hh = 0; hh < kMaxG; ++hh) s[hh] = valid ? D.tau * s[hh] : kNegInf;
#pragma unroll
        for (int hh = 0; hh < kMaxG; ++hh) {
            if (hh >= G) break;
            const float m_new = fmaxf(m[hh], wave_max(s[hh]));
            const float sc = expf(m[hh] - m_new);
            pj[hh] = valid ? expf(s[hh] - m_new) : 0.f;
            l[hh] = l[hh] * sc + wave_sum(pj[hh]);
#pragma unroll
            for (int p = 0; p < PL; ++p) acc[hh][p] *= sc;
            m[hh] = m_new;
        }
        const int nb = min(kWave, hi - j0);
        for (int jj = 0; jj < nb; ++jj) {
            const T* vr = sv + (size_t)(j0 + jj) * DD;
            float vv[PL];
#pragma unroll
            for (int p = 0; p < PL; ++p) vv[p] = to_f32(vr[lane + kWave * p]);
#pragma unroll
            for (int hh = 0; hh < kMaxG; ++hh) {
                if (hh >= G) break;
                const float pv = __shfl(pj[hh], jj, kWave);
#pragma unroll
                for (int p = 0; p < PL; ++p) acc[hh][p] = fmaf(pv, vv[p], acc[hh][p]);
            }
        }
    }
    for (int hh = 0; hh < G; ++hh) {
        float* part = w.part + (((size_t)b * D.Hq + g * G + hh) * w.splits + split) * (DD + 2);
        if (lane == 0) { part[0] = m[hh]; part[1] = l[hh]; }
#pragma unroll
        for (int p = 0; p < PL; ++p) part[2 + lane + kWave * p] = acc[hh][p];
    }
}

template <typename T, int DD>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeWork w, T* __restrict__ out,
                                                            int64_t* __restrict__ pos_dev, Dims D) {
    constexpr int PL = DD / kWave;
    const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    // the last launch of the step: every read of this step's positions is done
    if (pos_dev && h == 0 && lane == 0) pos_dev[b] += 1;
    const size_t bh = (size_t)b * D.Hq + h;
    const float* la = w.la + bh * (DD + 1);
    const float* wp = w.win + bh * (DD + 2);
    const float* pp = w.part + bh * w.splits * (DD + 2);
    // Linear terms sit at reference 0, so with linear mass the common
    // reference is max(0, the partials' maxima); without it (no routed linear
    // token) it is the partials' maximum alone, which may be negative: logits
    // far below 0 would otherwise underflow every weight and leave 0 / 0.
    float M = la[DD] > 0.f ? 0.f : kNegInf;
    if (wp[1] > 0.f) M = fmaxf(M, wp[0]);
    for (int s = 0; s < w.splits; ++s)
        if (pp[s * (DD + 2) + 1] > 0.f) M = fmaxf(M, pp[s * (DD + 2)]);
    const float fl = la[DD] > 0.f ? expf(-M) : 0.f;
    float l = la[DD] * fl;
    float acc[PL];
#pragma unroll
    for (int p = 0; p < PL; ++p) acc[p] = la[lane + kWave * p] * fl;
    if (wp[1] > 0.f) {
        const float f = expf(wp[0] - M);
        l += wp[1] * f;
#pragma unroll
        for (int p = 0; p < PL; ++p) acc[p] = fmaf(wp[2 + lane + kWave * p], f, acc[p]);
    }
    for (int s = 0; s < w.splits; ++s) {
        const float* ps = pp + s * (DD + 2);
        if (ps[1] > 0.f) {
            const float f = expf(ps[0] - M);
            l += ps[1] * f;
#pragma unroll
            for (int p = 0; p < PL; ++p) acc[p] = fmaf(ps[2 + lane + kWave * p], f, acc[p]);
        }
    }
    const float inv = 1.0f / l;
#pragma unroll
    for (int p = 0; p < PL; ++p) out[bh * DD + lane + kWave * p] = from_f32<T>(acc[p] * inv);
}

template <typename T, int DD>
hipError_t prep_t(const Dims& D, const void* q, const void* k, const void* v, const float* wq,
                  const float* wk, const float* gate, const CacheView& c, const DecodeWork& w,
                  hipStream_t s) {
    dim3 grid(D.Hkv, D.B);
    const T* qq = reinterpret_cast<const T*>(q);
    const T* kk = reinterpret_cast<const T*>(k);
    const T* vv = reinterpret_cast<const T*>(v);
    const int R = (D.W + kWave - 1) / kWave;
#define STILL_PREP(RR) hipLaunchKernelGGL((decode_prep_kernel<T, DD, RR>), grid, dim3(256), 0, s, qq, kk, vv, wq, wk, gate, c, w, D)
    if (R <= 1) STILL_PREP(1);
    else if (R <= 2) STILL_PREP(2);
    else if (R <= 4) STILL_PREP(4);
    else if (R <= 8) STILL_PREP(8);
    else STILL_PREP(16);
#undef STILL_PREP
    return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_prep(const Dims& D, const void* q, const void* k, const void* v,
                              const float* wphi_q, const float* wphi_k, const float* gate,
                              const CacheView& c, const DecodeWork& w, hipStream_t s) {
    if (D.d == 128)
        return D.bf16 ? prep_t<__bf16, 128>(D, q, k, v, wphi_q, wphi_k, gate, c, w, s)
                      : prep_t<float, 128>(D, q, k, v, wphi_q, wphi_k, gate, c, w, s);
    return D.bf16 ? prep_t<__bf16, 64>(D, q, k, v, wphi_q, wphi_k, gate, c, w, s)
                  : prep_t<float, 64>(D, q, k, v, wphi_q, wphi_k, gate, c, w, s);
}

hipError_t launch_decode_sel(const Dims& D, const void* q, const CacheView& c, const DecodeWork& w,
                             hipStream_t s) {
    if (D.lam == 0 || w.splits == 0) return hipSuccess;
    dim3 grid(w.splits, D.Hkv, D.B);
#define STILL_SEL(T, DD) hipLaunchKernelGGL((decode_sel_kernel<T, DD>), grid, dim3(64), 0, s, reinterpret_cast<const T*>(q), c, w, D)
    if (D.d == 128) {
        if (D.bf16) STILL_SEL(__bf16, 128); else STILL_SEL(float, 128);
    } else {
        if (D.bf16) STILL_SEL(__bf16, 64); else STILL_SEL(float, 64);
    }
#undef STILL_SEL
    return hipGetLastError();
}

hipError_t launch_decode_combine(const Dims& D, const DecodeWork& w, void* out, int64_t* pos_dev,
                                 hipStream_t s) {
    dim3 grid(D.Hq, D.B);
#define STILL_COMB(T, DD) hipLaunchKernelGGL((decode_combine_kernel<T, DD>), grid, dim3(64), 0, s, w, reinterpret_cast<T*>(out), pos_dev, D)
    if (D.d == 128) {
        if (D.bf16) STILL_COMB(__bf16, 128); else STILL_COMB(float, 128);
    } else {
        if (D.bf16) STILL_COMB(__bf16, 64); else STILL_COMB(float, 64);
    }
#undef STILL_COMB
    return hipGetLastError();
}

}  // namespace still
