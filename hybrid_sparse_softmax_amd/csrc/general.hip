// General STILL forward kernels: every supported shape (d in {64,128},
// any W, C, topk, GQA ratio), f32 or bf16 storage, fp32 arithmetic.
//
// Pipeline (Sec. 3.3 "Chunk-Wise Parallel Form" of the STILL paper):
//   phi_kernel          NP-Map of every query and key (Sec. 3.2)
//   head_scores_kernel  window softmax row + Self-Saliency per query head (Sec. 3.1)
//   select_kernel       group mean, per-chunk top-k, route flags (Sec. 3.3)
//   la_chunk_kernel     per-chunk sum of phi_k(k) v^T and phi_k(k) over LA tokens
//   la_scan_kernel      inclusive prefix of those sums over chunks (Appendix A.2 state)
//   main_general_kernel one wave per (b, t, h): LA read-out, then window and
//                       selected softmax terms, one shared normaliser (Fig. 2)
//   handoff_kernel      fills the decode cache as the recurrent form leaves it
#include "device_common.h"
#include "launch.h"
#include "np_map.h"

namespace still {

namespace {
constexpr float kNegInf = -__builtin_inff();

template <typename T>
__global__ __launch_bounds__(64) void phi_kernel(const T* __restrict__ x, const float* __restrict__ P,
                                                 const float* __restrict__ gate,
                                                 float* __restrict__ phi, int H, int hpp, int d,
                                                 int fd) {
    const int tok = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
    __shared__ float xs[128];
    __shared__ float ph[128];
    const T* xr = x + ((size_t)tok * H + h) * d;
    for (int i = lane; i < d; i += kWave) xs[i] = to_f32(xr[i]);
    __syncthreads();
    // a query's features carry its gate weight (the linear branch's weight)
    np_map_wave(xs, P + (size_t)(h / hpp) * (fd / 2) * d, d, fd, ph, lane,
                gate_weight(gate, (size_t)tok * H + h));
    __syncthreads();
    float* pr = phi + ((size_t)tok * H + h) * fd;
    for (int i = lane; i < fd; i += kWave) pr[i] = ph[i];
}

// Self-Saliency of query (b, t, h) over its window J_t = [max(0,t-W+1), t].
// Lane r*64+lane holds key j0 + r*64 + lane.  R = ceil(W / 64).
template <typename T, int R>
__global__ __launch_bounds__(64) void head_scores_kernel(const T* __restrict__ q,
                                                         const T* __restrict__ k,
                                                         float* __restrict__ hs, Dims D) {
    const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int g = h / D.G, d = D.d;
    __shared__ float qs[128];
    const T* qr = q + (((size_t)b * D.N + t) * D.Hq + h) * d;
    for (int i = lane; i < d; i += kWave) qs[i] = to_f32(qr[i]);
    __syncthreads();
    const int j0 = max(0, t - D.W + 1);
    const int n = t - j0 + 1;
    float s[R];
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int idx = r * kWave + lane;
        s[r] = kNegInf;
        if (idx < n) {
            const T* kr = k + (((size_t)b * D.N + j0 + idx) * D.Hkv + g) * d;
            float dot = 0.f;
            for (int i = 0; i < d; ++i) dot = fmaf(qs[i], to_f32(kr[i]), dot);
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
        e[r] = idx < n ? expf(s[r] - mx) : 0.f;
        sa += e[r];
        if (idx == n - 1) et = e[r]; else so += e[r];
    }
    sa = wave_sum(sa);
    so = wave_sum(so);
    et = wave_sum(et);
    float term = 0.f;
    if (D.route == kRouteSaliency) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int idx = r * kWave + lane;
            if (idx < n) term += saliency_term(e[r], idx == n - 1, et, sa, so, D.eps);
        }
        term = wave_sum(term);
    } else if (D.route == kRouteDiagonal) {
        term = et / sa;  // the own weight a_tt
    } else {
        // the own logit tau q_t.k_t (query-free criteria ignore this value)
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (r * kWave + lane == n - 1) term = s[r];
        term = wave_sum(term);
    }
    if (lane == 0) hs[((size_t)b * D.Hq + h) * D.N + t] = term;
}

// Top-lam of one complete chunk's n keys (sort keys in LDS) by one wave:
// route flags and the selected positions, ascending.
template <int R>
__device__ __forceinline__ void chunk_topk(const float* key, int n, int lam, int c0, int32_t* out,
                                           uint8_t* rt) {
    const int lane = threadIdx.x & 63;
    uint32_t kb[R];
#pragma unroll
    for (int r = 0; r < R; ++r) kb[r] = 64 * r + lane < n ? key_bits(key[64 * r + lane]) : 0u;
    bool f[R];
    int at[R];
    wave_topk<R>(kb, n, lam, f, at);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = 64 * r + lane;
        if (i < n) {
            rt[i] = f[r] ? kRouteSA : kRouteLA;
            if (f[r]) out[at[r]] = c0 + i;
        }
    }
}

// One block per (b, g, chunk): group mean of the head scores, then for a
// complete chunk the top-lam tokens by (score desc, position asc).
template <typename T>
__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ hs,
                                                     float* __restrict__ scores,
                                                     int32_t* __restrict__ sel_idx,
                                                     uint8_t* __restrict__ route,
                                                     const T* __restrict__ k, Dims D) {
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    extern __shared__ float sh[];
    float* key = sh;
    int* flag = reinterpret_cast<int*>(sh + D.C);
    const int c0 = c * D.C, n = min(D.C, D.N - c0);
    const size_t row = ((size_t)b * D.Hkv + g) * D.N + c0;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        float acc = 0.f;
        if (D.W > 0 && route_query_free(D.route)) {
            float kn = 0.f;
            if (D.route == kRouteKeyNorm) {
                const T* kr = k + (((size_t)b * D.N + c0 + i) * D.Hkv + g) * D.d;
                for (int e = 0; e < D.d; ++e) kn = fmaf(to_f32(kr[e]), to_f32(kr[e]), kn);
                kn = sqrtf(kn);
            }
            acc = query_free_score(D.route, kn, c0 + i, b, g, D.Hkv, D.C, D.lam);
        } else if (D.W > 0) {
            for (int hh = 0; hh < D.G; ++hh)
                acc += hs[((size_t)b * D.Hq + g * D.G + hh) * D.N + c0 + i];
            acc = acc / (float)D.G;
        }
        scores[row + i] = acc;
        key[i] = route_key(acc);
    }
    __syncthreads();
    uint8_t* rt = route + row;
    if (D.lam == 0 || n < D.C) {
        const uint8_t f = D.lam == 0 ? kRouteLA : kPending;
        for (int i = threadIdx.x; i < n; i += blockDim.x) rt[i] = f;
        return;
    }
    // radix top-lam of the chunk's keys by the first wave (R keys per lane)
    if (threadIdx.x < kWave) {
        int32_t* out = sel_idx + (((size_t)b * D.Hkv + g) * D.n_full + c) * D.lam;
        if (n <= kWave) chunk_topk<1>(key, n, D.lam, c0, out, rt);
        else if (n <= 4 * kWave) chunk_topk<4>(key, n, D.lam, c0, out, rt);
        else chunk_topk<16>(key, n, D.lam, c0, out, rt);
    }
}

// Per-chunk sums over the chunk's LA tokens: S[i][dim] = sum phi_k[i] v[dim],
// z[i] = sum phi_k[i].  Thread tid owns entries tid + 256 r.
template <typename T, int DD>
__global__ __launch_bounds__(256) void la_chunk_kernel(const float* __restrict__ phik,
                                                       const T* __restrict__ v,
                                                       const uint8_t* __restrict__ route,
                                                       float* __restrict__ lin, Dims D) {
    constexpr int E = DD * DD, PER = E / 256;
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    __shared__ float ph[32][DD];
    __shared__ float vv[32][DD];
    float acc[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r) acc[r] = 0.f;
    float zacc = 0.f;
    const int c0 = c * D.C, n = min(D.C, D.N - c0);
    for (int j0 = 0; j0 < n; j0 += 32) {
        const int nb = min(32, n - j0);
        __syncthreads();
        for (int x = tid; x < nb * DD; x += 256) {
            const int jj = x / DD, i = x % DD, pos = c0 + j0 + jj;
            const bool la = route[((size_t)b * D.Hkv + g) * D.N + pos] == kRouteLA;
            ph[jj][i] = la ? phik[(((size_t)b * D.N + pos) * D.Hkv + g) * DD + i] : 0.f;
            vv[jj][i] = to_f32(v[(((size_t)b * D.N + pos) * D.Hkv + g) * DD + i]);
        }
        __syncthreads();
        for (int jj = 0; jj < nb; ++jj) {
#pragma unroll
            for (int r = 0; r < PER; ++r) {
                const int e = tid + 256 * r;
                acc[r] = fmaf(ph[jj][e / DD], vv[jj][e % DD], acc[r]);
            }
            if (tid < DD) zacc += ph[jj][tid];
        }
    }
    float* out = lin + (((size_t)b * D.Hkv + g) * D.T + c) * (size_t)(DD * (DD + 1));
#pragma unroll
    for (int r = 0; r < PER; ++r) out[tid + 256 * r] = acc[r];
    if (tid < DD) out[E + tid] = zacc;
}

__global__ __launch_bounds__(256) void la_scan_kernel(float* __restrict__ lin, int cap_chunk,
                                                      float* __restrict__ cap_S,
                                                      float* __restrict__ cap_z, Dims D) {
    const int E = D.fd * D.d, E1 = E + D.fd;
    const int e = blockIdx.x * 256 + threadIdx.x, g = blockIdx.y, b = blockIdx.z;
    if (e >= E1) return;
    float* base = lin + ((size_t)b * D.Hkv + g) * D.T * (size_t)E1 + e;
    float run = 0.f;
    for (int c = 0; c < D.T; ++c) {
        run += base[(size_t)c * E1];
        base[(size_t)c * E1] = run;
        if (c == cap_chunk && cap_S) {
            if (e < E) cap_S[((size_t)b * D.Hkv + g) * E + e] = run;
            else cap_z[((size_t)b * D.Hkv + g) * D.fd + (e - E)] = run;
        }
    }
}

// One wave per query (b, t, h).  Lane owns output dims lane + 64 p.
template <typename T, int DD>
__global__ __launch_bounds__(64) void main_general_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ phiq, const float* __restrict__ phik,
    const uint8_t* __restrict__ route, const int32_t* __restrict__ sel_idx,
    const float* __restrict__ lin, T* __restrict__ out, float* __restrict__ stat, Dims D) {
    constexpr int PL = DD / kWave;
    const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int g = h / D.G;
    __shared__ float qs[DD];
    __shared__ float fq[DD];
    const size_t qoff = (((size_t)b * D.N + t) * D.Hq + h);
    for (int i = lane; i < DD; i += kWave) {
        qs[i] = to_f32(q[qoff * DD + i]);
        fq[i] = phiq[qoff * DD + i];
    }
    __syncthreads();
    auto krow = [&](int j) { return k + (((size_t)b * D.N + j) * D.Hkv + g) * DD; };
    auto vrow = [&](int j) { return v + (((size_t)b * D.N + j) * D.Hkv + g) * DD; };

    float acc[PL];
#pragma unroll
    for (int p = 0; p < PL; ++p) acc[p] = 0.f;
    float l = 0.f, m = 0.f;  // the linear terms' reference point is 0
    const int r_end = max(0, t - D.W + 1);  // routed tokens: j < r_end
    const int c_full = r_end / D.C;

    // linear attention: full chunks through the prefix state
    if (c_full >= 1) {
        const float* st = lin + (((size_t)b * D.Hkv + g) * D.T + (c_full - 1)) * (size_t)(DD * (DD + 1));
        for (int i = 0; i < DD; ++i) {
            const float f = fq[i];
#pragma unroll
            for (int p = 0; p < PL; ++p) acc[p] = fmaf(f, st[i * DD + lane + kWave * p], acc[p]);
        }
        float lp = 0.f;
        for (int i = lane; i < DD; i += kWave) lp = fmaf(fq[i], st[DD * DD + i], lp);
        l = wave_sum(lp);
    }
    // linear attention: LA tokens of the partly routed chunk
    const uint8_t* rt = route + ((size_t)b * D.Hkv + g) * D.N;
    for (int j0 = c_full * D.C; j0 < r_end; j0 += kWave) {
        const int j = j0 + lane;
        float w = 0.f;
        if (j < r_end && rt[j] == kRouteLA) {
            const float* pk = phik + (((size_t)b * D.N + j) * D.Hkv + g) * DD;
            for (int i = 0; i < DD; ++i) w = fmaf(fq[i], pk[i], w);
        }
        l += wave_sum(w);
        const int nb = min(kWave, r_end - j0);
        for (int jj = 0; jj < nb; ++jj) {
            const float wj = __shfl(w, jj, kWave);
            if (wj != 0.f) {
                const T* vr = vrow(j0 + jj);
#pragma unroll
                for (int p = 0; p < PL; ++p) acc[p] = fmaf(wj, to_f32(vr[lane + kWave * p]), acc[p]);
            }
        }
    }
    // Softmax terms, 64 keys at a time; jpos < 0 marks an empty lane.  With
    // linear mass the reference is max(0, max s), which keeps both kinds of
    // weight <= 1.  Without it (no routed linear token: t < W, every routed
    // token selected) the reference is the plain running maximum, which may
    // be negative: all logits far below 0 would otherwise underflow every
    // weight and leave 0 / 0.
    const bool lamass = l > 0.f;
    if (!lamass) m = kNegInf;
    auto sa_batch = [&](int jpos) {
        float s = kNegInf;
        if (jpos >= 0) {
            const T* kr = krow(jpos);
            float dot = 0.f;
            for (int i = 0; i < DD; ++i) dot = fmaf(qs[i], to_f32(kr[i]), dot);
            s = D.tau * dot;
        }
        const float m_new = fmaxf(m, wave_max(s));
        if (m_new == kNegInf) return;  // nothing visible yet
        const float sc = expf(m - m_new);
        const float pj = jpos >= 0 ? expf(s - m_new) : 0.f;
        l = l * sc + wave_sum(pj);
#pragma unroll
        for (int p = 0; p < PL; ++p) acc[p] *= sc;
        for (int jj = 0; jj < kWave; ++jj) {
            const int jp = __shfl(jpos, jj, kWave);
            if (jp >= 0) {
                const float pv = __shfl(pj, jj, kWave);
                const T* vr = vrow(jp);
#pragma unroll
                for (int p = 0; p < PL; ++p) acc[p] = fmaf(pv, to_f32(vr[lane + kWave * p]), acc[p]);
            }
        }
        m = m_new;
    };
    if (D.W > 0) {
        for (int j0 = max(0, t - D.W + 1); j0 <= t; j0 += kWave) {
            const int j = j0 + lane;
            sa_batch(j <= t ? j : -1);
        }
    }
    if (D.lam > 0 && r_end > 0) {
        const int32_t* sel = sel_idx + ((size_t)b * D.Hkv + g) * D.n_full * D.lam;
        const int n_cand = min(D.n_full, (r_end + D.C - 1) / D.C) * D.lam;
        for (int i0 = 0; i0 < n_cand; i0 += kWave) {
            const int i = i0 + lane;
            int jp = -1;
            if (i < n_cand) {
                const int pos = sel[i];
                if (pos < r_end) jp = pos;
            }
            sa_batch(jp);
        }
    }
    const float inv = 1.0f / l;
#pragma unroll
    for (int p = 0; p < PL; ++p) out[qoff * DD + lane + kWave * p] = from_f32<T>(acc[p] * inv);
    // optional statistics for a backward: (m, l, 0, exp(-m) / l with linear terms, else 0)
    if (stat && lane == 0) {
        stat[qoff * 4] = m;
        stat[qoff * 4 + 1] = l;
        stat[qoff * 4 + 2] = 0.f;
        stat[qoff * 4 + 3] = lamass ? expf(-m) * inv : 0.f;
    }
}

// Prefill -> decode hand-off for one (b, g): ring, route flags, pending
// scores, selected list, linear state (prefix chunk already in lin_S/lin_z,
// written by la_scan_kernel when cap_chunk >= 0).
template <typename T, int DD>
__global__ __launch_bounds__(256) void handoff_kernel(const T* __restrict__ k,
                                                      const T* __restrict__ v,
                                                      const float* __restrict__ wk,
                                                      const float* __restrict__ scores,
                                                      const int32_t* __restrict__ sel_idx,
                                                      const uint8_t* __restrict__ route,
                                                      int cap_chunk, CacheView c, Dims D) {
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const size_t bg = (size_t)b * D.Hkv + g;
    const int N = D.N, W = D.W, C = D.C;
    const uint8_t* rt = route + bg * N;
    // window ring and its route flags
    if (W > 0) {
        const int j0 = max(0, N - W), nr = N - j0;
        T* rk = reinterpret_cast<T*>(c.win_k) + bg * W * DD;
        T* rv = reinterpret_cast<T*>(c.win_v) + bg * W * DD;
        for (int x = tid; x < nr * DD; x += 256) {
            const int j = j0 + x / DD, i = x % DD;
            const size_t src = (((size_t)b * N + j) * D.Hkv + g) * DD + i;
            rk[(size_t)(j % W) * DD + i] = k[src];
            rv[(size_t)(j % W) * DD + i] = v[src];
        }
        for (int j = j0 + tid; j < N; j += 256)
            c.win_route[bg * W + j % W] = (j >= D.n_full * C) ? kPending : rt[j];
        for (int j = D.n_full * C + tid; j < N; j += 256)
            c.pend[bg * C + j % C] = scores[bg * N + j];
    }
    const int r_end = max(0, N - W);
    // selected tokens that already left the window, ascending
    __shared__ int s_count;
    if (D.lam > 0) {
        const int32_t* sel = sel_idx + bg * D.n_full * D.lam;
        const int n_cand = min(D.n_full, (r_end + C - 1) / C) * D.lam;
        if (tid == 0) {
            int cnt = 0;
            while (cnt < n_cand && sel[cnt] < r_end) ++cnt;
            s_count = cnt;
        }
        __syncthreads();
        const int cnt = min(s_count, c.cap);
        T* sk = reinterpret_cast<T*>(c.sel_k) + bg * c.cap * DD;
        T* sv = reinterpret_cast<T*>(c.sel_v) + bg * c.cap * DD;
        for (int x = tid; x < cnt * DD; x += 256) {
            const int r = x / DD, i = x % DD;
            const size_t src = (((size_t)b * N + sel[r]) * D.Hkv + g) * DD + i;
            sk[(size_t)r * DD + i] = k[src];
            sv[(size_t)r * DD + i] = v[src];
        }
        if (tid == 0) c.sel_count[bg] = cnt;
    } else if (c.sel_count && tid == 0) {
        c.sel_count[bg] = 0;
    }
    // linear state: chunks [0, c_full) come from the scan; add the rest
    const int c_full = r_end / C;
    float* S = c.lin_S + bg * D.fd * DD;
    float* z = c.lin_z + bg * D.fd;
    if (c_full - 1 != cap_chunk || cap_chunk < 0) {
        for (int e = tid; e < D.fd * DD; e += 256) S[e] = 0.f;
        for (int e = tid; e < D.fd; e += 256) z[e] = 0.f;
    }
    __shared__ float xs[DD], vs[DD], ph[DD];
    for (int j = c_full * C; j < r_end; ++j) {
        if (rt[j] != kRouteLA) continue;
        __syncthreads();
        const size_t src = (((size_t)b * N + j) * D.Hkv + g) * DD;
        for (int i = tid; i < DD; i += 256) {
            xs[i] = to_f32(k[src + i]);
            vs[i] = to_f32(v[src + i]);
        }
        __syncthreads();
        if (tid < kWave) np_map_wave(xs, wk + (size_t)g * (D.fd / 2) * DD, DD, D.fd, ph, tid);
        __syncthreads();
        for (int e = tid; e < D.fd * DD; e += 256) S[e] += ph[e / DD] * vs[e % DD];
        for (int e = tid; e < D.fd; e += 256) z[e] += ph[e];
    }
}

template <typename T>
hipError_t phi_t(const Dims& D, const void* x, int H, int hpp, const float* P, const float* gate,
                 float* phi, hipStream_t s) {
    dim3 grid(D.B * D.N, H);
    hipLaunchKernelGGL(phi_kernel<T>, grid, dim3(64), 0, s, reinterpret_cast<const T*>(x), P, gate,
                       phi, H, hpp, D.d, D.fd);
    return hipGetLastError();
}

template <typename T>
hipError_t scores_t(const Dims& D, const void* q, const void* k, float* hs, hipStream_t s) {
    dim3 grid(D.N, D.Hq, D.B);
    const T* qq = reinterpret_cast<const T*>(q);
    const T* kk = reinterpret_cast<const T*>(k);
    const int R = (D.W + kWave - 1) / kWave;
    if (R <= 1) hipLaunchKernelGGL((head_scores_kernel<T, 1>), grid, dim3(64), 0, s, qq, kk, hs, D);
    else if (R <= 2) hipLaunchKernelGGL((head_scores_kernel<T, 2>), grid, dim3(64), 0, s, qq, kk, hs, D);
    else if (R <= 4) hipLaunchKernelGGL((head_scores_kernel<T, 4>), grid, dim3(64), 0, s, qq, kk, hs, D);
    else if (R <= 8) hipLaunchKernelGGL((head_scores_kernel<T, 8>), grid, dim3(64), 0, s, qq, kk, hs, D);
    else hipLaunchKernelGGL((head_scores_kernel<T, 16>), grid, dim3(64), 0, s, qq, kk, hs, D);
    return hipGetLastError();
}

template <typename T, int DD>
hipError_t main_t(const Dims& D, const void* q, const void* k, const void* v, const float* phiq,
                  const float* phik, const uint8_t* route, const int32_t* sel_idx, const float* lin,
                  void* out, float* stat, hipStream_t s) {
    dim3 grid(D.N, D.Hq, D.B);
    hipLaunchKernelGGL((main_general_kernel<T, DD>), grid, dim3(64), 0, s,
                       reinterpret_cast<const T*>(q), reinterpret_cast<const T*>(k),
                       reinterpret_cast<const T*>(v), phiq, phik, route, sel_idx, lin,
                       reinterpret_cast<T*>(out), stat, D);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_phi(const Dims& D, const void* x, int H, int hpp, const float* P,
                      const float* gate, float* phi, hipStream_t s) {
    return D.bf16 ? phi_t<__bf16>(D, x, H, hpp, P, gate, phi, s)
                  : phi_t<float>(D, x, H, hpp, P, gate, phi, s);
}

hipError_t launch_head_scores(const Dims& D, const void* q, const void* k, float* hs, hipStream_t s) {
    return D.bf16 ? scores_t<__bf16>(D, q, k, hs, s) : scores_t<float>(D, q, k, hs, s);
}

hipError_t launch_select(const Dims& D, const float* hs, float* scores, int32_t* sel_idx,
                         uint8_t* route, const void* k, hipStream_t s) {
    dim3 grid(D.T, D.Hkv, D.B);
    const size_t shm = (size_t)D.C * (sizeof(float) + sizeof(int));
    if (D.bf16)
        hipLaunchKernelGGL(select_kernel<__bf16>, grid, dim3(256), shm, s, hs, scores, sel_idx, route,
                           reinterpret_cast<const __bf16*>(k), D);
    else
        hipLaunchKernelGGL(select_kernel<float>, grid, dim3(256), shm, s, hs, scores, sel_idx, route,
                           reinterpret_cast<const float*>(k), D);
    return hipGetLastError();
}

hipError_t launch_la_chunks(const Dims& D, const float* phik, const void* v, const uint8_t* route,
                            float* lin, hipStream_t s) {
    dim3 grid(D.T, D.Hkv, D.B);
    if (D.d == 128) {
        if (D.bf16) hipLaunchKernelGGL((la_chunk_kernel<__bf16, 128>), grid, dim3(256), 0, s, phik, reinterpret_cast<const __bf16*>(v), route, lin, D);
        else hipLaunchKernelGGL((la_chunk_kernel<float, 128>), grid, dim3(256), 0, s, phik, reinterpret_cast<const float*>(v), route, lin, D);
    } else {
        if (D.bf16) hipLaunchKernelGGL((la_chunk_kernel<__bf16, 64>), grid, dim3(256), 0, s, phik, reinterpret_cast<const __bf16*>(v), route, lin, D);
        else hipLaunchKernelGGL((la_chunk_kernel<float, 64>), grid, dim3(256), 0, s, phik, reinterpret_cast<const float*>(v), route, lin, D);
    }
    return hipGetLastError();
}

hipError_t launch_la_scan(const Dims& D, float* lin, int cap_chunk, float* cap_S, float* cap_z,
                          hipStream_t s) {
    const int E1 = D.fd * (D.d + 1);
    dim3 grid((E1 + 255) / 256, D.Hkv, D.B);
    hipLaunchKernelGGL(la_scan_kernel, grid, dim3(256), 0, s, lin, cap_chunk, cap_S, cap_z, D);
    return hipGetLastError();
}

hipError_t launch_main_general(const Dims& D, const void* q, const void* k, const void* v,
                               const float* phiq, const float* phik, const uint8_t* route,
                               const int32_t* sel_idx, const float* lin, void* out, float* stats,
                               hipStream_t s) {
    if (D.d == 128)
        return D.bf16 ? main_t<__bf16, 128>(D, q, k, v, phiq, phik, route, sel_idx, lin, out, stats, s)
                      : main_t<float, 128>(D, q, k, v, phiq, phik, route, sel_idx, lin, out, stats, s);
    return D.bf16 ? main_t<__bf16, 64>(D, q, k, v, phiq, phik, route, sel_idx, lin, out, stats, s)
                  : main_t<float, 64>(D, q, k, v, phiq, phik, route, sel_idx, lin, out, stats, s);
}

hipError_t launch_handoff(const Dims& D, const void* k, const void* v, const float* wphi_k,
                          const float* scores, const int32_t* sel_idx, const uint8_t* route,
                          int cap_chunk, const CacheView& c, hipStream_t s) {
    dim3 grid(D.Hkv, D.B);
#define STILL_HANDOFF(T, DD)                                                                  \
    hipLaunchKernelGGL((handoff_kernel<T, DD>), grid, dim3(256), 0, s,                        \
                       reinterpret_cast<const T*>(k), reinterpret_cast<const T*>(v), wphi_k, \
                       scores, sel_idx, route, cap_chunk, c, D)
    if (D.d == 128) {
        if (D.bf16) STILL_HANDOFF(__bf16, 128); else STILL_HANDOFF(float, 128);
    } else {
        if (D.bf16) STILL_HANDOFF(__bf16, 64); else STILL_HANDOFF(float, 64);
    }
#undef STILL_HANDOFF
    return hipGetLastError();
}

}  // namespace still
