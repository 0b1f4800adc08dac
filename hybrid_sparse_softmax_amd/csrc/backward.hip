// Backward pass of the STILL hybrid attention operator: gradients of
// L = sum(dout * out) w.r.t. q, k, v and the two NP-Map projections, with the
// routing held fixed (the selection is a constant mask; no gradient flows
// through the scores or the top-k).  The training this serves is the paper's
// two-stage linearization (Sec. 4.1 "Experimental Setups", training
// strategy; App. A.6.1), which backpropagates through the chunk-wise
// parallel form of Sec. 3.3.  Every supported shape, f32 or bf16 storage,
// fp32 arithmetic, fp32 gradients.
//
// Per query t of head h, with the sets of the forward (window + visible
// selected tokens SA_t, routed unselected tokens LA_t), weights
// w_j = exp(s_j - m) on SA_t and exp(-m) kappa_j on LA_t
// (kappa_j = phi_q(q_t) . phi_k(k_j)), l = sum w_j, o = sum w_j v_j / l and
// D_t = dout_t . o:
//   SA:  ds_j = (w_j / l)(dout_t . v_j - D_t)
//        dq_t += tau ds_j k_j,  dk_j += tau ds_j q_t,  dv_j += (w_j / l) dout_t
//   LA:  dkappa_j = c_t (dout_t . v_j - D_t)  with c_t = exp(-m) / l
//        dphi_q(t) = c_t (S_t dout_t - D_t z_t)    S_t, z_t: the LA state t reads
//        dphi_k(j) = U_j v_j - u_j,  dv_j = U_j^T phi_k(j)
//        with U_j = sum over t >= j + W (all heads of the group) of
//        c_t phi_q(t) dout_t^T and u_j = sum c_t D_t phi_q(t): a suffix sum
//        over query chunks plus the queries of one partial chunk.
// Then the NP-Map's vector-Jacobian product carries dphi to x and to P.
//
// Kernels, in launch order:
//   bwd_route_kernel   route flags and a clean ascending selected list per
//                      chunk from the caller's selection
//   (phi, la_chunk, la_scan of the forward: phi_q, phi_k and the LA prefix)
//   bwd_query_kernel   one wave per (b, two positions, g) for the group's heads:
//                      statistics m, l, D_t recomputed, dq's softmax part, dphi_q
//   bwd_uchunk_kernel  per query chunk: sum of c_t phi_q dout^T and c_t D_t phi_q
//   bwd_suffix_kernel  inclusive suffix of those sums over chunks
//   bwd_key_win_kernel one wave per four consecutive keys: their window
//                      queries' softmax terms (dk, dv) and the linear terms
//                      (dv, dphi_k)
//   bwd_key_sel_kernel one block per 16 selected keys: the softmax terms of
//                      the queries after their windows, added to dk, dv
//   np_vjp_kernel      NP-Map backward per (token, KV group): dx += ..., du
//   dw_partial_kernel  dP = sum du x^T over a slice of tokens
//   dw_reduce_kernel   sum of the slices
// On the matrix-core path (bf16, d = 128, W and C multiples of 64 up to 256,
// C <= W) every gradient term, the statistics, the NP-Map backward and the
// projection gradients run as MFMA kernels (prefill_mfma.hip,
// backward_mfma.hip) over 64-token tiles; bwd_route and bwd_suffix are
// shared with the general path.
#include "device_common.h"
#include "launch.h"
#include "row_ops.h"

namespace still {

namespace {

constexpr float kNegInfB = -__builtin_inff();

__global__ __launch_bounds__(256) void bwd_route_kernel(const int32_t* __restrict__ sel_in,
                                                        uint8_t* __restrict__ route,
                                                        int32_t* __restrict__ selw, Dims D) {
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    extern __shared__ int flag[];
    const int c0 = c * D.C, n = min(D.C, D.N - c0);
    uint8_t* rt = route + ((size_t)b * D.Hkv + g) * D.N + c0;
    if (D.lam == 0 || n < D.C) {
        const uint8_t f = D.lam == 0 ? kRouteLA : kPending;
        for (int i = threadIdx.x; i < n; i += blockDim.x) rt[i] = f;
        return;
    }
    for (int i = threadIdx.x; i < n; i += blockDim.x) flag[i] = 0;
    __syncthreads();
    const size_t row = (((size_t)b * D.Hkv + g) * D.n_full + c) * D.lam;
    for (int i = threadIdx.x; i < D.lam; i += blockDim.x) {
        const int pos = sel_in[row + i];
        if (pos >= c0 && pos < c0 + D.C) flag[pos - c0] = 1;  // other entries are ignored
    }
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) rt[i] = flag[i] ? kRouteSA : kRouteLA;
    if (threadIdx.x == 0) {
        int cnt = 0;
        for (int i = 0; i < n && cnt < D.lam; ++i)
            if (flag[i]) selw[row + cnt++] = c0 + i;
        for (; cnt < D.lam; ++cnt) selw[row + cnt] = -1;
    }
}

// One wave per KV head and two consecutive query positions (b, t0, t0 + 1,
// g), for all G query heads of the group: every key row a lane loads serves
// 2 G queries.  The query and dout rows, the same in every lane, are read
// through the scalar cache.  Lane owns output dims and features lane + 64 p.
// Two passes over the union of the two positions' softmax keys (each
// position masks the keys it does not see, so every pair counts once):
//   1. logits s_j and vd_j = dout . v_j: the reference m (max(0, max s)),
//      l = sum of weights and D_t = sum w_j vd_j / l (= dout . out), the
//      linear tokens entering through S_t, z_t and the partly covered chunk;
//   2. ds_j = (w_j / l)(vd_j - D_t), dq = tau sum ds_j k_j.
// Then dphi_q = c_t (S_t dout - D_t z_t + sum over the partly covered chunk's
// linear tokens of (vd_j - D_t) phi_k(j)), c_t = exp(-m) / l.  phi_q here is
// the gated feature gamma phi_q (gamma = 1 without a gate); the kernel writes
// gamma dphi_q for the NP-Map's VJP and dgate = (1 - gamma) phi_q . dphi_q.
// stat[(b, t, h)] = (m, l, D_t, c_t).
constexpr int kNP = 2;  // query positions per wave
template <typename T, int DD, int GM>
__global__ __launch_bounds__(64) void bwd_query_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ phiq, const float* __restrict__ phik,
    const uint8_t* __restrict__ route, const int32_t* __restrict__ selw,
    const float* __restrict__ lin, const float* __restrict__ gate, float* __restrict__ dq,
    float* __restrict__ dphiq, float* __restrict__ dgate, float* __restrict__ stat, Dims D) {
    constexpr int PL = DD / kWave;
    constexpr int R = kNP * GM;  // rows: position pp, head h -> pp GM + h
    const Item it = xcd_item((D.N + kNP - 1) / kNP, D.Hkv);
    const int t0 = it.x * kNP, g = it.y, b = it.z, lane = threadIdx.x;
    const int G = D.G;
    int tp[kNP], r_end[kNP];
    bool act[kNP];
#pragma unroll
    for (int pp = 0; pp < kNP; ++pp) {
        act[pp] = t0 + pp < D.N;  // a position past the end repeats the last one, writes nothing
        tp[pp] = min(t0 + pp, D.N - 1);
        r_end[pp] = max(0, tp[pp] - D.W + 1);  // routed tokens j < r_end
    }
    auto qoff = [&](int pp, int h) { return ((size_t)b * D.N + tp[pp]) * D.Hq + (size_t)g * G + h; };
    const T* qr[R];
    const T* dr[R];
    bool use[R];
#pragma unroll
    for (int pp = 0; pp < kNP; ++pp)
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            const int r = pp * GM + h;
            use[r] = h < G;
            const size_t o = qoff(pp, min(h, G - 1));
            qr[r] = q + o * DD;
            dr[r] = dout + o * DD;
        }
    __shared__ float fq[kNP][GM][DD];
    __shared__ float ds_[kNP][GM][DD];
    for (int x = lane; x < kNP * G * DD; x += kWave) {
        const int pp = x / (G * DD), h = (x / DD) % G, i = x % DD;
        const size_t o = qoff(pp, h);
        fq[pp][h][i] = phiq[o * DD + i];
        ds_[pp][h][i] = to_f32(dout[o * DD + i]);
    }
    __syncthreads();
    auto krow = [&](int j) { return k + (((size_t)b * D.N + j) * D.Hkv + g) * DD; };
    auto vrow = [&](int j) { return v + (((size_t)b * D.N + j) * D.Hkv + g) * DD; };
    auto pkrow = [&](int j) { return phik + (((size_t)b * D.N + j) * D.Hkv + g) * DD; };
    const uint8_t* rt = route + ((size_t)b * D.Hkv + g) * D.N;
    auto state_of = [&](int pp) {
        const int c_full = r_end[pp] / D.C;
        return c_full >= 1
            ? lin + (((size_t)b * D.Hkv + g) * D.T + (c_full - 1)) * (size_t)(DD * (DD + 1))
            : (const float*)nullptr;
    };

    // ---- linear part of pass 1 (reference 0), per position ----
    float y[R][PL];
    float l[R], dn[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        l[r] = dn[r] = 0.f;
#pragma unroll
        for (int p = 0; p < PL; ++p) y[r][p] = 0.f;
    }
#pragma unroll
    for (int pp = 0; pp < kNP; ++pp) {
        const float* st = state_of(pp);
        if (st) {
            float lp[GM], dp[GM];
#pragma unroll
            for (int h = 0; h < GM; ++h) lp[h] = dp[h] = 0.f;
#pragma unroll
            for (int p = 0; p < PL; ++p) {
                const int i = lane + kWave * p;
                const float4* row = reinterpret_cast<const float4*>(st + (size_t)i * DD);
                for (int e4 = 0; e4 < DD / 4; ++e4) {
                    const float4 rv = row[e4];
#pragma unroll
                    for (int h = 0; h < GM; ++h)
                        if (h < G) {
                            float x = y[pp * GM + h][p];
                            x = fmaf(rv.x, ds_[pp][h][4 * e4], x);
                            x = fmaf(rv.y, ds_[pp][h][4 * e4 + 1], x);
                            x = fmaf(rv.z, ds_[pp][h][4 * e4 + 2], x);
                            x = fmaf(rv.w, ds_[pp][h][4 * e4 + 3], x);
                            y[pp * GM + h][p] = x;
                        }
                }
                const float zi = st[DD * DD + i];
#pragma unroll
                for (int h = 0; h < GM; ++h) {
                    lp[h] = fmaf(fq[pp][h][i], zi, lp[h]);
                    dp[h] = fmaf(fq[pp][h][i], y[pp * GM + h][p], dp[h]);
                }
            }
#pragma unroll
            for (int h = 0; h < GM; ++h)
                if (h < G) {
                    l[pp * GM + h] = wave_sum(lp[h]);
                    dn[pp * GM + h] = wave_sum(dp[h]);
                }
        }
        const int cf0 = (r_end[pp] / D.C) * D.C;
        for (int j0 = cf0; j0 < r_end[pp]; j0 += kWave) {
            const int j = j0 + lane;
            float kap[GM], vd[GM];
#pragma unroll
            for (int h = 0; h < GM; ++h) kap[h] = vd[h] = 0.f;
            if (j < r_end[pp] && rt[j] == kRouteLA) {
                dot_multi<DD, GM>(fq[pp], pkrow(j), G, kap);
                dot_multi<DD, GM>(ds_[pp], vrow(j), G, vd);
            }
#pragma unroll
            for (int h = 0; h < GM; ++h)
                if (h < G) {
                    l[pp * GM + h] += wave_sum(kap[h]);
                    dn[pp * GM + h] += wave_sum(kap[h] * vd[h]);
                }
        }
    }

    // ---- the union of the positions' softmax keys ----
    const int t_hi = tp[kNP - 1];
    const int jw0 = max(0, tp[0] - D.W + 1);
    const int32_t* sel = selw + ((size_t)b * D.Hkv + g) * D.n_full * D.lam;
    const int n_cand = D.lam > 0 ? min(D.n_full, (r_end[kNP - 1] + D.C - 1) / D.C) * D.lam : 0;
    auto sees = [&](int pp, int jpos, bool win) {
        if (jpos < 0) return false;
        return win ? (jpos >= tp[pp] - D.W + 1 && jpos <= tp[pp]) : jpos < r_end[pp];
    };
    // Reference point of the weights: max(0, max s) when the query has linear
    // mass (both kinds of weight stay <= 1); the plain running maximum, which
    // may be negative, when it has none (t < W, every routed token selected),
    // so logits far below 0 cannot underflow every weight.  The key kernels
    // read the same reference from stat.
    float m[R], inv[R], Dt[R];
    bool la_mass[R];
    {
#pragma unroll
    for (int r = 0; r < R; ++r) {
        la_mass[r] = l[r] > 0.f;
        m[r] = la_mass[r] ? 0.f : kNegInfB;
    }
    auto pass1 = [&](int jpos, bool win) {
        bool ok[kNP];
        bool any = false;
#pragma unroll
        for (int pp = 0; pp < kNP; ++pp) {
            ok[pp] = sees(pp, jpos, win);
            any = any || ok[pp];
        }
        float s[R], vd[R];
        if (any) {
            dot_rows_u<DD, R>(qr, use, krow(jpos), s);
            dot_rows_u<DD, R>(dr, use, vrow(jpos), vd);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (use[r]) {
                const bool o = ok[r / GM];
                const float sh = o ? D.tau * s[r] : kNegInfB;
                const float m_new = fmaxf(m[r], wave_max(sh));
                if (m_new == kNegInfB) continue;  // nothing visible yet
                const float sc = expf(m[r] - m_new);
                const float pj = o ? expf(sh - m_new) : 0.f;
                l[r] = l[r] * sc + wave_sum(pj);
                dn[r] = dn[r] * sc + wave_sum(o ? pj * vd[r] : 0.f);
                m[r] = m_new;
            }
    };
    if (D.W > 0)
        for (int j0 = jw0; j0 <= t_hi; j0 += kWave) pass1(j0 + lane <= t_hi ? j0 + lane : -1, true);
    for (int i0 = 0; i0 < n_cand; i0 += kWave) pass1(i0 + lane < n_cand ? sel[i0 + lane] : -1, false);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        inv[r] = use[r] ? 1.0f / l[r] : 0.f;
        Dt[r] = dn[r] * inv[r];
    }

    // ---- pass 2: softmax part of dq ----
    float dqa[R][PL];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int p = 0; p < PL; ++p) dqa[r][p] = 0.f;
    auto pass2 = [&](int jpos, bool win) {
        bool ok[kNP];
        bool any = false;
#pragma unroll
        for (int pp = 0; pp < kNP; ++pp) {
            ok[pp] = sees(pp, jpos, win);
            any = any || ok[pp];
        }
        float dsj[R];
#pragma unroll
        for (int r = 0; r < R; ++r) dsj[r] = 0.f;
        if (any) {
            float s[R], vd[R];
            dot_rows_u<DD, R>(qr, use, krow(jpos), s);
            dot_rows_u<DD, R>(dr, use, vrow(jpos), vd);
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (use[r] && ok[r / GM]) dsj[r] = expf(D.tau * s[r] - m[r]) * inv[r] * (vd[r] - Dt[r]);
        }
        for (int jj = 0; jj < kWave; ++jj) {
            const int jp = __shfl(any ? jpos : -1, jj, kWave);
            if (jp >= 0) {
                const T* kr = krow(jp);
                float kv[PL];
#pragma unroll
                for (int p = 0; p < PL; ++p) kv[p] = to_f32(kr[lane + kWave * p]);
#pragma unroll
                for (int r = 0; r < R; ++r)
                    if (use[r]) {
                        const float w = __shfl(dsj[r], jj, kWave);
#pragma unroll
                        for (int p = 0; p < PL; ++p) dqa[r][p] = fmaf(w, kv[p], dqa[r][p]);
                    }
            }
        }
    };
    if (D.W > 0)
        for (int j0 = jw0; j0 <= t_hi; j0 += kWave) pass2(j0 + lane <= t_hi ? j0 + lane : -1, true);
    for (int i0 = 0; i0 < n_cand; i0 += kWave) pass2(i0 + lane < n_cand ? sel[i0 + lane] : -1, false);
#pragma unroll
    for (int pp = 0; pp < kNP; ++pp)
#pragma unroll
        for (int h = 0; h < GM; ++h)
            if (h < G && act[pp])
#pragma unroll
                for (int p = 0; p < PL; ++p)
                    dq[qoff(pp, h) * DD + lane + kWave * p] = D.tau * dqa[pp * GM + h][p];
    }

    // ---- dphi_q, per position ----
#pragma unroll
    for (int pp = 0; pp < kNP; ++pp) {
        const float* st = state_of(pp);
        float dfq[GM][PL];
#pragma unroll
        for (int h = 0; h < GM; ++h)
#pragma unroll
            for (int p = 0; p < PL; ++p)
                dfq[h][p] = st ? y[pp * GM + h][p] - Dt[pp * GM + h] * st[DD * DD + lane + kWave * p] : 0.f;
        const int cf0 = (r_end[pp] / D.C) * D.C;
        for (int j0 = cf0; j0 < r_end[pp]; j0 += kWave) {
            const int j = j0 + lane;
            float w[GM];
#pragma unroll
            for (int h = 0; h < GM; ++h) w[h] = 0.f;
            const bool la = j < r_end[pp] && rt[j] == kRouteLA;
            if (la) {
                dot_multi<DD, GM>(ds_[pp], vrow(j), G, w);
#pragma unroll
                for (int h = 0; h < GM; ++h) w[h] -= Dt[pp * GM + h];
            }
            const int nb = min(kWave, r_end[pp] - j0);
            for (int jj = 0; jj < nb; ++jj) {
                const int laj = __shfl((int)la, jj, kWave);
                if (laj) {
                    const float* pk = pkrow(j0 + jj);
                    float pv[PL];
#pragma unroll
                    for (int p = 0; p < PL; ++p) pv[p] = pk[lane + kWave * p];
#pragma unroll
                    for (int h = 0; h < GM; ++h)
                        if (h < G) {
                            const float wj = __shfl(w[h], jj, kWave);
#pragma unroll
                            for (int p = 0; p < PL; ++p) dfq[h][p] = fmaf(wj, pv[p], dfq[h][p]);
                        }
                }
            }
        }
#pragma unroll
        for (int h = 0; h < GM; ++h)
            if (h < G && act[pp]) {
                const int r = pp * GM + h;
                const size_t o = qoff(pp, h);
                // no linear mass: no linear term to differentiate
                const float cf = la_mass[r] ? expf(-m[r]) * inv[r] : 0.f;
                // cf dfq is the gradient w.r.t. the gated features fq = gamma phi_q:
                // phi_q gets gamma times it, the gate logit (1 - gamma) fq . (cf dfq)
                const float gw = gate_weight(gate, o);
#pragma unroll
                for (int p = 0; p < PL; ++p) dphiq[o * DD + lane + kWave * p] = gw * cf * dfq[h][p];
                if (dgate) {
                    float fd = 0.f;
#pragma unroll
                    for (int p = 0; p < PL; ++p) fd = fmaf(fq[pp][h][lane + kWave * p], dfq[h][p], fd);
                    fd = wave_sum(fd);
                    if (lane == 0) dgate[o] = (1.f - gw) * cf * fd;
                }
                if (lane == 0) {
                    stat[o * 4 + 0] = m[r];
                    stat[o * 4 + 1] = l[r];
                    stat[o * 4 + 2] = Dt[r];
                    stat[o * 4 + 3] = cf;
                }
            }
    }
}

// Per query chunk c of (b, g): U[i][e] = sum over its queries t and the
// group's heads of c_t phi_q[i] dout[e], u[i] = sum c_t D_t phi_q[i]
// (same (d + 1) fd layout as the LA state).  Thread tid owns entries tid + 256 r.
template <typename T, int DD>
__global__ __launch_bounds__(256) void bwd_uchunk_kernel(const float* __restrict__ phiq,
                                                         const T* __restrict__ dout,
                                                         const float* __restrict__ stat,
                                                         float* __restrict__ ust, Dims D) {
    constexpr int E = DD * DD, PER = E / 256;
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    __shared__ float ph[32][DD];
    __shared__ float dd[32][DD];
    __shared__ float cd[32];
    float acc[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r) acc[r] = 0.f;
    float uacc = 0.f;
    const int c0 = c * D.C, n = min(D.C, D.N - c0) * D.G;  // (t, h) pairs
    for (int r0 = 0; r0 < n; r0 += 32) {
        const int nb = min(32, n - r0);
        __syncthreads();
        for (int x = tid; x < nb * DD; x += 256) {
            const int rr = x / DD, i = x % DD, pr = r0 + rr;
            const int t = c0 + pr / D.G, h = g * D.G + pr % D.G;
            const size_t off = ((size_t)b * D.N + t) * D.Hq + h;
            ph[rr][i] = stat[off * 4 + 3] * phiq[off * DD + i];
            dd[rr][i] = to_f32(dout[off * DD + i]);
            if (i == 0) cd[rr] = stat[off * 4 + 2];
        }
        __syncthreads();
        for (int rr = 0; rr < nb; ++rr) {
#pragma unroll
            for (int r = 0; r < PER; ++r) {
                const int e = tid + 256 * r;
                acc[r] = fmaf(ph[rr][e / DD], dd[rr][e % DD], acc[r]);
            }
            if (tid < DD) uacc = fmaf(cd[rr], ph[rr][tid], uacc);
        }
    }
    float* out = ust + (((size_t)b * D.Hkv + g) * D.T + c) * (size_t)(DD * (DD + 1));
#pragma unroll
    for (int r = 0; r < PER; ++r) out[tid + 256 * r] = acc[r];
    if (tid < DD) out[E + tid] = uacc;
}

// ust16 (matrix-core path, else nullptr): the U part (e < fd d) of each
// suffix goes there in bf16, [B, Hkv, T, fd d], the operand precision of the
// key kernel that reads it; u stays in place in fp32.
__global__ __launch_bounds__(256) void bwd_suffix_kernel(float* __restrict__ ust, __bf16* __restrict__ ust16,
                                                         Dims D) {
    const int E1 = D.fd * (D.d + 1), EU = D.fd * D.d;
    const int e = blockIdx.x * 256 + threadIdx.x, g = blockIdx.y, b = blockIdx.z;
    if (e >= E1) return;
    const size_t bgT = ((size_t)b * D.Hkv + g) * D.T;
    float* base = ust + bgT * (size_t)E1 + e;
    __bf16* b16 = ust16 && e < EU ? ust16 + bgT * (size_t)EU + e : nullptr;
    float run = 0.f;
    // chunks from the last down, eight loads in flight at a time
    constexpr int kB = 8;
    for (int c1 = D.T; c1 > 0; c1 -= kB) {
        const int n = min(kB, c1);
        float x[kB];
#pragma unroll
        for (int i = 0; i < kB; ++i) x[i] = i < n ? base[(size_t)(c1 - 1 - i) * E1] : 0.f;
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            if (i >= n) break;
            run += x[i];
            const size_t c = (size_t)(c1 - 1 - i);
            if (b16) b16[c * EU] = (__bf16)run;
            else base[c * E1] = run;
        }
    }
}

constexpr int kKB = 4;  // keys per wave in the key-side kernels

// Softmax terms of KB keys (rows ks[i], vs[i] in LDS, positions jk[i], -1
// for none) against the query rows (t, h) with t in [t_lo, t_hi] and h in
// KV head g's group: each query row and dout row is loaded once for all KB
// keys.  A pair counts when mode 0: t in [j, j + W - 1] (the key's window
// queries), mode 1: t >= j + W (later queries of a selected key).
//   p = exp(s - m_t) / l_t,  ds = p (dout_t . v_j - D_t)
//   dka[i] += ds q_t,  dva[i] += p dout_t   (lane owns dims lane + 64 p)
template <typename T, int DD>
__device__ __forceinline__ void key_group_softmax(const T* __restrict__ q, const T* __restrict__ dout,
                                                  const float* __restrict__ stat,
                                                  const float (*ks)[DD], const float (*vs)[DD],
                                                  const int* jk, int t_lo, int t_hi, int mode,
                                                  int b, int g, const Dims& D, int lane,
                                                  float (*dka)[DD / kWave],
                                                  float (*dva)[DD / kWave]) {
    constexpr int PL = DD / kWave;
    const int G = D.G;
    const int n = t_hi >= t_lo ? (t_hi - t_lo + 1) * G : 0;
    auto row_of = [&](int pr) { return ((size_t)b * D.N + t_lo + pr / G) * D.Hq + (size_t)g * G + pr % G; };
    for (int i0 = 0; i0 < n; i0 += kWave) {
        const int pr = i0 + lane;
        float pj[kKB], dsj[kKB];
#pragma unroll
        for (int i = 0; i < kKB; ++i) pj[i] = dsj[i] = 0.f;
        if (pr < n) {
            const size_t o = row_of(pr);
            const int t = t_lo + pr / G;
            float s[kKB], vd[kKB];
            dot_multi<DD, kKB>(ks, q + o * DD, kKB, s);
            dot_multi<DD, kKB>(vs, dout + o * DD, kKB, vd);
            const float m = stat[o * 4 + 0], il = 1.0f / stat[o * 4 + 1], Dt = stat[o * 4 + 2];
#pragma unroll
            for (int i = 0; i < kKB; ++i) {
                const int j = jk[i];
                const bool ok = j >= 0 && (mode == 0 ? (t >= j && t <= j + D.W - 1) : t >= j + D.W);
                if (ok) {
                    pj[i] = expf(D.tau * s[i] - m) * il;
                    dsj[i] = pj[i] * (vd[i] - Dt);
                }
            }
        }
        const int nb = min(kWave, n - i0);
        for (int jj = 0; jj < nb; ++jj) {
            const size_t o = row_of(i0 + jj);
            float qe[PL], de[PL];
#pragma unroll
            for (int p = 0; p < PL; ++p) {
                qe[p] = to_f32(q[o * DD + lane + kWave * p]);
                de[p] = to_f32(dout[o * DD + lane + kWave * p]);
            }
#pragma unroll
            for (int i = 0; i < kKB; ++i) {
                const float w = __shfl(dsj[i], jj, kWave), pv = __shfl(pj[i], jj, kWave);
#pragma unroll
                for (int p = 0; p < PL; ++p) {
                    dka[i][p] = fmaf(w, qe[p], dka[i][p]);
                    dva[i][p] = fmaf(pv, de[p], dva[i][p]);
                }
            }
        }
    }
}

// One wave per (b, g, four consecutive keys j0 .. j0 + 3): the softmax terms
// of each key's window queries, and for a routed linear key everything its
// later queries contribute through the linear branch:
//   dv_j = U_j^T phi_k(j),  dphi_k(j) = U_j v_j - u_j
// (U_j: the inclusive suffix sum from the first chunk after j + W's chunk,
// plus the queries of j + W's chunk from j + W on, taken one by one).
// Writes dk (softmax part), dv and dphi_k of its keys.
template <typename T, int DD>
__global__ __launch_bounds__(64) void bwd_key_win_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ phiq, const float* __restrict__ phik,
    const uint8_t* __restrict__ route, const float* __restrict__ stat,
    const float* __restrict__ ust, float* __restrict__ dk, float* __restrict__ dv,
    float* __restrict__ dphik, Dims D) {
    constexpr int PL = DD / kWave;
    const Item it = xcd_item((D.N + kKB - 1) / kKB, D.Hkv);
    const int j0 = it.x * kKB, g = it.y, b = it.z, lane = threadIdx.x;
    __shared__ float ks[kKB][DD];
    __shared__ float vs[kKB][DD];
    __shared__ float fk[kKB][DD];
    int jk[kKB];
#pragma unroll
    for (int i = 0; i < kKB; ++i) jk[i] = j0 + i < D.N ? j0 + i : -1;
    auto koff = [&](int j) { return ((size_t)b * D.N + j) * D.Hkv + g; };
    for (int x = lane; x < kKB * DD; x += kWave) {
        const int i = x / DD, e = x % DD, j = min(j0 + i, D.N - 1);
        ks[i][e] = to_f32(k[koff(j) * DD + e]);
        vs[i][e] = to_f32(v[koff(j) * DD + e]);
        fk[i][e] = phik[koff(j) * DD + e];
    }
    __syncthreads();
    float dka[kKB][PL], dva[kKB][PL], dfa[kKB][PL];
#pragma unroll
    for (int i = 0; i < kKB; ++i)
#pragma unroll
        for (int p = 0; p < PL; ++p) dka[i][p] = dva[i][p] = dfa[i][p] = 0.f;
    if (D.W > 0)
        key_group_softmax<T, DD>(q, dout, stat, ks, vs, jk, j0, min(D.N - 1, j0 + kKB - 1 + D.W - 1),
                                 0, b, g, D, lane, dka, dva);
    // linear part, one pass per chunk c0 holding some key's first linear
    // query j + W: the suffix block c0 + 1 and the queries of chunk c0 are
    // read once for all keys of the group that share c0
    const int G = D.G;
    bool lak[kKB];
    int c0k[kKB];
#pragma unroll
    for (int i = 0; i < kKB; ++i) {
        const int j = jk[i];
        lak[i] = j >= 0 && j + D.W <= D.N - 1 && route[((size_t)b * D.Hkv + g) * D.N + j] == kRouteLA;
        c0k[i] = lak[i] ? (j + D.W) / D.C : -1;
    }
    int c_lo = D.T, c_hi = -1;
#pragma unroll
    for (int i = 0; i < kKB; ++i)
        if (lak[i]) {
            c_lo = min(c_lo, c0k[i]);
            c_hi = max(c_hi, c0k[i]);
        }
#pragma unroll 1
    for (int c0 = c_lo; c0 <= c_hi; ++c0) {
        bool mk[kKB];
        bool any = false;
        int t_a = D.N;
#pragma unroll
        for (int i = 0; i < kKB; ++i) {
            mk[i] = lak[i] && c0k[i] == c0;
            any = any || mk[i];
            if (mk[i]) t_a = min(t_a, jk[i] + D.W);
        }
        if (!any) continue;
        if (c0 + 1 < D.T) {
            const float* U = ust + (((size_t)b * D.Hkv + g) * D.T + c0 + 1) * (size_t)(DD * (DD + 1));
#pragma unroll 4
            for (int i = 0; i < DD; ++i) {
                float uv[PL];
#pragma unroll
                for (int p = 0; p < PL; ++p) uv[p] = U[(size_t)i * DD + lane + kWave * p];
#pragma unroll
                for (int kk = 0; kk < kKB; ++kk)
                    if (mk[kk]) {
                        const float f = fk[kk][i];
#pragma unroll
                        for (int p = 0; p < PL; ++p) dva[kk][p] = fmaf(f, uv[p], dva[kk][p]);
                    }
            }
#pragma unroll
            for (int p = 0; p < PL; ++p) {
                const int i = lane + kWave * p;
                const float4* row = reinterpret_cast<const float4*>(U + (size_t)i * DD);
                float x[kKB];
#pragma unroll
                for (int kk = 0; kk < kKB; ++kk) x[kk] = 0.f;
#pragma unroll 4
                for (int e4 = 0; e4 < DD / 4; ++e4) {
                    const float4 r = row[e4];
#pragma unroll
                    for (int kk = 0; kk < kKB; ++kk) {
                        x[kk] = fmaf(r.x, vs[kk][4 * e4], x[kk]);
                        x[kk] = fmaf(r.y, vs[kk][4 * e4 + 1], x[kk]);
                        x[kk] = fmaf(r.z, vs[kk][4 * e4 + 2], x[kk]);
                        x[kk] = fmaf(r.w, vs[kk][4 * e4 + 3], x[kk]);
                    }
                }
                const float zi = U[DD * DD + i];
#pragma unroll
                for (int kk = 0; kk < kKB; ++kk)
                    if (mk[kk]) dfa[kk][p] += x[kk] - zi;
            }
        }
        // queries of chunk c0 from the group's first linear query on
        const int t1 = min(D.N - 1, (c0 + 1) * D.C - 1);
        const int n_la = (t1 - t_a + 1) * G;
        auto row_of = [&](int pr) { return ((size_t)b * D.N + t_a + pr / G) * D.Hq + (size_t)g * G + pr % G; };
        for (int i0 = 0; i0 < n_la; i0 += kWave) {
            const int pr = i0 + lane;
            float wk_[kKB], wf[kKB];
#pragma unroll
            for (int kk = 0; kk < kKB; ++kk) wk_[kk] = wf[kk] = 0.f;
            if (pr < n_la) {
                const size_t o = row_of(pr);
                const int t = t_a + pr / G;
                float kap[kKB], vd[kKB];
                dot_multi<DD, kKB>(fk, phiq + o * DD, kKB, kap);
                dot_multi<DD, kKB>(vs, dout + o * DD, kKB, vd);
                const float cf = stat[o * 4 + 3], Dt = stat[o * 4 + 2];
#pragma unroll
                for (int kk = 0; kk < kKB; ++kk)
                    if (mk[kk] && t >= jk[kk] + D.W) {
                        wk_[kk] = cf * kap[kk];
                        wf[kk] = cf * (vd[kk] - Dt);
                    }
            }
            const int nb = min(kWave, n_la - i0);
            for (int jj = 0; jj < nb; ++jj) {
                const size_t o = row_of(i0 + jj);
                float de[PL], fe[PL];
#pragma unroll
                for (int p = 0; p < PL; ++p) {
                    de[p] = to_f32(dout[o * DD + lane + kWave * p]);
                    fe[p] = phiq[o * DD + lane + kWave * p];
                }
#pragma unroll
                for (int kk = 0; kk < kKB; ++kk)
                    if (mk[kk]) {
                        const float a = __shfl(wk_[kk], jj, kWave), c = __shfl(wf[kk], jj, kWave);
#pragma unroll
                        for (int p = 0; p < PL; ++p) {
                            dva[kk][p] = fmaf(a, de[p], dva[kk][p]);
                            dfa[kk][p] = fmaf(c, fe[p], dfa[kk][p]);
                        }
                    }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kKB; ++i) {
        if (jk[i] < 0) continue;
#pragma unroll
        for (int p = 0; p < PL; ++p) {
            const size_t e = koff(jk[i]) * DD + lane + kWave * p;
            dk[e] = D.tau * dka[i][p];
            dv[e] = dva[i][p];
            dphik[e] = dfa[i][p];
        }
    }
}

// One block of kSW waves per (b, g, kSW * kKB entries of the selected list);
// wave w takes entries kKB w .. kKB w + kKB - 1.  The softmax terms of every
// query after each selected key's window (t >= j + W), added to dk and dv
// (after bwd_key_win_kernel has written them; the entries of one (b, g)
// list are distinct positions, so no two waves share a key).  Tiles of 64
// query rows and their dout rows are loaded once per block, coalesced, into
// LDS (rows padded by 16 bytes so that 16 lanes reading 16 lanes' rows hit
// distinct banks), and every wave dots its keys against them.
constexpr int kSW = 4;
template <typename T, int DD>
__global__ __launch_bounds__(256) void bwd_key_sel_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const int32_t* __restrict__ selw, const float* __restrict__ stat,
    float* __restrict__ dk, float* __restrict__ dv, Dims D) {
    constexpr int PL = DD / kWave;
    constexpr int EPC = 16 / (int)sizeof(T);     // elements per 16-byte chunk
    constexpr int RS = DD + EPC;                 // padded row stride (elements)
    constexpr int CH = DD / EPC;                 // chunks per row
    const int n_list = D.n_full * D.lam;
    const Item it = xcd_item((n_list + kSW * kKB - 1) / (kSW * kKB), D.Hkv);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int e0 = it.x * kSW * kKB + wave * kKB, g = it.y, b = it.z;
    const int G = D.G;
    const int32_t* sel = selw + ((size_t)b * D.Hkv + g) * n_list;
    __shared__ float ks[kSW][kKB][DD];
    __shared__ float vs[kSW][kKB][DD];
    __shared__ __align__(16) T qt[kWave][RS];
    __shared__ __align__(16) T dt[kWave][RS];
    __shared__ float st3[kWave][3];
    __shared__ int tlo_w[kSW];
    int jk[kKB];
    int t_lo = D.N;
#pragma unroll
    for (int i = 0; i < kKB; ++i) {
        jk[i] = e0 + i < n_list ? sel[e0 + i] : -1;
        if (jk[i] >= 0) t_lo = min(t_lo, jk[i] + D.W);
    }
    auto koff = [&](int j) { return ((size_t)b * D.N + j) * D.Hkv + g; };
    for (int x = lane; x < kKB * DD; x += kWave) {
        const int i = x / DD, e = x % DD, j = max(jk[i], 0);
        ks[wave][i][e] = to_f32(k[koff(j) * DD + e]);
        vs[wave][i][e] = to_f32(v[koff(j) * DD + e]);
    }
    if (lane == 0) tlo_w[wave] = t_lo;
    __syncthreads();
    int tb = D.N;
#pragma unroll
    for (int w = 0; w < kSW; ++w) tb = min(tb, tlo_w[w]);
    const int n = tb <= D.N - 1 ? (D.N - tb) * G : 0;  // (t, h) rows from the block's first query on
    auto row_of = [&](int pr) { return ((size_t)b * D.N + tb + pr / G) * D.Hq + (size_t)g * G + pr % G; };
    float dka[kKB][PL], dva[kKB][PL];
#pragma unroll
    for (int i = 0; i < kKB; ++i)
#pragma unroll
        for (int p = 0; p < PL; ++p) dka[i][p] = dva[i][p] = 0.f;
    for (int i0 = 0; i0 < n; i0 += kWave) {
        __syncthreads();  // the previous tile is consumed
        for (int c = threadIdx.x; c < kWave * CH; c += kSW * kWave) {
            const int r = c / CH, part = c % CH, pr = i0 + r;
            if (pr < n) {
                const size_t o = row_of(pr) * DD + (size_t)part * EPC;
                *reinterpret_cast<uint4*>(&qt[r][part * EPC]) = *reinterpret_cast<const uint4*>(q + o);
                *reinterpret_cast<uint4*>(&dt[r][part * EPC]) = *reinterpret_cast<const uint4*>(dout + o);
            }
        }
        if (threadIdx.x < kWave && i0 + threadIdx.x < n) {
            const size_t o = row_of(i0 + threadIdx.x);
            st3[threadIdx.x][0] = stat[o * 4 + 0];
            st3[threadIdx.x][1] = 1.0f / stat[o * 4 + 1];
            st3[threadIdx.x][2] = stat[o * 4 + 2];
        }
        __syncthreads();
        const int pr = i0 + lane;
        float pj[kKB], dsj[kKB];
#pragma unroll
        for (int i = 0; i < kKB; ++i) pj[i] = dsj[i] = 0.f;
        if (pr < n) {
            const int t = tb + pr / G;
            float sv[kKB], vd[kKB];
            dot_multi<DD, kKB>(ks[wave], &qt[lane][0], kKB, sv);
            dot_multi<DD, kKB>(vs[wave], &dt[lane][0], kKB, vd);
            const float m = st3[lane][0], il = st3[lane][1], Dt = st3[lane][2];
#pragma unroll
            for (int i = 0; i < kKB; ++i)
                if (jk[i] >= 0 && t >= jk[i] + D.W) {
                    pj[i] = expf(D.tau * sv[i] - m) * il;
                    dsj[i] = pj[i] * (vd[i] - Dt);
                }
        }
        const int nb = min(kWave, n - i0);
        for (int jj = 0; jj < nb; ++jj) {
            float qe[PL], de[PL];
#pragma unroll
            for (int p = 0; p < PL; ++p) {
                qe[p] = to_f32(qt[jj][lane + kWave * p]);
                de[p] = to_f32(dt[jj][lane + kWave * p]);
            }
#pragma unroll
            for (int i = 0; i < kKB; ++i) {
                const float w = __shfl(dsj[i], jj, kWave), pv = __shfl(pj[i], jj, kWave);
#pragma unroll
                for (int p = 0; p < PL; ++p) {
                    dka[i][p] = fmaf(w, qe[p], dka[i][p]);
                    dva[i][p] = fmaf(pv, de[p], dva[i][p]);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kKB; ++i) {
        if (jk[i] < 0) continue;
#pragma unroll
        for (int p = 0; p < PL; ++p) {
            const size_t e = koff(jk[i]) * DD + lane + kWave * p;
            dk[e] += D.tau * dka[i][p];
            dv[e] += dva[i][p];
        }
    }
}

// NP-Map backward for the hpp heads of group gp of token tok, x[tok, gp hpp + h]
// with projection P[gp] (fd / 2 <= 64 rows, one per lane), one wave: the
// projection is read once for all hpp <= GM heads.  Per head:
//   a = softmax(z), bb = softmax(-z):  dz = a (da - <da, a>) - bb (db - <db, bb>)
//   z = ||x|| uh, uh = u / ||u||:       d||x|| = <dz, uh>, duh = ||x|| dz
//   du = (duh - <duh, uh> uh) / ||u||   (zero where u = 0: z is pinned to 0)
//   dx = d||x|| x / ||x|| + P^T du  (added into dx_out),  du stored for dP
template <typename T, int DD, int GM>
__global__ __launch_bounds__(64) void np_vjp_kernel(const T* __restrict__ x,
                                                    const float* __restrict__ Pall,
                                                    const float* __restrict__ dphi,
                                                    float* __restrict__ dx_out,
                                                    float* __restrict__ du_out, int H, int hpp,
                                                    int fd) {
    constexpr int PL = DD / kWave;
    const int tok = blockIdx.x, gp = blockIdx.y, lane = threadIdx.x;
    const int half = fd / 2;
    __shared__ float xs[GM][DD];
    __shared__ float dus[GM][64];
    const size_t row0 = (size_t)tok * H + (size_t)gp * hpp;  // head h: row0 + h
    for (int i = lane; i < hpp * DD; i += kWave) xs[i / DD][i % DD] = to_f32(x[row0 * DD + i]);
    __syncthreads();
    const float* P = Pall + (size_t)gp * half * DD;
    const bool act = lane < half;
    float u[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) u[h] = 0.f;
    if (act) {  // P rows are 16-byte aligned: the projections are checked aligned, d is 64 or 128
        const float4* pr = reinterpret_cast<const float4*>(P + (size_t)lane * DD);
#pragma unroll 4
        for (int i = 0; i < DD / 4; ++i) {
            const float4 w = pr[i];
#pragma unroll
            for (int h = 0; h < GM; ++h)
                if (h < hpp) {
                    u[h] = fmaf(w.x, xs[h][4 * i], u[h]);
                    u[h] = fmaf(w.y, xs[h][4 * i + 1], u[h]);
                    u[h] = fmaf(w.z, xs[h][4 * i + 2], u[h]);
                    u[h] = fmaf(w.w, xs[h][4 * i + 3], u[h]);
                }
        }
    }
    float rn[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
        rn[h] = 0.f;
        if (h >= hpp) continue;
        float ss = 0.f;
        for (int i = lane; i < DD; i += kWave) ss = fmaf(xs[h][i], xs[h][i], ss);
        const float nx = sqrtf(wave_sum(ss));
        const float nu = sqrtf(wave_sum(u[h] * u[h]));
        const float uh = nu > 0.f ? u[h] / nu : 0.f;
        const float z = nx * uh;
        const float m1 = wave_max(act ? z : kNegInfB), m2 = wave_max(act ? -z : kNegInfB);
        const float e1 = act ? expf(z - m1) : 0.f, e2 = act ? expf(-z - m2) : 0.f;
        const float a = e1 / wave_sum(e1), bb = e2 / wave_sum(e2);
        const size_t row = row0 + h;
        const float da = act ? dphi[row * fd + lane] : 0.f;
        const float db = act ? dphi[row * fd + half + lane] : 0.f;
        const float sa = wave_sum(da * a), sb = wave_sum(db * bb);
        const float dz = act ? a * (da - sa) - bb * (db - sb) : 0.f;
        const float dnx = nu > 0.f ? wave_sum(dz * uh) : 0.f;
        const float duh = nx * dz;
        const float proj = wave_sum(duh * uh);
        const float du = (nu > 0.f && act) ? (duh - proj * uh) / nu : 0.f;
        dus[h][lane] = du;
        rn[h] = nx > 0.f ? dnx / nx : 0.f;
        if (act) du_out[row * half + lane] = du;
    }
    __syncthreads();
    float acc[GM][PL];
#pragma unroll
    for (int h = 0; h < GM; ++h)
#pragma unroll
        for (int p = 0; p < PL; ++p) acc[h][p] = h < hpp ? rn[h] * xs[h][lane + kWave * p] : 0.f;
    for (int i = 0; i < half; ++i) {
        float pv[PL];
#pragma unroll
        for (int p = 0; p < PL; ++p) pv[p] = P[(size_t)i * DD + lane + kWave * p];
#pragma unroll
        for (int h = 0; h < GM; ++h)
            if (h < hpp)
#pragma unroll
                for (int p = 0; p < PL; ++p) acc[h][p] = fmaf(dus[h][i], pv[p], acc[h][p]);
    }
#pragma unroll
    for (int h = 0; h < GM; ++h)
        if (h < hpp)
#pragma unroll
            for (int p = 0; p < PL; ++p) dx_out[(row0 + h) * DD + lane + kWave * p] += acc[h][p];
}

// Partial dP[g] over token slice s: thread e owns column e of every row.
template <typename T, int DD>
__global__ __launch_bounds__(DD) void dw_partial_kernel(const T* __restrict__ x,
                                                        const float* __restrict__ du,
                                                        float* __restrict__ part, int ntok, int H,
                                                        int hpp, int half, int nslice) {
    const int g = blockIdx.x, sl = blockIdx.y, e = threadIdx.x;
    const int per = (ntok + nslice - 1) / nslice;
    const int tk0 = sl * per, tk1 = min(ntok, tk0 + per);
    float acc[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) acc[i] = 0.f;
    for (int tk = tk0; tk < tk1; ++tk) {
        for (int hh = 0; hh < hpp; ++hh) {
            const size_t row = (size_t)tk * H + g * hpp + hh;
            const float xe = to_f32(x[row * DD + e]);
            const float* dr = du + row * half;
#pragma unroll
            for (int i = 0; i < 64; ++i)
                if (i < half) acc[i] = fmaf(dr[i], xe, acc[i]);
        }
    }
    float* out = part + (((size_t)sl * gridDim.x + g) * half) * DD + e;
#pragma unroll
    for (int i = 0; i < 64; ++i)
        if (i < half) out[(size_t)i * DD] = acc[i];
}

__global__ __launch_bounds__(256) void dw_reduce_kernel(const float* __restrict__ part,
                                                        float* __restrict__ dw, int n, int nslice) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= n) return;
    // slices in order, eight loads in flight at a time
    constexpr int kB = 8;
    float s = 0.f;
    for (int s0 = 0; s0 < nslice; s0 += kB) {
        float x[kB];
#pragma unroll
        for (int i = 0; i < kB; ++i) x[i] = s0 + i < nslice ? part[(size_t)(s0 + i) * n + e] : 0.f;
#pragma unroll
        for (int i = 0; i < kB; ++i) s += x[i];
    }
    dw[e] = s;
}

__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ p, int n) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e < n) p[e] = 0.f;
}

template <typename T, int DD>
hipError_t bwd_t(const Dims& D, const BwdArgs& a, const BwdWork& w, hipStream_t s, BwdMark mark) {
    const T* q = reinterpret_cast<const T*>(a.q);
    const T* k = reinterpret_cast<const T*>(a.k);
    const T* v = reinterpret_cast<const T*>(a.v);
    const T* dout = reinterpret_cast<const T*>(a.dout);
    hipError_t e;
#define STILL_STEP(name, launch)                       \
    do {                                               \
        if ((e = mark.fn(mark.ctx, name)) != hipSuccess) return e; \
        launch;                                        \
        if ((e = hipGetLastError()) != hipSuccess) return e; \
    } while (0)
    STILL_STEP("bwd_route", hipLaunchKernelGGL(bwd_route_kernel, dim3(D.T, D.Hkv, D.B), dim3(256),
                                               (size_t)D.C * sizeof(int), s, a.sel_idx, w.route,
                                               w.selw, D));
    // the matrix-core kernels after the lists work in 64-token tiles (DT: the
    // tile dimensions, D itself when C = 64)
    const Dims& DT = w.tile;
    if (w.mfma) {
        // first pass and the softmax part of dq on the matrix cores
        if ((e = mark.fn(mark.ctx, "bwd_lists")) != hipSuccess) return e;
        if (D.C > 64) {
            if ((e = launch_bwd_lists_tiles(D, DT, w.selw, a.k, a.v, w.selw_t, w.ksel, w.vsel, w.list_off,
                                            a.wq, a.wk, w.wsplit, s)) != hipSuccess)
                return e;
        } else if ((e = launch_bwd_lists(D, w.selw, a.k, a.v, w.ksel, w.vsel, w.list_off, a.wq, a.wk,
                                         w.wsplit, s)) != hipSuccess) {
            return e;
        }
        // the keys' NP-Map features and the linear prefixes, unless the
        // forward's are given
        if (!w.lin_given) {
            if ((e = mark.fn(mark.ctx, "la_state")) != hipSuccess) return e;
            if ((e = launch_la_state(DT, a.k, a.v, w.wsplit, w.route, w.phik16, w.lin16, -1, s)) !=
                hipSuccess)
                return e;
            if ((e = mark.fn(mark.ctx, "la_scan16")) != hipSuccess) return e;
            if ((e = launch_la_group_scan(DT, w.lin16, -1, nullptr, nullptr, s)) != hipSuccess) return e;
        }
        // the statistics and gated query features: a first pass, or (given
        // the forward's out and statistics) the dq kernel's own prologue
        if (!a.stats) {
            if ((e = mark.fn(mark.ctx, "bwd_stats")) != hipSuccess) return e;
            if ((e = launch_hybrid_stats(DT, a.q, a.k, a.v, w.wsplit, w.phik16, w.route, w.ksel, w.vsel,
                                         w.lin16, a.gate, w.list_off, a.dout, w.stat, w.phiq, s)) !=
                hipSuccess)
                return e;
        }
        if ((e = mark.fn(mark.ctx, "bwd_dq")) != hipSuccess) return e;
        if ((e = launch_bwd_dq(DT, a.q, a.k, a.v, a.dout, w.route, w.ksel, w.vsel, w.list_off, w.stat,
                               w.phik16, w.lin16, a.gate, w.phiq, a.dq, w.duq,
                               a.gate ? a.dgate : nullptr, a.stats, a.out, w.wsplit, s)) != hipSuccess)
            return e;
    }
    // the queries' features carry their gate weights (phi~_q = gamma phi_q), so
    // every linear term below is the gated one (the matrix-core first pass
    // wrote them already)
    if (!w.mfma) {
        if ((e = mark.fn(mark.ctx, "phi_q")) != hipSuccess) return e;
        if ((e = launch_phi(D, a.q, D.Hq, D.G, a.wq, a.gate, w.phiq, s)) != hipSuccess) return e;
    }
    if (!w.mfma) {
        if ((e = mark.fn(mark.ctx, "phi_k")) != hipSuccess) return e;
        if ((e = launch_phi(D, a.k, D.Hkv, 1, a.wk, nullptr, w.phik, s)) != hipSuccess) return e;
        // the fp32 linear prefixes the query kernel reads (the matrix-core
        // dq kernel reads the bf16 ones)
        if ((e = mark.fn(mark.ctx, "la_chunk")) != hipSuccess) return e;
        if ((e = launch_la_chunks(D, w.phik, a.v, w.route, w.lin, s)) != hipSuccess) return e;
        if ((e = mark.fn(mark.ctx, "la_scan")) != hipSuccess) return e;
        if ((e = launch_la_scan(D, w.lin, -1, nullptr, nullptr, s)) != hipSuccess) return e;
    }
#define STILL_BWD_QUERY(GM)                                                               \
    hipLaunchKernelGGL((bwd_query_kernel<T, DD, GM>), dim3((D.N + kNP - 1) / kNP * D.Hkv * D.B), dim3(64), \
                       0, s, q, k,                                                                  \
                       v, dout, w.phiq, w.phik, w.route, w.selw, w.lin, a.gate, a.dq, w.dphiq,    \
                       a.dgate, w.stat, D)
    if (!w.mfma)
        STILL_STEP("bwd_query",
                   if (D.G == 1) STILL_BWD_QUERY(1); else if (D.G == 2) STILL_BWD_QUERY(2);
                   else if (D.G <= 4) STILL_BWD_QUERY(4); else STILL_BWD_QUERY(8));
#undef STILL_BWD_QUERY
    if (w.mfma) {
        if ((e = mark.fn(mark.ctx, "bwd_uchunk")) != hipSuccess) return e;
        if ((e = launch_bwd_key_lin(DT, a.v, a.dout, w.phiq, w.phik16, w.route, w.stat, w.ust, w.ust16, a.dv,
                                    a.k, w.wsplit, a.dk, w.duk, 0, s)) != hipSuccess)
            return e;
    } else {
        STILL_STEP("bwd_uchunk",
                   hipLaunchKernelGGL((bwd_uchunk_kernel<T, DD>), dim3(D.T, D.Hkv, D.B), dim3(256), 0,
                                      s, w.phiq, dout, w.stat, w.ust, D));
    }
    STILL_STEP("bwd_suffix",
               hipLaunchKernelGGL(bwd_suffix_kernel, dim3((D.fd * (D.d + 1) + 255) / 256, D.Hkv, D.B),
                                  dim3(256), 0, s, w.ust, reinterpret_cast<__bf16*>(w.ust16),
                                  w.mfma ? DT : D));
    if (w.mfma) {
        // linear terms first (dv, dphi_k), then the softmax terms on the matrix
        // cores: window keys (write dk, add to dv), then selected keys (add)
        if ((e = mark.fn(mark.ctx, "bwd_key_la")) != hipSuccess) return e;
        if ((e = launch_bwd_key_lin(DT, a.v, a.dout, w.phiq, w.phik16, w.route, w.stat, w.ust, w.ust16, a.dv,
                                    a.k, w.wsplit, a.dk, w.duk, 1, s)) != hipSuccess)
            return e;
        if ((e = mark.fn(mark.ctx, "bwd_kv_win")) != hipSuccess) return e;
        if ((e = launch_bwd_kv(DT, a.q, a.k, a.v, a.dout, w.route, w.ksel, w.vsel, w.selw_t, w.list_off,
                               w.stat, a.dk, a.dv, w.kvpart, 0, s)) != hipSuccess)
            return e;
        if ((e = mark.fn(mark.ctx, "bwd_kv_sel")) != hipSuccess) return e;
        if ((e = launch_bwd_kv(DT, a.q, a.k, a.v, a.dout, w.route, w.ksel, w.vsel, w.selw_t, w.list_off,
                               w.stat, a.dk, a.dv, w.kvpart, 1, s)) != hipSuccess)
            return e;
    } else {
    STILL_STEP("bwd_key_win",
               hipLaunchKernelGGL((bwd_key_win_kernel<T, DD>), dim3((D.N + kKB - 1) / kKB * D.Hkv * D.B),
                                  dim3(64), 0, s, q, k, v, dout, w.phiq, w.phik, w.route, w.stat,
                                  w.ust, a.dk, a.dv, w.dphik, D));
    if (D.lam > 0 && D.n_full > 0)
        STILL_STEP("bwd_key_sel",
                   hipLaunchKernelGGL((bwd_key_sel_kernel<T, DD>),
                                      dim3((D.n_full * D.lam + kSW * kKB - 1) / (kSW * kKB) * D.Hkv * D.B),
                                      dim3(kSW * kWave),
                                      0, s, q, k, v, dout, w.selw, w.stat, a.dk, a.dv, D));
    }
    const int ntok = D.B * D.N, half = D.fd / 2;
    const int nw = D.Hkv * half * DD;
    if (w.mfma) {
        // the projection gradients on the matrix cores (du in bf16 in the du
        // buffers, written by the NP-Map backwards inside the dq and key
        // linear kernels)
        if ((e = mark.fn(mark.ctx, "dw_q")) != hipSuccess) return e;
        if ((e = launch_dw_mfma(D, a.q, 0, w.duq, w.dwpart, w.nslice, s)) != hipSuccess) return e;
        STILL_STEP("dw_q_reduce", hipLaunchKernelGGL(dw_reduce_kernel, dim3((nw + 255) / 256), dim3(256),
                                                     0, s, w.dwpart, a.dwq, nw, w.nslice));
        if ((e = mark.fn(mark.ctx, "dw_k")) != hipSuccess) return e;
        if ((e = launch_dw_mfma(D, a.k, 1, w.duk, w.dwpart, w.nslice, s)) != hipSuccess) return e;
        STILL_STEP("dw_k_reduce", hipLaunchKernelGGL(dw_reduce_kernel, dim3((nw + 255) / 256), dim3(256),
                                                     0, s, w.dwpart, a.dwk, nw, w.nslice));
        return hipSuccess;
    }
#define STILL_NP_VJP_Q(GM)                                                                       \
    hipLaunchKernelGGL((np_vjp_kernel<T, DD, GM>), dim3(ntok, D.Hkv), dim3(64), 0, s, q, a.wq, w.dphiq, \
                       a.dq, w.duq, D.Hq, D.G, D.fd)
    STILL_STEP("np_vjp_q", if (D.G == 1) STILL_NP_VJP_Q(1); else if (D.G == 2) STILL_NP_VJP_Q(2);
                           else if (D.G <= 4) STILL_NP_VJP_Q(4); else STILL_NP_VJP_Q(8));
#undef STILL_NP_VJP_Q
    STILL_STEP("np_vjp_k",
               hipLaunchKernelGGL((np_vjp_kernel<T, DD, 1>), dim3(ntok, D.Hkv), dim3(64), 0, s, k,
                                  a.wk, w.dphik, a.dk, w.duk, D.Hkv, 1, D.fd));
    STILL_STEP("dw_q",
               hipLaunchKernelGGL((dw_partial_kernel<T, DD>), dim3(D.Hkv, w.nslice), dim3(DD), 0, s,
                                  q, w.duq, w.dwpart, ntok, D.Hq, D.G, half, w.nslice));
    STILL_STEP("dw_q_reduce", hipLaunchKernelGGL(dw_reduce_kernel, dim3((nw + 255) / 256), dim3(256),
                                                 0, s, w.dwpart, a.dwq, nw, w.nslice));
    STILL_STEP("dw_k",
               hipLaunchKernelGGL((dw_partial_kernel<T, DD>), dim3(D.Hkv, w.nslice), dim3(DD), 0, s,
                                  k, w.duk, w.dwpart, ntok, D.Hkv, 1, half, w.nslice));
    STILL_STEP("dw_k_reduce", hipLaunchKernelGGL(dw_reduce_kernel, dim3((nw + 255) / 256), dim3(256),
                                                 0, s, w.dwpart, a.dwk, nw, w.nslice));
#undef STILL_STEP
    return hipSuccess;
}

}  // namespace

int bwd_launch_count(bool) { return 16; }

hipError_t launch_bwd(const Dims& D, const BwdArgs& a, const BwdWork& w, hipStream_t s,
                      BwdMark mark) {
    if (D.d == 128) return D.bf16 ? bwd_t<__bf16, 128>(D, a, w, s, mark) : bwd_t<float, 128>(D, a, w, s, mark);
    return D.bf16 ? bwd_t<__bf16, 64>(D, a, w, s, mark) : bwd_t<float, 64>(D, a, w, s, mark);
}

hipError_t launch_zero(float* p, int n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace still
