// Future-KV-utility diagnostic of the STILL paper (full text App. A.7.4,
// Table 12): how much full causal attention each remote key receives from
// the queries after its window,
//   u[b, g, j] = sum over the query heads h of KV head g and the queries
//                t >= j + W of softmax_j'(tau q_t,h . k_j'), j' <= t.
// Compared with the tokens a routing criterion selected, it measures how
// well a causal local score predicts future use.  fp32 on the vector ALUs,
// every supported shape, f32 or bf16 storage.
//   util_rowstat_kernel  one wave per (b, t, g): the full causal softmax's
//                        reference m and normaliser l of every query head
//   util_colsum_kernel   one wave per (b, g, four consecutive keys): the
//                        weights of the queries after each key's window, summed
#include "device_common.h"
#include "launch.h"
#include "row_ops.h"

namespace still {

namespace {

constexpr int kUK = 4;  // keys per wave in the column sums

template <typename T, int DD, int GM>
__global__ __launch_bounds__(64) void util_rowstat_kernel(const T* __restrict__ q,
                                                          const T* __restrict__ k,
                                                          float* __restrict__ stat, Dims D) {
    const Item it = xcd_item(D.N, D.Hkv);
    const int t = it.x, g = it.y, b = it.z, lane = threadIdx.x;
    const int G = D.G;
    __shared__ float qs[GM][DD];
    const size_t qoff0 = ((size_t)b * D.N + t) * D.Hq + (size_t)g * G;
    for (int x = lane; x < G * DD; x += kWave) qs[x / DD][x % DD] = to_f32(q[(qoff0 + x / DD) * DD + x % DD]);
    __syncthreads();
    float m[GM], l[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
        m[h] = -__builtin_inff();
        l[h] = 0.f;
    }
    for (int j0 = 0; j0 <= t; j0 += kWave) {
        const int j = j0 + lane;
        float s[GM];
        if (j <= t) dot_multi<DD, GM>(qs, k + (((size_t)b * D.N + j) * D.Hkv + g) * DD, G, s);
#pragma unroll
        for (int h = 0; h < GM; ++h)
            if (h < G) {
                const float sh = j <= t ? D.tau * s[h] : -__builtin_inff();
                const float m_new = fmaxf(m[h], wave_max(sh));  // finite: key 0 is in the first batch
                l[h] = l[h] * expf(m[h] - m_new) + wave_sum(j <= t ? expf(sh - m_new) : 0.f);
                m[h] = m_new;
            }
    }
    if (lane == 0)
#pragma unroll
        for (int h = 0; h < GM; ++h)
            if (h < G) {
                stat[(qoff0 + h) * 2 + 0] = m[h];
                stat[(qoff0 + h) * 2 + 1] = l[h];
            }
}

template <typename T, int DD>
__global__ __launch_bounds__(64) void util_colsum_kernel(const T* __restrict__ q,
                                                         const T* __restrict__ k,
                                                         const float* __restrict__ stat,
                                                         float* __restrict__ util, Dims D) {
    const Item it = xcd_item((D.N + kUK - 1) / kUK, D.Hkv);
    const int j0 = it.x * kUK, g = it.y, b = it.z, lane = threadIdx.x;
    const int G = D.G;
    __shared__ float ks[kUK][DD];
    for (int x = lane; x < kUK * DD; x += kWave) {
        const int j = min(j0 + x / DD, D.N - 1);
        ks[x / DD][x % DD] = to_f32(k[(((size_t)b * D.N + j) * D.Hkv + g) * DD + x % DD]);
    }
    __syncthreads();
    const int t_lo = j0 + D.W;
    const int n = t_lo <= D.N - 1 ? (D.N - t_lo) * G : 0;
    float acc[kUK];
#pragma unroll
    for (int i = 0; i < kUK; ++i) acc[i] = 0.f;
    for (int pr = lane; pr < n; pr += kWave) {
        const int t = t_lo + pr / G;
        const size_t o = ((size_t)b * D.N + t) * D.Hq + (size_t)g * G + pr % G;
        float s[kUK];
        dot_multi<DD, kUK>(ks, q + o * DD, kUK, s);
        const float m = stat[o * 2 + 0], il = 1.0f / stat[o * 2 + 1];
#pragma unroll
        for (int i = 0; i < kUK; ++i)
            if (j0 + i < D.N && t >= j0 + i + D.W) acc[i] += expf(D.tau * s[i] - m) * il;
    }
#pragma unroll
    for (int i = 0; i < kUK; ++i) {
        const float tot = wave_sum(acc[i]);
        if (lane == 0 && j0 + i < D.N) util[((size_t)b * D.Hkv + g) * D.N + j0 + i] = tot;
    }
}

template <typename T, int DD>
hipError_t util_t(const Dims& D, const void* qv, const void* kv, float* stat, float* util,
                  hipStream_t s) {
    const T* q = reinterpret_cast<const T*>(qv);
    const T* k = reinterpret_cast<const T*>(kv);
    const dim3 rows(D.N * D.Hkv * D.B);
    if (D.G == 1) hipLaunchKernelGGL((util_rowstat_kernel<T, DD, 1>), rows, dim3(64), 0, s, q, k, stat, D);
    else if (D.G == 2) hipLaunchKernelGGL((util_rowstat_kernel<T, DD, 2>), rows, dim3(64), 0, s, q, k, stat, D);
    else if (D.G <= 4) hipLaunchKernelGGL((util_rowstat_kernel<T, DD, 4>), rows, dim3(64), 0, s, q, k, stat, D);
    else hipLaunchKernelGGL((util_rowstat_kernel<T, DD, 8>), rows, dim3(64), 0, s, q, k, stat, D);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((util_colsum_kernel<T, DD>), dim3((D.N + kUK - 1) / kUK * D.Hkv * D.B), dim3(64),
                       0, s, q, k, stat, util, D);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_future_utility(const Dims& D, const void* q, const void* k, float* stat,
                                 float* util, hipStream_t s) {
    if (D.d == 128)
        return D.bf16 ? util_t<__bf16, 128>(D, q, k, stat, util, s) : util_t<float, 128>(D, q, k, stat, util, s);
    return D.bf16 ? util_t<__bf16, 64>(D, q, k, stat, util, s) : util_t<float, 64>(D, q, k, stat, util, s);
}

}  // namespace still
