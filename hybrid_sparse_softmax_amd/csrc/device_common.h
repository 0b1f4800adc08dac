// Device helpers shared by the STILL kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace still {

constexpr int kWave = 64;

// route flag bytes (same values as the cache's win_route)
constexpr uint8_t kPending = 0, kRouteSA = 1, kRouteLA = 2;

// routing criteria (still.h STILL_ROUTE_*)
constexpr int kRouteSaliency = 0, kRouteDiagonal = 1, kRouteQK = 2, kRouteKeyNorm = 3,
              kRouteUniform = 4, kRouteRandom = 5;
__host__ __device__ constexpr bool route_query_free(int r) { return r >= kRouteKeyNorm; }

// splitmix64 (Steele, Lea and Flood 2014, in Vigna's formulation): one output
// for state x
__host__ __device__ inline uint64_t splitmix64(uint64_t x) {
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// score of token t of (sequence b, KV head g) under a query-free criterion;
// knorm = ||k_t|| (computed by the caller)
__host__ __device__ inline float query_free_score(int route, float knorm, int64_t t, int b, int g,
                                                  int Hkv, int C, int lam) {
    if (route == kRouteKeyNorm) return knorm;
    if (route == kRouteUniform) {
        const int off = (int)(t % C);  // selected offsets: floor(i C / lam), i < lam
        for (int i = 0; i < lam; ++i)
            if ((i * C) / lam == off) return 1.f;
        return 0.f;
    }
    const uint64_t x = ((uint64_t)((int64_t)b * Hkv + g) << 32) | (uint64_t)(uint32_t)t;
    return (float)(splitmix64(x) >> 40) * 0x1p-24f;
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
    return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
    return x;
}
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
    return x;
}

// log(1 + x) for x >= 0 in a few instructions: u = 1 + x rounded, then
// log(u) * x / (u - 1) cancels the rounding of u (D. Goldberg, "What every
// computer scientist should know about floating-point arithmetic", 1991);
// log(u) from the hardware base-2 logarithm, the quotient from the hardware
// reciprocal.
__device__ __forceinline__ float log1p_fast(float x) {
    const float u = 1.0f + x;
    if (u == 1.0f) return x;
    return __builtin_amdgcn_logf(u) * 0.69314718055994531f * (x * __builtin_amdgcn_rcpf(u - 1.0f));
}

// x / y through the hardware reciprocal (about 1 ulp each)
__device__ __forceinline__ float fast_div(float x, float y) { return x * __builtin_amdgcn_rcpf(y); }

// Weight of the linear branch from the gate logit of one (token, query head):
// gamma = sigmoid(g) (g = -inf gives 0, +inf gives 1); 1 without a gate.
__device__ __forceinline__ float gate_weight(const float* __restrict__ gate, size_t i) {
    return gate ? 1.f / (1.f + expf(-gate[i])) : 1.f;
}

// Sort key of a routing score: -0 counts as +0 and NaN ranks below every
// number, so that float comparison of keys gives the selection order.
__device__ __forceinline__ float route_key(float s) {
    if (s != s) return -__builtin_inff();
    return s == 0.0f ? 0.0f : s;
}

// Order-preserving map of a sort key (route_key: no NaN, no -0) to 32 bits:
// a larger key gives a larger unsigned value.
__device__ __forceinline__ uint32_t key_bits(float k) {
    const uint32_t u = __float_as_uint(k);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Per-chunk top-lam (full text Sec. 3.3, chunk-level selection) by one wave:
// the lam largest of the n <= 64 R keys it holds (position p = 64 r + lane in
// key[r], mapped by key_bits), ties to the lower position.  A radix select
// finds the lam-th largest value T from the top bit down, one ballot per
// bit and register (a candidate matches the bits fixed so far; if at least
// `need` candidates have the bit set, T has it, else those candidates are
// all kept and need shrinks by their count); then every key above T is
// kept, and of the keys equal to T the first `need` in position order (one
// more ballot per register gives each its rank).  O(32 R) wave steps
// instead of a rank count's O(C^2).  Every lane of the wave must call it;
// sel[r] says whether position 64 r + lane is kept, rank[r] its index among
// the kept positions in position order.
template <int R>
__device__ __forceinline__ void wave_topk(const uint32_t (&key)[R], int n, int lam, bool (&sel)[R],
                                          int (&rank)[R]) {
    const int lane = threadIdx.x & 63;
    uint32_t prefix = 0u, fixed = 0u;
    int need = lam;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t b = 1u << bit;
        int cnt = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const bool cand = 64 * r + lane < n && (key[r] & fixed) == prefix && (key[r] & b) != 0u;
            cnt += __popcll(__ballot(cand));
        }
        if (cnt >= need) prefix |= b;
        else need -= cnt;
        fixed |= b;
    }
    const uint64_t below = (1ull << lane) - 1ull;
    int ties = 0, kept = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool valid = 64 * r + lane < n;
        const uint64_t eq = __ballot(valid && key[r] == prefix);
        const bool s = valid && (key[r] > prefix || (key[r] == prefix && ties + __popcll(eq & below) < need));
        const uint64_t sm = __ballot(s);
        sel[r] = s;
        rank[r] = kept + __popcll(sm & below);
        ties += __popcll(eq);
        kept += __popcll(sm);
    }
}

// One Self-Saliency term.  For the diagonal (own) key:
//   a_t ln((a_t + eps)/eps) = a_t log1p(a_t / eps).
// For another key j of the row, with e_j the unnormalised weight, sa the row
// sum and so the row sum without the diagonal (a~_j = e_j / so):
//   a_j ln((a_j + eps)/(a~_j + eps)) = -a_j log1p((a~_j - a_j)/(a_j + eps)),
//   a~_j - a_j = e_j e_t / (so sa)  (no cancellation).
__device__ __forceinline__ float saliency_term(float e, bool is_diag, float et, float sa, float so,
                                               float eps) {
    if (e == 0.0f) return 0.0f;
    float a = e / sa;
    if (is_diag) return a * log1pf(a / eps);
    float diff = (e * et) / (so * sa);
    return -a * log1pf(diff / (a + eps));
}

}  // namespace still
