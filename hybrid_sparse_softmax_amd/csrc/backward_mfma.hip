// Key side of the STILL backward pass on the gfx950 matrix cores (bf16
// storage, head_dim 128, chunk 64, window 64 NWT), routing held fixed.
//
// For a key j and every query t that attends to it by softmax (its window
// t in [j, j + W - 1], and every later query t >= j + W when j is selected;
// full text Sec. 3.3), with P_tj = exp(tau q_t.k_j - m_t) / l_t and the
// first pass's statistics (m_t, l_t, D_t = dout_t . out_t):
//   dv_j += sum_t P_tj dout_t
//   dk_j += tau sum_t dS_tj q_t,   dS_tj = P_tj (dout_t . v_j - D_t)
// summed over the query heads of the KV group.  One wave owns 32 keys (K and
// V rows in registers as the B operands) and streams 64-query tiles of one
// head through LDS: per half tile of 32 queries
//   S  = Q K^T,  dP = dout V^T          (queries x keys)
//   dV^T += dout^T P,  dK^T += Q^T dS   (dims x keys, dS and P rounded to bf16)
// 64 products per wave and query tile.  Two launches:
//   window    keys of chunk c' in position order, query chunks c' .. c'+NWT
//             (causal in c'; in c'+NWT the window part plus, for a selected
//             key, the routed part); writes dk and adds to dv (which holds
//             the linear terms written before)
//   selected  the compact selected rows (positions from the selection),
//             every query chunk after their window: the visible rows of a
//             tile are a prefix (rows of chunks <= c - NWT - 1); adds to dk
//             and dv.
// The linear terms of dk / dv come from the fp32 kernels.
#include "launch.h"
#include "mfma_common.h"
#include "mfma_tiles.h"

namespace still {

namespace {
using namespace mt;

constexpr int kKW = 4;  // waves per block: 128 keys

// staged query tile of one head: rows t0 .. t0 + 63 (zero past N)
struct QTile {
    bf16 qs[kC * kKS];    // Q rows (A operand of S = Q K^T)
    bf16 ds[kC * kKS];    // dout rows (A operand of dP = dout V^T)
    bf16 qt[kD * kVS];    // Q^T (A operand of dK^T = Q^T dS)
    bf16 dt[kD * kVS];    // dout^T (A operand of dV^T = dout^T P)
    float lse2[kC];       // log2 of exp(m) l: P = 2^(s tau log2 e - lse2)
    float dd[kC];         // D = dout . out
};

__device__ __forceinline__ void stage_qtile(QTile& T, const bf16* __restrict__ q,
                                            const bf16* __restrict__ dout,
                                            const float* __restrict__ stat, const Dims& D, int b,
                                            int t0, int h, int tid, int nthr) {
    const int nv = min(kC, D.N - t0);
    const size_t ld = (size_t)D.Hq * kD;
    const size_t o = (((size_t)b * D.N + t0) * D.Hq + h) * kD;
    load_k_tile(q + o, ld, nv, T.qs, tid, nthr);
    load_k_tile(dout + o, ld, nv, T.ds, tid, nthr);
    load_vt_tile(q + o, ld, nv, T.qt, tid, nthr);
    load_vt_tile(dout + o, ld, nv, T.dt, tid, nthr);
    if (tid < kC) {
        float a = 0.f, dd = 0.f;
        if (tid < nv) {
            const f32x4 st = *reinterpret_cast<const f32x4*>(stat + ((((size_t)b * D.N + t0 + tid) * D.Hq + h) * 4));
            a = st[0] * kLog2e + __log2f(st[1]);
            dd = st[2];
        }
        T.lse2[tid] = a;
        T.dd[tid] = dd;
    }
}

// One wave's contribution of a staged query tile to its 32 keys.  vis(r)
// says whether query row r (0..63 of the tile) attends to this lane's key
// by softmax.
template <typename Vis>
__device__ __forceinline__ void key_tile(const QTile& T, const bf16x8 (&kf)[8], const bf16x8 (&vf)[8],
                                         float cl2, Vis vis, f32x16 (&dva)[4], f32x16 (&dka)[4]) {
    const int lane = threadIdx.x & 63, hf = lane >> 5, col = lane & 31;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        f32x16 s = zero16(), dp = zero16();
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            s = mfma32(ld_bf8(T.qs + (32 * qb + col) * kKS + 16 * st + 8 * hf), kf[st], s);
            dp = mfma32(ld_bf8(T.ds + (32 * qb + col) * kKS + 16 * st + 8 * hf), vf[st], dp);
        }
        // rows are queries 32 qb + acc_row(vv, hf), the column is the lane's key
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const int r0 = 32 * qb + acc_row(4 * v4, hf);
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(T.lse2 + r0);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(T.dd + r0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int vv = 4 * v4 + j;
                const float p = vis(r0 + j) ? __builtin_amdgcn_exp2f(fmaf(s[vv], cl2, -l4[j])) : 0.f;
                s[vv] = p;
                dp[vv] = p * (dp[vv] - d4[j]);
            }
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const bf16x8 pp = pack_acc(s, s2), pd = pack_acc(dp, s2);
            const int ks = 2 * qb + s2;  // queries 16 ks .. 16 ks + 15 of the tile
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                dva[dt] = mfma32(ld_bf8(T.dt + (32 * dt + col) * kVS + 16 * ks + 8 * hf), pp, dva[dt]);
                dka[dt] = mfma32(ld_bf8(T.qt + (32 * dt + col) * kVS + 16 * ks + 8 * hf), pd, dka[dt]);
            }
        }
    }
}

// B operand rows of key row `row` (bf16, 128 dims): dims 16 s + 8 hf .. +7
__device__ __forceinline__ void load_key_operand(const bf16* __restrict__ row, bf16x8 (&x)[8]) {
    const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int s = 0; s < 8; ++s) x[s] = ld_bf8(row + 16 * s + 8 * hf);
}

// window keys: block = 128 keys of chunks 2 cb, 2 cb + 1 of (b, g)
template <int NWT>
__global__ __launch_bounds__(kKW * 64) void bwd_kv_window_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const uint8_t* __restrict__ route, const float* __restrict__ stat,
    float* __restrict__ dk, float* __restrict__ dv, Dims D) {
    const int npair = (D.T + 1) / 2;
    const int cb = (int)(blockIdx.x % npair);
    const int bgi = (int)(blockIdx.x / npair);
    const int g = bgi % D.Hkv, b = bgi / D.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hf = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ck = 2 * cb + (wave >> 1);           // this wave's key chunk
    const int ok = 32 * (wave & 1) + col;          // the lane's key offset in it
    const int j = ck * kC + ok;
    const bool kvalid = j < D.N;
    const size_t bg = (size_t)b * D.Hkv + g;
    const int jr = min(j, D.N - 1);
    bf16x8 kf[8], vf[8];
    load_key_operand(k + (((size_t)b * D.N + jr) * D.Hkv + g) * kD, kf);
    load_key_operand(v + (((size_t)b * D.N + jr) * D.Hkv + g) * kD, vf);
    const bool ksel = kvalid && route[bg * D.N + jr] == kRouteSA;
    const float cl2 = D.tau * kLog2e;
    f32x16 dva[4], dka[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) dva[dt] = dka[dt] = zero16();

    __shared__ QTile T;
    const int c_first = 2 * cb, c_last = min(D.T - 1, 2 * cb + 1 + NWT);
    for (int qc = c_first; qc <= c_last; ++qc) {
        const int i = qc - ck;  // query chunk relative to this wave's key chunk
        const int t0 = qc * kC;
        for (int hh = 0; hh < D.G; ++hh) {
            __syncthreads();
            stage_qtile(T, q, dout, stat, D, b, t0, g * D.G + hh, tid, kKW * 64);
            __syncthreads();
            if (i < 0 || i > NWT || ck >= D.T) continue;
            const int nq = min(kC, D.N - t0);
            key_tile(T, kf, vf, cl2,
                     [&](int r) {
                         if (!kvalid || r >= nq) return false;
                         if (i == 0) return r >= ok;                   // causal
                         if (i < NWT) return true;                      // inside the window
                         return r < ok || ksel;                         // window part, routed selected
                     },
                     dva, dka);
        }
    }
    if (!kvalid) return;
    const size_t o = (((size_t)b * D.N + j) * D.Hkv + g) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const int e = 32 * dt + acc_row(4 * v4, hf);
            f32x4 a4, b4;
            const f32x4 v_old = *reinterpret_cast<const f32x4*>(dv + o + e);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                a4[jj] = D.tau * dka[dt][4 * v4 + jj];
                b4[jj] = v_old[jj] + dva[dt][4 * v4 + jj];
            }
            *reinterpret_cast<f32x4*>(dk + o + e) = a4;
            *reinterpret_cast<f32x4*>(dv + o + e) = b4;
        }
}

// selected keys: block = 128 consecutive compact rows of (b, g)
template <int NWT>
__global__ __launch_bounds__(kKW * 64) void bwd_kv_selected_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ ksel, const bf16* __restrict__ vsel,
    const bf16* __restrict__ dout, const int32_t* __restrict__ selw, const int* __restrict__ list_off,
    const float* __restrict__ stat, float* __restrict__ dk, float* __restrict__ dv, Dims D) {
    const int ntile = (D.n_full * D.lam + kKW * 32 - 1) / (kKW * 32);
    const int tb = (int)(blockIdx.x % ntile);
    const int bgi = (int)(blockIdx.x / ntile);
    const int g = bgi % D.Hkv, b = bgi / D.Hkv;
    const size_t bg = (size_t)b * D.Hkv + g;
    const int* loff = list_off + bg * (D.n_full + 1);
    const int total = loff[D.n_full];
    const int r_blk = tb * kKW * 32;
    if (r_blk >= total) return;  // every wave of the block leaves together
    const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hf = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = r_blk + 32 * wave + col;  // the lane's compact row
    const bool rvalid = r < total;
    // the row's chunk (loff[c] <= r < loff[c + 1]) and position
    int lo = 0, hi = D.n_full;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (loff[mid] <= min(r, total - 1)) lo = mid;
        else hi = mid;
    }
    const int crow = lo;
    const int pos = rvalid ? selw[(bg * D.n_full + crow) * D.lam + (r - loff[crow])] : 0;
    const size_t ldl = (size_t)D.Hkv * kD;
    const size_t rowo = ((size_t)b * sel_list_rows(D) * D.Hkv + g) * kD + (size_t)min(r, total - 1) * ldl;
    bf16x8 kf[8], vf[8];
    load_key_operand(ksel + rowo, kf);
    load_key_operand(vsel + rowo, vf);
    const float cl2 = D.tau * kLog2e;
    f32x16 dva[4], dka[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) dva[dt] = dka[dt] = zero16();

    // the block's first row belongs to chunk c0; query chunk qc sees the
    // rows of chunks <= qc - NWT - 1
    int c0 = 0;
    while (c0 + 1 < D.n_full && loff[c0 + 1] <= r_blk) ++c0;
    __shared__ QTile T;
    for (int qc = c0 + NWT + 1; qc < D.T; ++qc) {
        const int nvis = loff[min(qc - NWT, D.n_full)] - r_blk;  // visible rows: a prefix
        const int t0 = qc * kC;
        const int nq = min(kC, D.N - t0);
        for (int hh = 0; hh < D.G; ++hh) {
            __syncthreads();
            stage_qtile(T, q, dout, stat, D, b, t0, g * D.G + hh, tid, kKW * 64);
            __syncthreads();
            if (32 * wave >= nvis) continue;
            const bool rv = rvalid && 32 * wave + col < nvis;
            key_tile(T, kf, vf, cl2, [&](int rr) { return rv && rr < nq; }, dva, dka);
        }
    }
    if (!rvalid) return;
    const size_t o = (((size_t)b * D.N + pos) * D.Hkv + g) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const int e = 32 * dt + acc_row(4 * v4, hf);
            f32x4 a4 = *reinterpret_cast<const f32x4*>(dk + o + e);
            f32x4 b4 = *reinterpret_cast<const f32x4*>(dv + o + e);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                a4[jj] += D.tau * dka[dt][4 * v4 + jj];
                b4[jj] += dva[dt][4 * v4 + jj];
            }
            *reinterpret_cast<f32x4*>(dk + o + e) = a4;
            *reinterpret_cast<f32x4*>(dv + o + e) = b4;
        }
}

}  // namespace

hipError_t launch_bwd_kv(const Dims& D, const void* q, const void* k, const void* v, const void* dout,
                         const uint8_t* route, const void* ksel, const void* vsel,
                         const int32_t* selw, const int* list_off, const float* stat, float* dk,
                         float* dv, int phase, hipStream_t s) {
    const bf16* qq = reinterpret_cast<const bf16*>(q);
    const bf16* dd = reinterpret_cast<const bf16*>(dout);
    const int nwt = D.W / kC;
    if (phase == 0) {
        const unsigned nblk = (unsigned)((D.T + 1) / 2) * D.B * D.Hkv;
#define STILL_KVW(NWT)                                                                           \
    hipLaunchKernelGGL((bwd_kv_window_kernel<NWT>), dim3(nblk), dim3(kKW * 64), 0, s, qq,       \
                       reinterpret_cast<const bf16*>(k), reinterpret_cast<const bf16*>(v), dd,  \
                       route, stat, dk, dv, D)
        if (nwt == 1) STILL_KVW(1);
        else if (nwt == 2) STILL_KVW(2);
        else STILL_KVW(4);
#undef STILL_KVW
        return hipGetLastError();
    }
    if (D.lam == 0 || D.n_full == 0) return hipSuccess;
    const int ntile = (D.n_full * D.lam + kKW * 32 - 1) / (kKW * 32);
    const unsigned nblk = (unsigned)ntile * D.B * D.Hkv;
#define STILL_KVS(NWT)                                                                           \
    hipLaunchKernelGGL((bwd_kv_selected_kernel<NWT>), dim3(nblk), dim3(kKW * 64), 0, s, qq,     \
                       reinterpret_cast<const bf16*>(ksel), reinterpret_cast<const bf16*>(vsel), \
                       dd, selw, list_off, stat, dk, dv, D)
    if (nwt == 1) STILL_KVS(1);
    else if (nwt == 2) STILL_KVS(2);
    else STILL_KVS(4);
#undef STILL_KVS
    return hipGetLastError();
}

}  // namespace still
