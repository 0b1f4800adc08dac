// The STILL backward pass on the gfx950 matrix cores (bf16 storage,
// head_dim 128, 64-token tiles, window 64 NWT), routing held fixed: every
// kernel of the matrix-core path but the lists and the first pass (the
// forward's main kernel with statistics, prefill_mfma.hip; skipped when the
// forward's statistics are given).
//
// Softmax terms.  For a key j and every query t that attends to it by
// softmax (its window t in [j, j + W - 1], and every later query t >= j + W
// when j is selected; full text Sec. 3.3), with P_tj = exp(tau q_t.k_j -
// m_t) / l_t and the first pass's statistics (m_t, l_t, D_t = dout_t . out_t):
//   dv_j += sum_t P_tj dout_t
//   dk_j += tau sum_t dS_tj q_t,   dS_tj = P_tj (dout_t . v_j - D_t)
//   dq_t += tau sum_j dS_tj k_j
// summed over the query heads of the KV group.  Key kernels: one wave owns
// 32 keys (K and V rows in registers as the B operands) and streams 64-query
// tiles of one head through LDS: per half tile of 32 queries
//   S  = Q K^T,  dP = dout V^T          (queries x keys)
//   dV^T += dout^T P,  dK^T += Q^T dS   (dims x keys, dS and P rounded to bf16)
// 64 products per wave and query tile.  Two launches:
//   window    keys of chunk c' in position order, query chunks c' .. c'+NWT
//             (causal in c'; in c'+NWT the window part plus, for a selected
//             key, the routed part); adds to dk and dv (which hold the
//             NP-Map and linear terms written before)
//   selected  the compact selected rows (positions from the selection),
//             every query chunk after their window: the visible rows of a
//             tile are a prefix (rows of chunks <= c - NWT - 1); adds to dk
//             and dv.
// The query kernel streams the forward's key tiles for dq, then forms the
// gradient of the queries' features (dphi_q, dgate) and carries it through
// their NP-Map backward into dq.  The keys' linear terms with their NP-Map
// backward, and the projection gradients, follow below.
#include "launch.h"
#include "mfma_common.h"
#include "mfma_tiles.h"
#include "row_ops.h"

namespace still {

namespace {
using namespace mt;


// key kernels: the window kernel's block takes kWinKPB key chunks (two
// waves per chunk), the selected kernel's kSelW waves of 32 compact rows
constexpr int kWinKPB = 2;
constexpr int kSelW = 4;

// staged query tile of one head: rows t0 .. t0 + 63 (zero past N)
struct QTile {
    bf16 qs[kC * kKS];    // Q rows (A operand of S = Q K^T)
    bf16 ds[kC * kKS];    // dout rows (A operand of dP = dout V^T)
    bf16 qt[kD * kVS];    // Q^T (A operand of dK^T = Q^T dS)
    bf16 dt[kD * kVS];    // dout^T (A operand of dV^T = dout^T P)
    float lse2[kC];       // log2 of exp(m) l: P = 2^(s tau log2 e - lse2)
    float dd[kC];         // D = dout . out
};

// Streams the query tiles of steps 0 .. nstep-1 (step n: the 64 queries
// from t0 of head h, step_of(n, t0, h)) through two LDS buffers for a block
// of 512 threads, calling body(n, tile) for each step with every wave.  The
// Q and dout rows (padded layout; rows past N repeat the last one) and the
// raw statistics of step n+1 come by DMA (global_load_lds) while step n is
// computed; once they have landed, the block builds the transposed copies
// (Q by threads 0-255, dout by 256-511) and the statistics in LDS.
template <typename StepOf, typename Body>
__device__ __forceinline__ void stream_qtiles(QTile (&T2)[2], float (&rawst)[2][kC * 4], int nstep,
                                              StepOf step_of, Body body, const bf16* __restrict__ q,
                                              const bf16* __restrict__ dout, const float* __restrict__ stat,
                                              const Dims& D, int b) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    auto issue = [&](int n) {
        int t0, h;
        step_of(n, t0, h);
        const int nv = min(kC, D.N - t0);
        const size_t o = (((size_t)b * D.N + t0) * D.Hq + h) * kD;
        QTile& B = T2[n & 1];
        const unsigned qd = (unsigned)(size_t)(lds_void*)B.qs, dd = (unsigned)(size_t)(lds_void*)B.ds;
        for (int x = wv; x < kKPieces; x += 8) {
            stage_k_piece_u(x, q + o, D.Hq * kD, nv, qd);
            stage_k_piece_u(x, dout + o, D.Hq * kD, nv, dd);
        }
        if (wv == 7) {
            const float* ss = stat + (((size_t)b * D.N + t0 + min(lane, nv - 1)) * D.Hq + h) * 4;
            dma16_untracked(reinterpret_cast<const bf16*>(ss), (unsigned)(size_t)(lds_void*)rawst[n & 1]);
        }
    };
    auto finish = [&](int n) {
        int t0, h;
        step_of(n, t0, h);
        const int nv = min(kC, D.N - t0);
        QTile& B = T2[n & 1];
        const bf16* src = tid < 256 ? B.qs : B.ds;
        bf16* dst = tid < 256 ? B.qt : B.dt;
        const int x = tid & 255, kq = x & 15, oct = x >> 4;  // rows 4 kq .. +3, columns 8 oct .. +7
        bf16x8 r4[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) r4[rr] = ld_bf8(src + (4 * kq + rr) * kKS + 8 * oct);
        const int pos = kperm(4 * kq);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16x4 t4;
            t4[0] = r4[0][e];
            t4[1] = r4[1][e];
            t4[2] = r4[2][e];
            t4[3] = r4[3][e];
            *reinterpret_cast<bf16x4*>(dst + (8 * oct + e) * kVS + pos) = t4;
        }
        if (tid < kC) {
            const f32x4 st = *reinterpret_cast<const f32x4*>(rawst[n & 1] + 4 * tid);
            B.lse2[tid] = tid < nv ? st[0] * kLog2e + __log2f(st[1]) : 0.f;  // P = 2^(s tau log2 e - lse2)
            B.dd[tid] = tid < nv ? st[2] : 0.f;
        }
    };
    if (nstep > 0) issue(0);
    for (int n = 0; n < nstep; ++n) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's share of step n
        __syncthreads();                      // every share landed; step n-1 is done
        finish(n);
        __syncthreads();
        if (n + 1 < nstep) issue(n + 1);  // into the buffer of step n-1
        body(n, T2[n & 1]);
    }
}

// One staged query tile's contribution to a block's key groups of 32 keys,
// each group shared by two waves (on one SIMD): role 0 holds the group's K
// rows and forms S = Q K^T, P and dV^T += dout^T P; role 1 holds the V rows
// and forms dP = dout V^T, then dS = P (dP - D) with the P its partner
// hands over through LDS (bf16, packed as the value product's operand, lane
// for lane), and dK^T += Q^T dS.  vis(r) says whether query row r (0..63 of
// the tile) attends to the lane's key by softmax; act (wave-uniform) whether
// the group has a key the tile's queries see.  Every wave of the block calls
// it (one barrier inside).
template <int NG, typename Vis>
__device__ __forceinline__ void key_tile_split(const QTile& T, const bf16x8 (&kv)[8], int role, int grp,
                                               float cl2, bool act, Vis vis,
                                               bf16x8 (&pbuf)[NG][2][2][64], f32x16 (&acc)[4]) {
    const int lane = threadIdx.x & 63, hf = lane >> 5, col = lane & 31;
    f32x16 x[2];  // role 0: P, role 1: dP (rows: queries 32 qb + acc_row, column: the lane's key)
    if (act) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            x[qb] = zero16();
            const bf16* A = role == 0 ? T.qs : T.ds;
#pragma unroll
            for (int st = 0; st < 8; ++st)
                x[qb] = mfma32(ld_bf8(A + (32 * qb + col) * kKS + 16 * st + 8 * hf), kv[st], x[qb]);
            if (role == 0) {
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const int r0 = 32 * qb + acc_row(4 * v4, hf);
                    const f32x4 l4 = *reinterpret_cast<const f32x4*>(T.lse2 + r0);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int vv = 4 * v4 + j;
                        x[qb][vv] = vis(r0 + j) ? __builtin_amdgcn_exp2f(fmaf(x[qb][vv], cl2, -l4[j])) : 0.f;
                    }
                }
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) pbuf[grp][qb][s2][lane] = pack_acc(x[qb], s2);
            }
        }
    }
    __syncthreads();  // every group's P is in pbuf
    if (!act) return;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            bf16x8 pk = pbuf[grp][qb][s2][lane];
            if (role == 1) {
                // dS on the same accumulator elements (element j of k-step s2
                // is element 8 s2 + j)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int vv = 8 * s2 + j;
                    pk[j] = (bf16)((float)pk[j] * (x[qb][vv] - T.dd[32 * qb + acc_row(vv, hf)]));
                }
            }
            const int ks = 2 * qb + s2;  // queries 16 ks .. 16 ks + 15 of the tile
            const bf16* A = role == 0 ? T.dt : T.qt;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                acc[dt] = mfma32(ld_bf8(A + (32 * dt + col) * kVS + 16 * ks + 8 * hf), pk, acc[dt]);
        }
}

// B operand rows of key row `row` (bf16, 128 dims): dims 16 s + 8 hf .. +7
__device__ __forceinline__ void load_key_operand(const bf16* __restrict__ row, bf16x8 (&x)[8]) {
    const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int s = 0; s < 8; ++s) x[s] = ld_bf8(row + 16 * s + 8 * hf);
}

// window keys: block = 128 keys of chunks 2 cb, 2 cb + 1 of (b, g), four
// groups of 32 keys, two waves each (key_tile_split)
template <int NWT, int KPB>
__global__ __launch_bounds__(KPB * 256) __attribute__((amdgpu_waves_per_eu(2))) void bwd_kv_window_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const uint8_t* __restrict__ route, const float* __restrict__ stat,
    float* __restrict__ dk, float* __restrict__ dv, Dims D) {
    static_assert(KPB * 256 == 512, "stream_qtiles takes blocks of 512 threads");
    const int npair = (D.T + KPB - 1) / KPB;
    const int cb = (int)(blockIdx.x % npair);
    const int bgi = (int)(blockIdx.x / npair);
    const int g = bgi % D.Hkv, b = bgi / D.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hf = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave = wv % (2 * KPB), role = wv / (2 * KPB);  // key group; 0: P and dv, 1: dS and dk
    const int ck = KPB * cb + (wave >> 1);         // this group's key chunk
    const int ok = 32 * (wave & 1) + col;          // the lane's key offset in it
    const int j = ck * kC + ok;
    const bool kvalid = j < D.N;
    const size_t bg = (size_t)b * D.Hkv + g;
    const int jr = min(j, D.N - 1);
    bf16x8 kv[8];  // role 0: K rows, role 1: V rows
    load_key_operand((role == 0 ? k : v) + (((size_t)b * D.N + jr) * D.Hkv + g) * kD, kv);
    const bool ksel = kvalid && route[bg * D.N + jr] == kRouteSA;
    const float cl2 = D.tau * kLog2e;
    f32x16 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = zero16();

    __shared__ QTile T2[2];
    __shared__ __align__(16) float rawst[2][kC * 4];
    __shared__ __align__(16) bf16x8 pbuf[2 * KPB][2][2][64];
    // steps: query chunks c_first .. c_last, every head of the group
    const int c_first = KPB * cb, c_last = min(D.T - 1, KPB * cb + KPB - 1 + NWT);
    stream_qtiles(
        T2, rawst, (c_last - c_first + 1) * D.G,
        [&](int n, int& t0, int& h) {
            t0 = (c_first + n / D.G) * kC;
            h = g * D.G + n % D.G;
        },
        [&](int n, const QTile& T) {
            const int qc = c_first + n / D.G;
            const int i = qc - ck;  // query chunk relative to this group's key chunk
            const int nq = min(kC, D.N - qc * kC);
            key_tile_split(T, kv, role, wave, cl2, !(i < 0 || i > NWT || ck >= D.T),
                           [&](int r) {
                               if (!kvalid || r >= nq) return false;
                               if (i == 0) return r >= ok;                   // causal
                               if (i < NWT) return true;                      // inside the window
                               return r < ok || ksel;                         // window part, routed selected
                           },
                           pbuf, acc);
        },
        q, dout, stat, D, b);
    if (!kvalid) return;
    // role 0 adds to dv, role 1 tau times its sums to dk
    const size_t o = (((size_t)b * D.N + j) * D.Hkv + g) * kD;
    float* dst = role == 1 ? dk : dv;
    const float sc = role == 1 ? D.tau : 1.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const int e = 32 * dt + acc_row(4 * v4, hf);
            f32x4 a4 = *reinterpret_cast<const f32x4*>(dst + o + e);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) a4[jj] += sc * acc[dt][4 * v4 + jj];
            *reinterpret_cast<f32x4*>(dst + o + e) = a4;
        }
}

// selected keys: block = 128 consecutive compact rows of (b, g) and one of
// kSelSeg segments of the query chunks after their window (rows of early
// chunks meet many more query chunks than late ones; the segments spread
// that work over blocks).  Segment 0 adds its sums to dk and dv; the others
// write theirs to part [kSelSeg - 1][B, Hkv, n_full lam][2 d] (zeros for an
// empty segment), which bwd_kv_merge_kernel adds afterwards: no atomics, a
// fixed order of summation.
constexpr int kSelSeg = 2;
template <int NWT, int KW>
__global__ __launch_bounds__(KW * 128) __attribute__((amdgpu_waves_per_eu(2))) void bwd_kv_selected_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ ksel, const bf16* __restrict__ vsel,
    const bf16* __restrict__ dout, const int32_t* __restrict__ selw, const int* __restrict__ list_off,
    const float* __restrict__ stat, float* __restrict__ dk, float* __restrict__ dv,
    float* __restrict__ part, Dims D) {
    static_assert(KW * 128 == 512, "stream_qtiles takes blocks of 512 threads");
    // blocks in order of (row tile, segment), every (b, g) side by side:
    // earlier row tiles meet more query chunks, so the longest go first
    const int nbg = D.B * D.Hkv;
    const int bgi = (int)(blockIdx.x % nbg);
    const int sg = (int)((blockIdx.x / nbg) % kSelSeg);
    const int tb = (int)(blockIdx.x / nbg / kSelSeg);
    const int g = bgi % D.Hkv, b = bgi / D.Hkv;
    const size_t bg = (size_t)b * D.Hkv + g;
    const int* loff = list_off + bg * (D.n_full + 1);
    const int total = loff[D.n_full];
    const int r_blk = tb * KW * 32;
    if (r_blk >= total) return;  // every wave of the block leaves together
    const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hf = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave = wv % KW, role = wv / KW;  // key group; 0: P and dv, 1: dS and dk
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
    bf16x8 kv[8];  // role 0: K rows, role 1: V rows
    load_key_operand((role == 0 ? ksel : vsel) + rowo, kv);
    const float cl2 = D.tau * kLog2e;
    f32x16 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = zero16();
    __shared__ __align__(16) bf16x8 pbuf[KW][2][2][64];

    // the block's first row belongs to chunk c0; query chunk qc sees the
    // rows of chunks <= qc - NWT - 1; this block takes segment sg of the
    // query chunks c0 + NWT + 1 .. T - 1
    int c0 = 0;
    while (c0 + 1 < D.n_full && loff[c0 + 1] <= r_blk) ++c0;
    const int qa = c0 + NWT + 1, nq_all = max(0, D.T - qa);
    const int seg_len = (nq_all + kSelSeg - 1) / kSelSeg;
    const int q_lo = qa + sg * seg_len, q_hi = min(D.T, q_lo + seg_len);
    __shared__ QTile T2[2];
    __shared__ __align__(16) float rawst[2][kC * 4];
    // steps: query chunks q_lo .. q_hi - 1, every head of the group
    stream_qtiles(
        T2, rawst, (q_hi - q_lo) * D.G,
        [&](int n, int& t0, int& h) {
            t0 = (q_lo + n / D.G) * kC;
            h = g * D.G + n % D.G;
        },
        [&](int n, const QTile& T) {
            const int qc = q_lo + n / D.G;
            const int nvis = loff[min(qc - NWT, D.n_full)] - r_blk;  // visible rows: a prefix
            const int nq = min(kC, D.N - qc * kC);
            const bool rv = rvalid && 32 * wave + col < nvis;
            key_tile_split(T, kv, role, wave, cl2, 32 * wave < nvis, [&](int rr) { return rv && rr < nq; },
                           pbuf, acc);
        },
        q, dout, stat, D, b);
    if (!rvalid) return;
    // role 0's sums are dv's, role 1's (times tau) dk's
    const float sc = role == 1 ? D.tau : 1.f;
    if (sg > 0) {
        float* pr = part + (((size_t)(sg - 1) * D.B * D.Hkv + bg) * ((size_t)D.n_full * D.lam) + r) * (2 * kD) +
                    (role == 1 ? 0 : kD);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int e = 32 * dt + acc_row(4 * v4, hf);
                f32x4 a4;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) a4[jj] = sc * acc[dt][4 * v4 + jj];
                *reinterpret_cast<f32x4*>(pr + e) = a4;
            }
        return;
    }
    const size_t o = (((size_t)b * D.N + pos) * D.Hkv + g) * kD;
    float* dst = role == 1 ? dk : dv;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const int e = 32 * dt + acc_row(4 * v4, hf);
            f32x4 a4 = *reinterpret_cast<const f32x4*>(dst + o + e);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) a4[jj] += sc * acc[dt][4 * v4 + jj];
            *reinterpret_cast<f32x4*>(dst + o + e) = a4;
        }
}

// Adds the later segments' sums of every compact row to dk and dv of its
// position: one wave per row, four floats per lane (dk then dv).
__global__ __launch_bounds__(256) void bwd_kv_merge_kernel(const float* __restrict__ part,
                                                           const int32_t* __restrict__ selw,
                                                           const int* __restrict__ list_off,
                                                           float* __restrict__ dk, float* __restrict__ dv,
                                                           Dims D) {
    const int g = blockIdx.y, b = blockIdx.z;
    const size_t bg = (size_t)b * D.Hkv + g;
    const int* loff = list_off + bg * (D.n_full + 1);
    const int total = loff[D.n_full];
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (r >= total) return;
    int lo = 0, hi = D.n_full;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (loff[mid] <= r) lo = mid;
        else hi = mid;
    }
    const int pos = selw[(bg * D.n_full + lo) * D.lam + (r - loff[lo])];
    const size_t rows = (size_t)D.n_full * D.lam;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int sg = 1; sg < kSelSeg; ++sg)
        acc += *reinterpret_cast<const f32x4*>(part + (((size_t)(sg - 1) * D.B * D.Hkv + bg) * rows + r) * (2 * kD) + 4 * lane);
    float* dst = (lane < kD / 4 ? dk : dv) + (((size_t)b * D.N + pos) * D.Hkv + g) * kD + 4 * (lane % (kD / 4));
    *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<const f32x4*>(dst) + acc;
}


// ---------------------------------------------------------------------------
// Query side: dq's softmax part, the linear terms of the queries' gated
// features, and their NP-Map backward.  Block = HB query heads of KV head g x
// the 64 queries of chunk c (two waves per head, 32 queries each), the key
// tiles of the forward (window chunks c-NWT+1 .. c, the compact selected
// rows, and the partly covered chunk c-NWT last, each with its mask).  Per
// tile, with the statistics (m, l, D) and P = exp(tau q.k - m) / l:
//   S^T  = K Q^T           (logits, keys x queries)
//   dP^T = V dout^T        (dout . v_j)
//   dS^T = P^T (dP^T - D)  rounded to bf16 as the forward rounds P
//   dQ^T += K^T dS^T       (K read transposed from LDS)
// Then, for a query with linear mass (c_t = exp(-m) / l > 0; full text
// Sec. 3.3, the chunk-wise linear branch with the shared normaliser), the
// gradient w.r.t. its gated features fq = gamma phi_q:
//   dfq = c_t (S dout - D z + sum over the routed unselected keys j of
//         chunk c-NWT at or below the query's offset of (dout . v_j - D) phi_k(j))
// with S, z the linear prefix of chunks <= c-NWT-1 (within-run part plus the
// earlier runs', summed in fp32 and rounded to bf16 once), on the matrix
// cores in the prefix's feature order.  dphi_q = gamma dfq goes through the
// NP-Map backward into dQ^T; the same pass gives gamma phi_q (bf16) for the
// kernels after this one and the gate logit's gradient gamma (1 - gamma)
// phi_q . dfq.  dq = tau (dQ^T)^T plus the norm term is written once, fp32.
template <int HB, int NWT>
__global__ __launch_bounds__(HB * 128) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const uint8_t* __restrict__ route,
    const bf16* __restrict__ ksel, const bf16* __restrict__ vsel, const int* __restrict__ list_off,
    float* __restrict__ stat, const bf16* __restrict__ phik, LinBufs L,
    const float* __restrict__ gate, bf16* __restrict__ phiq, float* __restrict__ dq,
    bf16* __restrict__ du_out, float* __restrict__ dgate, const float* __restrict__ stat_in,
    const bf16* __restrict__ out, const bf16* __restrict__ wqh, const bf16* __restrict__ wql, Dims D) {
    constexpr int NW = HB * 2;
    const int HG = D.G / HB;
    const int per_c = D.B * D.Hkv * HG;
    const int c = D.T - 1 - (int)(blockIdx.x / per_c);
    int r = (int)(blockIdx.x % per_c);
    const int hg = r % HG;
    r /= HG;
    const int g = r % D.Hkv, b = r / D.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, col = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qh = wave / HB;
    const int h = g * D.G + hg * HB + wave % HB;
    const int t0 = c * kC;
    const int oq = 32 * qh + col;
    const size_t bg = (size_t)b * D.Hkv + g;
    const float cl2 = D.tau * kLog2e;
    const int* loff = list_off + bg * (D.n_full + 1);
    const int nrows = c > NWT ? loff[c - NWT] : 0;
    const int ntile = NWT + 1 + (nrows + kC - 1) / kC;
    const int first = c >= NWT ? 0 : NWT - c;
    const int tla = t0 - NWT * kC;
    const size_t ldkv = (size_t)D.Hkv * kD;

    // Everything the block reads from memory beyond its own query rows comes
    // straight into LDS (global_load_lds), requested one step ahead:
    //   buffers 0, 1: the key tiles, double buffered (the next tile lands
    //     while the current one is computed): K and V rows in the padded
    //     K-tile layout (row reads for the logits and dout . v), K rows again
    //     in the swizzled V-tile layout (transposed reads of dQ^T += K^T dS^T);
    //   phkt: the phi_k rows of chunk c-NWT (swizzled V-tile layout), from
    //     the start;
    //   during the last tile, the linear prefix's two bf16 matrices (64 KB)
    //     into the other buffer (50 KB) and the overflow area, with the two
    //     z vectors; they are summed into the last tile's buffer after it;
    //   then the NP-Map projection (rows permuted for the NP-Map backward)
    //     into the other buffer, in the key tiles' three layouts.
    // Tile order: with c >= NWT the partly covered chunk c-NWT (tile 0) comes
    // last, and its dout . v products also give the linear terms' weights.
    constexpr int kBuf = 2 * kKTile + kVTile;  // elements of one buffer
    constexpr int kBufPieces = kBuf / 512;     // its 1 KB pieces (50)
    constexpr int kRawPieces = 2 * kD * kD / 512;  // the prefix's two matrices (64)
    constexpr int kOver = (kRawPieces - kBufPieces) * 512;  // overflow elements
    __shared__ __align__(16) bf16 smem[2 * kBuf + kVTile + kOver + 2 * kD * 2];
    const unsigned lds0 = (unsigned)(size_t)(lds_void*)smem;
    auto kpb = [&](int j) { return smem + j * kBuf; };
    auto vpb = [&](int j) { return smem + j * kBuf + kKTile; };
    auto ktb = [&](int j) { return smem + j * kBuf + 2 * kKTile; };
    const bf16* phkt = smem + 2 * kBuf;
    constexpr int kOverOff = 2 * kBuf + kVTile;  // overflow area, then lz | gz
    // LDS element offset of 1 KB piece x of the staged prefix (x < 32: the
    // within-run part, x >= 32: the earlier runs'), buffer jr first
    auto raw_piece = [&](int jr, int x) { return x < kBufPieces ? jr * kBuf + 512 * x : kOverOff + 512 * (x - kBufPieces); };
    const int nt = ntile - first;  // tiles in the loop (>= 2 when c >= NWT)
    auto tile_at = [&](int pos) { return first > 0 ? first + pos : (pos + 1 < nt ? pos + 1 : 0); };
    // rows of tile i: a window chunk from k / v, or compact rows; every tile
    // has nv >= 1 valid rows, and rows past nv repeat row nv - 1 (masked)
    auto stage = [&](int pos) {
        const int i = tile_at(pos);
        const bf16 *srck, *srcv;
        int nv;
        if (i <= NWT) {
            const int tc = c - NWT + i;
            nv = min(kC, D.N - tc * kC);
            const size_t off = (((size_t)b * D.N + (size_t)tc * kC) * D.Hkv + g) * kD;
            srck = k + off;
            srcv = v + off;
        } else {
            const int r0 = (i - NWT - 1) * kC;
            nv = min(kC, nrows - r0);
            const size_t off = ((size_t)b * sel_list_rows(D) * D.Hkv + g) * kD + (size_t)r0 * ldkv;
            srck = ksel + off;
            srcv = vsel + off;
        }
        const unsigned j = (unsigned)(pos & 1);
        const unsigned kd = lds0 + 2u * j * kBuf, vd = kd + 2u * kKTile, td = kd + 4u * kKTile;
        for (int x = wave; x < kKPieces; x += NW) {
            stage_k_piece_u(x, srck, (int)ldkv, nv, kd);
            stage_k_piece_u(x, srcv, (int)ldkv, nv, vd);
        }
        for (int x = wave; x < kVPieces; x += NW) stage_v_piece_u(x, srck, (int)ldkv, nv, td);
    };
    stage(0);  // lands during the prologue (buffer 0)
    if (c >= NWT) {
        const bf16* pk = phik + (bg * D.N + tla) * kD;
        const unsigned pd = lds0 + 2u * (2 * kBuf);
        for (int x = wave; x < kVPieces; x += NW) stage_v_piece_u(x, pk, kD, kC, pd);
    }
    int voff[4];
    vt_lane_offsets(voff);

    // route flags of chunk c-NWT (requested with the query rows)
    const uint8_t rtf = c >= NWT ? route[bg * D.N + tla + lane] : (uint8_t)0;
    // the lane's query: Q and dout operands, statistics
    const int tq = min(t0 + oq, D.N - 1);
    const size_t qo = ((size_t)b * D.N + tq) * D.Hq + h;
    bf16x8 qf[8], df[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) {
        qf[st] = ld_bf8(q + qo * kD + 16 * st + 8 * hf);
        df[st] = ld_bf8(dout + qo * kD + 16 * st + 8 * hf);
    }
    f32x4 stq;
    if (stat_in) {
        // from the forward: (m, l, -, c) of the query, and its output for
        // D = dout . out (the lane's 64 dims plus the other half's); the
        // statistics go to stat for the kernels after this one (the gated
        // features gamma phi_q follow from the NP-Map backward below)
        stq = *reinterpret_cast<const f32x4*>(stat_in + qo * 4);
        float dd = 0.f;
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const bf16x8 o8 = ld_bf8(out + qo * kD + 16 * st + 8 * hf);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x2 a2 = {o8[2 * j], o8[2 * j + 1]};
                const bf16x2 b2 = {df[st][2 * j], df[st][2 * j + 1]};
                dd = __builtin_amdgcn_fdot2_f32_bf16(a2, b2, dd, false);
            }
        }
        stq[2] = dd + xor32(dd);
        if (hf == 0 && t0 + oq < D.N) *reinterpret_cast<f32x4*>(stat + qo * 4) = stq;
    } else {
        stq = *reinterpret_cast<const f32x4*>(stat + qo * 4);
    }
    const float lse2 = stq[0] * kLog2e + __log2f(stq[1]);  // P = 2^(s cl2 - lse2)
    const float dq_d = stq[2];
    uint64_t selmask = 0;
    if (c >= NWT) selmask = __ballot(rtf == kRouteSA);

    f32x16 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = zero16();

    // the first tile and phi_k have landed (each wave waits for its own
    // staging, then the barrier)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    const int ngroups = (D.n_full + D.ng - 1) / D.ng;
    const int cq = c - NWT - 1, run = c > NWT ? cq / D.ng : 0;  // the prefix's last chunk, its run
    auto stage_prefix = [&](int jr) {
        const bf16* shg = reinterpret_cast<const bf16*>(L.sh) + (bg * D.n_full + cq) * (size_t)(kD * kD);
        const bf16* ghg = reinterpret_cast<const bf16*>(L.gh) + (bg * ngroups + run) * (size_t)(kD * kD);
        for (int x = wave; x < kRawPieces; x += NW)
            dma16_untracked((x < 32 ? shg + 512 * x : ghg + 512 * (x - 32)) + 8 * lane,
                            lds0 + 2u * (unsigned)raw_piece(jr, x));
        if (wave == NW - 1) {
            const float* zs = lane < 32 ? L.lz + (bg * D.n_full + cq) * kD + 4 * lane
                                        : L.gz + (bg * ngroups + run) * kD + 4 * (lane - 32);
            dma16_untracked(reinterpret_cast<const bf16*>(zs), lds0 + 2u * (kOverOff + kOver));
        }
    };
    // one tile: position pos in the order above; lin (tile 0 only) also
    // packs the linear terms' weights dout . v_j - D of the routed
    // unselected keys at or below the query's offset into wl
    auto tile = [&](int pos, bool lin, bf16x8 (&wl)[4]) __attribute__((always_inline)) {
        if (pos + 1 < nt) stage(pos + 1);  // into the buffer of position pos-1
        if (lin && c > NWT) stage_prefix((pos & 1) ^ 1);
        const int i = tile_at(pos), j = pos & 1;
        const bf16* kr = kpb(j);
        const bf16* vr = vpb(j);
        const bf16* ktr = ktb(j);
        uint64_t hi_m, lo_m;
        if (i == 0) {
            hi_m = ~0ull;
            lo_m = selmask;
        } else if (i < NWT) {
            hi_m = lo_m = ~0ull;
        } else if (i == NWT) {
            hi_m = 0ull;
            lo_m = ~0ull;
        } else {
            const int nv = min(kC, nrows - (i - NWT - 1) * kC);
            hi_m = lo_m = nv == kC ? ~0ull : (1ull << nv) - 1ull;
        }
        f32x16 sc[2], dp[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            sc[jj] = zero16();
            dp[jj] = zero16();
        }
#pragma unroll
        for (int st = 0; st < 8; ++st)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                sc[jj] = mfma32(ld_bf8(kr + (32 * jj + col) * kKS + 16 * st + 8 * hf), qf[st], sc[jj]);
                dp[jj] = mfma32(ld_bf8(vr + (32 * jj + col) * kKS + 16 * st + 8 * hf), df[st], dp[jj]);
            }
        if (lin) {
            f32x16 w[2];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) {
                    const int rk = 32 * jj + acc_row(vv, hf);
                    const bool la = rk <= oq && !((selmask >> rk) & 1ull);
                    w[jj][vv] = la ? dp[jj][vv] - dq_d : 0.f;
                }
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) wl[s4] = pack_acc(w[s4 >> 1], s4 & 1);
        }
        // key row rk counts for the lane's query when bit rk of
        // (rk > oq ? hi_m : lo_m) is set
        const uint64_t gt = oq >= 63 ? 0ull : ~0ull << (oq + 1);
        const uint64_t mm = ((hi_m & gt) | (lo_m & ~gt)) >> (4 * hf);
        const uint32_t mw[2] = {(uint32_t)mm, (uint32_t)(mm >> 32)};
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) {
                const bool ok = (mw[jj] >> (8 * (vv >> 2) + (vv & 3))) & 1u;
                const float p = ok ? __builtin_amdgcn_exp2f(fmaf(sc[jj][vv], cl2, -lse2)) : 0.f;
                sc[jj][vv] = p * (dp[jj][vv] - dq_d);
            }
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const bf16x8 pa = pack_acc(sc[s4 >> 1], s4 & 1);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) acc[dt] = mfma32(vt_frag(ktr, voff, dt, s4), pa, acc[dt]);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next tile landed
        __syncthreads();
    };
    const int nloop = c >= NWT ? nt - 1 : nt;
    for (int pos = 0; pos < nloop; ++pos) {
        bf16x8 unused[4];
        tile(pos, false, unused);
    }
    bf16x8 wl[4];
    if (c >= NWT) tile(nt - 1, true, wl);
    const bool qvalid = t0 + oq < D.N;
    const int jl = (nt - 1) & 1, jp = jl ^ 1;  // the last tile's buffer, the other one
    // the NP-Map projection of KV head g (high and low parts, 64 rows each)
    // into buffer jp, rows permuted (LDS row r = projection row kperm(r)):
    // both parts in the padded layout, the high part again swizzled
    const bf16* ph = wqh + (size_t)g * (kD / 2) * kD;
    const bf16* pl = wql + (size_t)g * (kD / 2) * kD;
    auto stage_proj = [&]() {
        const unsigned kd = lds0 + 2u * jp * kBuf;
        for (int x = wave; x < kKPieces; x += NW) {
            const int pp = 64 * x + lane, row = pp / 17, slot = min(pp - 17 * row, 15);
            const int so = kperm(row) * kD + 8 * slot;
            dma16_untracked(ph + so, kd + 1024u * x);
            dma16_untracked(pl + so, kd + 2u * kKTile + 1024u * x);
        }
        for (int x = wave; x < kVPieces; x += NW) {
            const int row = 4 * x + (lane >> 4), slot = (lane & 15) ^ vswz(row);
            dma16_untracked(ph + kperm(row) * kD + 8 * slot, kd + 4u * kKTile + 1024u * x);
        }
    };

    // ---- linear terms: dfq^T (rows = feature positions p of the prefix's
    // order, feature kperm(p); column = the lane's query) ----
    f32x16 dfq[4];
#pragma unroll
    for (int ft = 0; ft < 4; ++ft) dfq[ft] = zero16();
    if (c > NWT) {
        // prefix of chunks <= c-NWT-1 into sT[p][e] (the stored S^T rows are
        // [e][p]; kD rows of kKS over the last tile's K and V rows): the
        // within-run part of chunk c-NWT-1 plus its run's exclusive prefix,
        // summed in fp32
        bf16* sT = kpb(jl);
        for (int x = tid; x < 32 * 16; x += NW * 64) {
            const int eq = x & 31, oct = x >> 5;  // dims 4 eq .. +3, positions 8 oct .. +7
            bf16x8 rr[4];
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const int o = (4 * eq + e4) * kD + 8 * oct;  // element of a stored matrix
                const bf16x8 a8 = ld_bf8(smem + raw_piece(jp, o >> 9) + (o & 511));
                const bf16x8 b8 = ld_bf8(smem + raw_piece(jp, 32 + (o >> 9)) + (o & 511));
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) rr[e4][jj] = (bf16)((float)a8[jj] + (float)b8[jj]);
            }
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                bf16x4 t4;
                t4[0] = rr[0][jj];
                t4[1] = rr[1][jj];
                t4[2] = rr[2][jj];
                t4[3] = rr[3][jj];
                *reinterpret_cast<bf16x4*>(sT + (8 * oct + jj) * kKS + 4 * eq) = t4;
            }
        }
        __syncthreads();  // sT complete, the stored matrices consumed
    }
    stage_proj();
    if (c >= NWT) {
        // chunk c-NWT: the weights from its tile, times phi_k^T (transposed
        // reads of its staged rows)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
            for (int ft = 0; ft < 4; ++ft) dfq[ft] = mfma32(vt_frag(phkt, voff, ft, s4), wl[s4], dfq[ft]);
    }
    if (c > NWT) {
        const bf16* sT = kpb(jl);
#pragma unroll
        for (int ft = 0; ft < 4; ++ft)
#pragma unroll
            for (int st = 0; st < 8; ++st)
                dfq[ft] = mfma32(ld_bf8(sT + (32 * ft + col) * kKS + 16 * st + 8 * hf), df[st], dfq[ft]);
        const float* lz = reinterpret_cast<const float*>(smem + kOverOff + kOver);
        const float* gz = lz + kD;
#pragma unroll
        for (int ft = 0; ft < 4; ++ft)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int p0 = 32 * ft + acc_row(4 * v4, hf);
                const f32x4 z1 = *reinterpret_cast<const f32x4*>(lz + p0);
                const f32x4 z2 = *reinterpret_cast<const f32x4*>(gz + p0);
#pragma unroll
                for (int j = 0; j < 4; ++j) dfq[ft][4 * v4 + j] -= dq_d * (z1[j] + z2[j]);
            }
    }
    // the query row again (read back rather than kept live through the
    // linear phase)
    bf16x8 xq[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) xq[st] = ld_bf8(q + qo * kD + 16 * st + 8 * hf);
    // dphi_q = gamma c_t dfq (the ungated features' gradient) and, for the
    // gate logit, dgate = gamma (1 - gamma) c_t phi_q . dfq: dfq stays
    // unscaled, the scale enters dz
    const float cf = stq[3];
    const float gw = gate_weight(gate, qo);

    // ---- NP-Map backward of the query (full text Sec. 3.2; the map
    // u = P q, z = ||q|| u / ||u||, phi = [softmax(z); softmax(-z)]):
    //   dz = phi+ (dphi+ - <phi+, dphi+>) - phi- (dphi- - <phi-, dphi->)
    //   du = ||q|| (dz - uh <uh, dz>) / ||u||,  dq += P^T du + (<uh, dz> / ||q||) q
    // and du (bf16) for the projection gradient.  dfq's row 32 ft + r (ft <
    // 2) is the gradient of phi+ at feature kperm(32 ft + r) (ft >= 2: phi-
    // of feature kperm(32 (ft - 2) + r)), so the projection's rows are
    // staged in that order (LDS row r = P row kperm(r)): u then comes out of
    // the matrix cores with the same rows, and P^T is staged in natural
    // order for dQ^T = P^T dU^T, whose contraction positions are the features.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the projection has landed
    __syncthreads();
    const bf16* ks = kpb(jp);  // high part, rows permuted
    const bf16* vs = vpb(jp);  // low part, rows permuted
    const bf16* pt = ktb(jp);  // high part swizzled: transposed reads give P^T in feature order
    f32x16 u[2];
    u[0] = zero16();
    u[1] = zero16();
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
        for (int ft = 0; ft < 2; ++ft) {
            u[ft] = mfma32(ld_bf8(ks + (32 * ft + col) * kKS + 16 * st + 8 * hf), xq[st], u[ft]);
            u[ft] = mfma32(ld_bf8(vs + (32 * ft + col) * kKS + 16 * st + 8 * hf), xq[st], u[ft]);
        }
    float nx = 0.f, nu = 0.f, umax = -__builtin_inff(), umin = __builtin_inff();
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x2 x2 = {xq[st][2 * j], xq[st][2 * j + 1]};
            nx = __builtin_amdgcn_fdot2_f32_bf16(x2, x2, nx, false);
        }
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) {
            nu = fmaf(u[ft][vv], u[ft][vv], nu);
            umax = vmax(umax, u[ft][vv]);
            umin = vmin(umin, u[ft][vv]);
        }
    nx = sqrtf(nx + xor32(nx));
    nu = sqrtf(nu + xor32(nu));
    umax = vmax(umax, xor32(umax));
    umin = vmin(umin, xor32(umin));
    const float iu = nu > 0.f ? 1.f / nu : 0.f;  // uh = u iu (0 when u = 0)
    const float scl = nx * iu * kLog2e;           // z log2(e) = scl u
    float ep[2][16], en[2][16], sp = 0.f, sn = 0.f, sa = 0.f, sb = 0.f;
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) {
            ep[ft][vv] = __builtin_amdgcn_exp2f(fmaf(u[ft][vv], scl, -scl * umax));
            en[ft][vv] = __builtin_amdgcn_exp2f(fmaf(u[ft][vv], -scl, scl * umin));
            sp += ep[ft][vv];
            sn += en[ft][vv];
            sa = fmaf(ep[ft][vv], dfq[ft][vv], sa);
            sb = fmaf(en[ft][vv], dfq[ft + 2][vv], sb);
        }
    sp = 1.f / (sp + xor32(sp));
    sn = 1.f / (sn + xor32(sn));
    sa = (sa + xor32(sa)) * sp;  // phi+ . dfq+
    sb = (sb + xor32(sb)) * sn;  // phi- . dfq-
    if (dgate && hf == 0 && qvalid) dgate[qo] = gw * (1.f - gw) * cf * (sa + sb);
    if (stat_in && qvalid) {
        // gamma phi_q (bf16) for the kernels after this one, in the features'
        // storage order (position p holds feature kperm(p), as phi_k): rows
        // 32 ft + acc_row(4 v4, hf) .. +3 are four consecutive positions
        bf16* pr = phiq + qo * kD;
#pragma unroll
        for (int ft = 0; ft < 2; ++ft)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                bf16x4 a4, b4;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    a4[j] = (bf16)(gw * sp * ep[ft][4 * v4 + j]);
                    b4[j] = (bf16)(gw * sn * en[ft][4 * v4 + j]);
                }
                const int p0 = 32 * ft + acc_row(4 * v4, hf);
                *reinterpret_cast<bf16x4*>(pr + p0) = a4;
                *reinterpret_cast<bf16x4*>(pr + 64 + p0) = b4;
            }
    }
    const float dsc = gw * cf;  // dphi_q = dsc dfq
    float dnx = 0.f;
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) {
            const float z =
                dsc * (ep[ft][vv] * sp * (dfq[ft][vv] - sa) - en[ft][vv] * sn * (dfq[ft + 2][vv] - sb));
            ep[ft][vv] = z;
            dnx = fmaf(z, u[ft][vv] * iu, dnx);
        }
    dnx += xor32(dnx);
    const float cu = nx * iu;
    f32x16 dua[2];
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) dua[ft][vv] = cu * (ep[ft][vv] - dnx * u[ft][vv] * iu);
    // dQ^T += P^T dU^T / tau into the softmax part's accumulators (dq =
    // tau acc): the packed du rows are contraction positions = features
    {
        const float itau = 1.f / D.tau;
#pragma unroll
        for (int ft = 0; ft < 2; ++ft)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                f32x16 dsc = dua[ft];
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) dsc[vv] *= itau;
                const bf16x8 pd = pack_acc(dsc, s2);
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
                    acc[dt] = mfma32(vt_frag(pt, voff, dt, 2 * ft + s2), pd, acc[dt]);
            }
    }
    if (!qvalid) return;
    const float rn = nx > 0.f ? dnx / nx : 0.f;
    {
        float* dr = dq + qo * kD;
        const bf16* qrow = q + qo * kD;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int e = 32 * dt + acc_row(4 * v4, hf);
                const bf16x4 x4 = *reinterpret_cast<const bf16x4*>(qrow + e);
                f32x4 a4;
#pragma unroll
                for (int j = 0; j < 4; ++j) a4[j] = D.tau * acc[dt][4 * v4 + j] + rn * (float)x4[j];
                *reinterpret_cast<f32x4*>(dr + e) = a4;
            }
    }
    // du of row rho = token G + (h - g G) of group g, natural feature order:
    // four consecutive rows of dua hold four consecutive features
    {
        const size_t nrho = (size_t)D.B * D.N * D.G;
        const size_t rho = ((size_t)b * D.N + tq) * D.G + (h - g * D.G);
        bf16* dur = du_out + ((size_t)g * nrho + rho) * (kD / 2);
#pragma unroll
        for (int ft = 0; ft < 2; ++ft)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                bf16x4 d4;
#pragma unroll
                for (int j = 0; j < 4; ++j) d4[j] = (bf16)dua[ft][4 * v4 + j];
                *reinterpret_cast<bf16x4*>(dur + kperm(32 * ft + acc_row(4 * v4, hf))) = d4;
            }
    }
}

// ---------------------------------------------------------------------------
// Key side of the linear branch (full text Sec. 3.3, chunk-wise linear
// attention under the shared normaliser).  A routed unselected key j of
// chunk cj reaches every query t >= j + W through the linear state:
//   dv_j += U_j^T phi_k(j),  dphi_k(j) = U_j v_j - u_j,
//   U_j = sum over those queries (all heads of the group) of c_t fq_t dout_t^T,
//   u_j = sum c_t D_t fq_t    (fq = gamma phi_q, c_t = exp(-m) / l)
// = the chunk sums of chunks >= cj + NWT + 1 (an inclusive suffix over
// chunks) plus the queries of chunk cj + NWT at or after the key's offset.
// ---------------------------------------------------------------------------

// Chunk sums per query chunk c of (b, g): U[i][e] = sum over its queries t
// and the group's heads of c_t fq_t[i] dout_t[e], u[i] = sum c_t D_t fq_t[i]
// (i: the features' storage position, the order fq is stored in)
// (the fp32 layout [i][e] then u, (d + 1) d' floats).  Per head, (c fq)^T and
// dout^T are staged with the queries as contraction index; wave w owns
// features 32 w .. 32 w + 31.
__global__ __launch_bounds__(256) void bwd_uchunk_mfma_kernel(const bf16* __restrict__ phiq,
                                                              const bf16* __restrict__ dout,
                                                              const float* __restrict__ stat,
                                                              float* __restrict__ ust, Dims D) {
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hf = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    __shared__ __align__(16) bf16 ft[kD * kVS];  // (c fq)^T: [feature][kperm(query)]
    __shared__ __align__(16) bf16 dtt[kD * kVS]; // dout^T:   [dim][kperm(query)]
    __shared__ float dq_[kC];                     // D_t, at kperm(query)
    const int t0 = c * kC, nv = min(kC, D.N - t0);
    f32x16 acc[4];
#pragma unroll
    for (int et = 0; et < 4; ++et) acc[et] = zero16();
    float uacc = 0.f;
    for (int hh = 0; hh < D.G; ++hh) {
        const int h = g * D.G + hh;
        const size_t o0 = ((size_t)b * D.N + t0) * D.Hq + h;
        __syncthreads();
        for (int x = tid; x < 16 * 16; x += 256) {
            const int kq = x & 15, oct = x >> 4;
            bf16x8 rr[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int row = 4 * kq + q4;
                if (row < nv) {
                    const size_t o = o0 + (size_t)row * D.Hq;
                    // fq in the features' storage order: U's rows are positions
                    const float cf = stat[o * 4 + 3];
                    const bf16x8 a = ld_bf8(phiq + o * kD + 8 * oct);
#pragma unroll
                    for (int l = 0; l < 8; ++l) rr[q4][l] = (bf16)(cf * (float)a[l]);
                } else {
                    rr[q4] = zero_bf8();
                }
            }
            const int pos = kperm(4 * kq);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bf16x4 t4;
                t4[0] = rr[0][e];
                t4[1] = rr[1][e];
                t4[2] = rr[2][e];
                t4[3] = rr[3][e];
                *reinterpret_cast<bf16x4*>(ft + (8 * oct + e) * kVS + pos) = t4;
            }
        }
        load_vt_tile(dout + o0 * kD, (size_t)D.Hq * kD, nv, dtt, tid, 256);
        if (tid < kC) dq_[kperm(tid)] = tid < nv ? stat[(o0 + (size_t)tid * D.Hq) * 4 + 2] : 0.f;
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 a = ld_bf8(ft + (32 * wave + col) * kVS + 16 * ks + 8 * hf);
#pragma unroll
            for (int et = 0; et < 4; ++et)
                acc[et] = mfma32(a, ld_bf8(dtt + (32 * et + col) * kVS + 16 * ks + 8 * hf), acc[et]);
        }
        if (tid < kD) {
            const bf16* fr = ft + tid * kVS;
            for (int p = 0; p < kC; ++p) uacc = fmaf((float)fr[p], dq_[p], uacc);
        }
    }
    float* out = ust + (((size_t)b * D.Hkv + g) * D.T + c) * (size_t)(kD * (kD + 1));
#pragma unroll
    for (int et = 0; et < 4; ++et)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv)
            out[(size_t)(32 * wave + acc_row(vv, hf)) * kD + 32 * et + col] = acc[et][vv];
    if (tid < kD) out[kD * kD + tid] = uacc;
}

// Per key chunk cj of (b, g), 64 keys: the linear terms above.  Waves 0 / 1
// take keys 0-31 / 32-63 for dphi_k (rows: feature positions p of phi_k's
// storage order, feature kperm(p)), waves 2 / 3 the same keys for dv (rows:
// dims).  The suffix sum U of chunks >= cj + NWT + 1 is staged in bf16 twice
// (rows of positions p, and transposed); then, per head, the 64 queries of
// chunk cj + NWT (fq with permuted features, fq^T, dout, dout^T).  Writes dv
// (the linear part; the softmax kernels add theirs) and dphi_k (feature
// order) of every key of the chunk, zeros for keys with no linear term.
template <int NWT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void bwd_key_lin_kernel(
    const bf16* __restrict__ v, const bf16* __restrict__ dout, const bf16* __restrict__ phiq,
    const bf16* __restrict__ phik16, const uint8_t* __restrict__ route, const float* __restrict__ stat,
    const float* __restrict__ ust, const bf16* __restrict__ ust16, float* __restrict__ dv,
    const bf16* __restrict__ k,
    const bf16* __restrict__ wkh, const bf16* __restrict__ wkl, float* __restrict__ dk,
    bf16* __restrict__ du_out, Dims D) {
    const Item it = xcd_item(D.T, D.Hkv);
    const int cj = it.x, g = it.y, b = it.z;
    const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hf = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kh = wave & 1, role = wave >> 1;  // role 0: dphi_k, 1: dv
    const size_t bg = (size_t)b * D.Hkv + g;
    const int rk = 32 * kh + col;  // the lane's key offset in chunk cj
    const int j = cj * kC + rk;
    const int c0 = cj + NWT;  // chunk of the first linear query
    const bool has_q = c0 < D.T;
    const bool la = j < D.N && has_q && j + D.W <= D.N - 1 && route[bg * D.N + j] == kRouteLA;
    const int jr = min(j, D.N - 1);
    bf16x8 bop[8];  // role 0: v_j (dims), role 1: phi_k(j) (storage positions)
    if (role == 0) load_key_operand(v + (((size_t)b * D.N + jr) * D.Hkv + g) * kD, bop);
    else load_key_operand(phik16 + (bg * D.N + jr) * kD, bop);
    // one area: U and U^T (bf16), then per head fq, fq^T, dout, dout^T
    __shared__ __align__(16) bf16 sm[2 * kC * kKS + 2 * kD * kVS];
    __shared__ float cq[kC], dq_[kC];
    __shared__ __align__(16) float rawst[2][kC * 4];  // raw statistics of the staged heads
    f32x16 acc[4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) acc[t4] = zero16();
    if (has_q && c0 + 1 < D.T) {
        const float* U = ust + (bg * D.T + c0 + 1) * (size_t)(kD * (kD + 1));  // its u
        const bf16* U16 = ust16 + (bg * D.T + c0 + 1) * (size_t)(kD * kD);     // its U, bf16
        bf16* ub = sm;              // [p][e], kKS
        bf16* ut = sm + kD * kKS;   // [e][p], kKS
        for (int x = tid; x < kD * 16; x += 256) {
            const int pp = x >> 4, oct = x & 15;  // U's rows are the features' storage positions
            const bf16x8 r = ld_bf8(U16 + (size_t)pp * kD + 8 * oct);
            st_bf8(ub + pp * kKS + 8 * oct, r);
#pragma unroll
            for (int e = 0; e < 8; ++e) ut[(8 * oct + e) * kKS + pp] = r[e];
        }
        __syncthreads();
        const bf16* A = role == 0 ? ub : ut;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
            for (int st = 0; st < 8; ++st)
                acc[t4] = mfma32(ld_bf8(A + (32 * t4 + col) * kKS + 16 * st + 8 * hf), bop[st], acc[t4]);
        if (role == 0) {
            // - u (feature order)
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) acc[t4][vv] -= U[kD * kD + 32 * t4 + acc_row(vv, hf)];
        }
    }
    if (has_q) {
        const int tq0 = c0 * kC, nq = min(kC, D.N - tq0);
        // Per head: fq [q][p] and dout [q][e] rows (kKS; rows past N repeat
        // the last one, with weight c = 0) in one of two buffers, requested by
        // DMA while the previous head is computed (head 0 after the suffix
        // products, whose operands fill both); their transposes are read from
        // the same rows (ds_read_b64_tr_b16).
        int poff[4];
        kt_pad_lane_offsets(poff);
        const unsigned lds_sm = (unsigned)(size_t)(lds_void*)sm;
        auto issue = [&](int hh) {
            const size_t o0 = ((size_t)b * D.N + tq0) * D.Hq + g * D.G + hh;
            const unsigned fb = lds_sm + 4u * kKTile * (unsigned)(hh & 1), db = fb + 2u * kKTile;
            for (int x = wave; x < kKPieces; x += 4) {
                stage_k_piece_u(x, phiq + o0 * kD, D.Hq * kD, nq, fb);
                stage_k_piece_u(x, dout + o0 * kD, D.Hq * kD, nq, db);
            }
            if (wave == 3)
                dma16_untracked(reinterpret_cast<const bf16*>(stat + (o0 + (size_t)min(lane, nq - 1) * D.Hq) * 4),
                                (unsigned)(size_t)(lds_void*)rawst[hh & 1]);
        };
        __syncthreads();  // the suffix products' reads of sm are done
        issue(0);
        for (int hh = 0; hh < D.G; ++hh) {
            const bf16* fq = sm + 2 * kKTile * (hh & 1);
            const bf16* dr = fq + kKTile;
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's share of head hh
            __syncthreads();                      // every share landed; head hh-1 is done
            if (tid < kC) {
                const f32x4 s4 = *reinterpret_cast<const f32x4*>(rawst[hh & 1] + 4 * tid);
                cq[tid] = tid < nq ? s4[3] : 0.f;
                dq_[tid] = tid < nq ? s4[2] : 0.f;
            }
            __syncthreads();
            if (hh + 1 < D.G) issue(hh + 1);  // into the buffer of head hh-1
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                // rows: queries 32 qb + acc_row, column: the lane's key
                f32x16 x = zero16();
                const bf16* A = role == 0 ? dr : fq;
#pragma unroll
                for (int st = 0; st < 8; ++st)
                    x = mfma32(ld_bf8(A + (32 * qb + col) * kKS + 16 * st + 8 * hf), bop[st], x);
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const int r0 = 32 * qb + acc_row(4 * v4, hf);
                    const f32x4 c4 = *reinterpret_cast<const f32x4*>(cq + r0);
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(dq_ + r0);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int vv = 4 * v4 + jj;
                        const bool ok = la && r0 + jj >= rk;  // query at or after the key's offset
                        // role 0: c_t (dout . v_j - D_t); role 1: c_t fq . phi_k(j)
                        x[vv] = ok ? c4[jj] * (role == 0 ? x[vv] - d4[jj] : x[vv]) : 0.f;
                    }
                }
                const bf16* At = role == 0 ? fq : dr;
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const bf16x8 pw = pack_acc(x, s2);
                    const int ks = 2 * qb + s2;
#pragma unroll
                    for (int t4 = 0; t4 < 4; ++t4) acc[t4] = mfma32(kt_pad_frag(At, poff, t4, ks), pw, acc[t4]);
                }
            }
        }
    }
    // The keys' NP-Map backward follows in the role-0 waves (0, 1), with
    // dphi_k = their acc (zero for keys with no linear term), as the
    // queries' in bwd_dq_kernel: the projection's rows staged in the order
    // of acc's rows (LDS row r = P row kperm(r)), P^T in natural order, by
    // the whole block before the roles part; it writes dk = P^T du +
    // (<uh, dz> / ||k||) k (the softmax kernels add their terms afterwards)
    // and du (bf16, rows = tokens) for the projection gradient.
    bf16* ks = sm;
    bf16* vs = sm + kC * kKS;
    bf16* kt = sm + 2 * kC * kKS;
    __syncthreads();  // every wave's reads of sm are done
    {
        const bf16* ph = wkh + (size_t)g * (kD / 2) * kD;
        const bf16* pl = wkl + (size_t)g * (kD / 2) * kD;
        for (int x = tid; x < kC * 16; x += 256) {
            const int row = x >> 4, piece = x & 15;
            const size_t src = (size_t)kperm(row) * kD + 8 * piece;
            st_bf8(ks + row * kKS + 8 * piece, ld_bf8(ph + src));
            st_bf8(vs + row * kKS + 8 * piece, ld_bf8(pl + src));
        }
        for (int x = tid; x < 16 * 16; x += 256) {
            const int kq = x & 15, oct = x >> 4;
            bf16x8 r4[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) r4[rr] = ld_bf8(ph + (size_t)(4 * kq + rr) * kD + 8 * oct);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bf16x4 t4;
                t4[0] = r4[0][e];
                t4[1] = r4[1][e];
                t4[2] = r4[2][e];
                t4[3] = r4[3][e];
                *reinterpret_cast<bf16x4*>(kt + (8 * oct + e) * kVS + 4 * kq) = t4;
            }
        }
    }
    __syncthreads();
    const size_t o = (((size_t)b * D.N + jr) * D.Hkv + g) * kD;
    if (role == 1) {
        if (j >= D.N) return;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int r0 = 32 * t4 + acc_row(4 * v4, hf);
                f32x4 w4;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) w4[jj] = la ? acc[t4][4 * v4 + jj] : 0.f;
                *reinterpret_cast<f32x4*>(dv + o + r0) = w4;
            }
        return;
    }
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) acc[t4][vv] = la ? acc[t4][vv] : 0.f;
    bf16x8 xk[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) xk[st] = ld_bf8(k + o + 16 * st + 8 * hf);
    f32x16 u[2];
    u[0] = zero16();
    u[1] = zero16();
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
        for (int ft = 0; ft < 2; ++ft) {
            u[ft] = mfma32(ld_bf8(ks + (32 * ft + col) * kKS + 16 * st + 8 * hf), xk[st], u[ft]);
            u[ft] = mfma32(ld_bf8(vs + (32 * ft + col) * kKS + 16 * st + 8 * hf), xk[st], u[ft]);
        }
    float nx = 0.f, nu = 0.f, umax = -__builtin_inff(), umin = __builtin_inff();
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const bf16x2 x2 = {xk[st][2 * jj], xk[st][2 * jj + 1]};
            nx = __builtin_amdgcn_fdot2_f32_bf16(x2, x2, nx, false);
        }
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) {
            nu = fmaf(u[ft][vv], u[ft][vv], nu);
            umax = vmax(umax, u[ft][vv]);
            umin = vmin(umin, u[ft][vv]);
        }
    nx = sqrtf(nx + xor32(nx));
    nu = sqrtf(nu + xor32(nu));
    umax = vmax(umax, xor32(umax));
    umin = vmin(umin, xor32(umin));
    const float iu = nu > 0.f ? 1.f / nu : 0.f;
    const float scl = nx * iu * kLog2e;
    float ep[2][16], en[2][16], sp = 0.f, sn = 0.f, sa = 0.f, sb = 0.f;
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) {
            ep[ft][vv] = __builtin_amdgcn_exp2f(fmaf(u[ft][vv], scl, -scl * umax));
            en[ft][vv] = __builtin_amdgcn_exp2f(fmaf(u[ft][vv], -scl, scl * umin));
            sp += ep[ft][vv];
            sn += en[ft][vv];
            sa = fmaf(ep[ft][vv], acc[ft][vv], sa);
            sb = fmaf(en[ft][vv], acc[ft + 2][vv], sb);
        }
    sp = 1.f / (sp + xor32(sp));
    sn = 1.f / (sn + xor32(sn));
    sa = (sa + xor32(sa)) * sp;
    sb = (sb + xor32(sb)) * sn;
    float dnx = 0.f;
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) {
            const float z = ep[ft][vv] * sp * (acc[ft][vv] - sa) - en[ft][vv] * sn * (acc[ft + 2][vv] - sb);
            ep[ft][vv] = z;
            dnx = fmaf(z, u[ft][vv] * iu, dnx);
        }
    dnx += xor32(dnx);
    const float cu = nx * iu;
    f32x16 dua[2];
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) dua[ft][vv] = cu * (ep[ft][vv] - dnx * u[ft][vv] * iu);
    f32x16 dxt[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) dxt[dt] = zero16();
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const bf16x8 pd = pack_acc(dua[ft], s2);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                dxt[dt] = mfma32(ld_bf8(kt + (32 * dt + col) * kVS + 32 * ft + 16 * s2 + 8 * hf), pd, dxt[dt]);
        }
    if (j >= D.N) return;
    const float rn = nx > 0.f ? dnx / nx : 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const int e = 32 * dt + acc_row(4 * v4, hf);
            const bf16x4 x4 = *reinterpret_cast<const bf16x4*>(k + o + e);
            f32x4 a4;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) a4[jj] = dxt[dt][4 * v4 + jj] + rn * (float)x4[jj];
            *reinterpret_cast<f32x4*>(dk + o + e) = a4;
        }
    bf16* dur = du_out + ((size_t)g * D.B * D.N + (size_t)b * D.N + j) * (kD / 2);
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            bf16x4 d4;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) d4[jj] = (bf16)dua[ft][4 * v4 + jj];
            *reinterpret_cast<bf16x4*>(dur + kperm(32 * ft + acc_row(4 * v4, hf))) = d4;
        }
}

// ---------------------------------------------------------------------------
// Projection gradient dP[g] = sum over the rows rho of group g of du x^T,
// partial over one slice of rows per block: 64-row tiles of dU and X staged
// transposed (rows as the contraction index), each wave one 32-feature by
// 64-dim quarter of dP.
__global__ __launch_bounds__(256) void dw_mfma_kernel(const bf16* __restrict__ x,
                                                      const bf16* __restrict__ du,
                                                      float* __restrict__ part, int ntok, int H,
                                                      int hpp, int nslice) {
    constexpr int kF = kD / 2;
    const int sl = blockIdx.x, g = blockIdx.y, G8 = gridDim.y;
    const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hf = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ftile = wave & 1, dpair = wave >> 1;
    const int nrho = ntok * hpp;
    const int per = ((nrho + nslice - 1) / nslice + kC - 1) / kC * kC;
    const int r0 = sl * per, r1 = min(nrho, r0 + per);
    __shared__ __align__(16) bf16 dut[kF * kVS];
    __shared__ __align__(16) bf16 xt[kD * kVS];
    f32x16 acc[2];
    acc[0] = zero16();
    acc[1] = zero16();
    const bf16* dug = du + (size_t)g * nrho * kF;
    for (int rb = r0; rb < r1; rb += kC) {
        const int nv = min(kC, r1 - rb);
        __syncthreads();
        // dU^T: dut[f * kVS + kperm(r)] = du[rb + r][f]
        load_vt_tile64(dug + (size_t)rb * kF, kF, nv, dut, tid, 256);
        // X^T: xt[e * kVS + kperm(r)] = x[row(rb + r)][e]
        for (int xi = tid; xi < 16 * 16; xi += 256) {
            const int kq = xi & 15, oct = xi >> 4;
            bf16x8 rr[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int r = 4 * kq + q4;
                const int rho = rb + r;
                const size_t xr = (size_t)(rho / hpp) * H + (size_t)g * hpp + rho % hpp;
                rr[q4] = r < nv ? ld_bf8(x + xr * kD + 8 * oct) : zero_bf8();
            }
            const int pos = kperm(4 * kq);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bf16x4 t4;
                t4[0] = rr[0][e];
                t4[1] = rr[1][e];
                t4[2] = rr[2][e];
                t4[3] = rr[3][e];
                *reinterpret_cast<bf16x4*>(xt + (8 * oct + e) * kVS + pos) = t4;
            }
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 a = ld_bf8(dut + (32 * ftile + col) * kVS + 16 * ks + 8 * hf);
#pragma unroll
            for (int jd = 0; jd < 2; ++jd)
                acc[jd] = mfma32(a, ld_bf8(xt + (32 * (2 * dpair + jd) + col) * kVS + 16 * ks + 8 * hf), acc[jd]);
        }
    }
    // rows f = 32 ftile + acc_row, column e = 32 (2 dpair + jd) + col
    float* out = part + ((size_t)sl * G8 + g) * kF * kD;
#pragma unroll
    for (int jd = 0; jd < 2; ++jd)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv)
            out[(size_t)(32 * ftile + acc_row(vv, hf)) * kD + 32 * (2 * dpair + jd) + col] = acc[jd][vv];
}

}  // namespace

hipError_t launch_bwd_dq(const Dims& D, const void* q, const void* k, const void* v, const void* dout,
                         const uint8_t* route, const void* ksel, const void* vsel,
                         const int* list_off, float* stat, const void* phik16, const LinBufs& L,
                         const float* gate, void* phiq, float* dq, void* du, float* dgate,
                         const float* stat_in, const void* out, const void* wsplit, hipStream_t s) {
    const int HB = D.G >= 4 ? 4 : D.G;  // query heads per block, two waves each
    const int n = D.Hkv * (kD / 2) * kD;
    const bf16* wqh = reinterpret_cast<const bf16*>(wsplit);
    const bf16* wql = wqh + n;
    const unsigned nblk = (unsigned)D.T * D.B * D.Hkv * (D.G / HB);
    const int nwt = D.W / kC;
#define STILL_DQ1(H, NWT)                                                                        \
    hipLaunchKernelGGL((bwd_dq_kernel<H, NWT>), dim3(nblk), dim3(128 * H), 0, s,                \
                       reinterpret_cast<const bf16*>(q), reinterpret_cast<const bf16*>(k),      \
                       reinterpret_cast<const bf16*>(v), reinterpret_cast<const bf16*>(dout),   \
                       route, reinterpret_cast<const bf16*>(ksel),                                \
                       reinterpret_cast<const bf16*>(vsel), list_off, stat,                       \
                       reinterpret_cast<const bf16*>(phik16), L, gate, reinterpret_cast<bf16*>(phiq), dq,           \
                       reinterpret_cast<bf16*>(du), dgate,                                            \
                       stat_in, reinterpret_cast<const bf16*>(out), wqh, wql, D)
#define STILL_DQ(H)                \
    do {                           \
        if (nwt == 1)              \
            STILL_DQ1(H, 1);       \
        else if (nwt == 2)         \
            STILL_DQ1(H, 2);       \
        else                       \
            STILL_DQ1(H, 4);       \
    } while (0)
    if (HB == 4) STILL_DQ(4);
    else if (HB == 2) STILL_DQ(2);
    else STILL_DQ(1);
#undef STILL_DQ
#undef STILL_DQ1
    return hipGetLastError();
}

hipError_t launch_bwd_key_lin(const Dims& D, const void* v, const void* dout, const void* phiq,
                              const void* phik16, const uint8_t* route, const float* stat, float* ust,
                              const void* ust16, float* dv, const void* k, const void* wsplit, float* dk,
                              void* du16, int phase, hipStream_t s) {
    if (phase == 0) {
        hipLaunchKernelGGL(bwd_uchunk_mfma_kernel, dim3(D.T, D.Hkv, D.B), dim3(256), 0, s,
                           reinterpret_cast<const bf16*>(phiq), reinterpret_cast<const bf16*>(dout), stat, ust,
                           D);
        return hipGetLastError();
    }
    const unsigned nblk = (unsigned)D.T * D.Hkv * D.B;
    const int nwt = D.W / kC;
    const size_t part = (size_t)D.Hkv * (kD / 2) * kD;
    const bf16* wkh = reinterpret_cast<const bf16*>(wsplit) + 2 * part;  // [wq hi, wq lo, wk hi, wk lo]
#define STILL_KL(NWT)                                                                            \
    hipLaunchKernelGGL((bwd_key_lin_kernel<NWT>), dim3(nblk), dim3(256), 0, s,                  \
                       reinterpret_cast<const bf16*>(v), reinterpret_cast<const bf16*>(dout),   \
                       reinterpret_cast<const bf16*>(phiq), reinterpret_cast<const bf16*>(phik16), route, \
                       stat, ust, reinterpret_cast<const bf16*>(ust16), dv,                         \
                       reinterpret_cast<const bf16*>(k), wkh, wkh + part, dk,                         \
                       reinterpret_cast<bf16*>(du16), D)
    if (nwt == 1) STILL_KL(1);
    else if (nwt == 2) STILL_KL(2);
    else STILL_KL(4);
#undef STILL_KL
    return hipGetLastError();
}

size_t bwd_kv_part_floats(const Dims& D) {
    return (size_t)(kSelSeg - 1) * D.B * D.Hkv * D.n_full * D.lam * (2 * kD);
}

hipError_t launch_bwd_kv(const Dims& D, const void* q, const void* k, const void* v, const void* dout,
                         const uint8_t* route, const void* ksel, const void* vsel,
                         const int32_t* selw, const int* list_off, const float* stat, float* dk,
                         float* dv, float* part, int phase, hipStream_t s) {
    const bf16* qq = reinterpret_cast<const bf16*>(q);
    const bf16* dd = reinterpret_cast<const bf16*>(dout);
    const int nwt = D.W / kC;
    if (phase == 0) {
        const unsigned nblk = (unsigned)((D.T + kWinKPB - 1) / kWinKPB) * D.B * D.Hkv;
#define STILL_KVW(NWT)                                                                           \
    hipLaunchKernelGGL((bwd_kv_window_kernel<NWT, kWinKPB>), dim3(nblk), dim3(kWinKPB * 256), 0, s, qq, \
                       reinterpret_cast<const bf16*>(k), reinterpret_cast<const bf16*>(v), dd,  \
                       route, stat, dk, dv, D)
        if (nwt == 1) STILL_KVW(1);
        else if (nwt == 2) STILL_KVW(2);
        else STILL_KVW(4);
#undef STILL_KVW
        return hipGetLastError();
    }
    if (D.lam == 0 || D.n_full == 0) return hipSuccess;
    const int ntile = (D.n_full * D.lam + kSelW * 32 - 1) / (kSelW * 32);
    const unsigned nblk = (unsigned)ntile * kSelSeg * D.B * D.Hkv;
#define STILL_KVS(NWT)                                                                           \
    hipLaunchKernelGGL((bwd_kv_selected_kernel<NWT, kSelW>), dim3(nblk), dim3(kSelW * 128), 0, s, qq, \
                       reinterpret_cast<const bf16*>(ksel), reinterpret_cast<const bf16*>(vsel), \
                       dd, selw, list_off, stat, dk, dv, part, D)
    if (nwt == 1) STILL_KVS(1);
    else if (nwt == 2) STILL_KVS(2);
    else STILL_KVS(4);
#undef STILL_KVS
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || kSelSeg == 1) return e;
    hipLaunchKernelGGL(bwd_kv_merge_kernel, dim3((D.n_full * D.lam + 3) / 4, D.Hkv, D.B), dim3(256), 0, s,
                       part, selw, list_off, dk, dv, D);
    return hipGetLastError();
}

// NP-Map backward of one side (q: H = Hq, hpp = G, projection parts 0 / 1;
// k: H = Hkv, hpp = 1, parts 2 / 3 of wsplit) and its projection gradient
hipError_t launch_dw_mfma(const Dims& D, const void* x, int side, const void* du16, float* part,
                          int nslice, hipStream_t s) {
    const int H = side == 0 ? D.Hq : D.Hkv, hpp = side == 0 ? D.G : 1;
    hipLaunchKernelGGL(dw_mfma_kernel, dim3(nslice, D.Hkv), dim3(256), 0, s,
                       reinterpret_cast<const bf16*>(x), reinterpret_cast<const bf16*>(du16), part,
                       D.B * D.N, H, hpp, nslice);
    return hipGetLastError();
}

}  // namespace still
