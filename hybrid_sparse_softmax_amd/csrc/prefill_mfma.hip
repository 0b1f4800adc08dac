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
//   la_state_kernel     NP-Map of the keys (Sec. 3.2, MFMA projection),
//                       phi_k rows for the read-out, and running sums of
//                       phi_k v^T over unselected tokens (MFMA; Appendix A.2
//                       state) along runs of consecutive chunks
//   la_group_scan_kernel  prefix over the runs' totals
//   hybrid_main_kernel  per query chunk: linear prefix read-out, chunk c-NWT
//                       (window, routed selected and routed linear tokens),
//                       chunks c-NWT+1 .. c (window; causal in chunk c),
//                       then every selected token of chunks <= c-NWT-1
//                       from the compact list; one online normaliser shared
//                       by both branches (Fig. 2)
//
// Chunks are 64 tokens and the window W = 64 NWT (NWT = 1, 2 or 4).  Routing:
// token j is routed for query t once j <= t - W, so for a query of chunk c
// the tokens of chunk c-NWT at an offset <= its own are routed (their
// chunk's decision is final), later ones are still in its window.
#include <type_traits>

#include "launch.h"
#include "mfma_common.h"
#include "mfma_tiles.h"

namespace still {

namespace {
using namespace mt;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr int kFS = kC + 4;     // LDS row stride (floats) of transposed phi_k
constexpr int kHS = kD + 8;     // LDS row stride (elements) of a staged state's bf16 parts
constexpr float kLazy = 8.0f;   // rescale only when the running max grows by more (log2 units)

enum { kModePrev = 0, kModeDiag = 1, kModeSparse = 2 };

// Q operand of one wave: tokens t0 .. t0+63 of head h; qf[qt][s] holds
// token t0 + 32 qt + l%32, dims 16 s + 8 (l/32) .. +7.  Tokens beyond N
// repeat token N-1 (their outputs are never written).
__device__ __forceinline__ void load_q(const bf16* __restrict__ q, const Dims& D, int b, int t0,
                                       int h, bf16x8 (&qf)[2][8]) {
    const int lane = threadIdx.x & 63, hf = lane >> 5, col = lane & 31;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int t = min(t0 + 32 * qt + col, D.N - 1);
        const bf16* row = q + (((size_t)b * D.N + t) * D.Hq + h) * kD + 8 * hf;
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[qt][s] = ld_bf8(row + 16 * s);
    }
}

// ---------------------------------------------------------------------------
// window scores, selection, gather
// ---------------------------------------------------------------------------
// NP-Map projections of KV head g (fp32) as bf16 high and low parts for the
// matrix-core products that use them (the projection equals high + low up to
// the rounding of low): wsplit = [wq high, wq low, wk high, wk low], each
// Hkv * (d'/2) * d elements.  nthr threads, 16 floats each per pass.
__device__ __forceinline__ void split_projections(const float* __restrict__ wq, const float* __restrict__ wk,
                                                  bf16* __restrict__ wsplit, int Hkv, int g, int nthr) {
    const int n = Hkv * (kD / 2) * kD, per = (kD / 2) * kD;
    for (int i0 = 4 * threadIdx.x; i0 < 2 * per; i0 += 16 * nthr) {
        f32x4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = min(i0 + 4 * nthr * u, 2 * per - 4), which = i / per, e = g * per + i % per;
            x[u] = *reinterpret_cast<const f32x4*>((which ? wk : wq) + e);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + 4 * nthr * u;
            if (i >= 2 * per) break;
            const int which = i / per, e = g * per + i % per;
            bf16x4 hi, lo;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                hi[j] = (bf16)x[u][j];
                lo[j] = (bf16)(x[u][j] - (float)hi[j]);
            }
            *reinterpret_cast<bf16x4*>(wsplit + (size_t)2 * n * which + e) = hi;
            *reinterpret_cast<bf16x4*>(wsplit + (size_t)2 * n * which + n + e) = lo;
        }
    }
}

// NWT = W / 64: the window of a query spans NWT chunks back from its own.
// chunk: the true chunk length.  When it exceeds 64 (D then counts 64-token
// tiles) the block writes its tile's scores and the projection split and
// stops there; chunk_select_kernel selects per chunk.
template <int NW, int NWT>
__global__ __launch_bounds__(NW * 64) void win_select_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    float* __restrict__ scores, int32_t* __restrict__ sel_idx, uint8_t* __restrict__ route,
    bf16* __restrict__ ksel, bf16* __restrict__ vsel, const float* __restrict__ wq,
    const float* __restrict__ wk, bf16* __restrict__ wsplit, int chunk, Dims D) {
    const bool score_only = chunk > kC;
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, col = lane & 31;
    const int t0 = c * kC;
    const size_t bg = (size_t)b * D.Hkv + g;
    __shared__ float hsc[8][kC];
    __shared__ float key_s[kC];
    __shared__ int flag_s[kC];
    __shared__ int pos_s[kC];
    // K rows of chunks c-NWT .. c, staged once for all heads (K tile layout;
    // rows before token 0 are never loaded and only ever masked)
    __shared__ __align__(16) bf16 kwin[(NWT + 1) * kKTile];
    const bf16* kown = kwin + NWT * kKTile;  // this chunk's key rows
    {
        const size_t ldkv = (size_t)D.Hkv * kD;
        for (int i = 0; i <= NWT; ++i) {
            const int tc = c - NWT + i;
            if (tc < 0) continue;
            const bf16* src = k + (((size_t)b * D.N + (size_t)tc * kC) * D.Hkv + g) * kD;
            for (int j = wave; j < kKPieces; j += NW) stage_k_piece(j, src, ldkv, min(kC, D.N - tc * kC), kwin + i * kKTile);
        }
    }
    // this chunk's value rows, requested now for the gather at the end:
    // piece x = tid + 64 NW i is row x / 16, dims 8 (x % 16) .. +7
    constexpr int kVP = kC * 16 / (NW * 64);
    bf16x8 vrow[kVP];
    if (c < D.n_full && !score_only) {
#pragma unroll
        for (int i = 0; i < kVP; ++i) {
            const int x = tid + NW * 64 * i;
            vrow[i] = ld_bf8(v + (((size_t)b * D.N + t0 + (x >> 4)) * D.Hkv + g) * kD + 8 * (x & 15));
        }
    }
    // Q operand of query half qt of head hh (the next one is requested while
    // the current one is scored)
    auto load_q = [&](bf16x8 (&qd)[8], int hh, int qt) {
        const int t = min(t0 + 32 * qt + col, D.N - 1);
        const bf16* row = q + (((size_t)b * D.N + t) * D.Hq + g * D.G + hh) * kD + 8 * hf;
#pragma unroll
        for (int s = 0; s < 8; ++s) qd[s] = ld_bf8(row + 16 * s);
    };
    bf16x8 qf[8], qn[8];
    if (wave < D.G) load_q(qf, wave, 0);
    const float tl2 = D.tau * kLog2e;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();

    // query-free criteria need no window rows
    for (int hh = route_query_free(D.route) ? D.G : wave; hh < D.G; hh += NW) {
#pragma unroll 1
        for (int qt = 0; qt < 2; ++qt) {
            {
                const int nh = qt == 0 ? hh : hh + NW, nq = qt ^ 1;
                if (nh < D.G) load_q(qn, nh, nq);
            }
            // logits against keys t0-64 NWT .. t0+63 (key index kk = 32 kt +
            // row); the window of query offset qo is kk in [qo+1, qo+64 NWT],
            // inside key subtiles kt = qt .. qt+2 NWT
            constexpr int NS = 2 * NWT + 1, NSLOT = 2 * NWT;
            f32x16 sc[NS];
#pragma unroll
            for (int j = 0; j < NS; ++j) sc[j] = zero16();
#pragma unroll
            for (int s = 0; s < 8; ++s) {
#pragma unroll
                for (int j = 0; j < NS; ++j) {
                    const int kt = qt + j;
                    const bf16x8 a = ld_bf8(kwin + (kt >> 1) * kKTile + (32 * (kt & 1) + col) * kKS + 16 * s + 8 * hf);
                    sc[j] = mfma32(a, qf[s], sc[j]);
                }
            }
            const int qo = 32 * qt + col;  // query offset in the chunk; its own key is kk = qo + 64 NWT
            // The window [qo+1, qo+64 NWT] holds all of subtiles qt+1 ..
            // qt+2NWT-1, the rows of subtile qt above the query's offset and
            // the other rows of subtile qt+2NWT: the last two are
            // complementary, so each lane keeps 32 NWT entries: sc[1 ..
            // 2NWT-1] in place and the merged pair in sc[0] (the query's own
            // key among them).  Keys before token 0 drop out.
            const int kbase = t0 - NWT * kC;  // position of kk = 0
            float mx = kNegInf, lown = 0.f;  // lown: the own logit (one lane of the pair)
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) {
                const int r = acc_row(vv, hf);
                if (r == col) lown = D.tau * sc[NSLOT][vv];
#pragma unroll
                for (int j = 1; j < NSLOT; ++j) {
                    const int kk = 32 * (qt + j) + r;
                    const float x = kbase + kk >= 0 ? tl2 * sc[j][vv] : kNegInf;  // log2 units
                    sc[j][vv] = x;
                    mx = vmax(mx, x);
                }
                {
                    const bool lo = r > col;
                    const int kk = lo ? 32 * qt + r : 32 * (qt + NSLOT) + r;
                    const float x = kbase + kk >= 0 ? tl2 * (lo ? sc[0][vv] : sc[NSLOT][vv]) : kNegInf;
                    sc[0][vv] = x;
                    mx = vmax(mx, x);
                }
            }
            mx = vmax(mx, xor32(mx));
            float sa = 0.f, so = 0.f, et = 0.f;
#pragma unroll
            for (int j = 0; j < NSLOT; ++j)
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) {
                    const float x = sc[j][vv];
                    const float e = x == kNegInf ? 0.f : __builtin_amdgcn_exp2f(x - mx);
                    sc[j][vv] = e;
                    sa += e;
                    if (j == 0 && acc_row(vv, hf) == col) et += e;  // the query's own key
                    else so += e;
                }
            sa += xor32(sa);
            so += xor32(so);
            et += xor32(et);
            // Score = sum_j a_j ln((a_j + eps) / (a~_j + eps)) with a_j = e_j / sa
            // and the leave-one-out a~_j = e_j / so (j != t), a~_t = 0:
            //   own key:    a_t log1p(a_t / eps)
            //   other keys: -a_j log1p(r e_j / (e_j + eps sa)),  r = e_t / so
            const float isa = 1.f / sa;
            float term = 0.f;
            if (D.route == kRouteSaliency) {
                const float r = so > 0.f ? et / so : 0.f;
                const float esa = D.eps * sa;
#pragma unroll
                for (int j = 0; j < NSLOT; ++j)
#pragma unroll
                    for (int vv = 0; vv < 16; ++vv) {
                        const float e = sc[j][vv];
                        const float tj = -(e * isa) * log1p_fast(fast_div(r * e, e + esa));
                        term += (e > 0.f && !(j == 0 && acc_row(vv, hf) == col)) ? tj : 0.f;
                    }
                term += xor32(term);
                const float at = et * isa;  // the query's own key, once
                term += at * log1pf(at / D.eps);
            } else if (D.route == kRouteDiagonal) {
                term = et * isa;  // the own weight a_tt
            } else {
                term = lown + xor32(lown);  // the own logit tau q_t.k_t
            }
            if (hf == 0) hsc[hh][qo] = term;
#pragma unroll
            for (int s = 0; s < 8; ++s) qf[s] = qn[s];
        }
    }
    __syncthreads();
    const int nq = min(kC, D.N - t0);
    if (tid < nq) {
        float sig;
        if (route_query_free(D.route)) {
            float kn = 0.f;
            if (D.route == kRouteKeyNorm) {
                const bf16* kr = kown + tid * kKS;  // this chunk's key rows
                for (int e = 0; e < kD; ++e) kn = fmaf((float)kr[e], (float)kr[e], kn);
                kn = sqrtf(kn);
            }
            sig = query_free_score(D.route, kn, t0 + tid, b, g, D.Hkv, chunk, D.lam);
        } else {
            float acc = 0.f;
            for (int hh = 0; hh < D.G; ++hh) acc += hsc[hh][tid];
            sig = acc / (float)D.G;
        }
        scores[bg * D.N + t0 + tid] = sig;
        key_s[tid] = route_key(sig);
    }
    if (score_only) {
        if (c == 0 && b == 0) split_projections(wq, wk, wsplit, D.Hkv, g, NW * 64);
        return;
    }
    __syncthreads();
    uint8_t* rt = route + bg * D.N + t0;
    // the compact lists' last 64 rows: this chunk's tokens when it is the
    // open one (rows past N repeat token N-1), zeros after a complete last chunk
    const size_t ldkv = (size_t)D.Hkv * kD;
    const size_t list0 = ((size_t)b * sel_list_rows(D) * D.Hkv + g) * kD;  // row 0 of (b, g)
    if (c == D.T - 1) {
        const size_t pad = list0 + (size_t)D.n_full * D.lam * ldkv;
        const bool open = c >= D.n_full;
        for (int x = tid; x < kC * 16; x += NW * 64) {
            const int p = x >> 4, piece = x & 15;
            const size_t src = (((size_t)b * D.N + min(t0 + p, D.N - 1)) * D.Hkv + g) * kD + 8 * piece;
            st_bf8(ksel + pad + p * ldkv + 8 * piece, open ? ld_bf8(k + src) : zero_bf8());
            st_bf8(vsel + pad + p * ldkv + 8 * piece, open ? ld_bf8(v + src) : zero_bf8());
        }
    }
    // the first chunk's blocks of sequence 0 also split the projections
    if (c == 0 && b == 0) split_projections(wq, wk, wsplit, D.Hkv, g, NW * 64);
    if (c >= D.n_full) {  // the open chunk: no decision yet
        if (tid < nq) rt[tid] = kPending;
        return;
    }
    const size_t base = (bg * D.n_full + c) * D.lam;
    if (wave == 0) {
        // the chunk's 64 keys, one per lane: radix top-lam by ballots
        const uint32_t kb[1] = {key_bits(key_s[lane])};
        bool f[1] = {false};
        int at[1] = {0};
        if (D.lam > 0) wave_topk<1>(kb, kC, D.lam, f, at);
        rt[lane] = f[0] ? kRouteSA : kRouteLA;
        if (f[0]) sel_idx[base + at[0]] = t0 + lane;
        pos_s[lane] = f[0] ? at[0] : -1;
    }
    __syncthreads();
    // each selected row goes to its place in the compact lists (K from LDS,
    // V from the rows requested at the start)
#pragma unroll
    for (int i = 0; i < kVP; ++i) {
        const int x = tid + NW * 64 * i, p = x >> 4, piece = x & 15, at = pos_s[p];
        if (at >= 0) {
            const size_t dst = list0 + ((size_t)c * D.lam + at) * ldkv + 8 * piece;
            st_bf8(ksel + dst, ld_bf8(kown + p * kKS + 8 * piece));
            st_bf8(vsel + dst, vrow[i]);
        }
    }
}

// Selection for chunks of C = 64 CT tokens (CT = 2 or 4; the window W >= C):
// one block per (chunk, KV head, sequence) takes the top-lam of the chunk's
// C window scores (written by win_select_kernel in score mode; ties to the
// lower position), writes sel_idx, the chunk's route flags, its selected K/V
// rows at rows c lam + rank of the compact lists (list_rows rows per
// sequence), and the per-tile list offsets loff[tau] = number of compact rows
// at positions below 64 tau, tau = 0 .. N / 64, for the tiles of this chunk;
// the lists are in position order, so the selected tokens a query sees
// beyond its window are a prefix of them.  The open chunk gets pending
// flags and no rows; the last chunk's block writes the copy of an incomplete
// last tile behind the selected rows (rows past N repeat token N-1; zeros
// when N is a multiple of 64).  D holds the chunk dimensions.
template <int CT>
__global__ __launch_bounds__(256) void chunk_select_kernel(
    const float* __restrict__ scores, const bf16* __restrict__ k, const bf16* __restrict__ v,
    int32_t* __restrict__ sel_idx, uint8_t* __restrict__ route, bf16* __restrict__ ksel,
    bf16* __restrict__ vsel, int* __restrict__ loff, int list_rows, Dims D) {
    constexpr int CC = kC * CT;
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, lane = tid & 63;
    const size_t bg = (size_t)b * D.Hkv + g;
    const int t0 = c * CC, n64 = D.N / kC;
    const bool complete = c < D.n_full;
    __shared__ int pos_s[CC];
    __shared__ int cnt_s[CT];
    uint8_t* rt = route + bg * D.N + t0;
    if (tid < 64) {
        if (complete) {
            uint32_t kb[CT];
            bool f[CT];
            int at[CT];
#pragma unroll
            for (int r = 0; r < CT; ++r) {
                kb[r] = key_bits(route_key(scores[bg * D.N + t0 + 64 * r + lane]));
                f[r] = false;
                at[r] = 0;
            }
            if (D.lam > 0) wave_topk<CT>(kb, CC, D.lam, f, at);
            const size_t base = (bg * D.n_full + c) * D.lam;
#pragma unroll
            for (int r = 0; r < CT; ++r) {
                rt[64 * r + lane] = f[r] ? kRouteSA : kRouteLA;
                if (f[r]) sel_idx[base + at[r]] = t0 + 64 * r + lane;
                pos_s[64 * r + lane] = f[r] ? at[r] : -1;
                const int n = __popcll(__ballot(f[r]));
                if (lane == 0) cnt_s[r] = n;
            }
        } else {
#pragma unroll
            for (int r = 0; r < CT; ++r) {
                if (t0 + 64 * r + lane < D.N) rt[64 * r + lane] = kPending;
                pos_s[64 * r + lane] = -1;
                if (lane == 0) cnt_s[r] = 0;
            }
        }
    }
    __syncthreads();
    if (tid <= CT) {
        // tiles of this chunk, and the tile right after the last chunk when
        // that chunk is complete
        const int tau = c * CT + tid;
        if (tau <= n64 && (tid < CT || c == D.T - 1)) {
            int val = D.lam * c;
            for (int r = 0; r < tid; ++r) val += cnt_s[r];
            loff[bg * (n64 + 1) + tau] = val;
        }
    }
    const size_t ldkv = (size_t)D.Hkv * kD;
    const size_t list0 = ((size_t)b * list_rows * D.Hkv + g) * kD;  // row 0 of (b, g)
    if (complete) {
        for (int x = tid; x < CC * 16; x += 256) {
            const int p = x >> 4, piece = x & 15, at = pos_s[p];
            if (at >= 0) {
                const size_t src = (((size_t)b * D.N + t0 + p) * D.Hkv + g) * kD + 8 * piece;
                const size_t dst = list0 + ((size_t)c * D.lam + at) * ldkv + 8 * piece;
                st_bf8(ksel + dst, ld_bf8(k + src));
                st_bf8(vsel + dst, ld_bf8(v + src));
            }
        }
    }
    if (c == D.T - 1) {
        const size_t pad = list0 + (size_t)D.n_full * D.lam * ldkv;
        const bool open = D.N % kC != 0;
        const int tt0 = n64 * kC;
        for (int x = tid; x < kC * 16; x += 256) {
            const int p = x >> 4, piece = x & 15;
            const size_t src = (((size_t)b * D.N + min(tt0 + p, D.N - 1)) * D.Hkv + g) * kD + 8 * piece;
            st_bf8(ksel + pad + p * ldkv + 8 * piece, open ? ld_bf8(k + src) : zero_bf8());
            st_bf8(vsel + pad + p * ldkv + 8 * piece, open ? ld_bf8(v + src) : zero_bf8());
        }
    }
}

// Workgroup barrier that settles only this wave's LDS accesses (lgkmcnt), not
// its outstanding global loads, stores or tile staging: staged rows are
// waited for explicitly (vmcnt) at the barrier that publishes them.  The
// empty asm statements keep the compiler from moving memory accesses across
// the barrier.
__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// NP-Map of keys and linear-attention prefixes (complete chunks only)
// ---------------------------------------------------------------------------
// One block walks a run of D.ng consecutive chunks of one (b, KV head),
// keeping the running sums in its MFMA accumulators, and writes for each
// chunk c the prefix within its run,
//   S^T[dim][kperm(f)] = sum over the LA tokens of the run's chunks <= c of
//   v[dim] phi_k[f],   z[kperm(f)] = sum of phi_k[f],
// as S^T rows in bf16 (the read-out's operand precision, L.sh) and z in fp32
// (L.lz).  The fp32 state at the run's last chunk (its total, L.ltot) and at
// the hand-off chunk (L.lcap) is kept for the scan.  la_group_scan_kernel
// then forms each run's exclusive prefix over the earlier runs, so the full
// prefix of chunk c is the within-run prefix plus the prefix of run c / ng.
__global__ __launch_bounds__(256) void la_state_kernel(const bf16* __restrict__ k,
                                                       const bf16* __restrict__ v,
                                                       const bf16* __restrict__ wkh,
                                                       const bf16* __restrict__ wkl,
                                                       const uint8_t* __restrict__ route,
                                                       bf16* __restrict__ phik, LinBufs L,
                                                       int cap_chunk, Dims D) {
    const int grp = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, col = lane & 31;
    const size_t bg = (size_t)b * D.Hkv + g;
    const int c_lo = grp * D.ng, c_hi = min(D.n_full, c_lo + D.ng);
    __shared__ __align__(16) bf16 vt[kD * kVS];
    __shared__ __align__(16) float ft[kD * kFS];

    f32x16 acc[4];  // S^T rows 32 wave + .., feature tiles f4; running over the run
#pragma unroll
    for (int f4 = 0; f4 < 4; ++f4) acc[f4] = zero16();
    float zacc = 0.f;  // threads < 128: z of feature tid
    // Each chunk's keys (waves 0-1, one token per lane) and values (waves
    // 2-3, four rows x 8 dims per item, two items per lane) are loaded into
    // registers one chunk ahead, so their latency overlaps the previous
    // chunk's products; barriers wait for LDS only, never for the stores.
    bf16x8 xb[1][8];
    uint8_t rtok = 0;
    bf16x8 vr[2][4];
    auto load_chunk = [&](int c) {
        const int t0 = c * kC;
        if (wave < 2) {
            const int tok = t0 + 32 * wave + col;
            const bf16* kr = k + (((size_t)b * D.N + tok) * D.Hkv + g) * kD + 8 * hf;
#pragma unroll
            for (int s = 0; s < 8; ++s) xb[0][s] = ld_bf8(kr + 16 * s);
            rtok = route[bg * D.N + tok];
        } else {
            const bf16* src = v + (((size_t)b * D.N + t0) * D.Hkv + g) * kD;
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int x = tid - 128 + 128 * it, kq = x & 15, oct = x >> 4;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    vr[it][rr] = ld_bf8(src + (size_t)(4 * kq + rr) * D.Hkv * kD + 8 * oct);
            }
        }
    };
    if (c_lo < c_hi) load_chunk(c_lo);
    for (int c = c_lo; c < c_hi; ++c) {
        const int t0 = c * kC;
        if (wave < 2) {
            const int tt = wave;
            const int tok = t0 + 32 * tt + col;
            f32x16 phi[1][2][2];
            np_map_mfma<1>(xb, wkh + (size_t)g * (kD / 2) * kD, wkl + (size_t)g * (kD / 2) * kD, kD, phi);
            // phi_k row of the token, features in kperm order, for the read-out
            bf16* pr = phik + (bg * D.N + tok) * kD;
#pragma unroll
            for (int sgn = 0; sgn < 2; ++sgn)
#pragma unroll
                for (int f2 = 0; f2 < 2; ++f2)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        st_bf8(pr + 64 * sgn + 32 * f2 + 16 * s2 + 8 * hf, pack_acc(phi[0][sgn][f2], s2));
            const bool la = rtok == kRouteLA;
            const int tp = kperm(32 * tt + col);
#pragma unroll
            for (int sgn = 0; sgn < 2; ++sgn)
#pragma unroll
                for (int f2 = 0; f2 < 2; ++f2)
#pragma unroll
                    for (int vv = 0; vv < 16; ++vv)
                        ft[(64 * sgn + 32 * f2 + acc_row(vv, hf)) * kFS + tp] = la ? phi[0][sgn][f2][vv] : 0.f;
        } else {
            // values transposed into LDS: vt[dim][kperm(token)], as load_vt_tile
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int x = tid - 128 + 128 * it, kq = x & 15, oct = x >> 4;
                const int pos = kperm(4 * kq);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    bf16x4 t4;
                    t4[0] = vr[it][0][e];
                    t4[1] = vr[it][1][e];
                    t4[2] = vr[it][2][e];
                    t4[3] = vr[it][3][e];
                    *reinterpret_cast<bf16x4*>(vt + (8 * oct + e) * kVS + pos) = t4;
                }
            }
        }
        if (c + 1 < c_hi) load_chunk(c + 1);
        lds_barrier();
        constexpr int E1 = (kD + 1) * kD;
        const int ngroups = (D.n_full + D.ng - 1) / D.ng;
        bf16* oh = reinterpret_cast<bf16*>(L.sh) + (bg * D.n_full + c) * (size_t)(kD * kD);
        // fp32 copies: the run total (last chunk of the run), the hand-off chunk
        float* of = c == c_hi - 1 ? L.ltot + (bg * ngroups + grp) * (size_t)E1 : nullptr;
        float* oc = c == cap_chunk ? L.lcap + bg * (size_t)E1 : nullptr;
        const int dt = wave;  // dims 32 dt .. 32 dt + 31
        // S (rows = features, columns = dims) on the matrix cores, so a lane
        // holds dim 32 dt + l%32 and features 32 f4 + acc_row(vv, l/32):
        // elements 0-7 and 8-15 land at kperm positions 32 f4 + 8 hf + 0..7
        // and 32 f4 + 16 + 8 hf + 0..7 of the S^T row, two 16-byte stores
#pragma unroll
        for (int f4 = 0; f4 < 4; ++f4) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 a = ld_bf8(vt + (32 * dt + col) * kVS + 16 * ks + 8 * hf);
                bf16x8 hi, lo;
                ld_split8(ft + (32 * f4 + col) * kFS + 16 * ks + 8 * hf, hi, lo);
                acc[f4] = mfma32(hi, a, acc[f4]);
                acc[f4] = mfma32(lo, a, acc[f4]);
            }
            const int e0 = (32 * dt + col) * kD + 32 * f4 + 8 * hf;  // elements 0-7; 8-15 at e0 + 16
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                st_bf8(oh + e0 + 16 * h2, pack_acc(acc[f4], h2));
                if (of) {
                    *reinterpret_cast<f32x4*>(of + e0 + 16 * h2) =
                        f32x4{acc[f4][8 * h2], acc[f4][8 * h2 + 1], acc[f4][8 * h2 + 2], acc[f4][8 * h2 + 3]};
                    *reinterpret_cast<f32x4*>(of + e0 + 16 * h2 + 4) =
                        f32x4{acc[f4][8 * h2 + 4], acc[f4][8 * h2 + 5], acc[f4][8 * h2 + 6], acc[f4][8 * h2 + 7]};
                }
                if (oc) {
                    *reinterpret_cast<f32x4*>(oc + e0 + 16 * h2) =
                        f32x4{acc[f4][8 * h2], acc[f4][8 * h2 + 1], acc[f4][8 * h2 + 2], acc[f4][8 * h2 + 3]};
                    *reinterpret_cast<f32x4*>(oc + e0 + 16 * h2 + 4) =
                        f32x4{acc[f4][8 * h2 + 4], acc[f4][8 * h2 + 5], acc[f4][8 * h2 + 6], acc[f4][8 * h2 + 7]};
                }
            }
        }
        if (tid < kD) {
            float z = 0.f;
            for (int t = 0; t < kC; ++t) z += ft[tid * kFS + t];
            zacc += z;
            const int fz = kperm(tid);
            L.lz[(bg * D.n_full + c) * kD + fz] = zacc;
            if (of) of[kD * kD + fz] = zacc;
            if (oc) oc[kD * kD + fz] = zacc;
        }
        lds_barrier();  // the next chunk overwrites vt and ft
    }
}

// Exclusive prefix over runs: the prefix of run r is the sum of the totals of
// runs < r, written as S^T rows in bf16 (L.gh) and z in fp32 (L.gz); the full
// fp32 prefix of chunk cap_chunk also goes into the decode cache's lin_S
// [f][dim] / lin_z [f].
__global__ __launch_bounds__(256) void la_group_scan_kernel(LinBufs L, int ngroups, int cap_chunk,
                                                            float* __restrict__ cap_S,
                                                            float* __restrict__ cap_z, Dims D) {
    constexpr int E1 = (kD + 1) * kD;
    const int e = blockIdx.x * 256 + threadIdx.x, g = blockIdx.y, b = blockIdx.z;
    if (e >= E1) return;
    const size_t bg = (size_t)b * D.Hkv + g;
    const float* tot_e = L.ltot + bg * ngroups * (size_t)E1 + e;
    const bool is_s = e < kD * kD;
    bf16* gh = reinterpret_cast<bf16*>(L.gh) + bg * (size_t)ngroups * (kD * kD) + e;
    float* gz = L.gz + bg * (size_t)ngroups * kD + (is_s ? 0 : e - kD * kD);
    float run = 0.f;
    // the runs' totals are requested 16 at a time (independent loads), then
    // summed in order
    constexpr int kBatch = 16;
    for (int g0 = 0; g0 < ngroups; g0 += kBatch) {
        float tot[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) tot[i] = tot_e[(size_t)min(g0 + i, ngroups - 1) * E1];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int grp = g0 + i;
            if (grp >= ngroups) break;
            if (is_s) gh[(size_t)grp * (kD * kD)] = (bf16)run;
            else gz[(size_t)grp * kD] = run;
            const int first = grp * D.ng, last = min(D.n_full, first + D.ng) - 1;
            if (cap_S && cap_chunk >= first && cap_chunk <= last) {
                const float val = run + L.lcap[bg * E1 + e];
                const int row = e / kD, f = kperm(e % kD);
                if (row < kD) cap_S[(bg * kD + f) * kD + row] = val;
                else cap_z[bg * kD + f] = val;
            }
            run += tot[i];
        }
    }
}

// ---------------------------------------------------------------------------
// hybrid output
// ---------------------------------------------------------------------------
// one staging wave's instructions w, w + NS, ... of a K or V tile
template <int NS>
__device__ __forceinline__ void stage_k_share_u(const bf16* __restrict__ src, int ld, int nv, unsigned dst,
                                                int w) {
#pragma unroll
    for (int t = 0; t < (kKPieces + NS - 1) / NS; ++t)
        if (w + NS * t < kKPieces) stage_k_piece_u(w + NS * t, src, ld, nv, dst);
}

template <int NS>
__device__ __forceinline__ void stage_v_share_u(const bf16* __restrict__ src, int ld, int nv, unsigned dst,
                                                int w) {
#pragma unroll
    for (int t = 0; t < (kVPieces + NS - 1) / NS; ++t)
        if (w + NS * t < kVPieces) stage_v_piece_u(w + NS * t, src, ld, nv, dst);
}


// Scheduling pattern for one pair of products (value, logits) of the
// software-pipelined loop: product, R1 LDS reads, NV vector instructions,
// product, R2 LDS reads, NV vector instructions.
template <int R1, int R2, int NV>
__device__ __forceinline__ void sched_step_pair() {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (R1 > 0) __builtin_amdgcn_sched_group_barrier(0x100, R1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (R2 > 0) __builtin_amdgcn_sched_group_barrier(0x100, R2, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
}


// Workgroup barrier taken only when en != 0 (wave-uniform), after this wave's
// staging loads have landed (vmcnt); its LDS reads are not waited for.  The
// test and skip sit inside the asm statement, so the caller's code stays one
// basic block and its scheduling barriers keep their hold.
__device__ __forceinline__ void staged_barrier_if(int en) {
    const int e = __builtin_amdgcn_readfirstlane(en);
    __asm__ volatile("s_cmp_eq_u32 %0, 0\n\ts_cbranch_scc1 1f\n\ts_waitcnt vmcnt(0)\n\ts_barrier\n1:"
                     :
                     : "s"(e)
                     : "memory", "scc");
}

// Matrix phase of the lock-step output loop: the value product of the
// previous tile (V in vread, operand pb) and the logits of the current one
// (K in kread) on the matrix cores.
__device__ __forceinline__ void matrix_phase(f32x16 (&o)[4], f32x16 (&sc)[2], const bf16x8 (&pb)[4],
                                             const bf16x8 (&qf)[8], const int (&voff)[4],
                                             const bf16* __restrict__ kread, const bf16* __restrict__ vread) {
    const int lane = threadIdx.x & 63, hf = lane >> 5, col = lane & 31;
    const bf16* kt = kread + col * kKS + 8 * hf;
    bf16x8 fv[16], fk[16];
#pragma unroll
    for (int st = 0; st < 16; ++st) {
        fv[st] = vt_frag(vread, voff, st & 3, st >> 2);
        fk[st] = ld_bf8(kt + 32 * (st & 1) * kKS + 16 * (st >> 1));
    }
    sc[0] = zero16();
    sc[1] = zero16();
#pragma unroll
    for (int st = 0; st < 16; ++st) {
        o[st & 3] = mfma32(fv[st], pb[st >> 2], o[st & 3]);
        sc[st & 1] = mfma32(fk[st], qf[st >> 1], sc[st & 1]);
    }
}

// Block = HB query heads of KV head g x the 64 tokens of chunk c; two waves
// per head, each owning 32 queries, so two waves share every SIMD and one's
// softmax arithmetic overlaps the other's matrix products.  Key tiles, in
// order: chunks c-NWT .. c (the window, NWT = W / 64; chunk c-NWT also holds
// the routed selected tokens at or below the query's offset), then the
// compact selected rows of chunks <= c-NWT-1, 64 at a time; each tile is
// staged in one of two LDS buffers while the previous one is computed.
// Blocks are issued longest first (largest c); consecutive blocks take
// different KV heads, so each XCD's L2 keeps few compact lists.
//
// stat (not STATS, when not null): with the output, each query head's (m, l,
// 0, c) as below, for a backward that starts from them.
// STATS (the backward's first pass): instead of the output, each query head
// writes (m, l, D, c) to stat: the reference m in natural units, the
// normaliser l at that reference (linear terms included), D = dout . out
// (out = O / l in fp32), and c = exp(-m) / l when the query has linear mass
// (else 0).  list_off (when not null) gives the compact rows of chunk c as
// rows list_off[c] .. list_off[c + 1] - 1 of (b, g) (n_full + 1 entries, the
// last the open chunk's copy), for lists built from a given selection whose
// chunks may hold fewer than lam rows.  STATS also writes each query head's
// gated NP-Map features gamma phi_q (bf16, in the features' storage order:
// position p holds feature kperm(p), as for phi_k) to phiq_out (zeros for
// queries with no routed token).
template <int HB, int NWT, bool STATS = false>
__global__ __launch_bounds__(HB * 128) void hybrid_main_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ wqh, const bf16* __restrict__ wql, const bf16* __restrict__ phik,
    const uint8_t* __restrict__ route,
    const bf16* __restrict__ ksel, const bf16* __restrict__ vsel, LinBufs L,
    const float* __restrict__ gate, bf16* __restrict__ out, const int* __restrict__ list_off,
    const bf16* __restrict__ dout, float* __restrict__ stat, bf16* __restrict__ phiq_out, Dims D) {
    constexpr int NW = HB * 2;  // waves
    const int HG = D.G / HB;
    const int per_c = D.B * D.Hkv * HG;
    const int c = D.T - 1 - (int)(blockIdx.x / per_c);
    int r = (int)(blockIdx.x % per_c);
    const int hg = r % HG;
    r /= HG;
    const int g = r % D.Hkv, b = r / D.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, col = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // waves 0..HB-1 take the first 32 queries of their head, waves HB.. the
    // last 32; with HB = 4 the two halves of a head share a SIMD
    const int qh = wave / HB;  // wave-uniform (scalar)
    const int h = g * D.G + hg * HB + wave % HB;
    const int t0 = c * kC;
    const int oq = 32 * qh + col;                  // this lane's query offset in the chunk
    const size_t bg = (size_t)b * D.Hkv + g;
    const float cl2 = D.tau * kLog2e;

    // K of tile i in kbuf(i) (two buffers), V of tile i in vbuf(i) (three: the
    // second query half still reads the previous tile's values after the
    // barrier that lets the first half stage the next ones).  The linear
    // prefix S^T rows (then z) follow; the epilogue reuses the front.
    constexpr int kNV = 3;
    // staged linear prefix: S^T rows in bf16 [kD][kHS], then z as kD floats
    // (from float kZOff); the epilogue reuses the same bytes
    constexpr int kZOff = kD * kHS / 2;
    constexpr int kPrefixFloats = kZOff + kD;
    // the same bytes first hold the prologue's projection parts and phi_k rows
    // (three K-tile layouts) and last the output tiles (HB * 32 * kKS floats)
    constexpr int kPreFloats = 3 * kKTile / 2;
    constexpr int kStsA = kPrefixFloats > kPreFloats ? kPrefixFloats : kPreFloats;
    // behind the prologue data: rows 64-127 of the earlier runs' prefix
    // (16 KB) and the two z vectors (1 KB), parked there by the first round trip
    constexpr int kParkFloats = kPreFloats + kD * kD / 4 + 2 * kD;
    constexpr int kStsB = kStsA > kParkFloats ? kStsA : kParkFloats;
    constexpr int kStsFloats = kStsB > HB * 32 * kKS ? kStsB : HB * 32 * kKS;
    __shared__ __align__(16) bf16 smem[2 * kKTile + kNV * kVTile];
    __shared__ __align__(16) float sts[kStsFloats];
    auto kbuf = [&](int i) { return smem + (i & 1) * kKTile; };
    auto vbuf = [&](int i) { return smem + 2 * kKTile + ((i + 3) % 3) * kVTile; };  // i >= -1

    // tiles: i <= NWT = chunk c-NWT+i (those before chunk 0 are skipped),
    // NWT+1.. = compact selected rows of chunks <= c-NWT-1
    const int* loff = list_off ? list_off + bg * (D.n_full + 1) : nullptr;
    const int nrows = c > NWT ? (loff ? loff[c - NWT] : (c - NWT) * D.lam) : 0;
    const int tail_row = loff ? loff[D.n_full] : D.n_full * D.lam;  // the open chunk's copy
    const int ntile = NWT + 1 + (nrows + kC - 1) / kC;
    const int first = c >= NWT ? 0 : NWT - c;
    const int tla = t0 - NWT * kC;  // first token of chunk c-NWT (the partly routed one)
    // compact lists of (b, g): rows ldkv elements apart, like k and v
    const size_t ldkv = (size_t)D.Hkv * kD;
    const bf16* kb = ksel + ((size_t)b * sel_list_rows(D) * D.Hkv + g) * kD;
    const bf16* vb = vsel + ((size_t)b * sel_list_rows(D) * D.Hkv + g) * kD;
    // rows of tile i: source offset (elements, K and V alike), row stride,
    // valid count, and whether the rows come from the compact lists.  Every
    // tile has 64 readable rows ldkv apart: an incomplete last chunk is read
    // from its copy at the end of the compact lists.
    auto tile_src = [&](int i, size_t& off, size_t& ld, int& nv, bool& compact) {
        ld = ldkv;
        if (i <= NWT) {
            const int tc = c - NWT + i;
            nv = min(kC, D.N - tc * kC);
            compact = nv < kC;
            off = compact ? (size_t)tail_row * ldkv
                          : (((size_t)b * D.N + (size_t)tc * kC) * D.Hkv + g) * kD;
        } else {
            const int r0 = (i - NWT - 1) * kC;
            off = (size_t)r0 * ldkv;
            nv = min(kC, nrows - r0);
            compact = true;
        }
    };
    // issue this wave's share of the staging instructions of K and/or V of
    // tile i; they complete by the wave's next vmcnt(0)
    auto stage = [&](int i, bool do_k, bool do_v) {
        size_t off, ld;
        int nv;
        bool cp;
        tile_src(i, off, ld, nv, cp);
        if (do_k)
            for (int j = wave; j < kKPieces; j += NW) stage_k_piece(j, (cp ? kb : k) + off, ld, nv, kbuf(i));
        if (do_v)
            for (int j = wave; j < kVPieces; j += NW) stage_v_piece(j, (cp ? vb : v) + off, ld, nv, vbuf(i));
    };
    int voff[4];
    vt_lane_offsets(voff);

    // The prologue's reads are requested together: the first tile; into the
    // prefix area (free until the prefix itself is written there) the NP-Map
    // projection parts and the phi_k rows of chunk c-NWT, in the K tile
    // layout; the route flags of chunk c-NWT; Q.  The prefix rows follow once
    // the projections and phi_k rows have been used.
    // (written before the staging below is issued)
    stage(first, true, true);
    bf16* pre = reinterpret_cast<bf16*>(sts);  // [W high | W low | phi_k rows], kKTile each
    {
        const bf16* wh = wqh + (size_t)g * (kD / 2) * kD;
        const bf16* wl_ = wql + (size_t)g * (kD / 2) * kD;
        for (int j = wave; j < kKPieces; j += NW) {
            stage_k_piece(j, wh, kD, kD / 2, pre);
            stage_k_piece(j, wl_, kD, kD / 2, pre + kKTile);
        }
        if (c >= NWT) {
            const bf16* pk = phik + (bg * D.N + tla) * kD;
            for (int j = wave; j < kKPieces; j += NW) stage_k_piece(j, pk, kD, kC, pre + 2 * kKTile);
        }
    }
    // The linear prefix of chunks <= c-NWT-1 (bf16 S^T rows, 32 KB each: the
    // within-run part sh of chunk c-NWT-1 and the earlier runs' part gh) and
    // their z vectors come with the same round trip, straight into LDS areas
    // the prologue leaves free: sh into V buffers 1-2, gh rows 0-63 into K
    // buffer 1, rows 64-127 and the z vectors (lz | gz) behind the prologue
    // data in sts.  (When there is a prefix, c > NWT, the first tile is tile 0 in K buffer 0 and V
    // buffer 0.)
    const int ngroups = (D.n_full + D.ng - 1) / D.ng;
    const char* park_sh = reinterpret_cast<const char*>(smem + 2 * kKTile + kVTile);
    const char* park_gh0 = reinterpret_cast<const char*>(smem + kKTile);
    const char* park_gh1 = reinterpret_cast<const char*>(sts + kPreFloats);
    const float* park_z = sts + kPreFloats + kD * kD / 4;
    if (c > NWT) {
        const int cp = c - NWT - 1, run = cp / D.ng;
        const bf16* shg = reinterpret_cast<const bf16*>(L.sh) + (bg * D.n_full + cp) * (size_t)(kD * kD);
        const bf16* ghg = reinterpret_cast<const bf16*>(L.gh) + (bg * ngroups + run) * (size_t)(kD * kD);
        // instruction j moves bytes 1024 j .. 1024 j + 1023 of a matrix
        for (int j = wave; j < 32; j += NW) {
            dma16(shg + 512 * j + 8 * lane, (bf16*)park_sh + 512 * j);
            dma16(ghg + 512 * j + 8 * lane, (bf16*)(j < 16 ? park_gh0 : park_gh1) + 512 * (j & 15));
        }
        if (wave == NW - 1) {
            const float* zsrc = lane < 32 ? L.lz + (bg * D.n_full + cp) * kD + 4 * lane
                                          : L.gz + (bg * ngroups + run) * kD + 4 * (lane - 32);
            dma16(reinterpret_cast<const bf16*>(zsrc), (bf16*)park_z);
        }
    }
    const uint8_t rt = c >= NWT ? route[bg * D.N + tla + lane] : 0;
    // Q operand: qf[s] holds query t0 + oq (tokens past N repeat N-1, never
    // written), dims 16 s + 8 hf .. +7
    bf16x8 qf[1][8];
    {
        const int t = min(t0 + oq, D.N - 1);
        const bf16* row = q + (((size_t)b * D.N + t) * D.Hq + h) * kD + 8 * hf;
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[0][s] = ld_bf8(row + 16 * s);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): everything above
    __syncthreads();

    // running state of the lane's query: reference point m2 (log2 units,
    // starts at 0, the linear terms' reference; see nola below for queries
    // without linear terms), partial normaliser ls of
    // this half's rows; O^T tiles o[dt]: rows = dims 32 dt + .., column = query
    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = zero16();
    float m2 = 0.f, ls = 0.f;
    uint64_t selmask = 0;

    if (c >= NWT) {
        selmask = __ballot(rt == kRouteSA);
        f32x16 phi[1][2][2];
        np_map_mfma<1>(qf, pre, pre + kKTile, kKS, phi);
        if (gate) {
            // the query's features carry its gate weight, so both the linear
            // numerator and denominator below do
            const int tg = min(t0 + oq, D.N - 1);
            const float gw = gate_weight(gate, ((size_t)b * D.N + tg) * D.Hq + h);
#pragma unroll
            for (int sgn = 0; sgn < 2; ++sgn)
#pragma unroll
                for (int f2 = 0; f2 < 2; ++f2)
#pragma unroll
                    for (int vv = 0; vv < 16; ++vv) phi[0][sgn][f2][vv] *= gw;
        }
        if constexpr (STATS) {
            // this lane's 64 features of its query, 64 sgn + 32 f2 + acc_row(..),
            // at their storage positions (position p holds feature kperm(p))
            if (t0 + oq < D.N) {
                bf16* pr = phiq_out + (((size_t)b * D.N + t0 + oq) * D.Hq + h) * kD;
#pragma unroll
                for (int sgn = 0; sgn < 2; ++sgn)
#pragma unroll
                    for (int f2 = 0; f2 < 2; ++f2)
#pragma unroll
                        for (int v4 = 0; v4 < 4; ++v4) {
                            bf16x4 x4;
#pragma unroll
                            for (int j = 0; j < 4; ++j) x4[j] = (bf16)phi[0][sgn][f2][4 * v4 + j];
                            *reinterpret_cast<bf16x4*>(pr + kperm(64 * sgn + 32 * f2 + acc_row(4 * v4, hf))) = x4;
                        }
            }
        }

        bf16x8 phb[2][2][2];  // [sgn][ft][s2]
#pragma unroll
        for (int sgn = 0; sgn < 2; ++sgn)
#pragma unroll
            for (int f2 = 0; f2 < 2; ++f2) {
                phb[sgn][f2][0] = pack_acc(phi[0][sgn][f2], 0);
                phb[sgn][f2][1] = pack_acc(phi[0][sgn][f2], 1);
            }
        {
            // routed linear tokens of chunk c-NWT (offset <= the query's, not
            // selected): weight phi_k(k_j) . phi_q(q_t) at reference point 0
            f32x16 wl[2];  // rows = keys, column = query
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                wl[kt] = zero16();
                const bf16* pk = pre + 2 * kKTile + (32 * kt + col) * kKS + 8 * hf;
#pragma unroll
                for (int sgn = 0; sgn < 2; ++sgn)
#pragma unroll
                    for (int f2 = 0; f2 < 2; ++f2)
#pragma unroll
                        for (int s2 = 0; s2 < 2; ++s2)
                            wl[kt] = mfma32(ld_bf8(pk + 64 * sgn + 32 * f2 + 16 * s2), phb[sgn][f2][s2], wl[kt]);
            }
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) {
                    const int rk = 32 * kt + acc_row(vv, hf);
                    const bool la = rk <= oq && !((selmask >> rk) & 1ull);
                    const float p = la ? wl[kt][vv] : 0.f;
                    wl[kt][vv] = p;
                    ls += p;
                }
            const bf16* vt = vbuf(first);  // tile 0 = chunk c-NWT
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 pa = pack_acc(wl[ks >> 1], ks & 1);
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) o[dt] = mfma32(vt_frag(vt, voff, dt, ks), pa, o[dt]);
            }
        }
        if (c > NWT) {
            // prefix of chunks <= c-NWT-1 (within-run part + earlier runs), staged
            // in LDS once for all waves (over the projections and phi_k rows,
            // now read): S^T rounded to bf16 (the MFMA operand, the precision
            // of every other product on this path), z in fp32
            // within-run prefix of chunk c-NWT-1 plus the prefix of its run: the
            // S^T rows arrive in bf16 (pieces of 4) and are added in fp32 and
            // rounded once; z is fp32 throughout
            constexpr int kSPieces = kD * kD / 4, kSPer = (kSPieces + 64 * NW - 1) / (64 * NW);
            __syncthreads();
            bf16* sth = reinterpret_cast<bf16*>(sts);
            // piece x: elements 4x .. 4x+3 of the S^T rows (row 4x / kD)
#pragma unroll
            for (int t = 0; t < kSPer; ++t) {
                const int x = tid + 64 * NW * t;
                if (x < kSPieces) {
                    const bf16x4 sa = *reinterpret_cast<const bf16x4*>(park_sh + 8 * x);
                    const bf16x4 sg = *reinterpret_cast<const bf16x4*>(
                        x < kSPieces / 2 ? park_gh0 + 8 * x : park_gh1 + 8 * (x - kSPieces / 2));
                    bf16x4 hi;
#pragma unroll
                    for (int j = 0; j < 4; ++j) hi[j] = (bf16)((float)sa[j] + (float)sg[j]);
                    *reinterpret_cast<bf16x4*>(sth + (4 * x / kD) * kHS + (4 * x) % kD) = hi;
                }
            }
            if (tid < kD / 4)
                *reinterpret_cast<f32x4*>(&sts[kZOff + 4 * tid]) =
                    *reinterpret_cast<const f32x4*>(park_z + 4 * tid) +
                    *reinterpret_cast<const f32x4*>(park_z + kD + 4 * tid);
            __syncthreads();
            // normaliser of the linear prefix (chunks <= c-NWT-1): phi_q . z, with
            // the same bf16 features as the numerator's products
            float acc = 0.f;
#pragma unroll
            for (int sgn = 0; sgn < 2; ++sgn)
#pragma unroll
                for (int f2 = 0; f2 < 2; ++f2)
#pragma unroll
                    for (int vv = 0; vv < 16; ++vv)
                        acc = fmaf(sts[kZOff + kperm(64 * sgn + 32 * f2 + acc_row(vv, hf))],
                                   (float)phb[sgn][f2][vv >> 3][vv & 7], acc);
            ls += acc;
            // numerator of the linear prefix: O^T += S^T phi_q
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int sgn = 0; sgn < 2; ++sgn)
#pragma unroll
                    for (int f2 = 0; f2 < 2; ++f2)
#pragma unroll
                        for (int s2 = 0; s2 < 2; ++s2) {
                            const bf16* sr = reinterpret_cast<const bf16*>(sts) + (32 * dt + col) * kHS +
                                             64 * sgn + 32 * f2 + 16 * s2 + 8 * hf;
                            o[dt] = mfma32(ld_bf8(sr), phb[sgn][f2][s2], o[dt]);
                        }
        }
    }

    if constexpr (STATS) {
        if (c < NWT && t0 + oq < D.N) {  // no routed token yet: no linear term
            bf16* pr = phiq_out + (((size_t)b * D.N + t0 + oq) * D.Hq + h) * kD;
            const bf16x4 z4 = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
#pragma unroll
            for (int x = 0; x < 16; ++x) *reinterpret_cast<bf16x4*>(pr + 32 * (x >> 2) + acc_row(4 * (x & 3), hf)) = z4;
        }
    }
    // A query with no linear mass (t < W, or every routed token of its
    // chunks selected) has nothing at the linear reference 0, so its
    // reference need not stay >= 0: at the first tile with a key it can see,
    // m2 moves to that tile's maximum, up or down.  Logits far below 0
    // would otherwise underflow every weight and leave 0 / 0.  The flag is
    // the same in both lanes of a query.
    bool nola = !(ls + xor32(ls) > 0.f);
    const bool lamass = !nola;

    // logits of tile i (K^T Q on the matrix cores)
    auto qk = [&](int i, f32x16 (&sc)[2]) {
        const bf16* ks = kbuf(i);
        sc[0] = zero16();
        sc[1] = zero16();
#pragma unroll
        for (int s = 0; s < 8; ++s) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                sc[kt] = mfma32(ld_bf8(ks + (32 * kt + col) * kKS + 16 * s + 8 * hf), qf[0][s], sc[kt]);
        }
    };
    // softmax terms of tile i, in place: key row rk counts for the lane's
    // query when bit rk of (rk > oq ? hi_m : lo_m) is set
    // softmax terms of tile i, in place, in three steps.  Masking: key row
    // rk counts for the lane's query when bit rk of (rk > oq ? hi_m : lo_m)
    // is set.
    auto softmax_mask = [&](int i, f32x16 (&sc)[2]) -> bool {
        // chunk c-NWT (i = 0): window keys (offset above the query's) and
        // routed selected keys; chunk c (i = NWT): causal; chunks between:
        // inside every query's window; compact rows: the valid ones.  Written
        // as selects on wave-uniform values (no branches).
        const int nvc = nrows - (i - NWT - 1) * kC;
        const uint64_t part = nvc >= kC ? ~0ull : (1ull << (nvc & 63)) - 1ull;
        const bool win = i <= NWT;
        const uint64_t hi_m = win ? (i == NWT ? 0ull : ~0ull) : part;
        const uint64_t lo_m = win ? (i == 0 ? selmask : ~0ull) : part;
        if ((hi_m & lo_m) != ~0ull) {
            // edge tiles only: masked key rows drop out of the softmax.  The
            // lane's combined mask, shifted down by 4 hf, holds the bit of
            // element vv of accumulator kt at 32 kt + 8 (vv / 4) + vv % 4.
            __asm__ volatile("");
            const uint64_t gt = oq >= 63 ? 0ull : ~0ull << (oq + 1);
            const uint64_t mm = ((hi_m & gt) | (lo_m & ~gt)) >> (4 * hf);
            const uint32_t mw[2] = {(uint32_t)mm, (uint32_t)(mm >> 32)};
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int vv = 0; vv < 16; ++vv)
                    if (!((mw[kt] >> (8 * (vv >> 2) + (vv & 3))) & 1u)) sc[kt][vv] = kNegInf;
            return true;
        }
        return false;
    };
    // reference point: when the tile's maximum exceeds m2 by more than kLazy
    // (log2 units) the reference moves up to the next integer at or above it
    // and the running sums scale by al, an exact power of two (returns true;
    // the caller scales O)
    auto softmax_ref = [&](const f32x16 (&sc)[2], float& al) -> bool {
        float tmax = kNegInf;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) tmax = vmax(tmax, sc[kt][vv]);
        const float tm2 = half_pair_max(tmax) * cl2;
        const bool down = nola && tm2 > kNegInf;
        if (__any(tm2 > m2 + kLazy || down)) {
            // a rare path: keep the compiler from speculating it into every tile
            __asm__ volatile("");
            float mn = ceilf(fmaxf(m2, tm2));
            al = __builtin_amdgcn_exp2f(m2 - mn);
            if (down) {
                // first visible key of a query without linear mass: nothing
                // is summed yet (O and ls are 0), the reference takes this
                // tile's maximum
                mn = ceilf(tm2);
                al = 0.f;
                nola = false;
            }
            m2 = mn;
            ls *= al;
            return true;
        }
        return false;
    };
    auto softmax_exp = [&](f32x16 (&sc)[2]) {
        const float nm = -m2;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) {
                // the normaliser sums the bf16 probabilities the value product
                // uses, so O / l is their exact weighted mean
                const float p = (float)(bf16)__builtin_amdgcn_exp2f(fmaf(sc[kt][vv], cl2, nm));
                sc[kt][vv] = p;
                ls += p;
            }
    };
    auto softmax = [&](int i, f32x16 (&sc)[2]) {
        softmax_mask(i, sc);
        float al = 1.f;
        if (softmax_ref(sc, al)) {
            __asm__ volatile("");
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) o[dt][vv] *= al;
        }
        softmax_exp(sc);
    };

    f32x16 sc[2];
    if constexpr (HB == 4) {
        // Software-pipelined loop, the same in every wave: iteration s runs
        // the value product of tile s-1 and the logits of tile s+1 on the
        // matrix cores while the vector units work through the softmax of
        // tile s, all in one instruction stream, so each wave keeps its
        // products and its exp arithmetic in flight together.  Iteration s
        // reads K of s+1 and V of s-1 and stages K of s+2 and V of s (LDS
        // straight from global memory, untracked, settled before the
        // iteration's barrier).  The first value product runs on zero
        // probabilities over the zero-filled spare V buffer.
        const unsigned lds0 = (unsigned)(size_t)(lds_void*)smem;
        // first row of tile i in k / v or the compact lists (every tile has 64
        // readable rows ldkv apart): window chunks c-NWT+i (chunk c, when
        // incomplete, from its copy), then compact rows 64 (i - NWT - 1) on
        const int64_t tstride = (int64_t)kC * (int64_t)ldkv;
        const int64_t win0 = (((int64_t)b * D.N + (int64_t)(c - NWT) * kC) * D.Hkv + g) * kD;
        const bool open_c = D.N - t0 < kC;
        auto tile_ptr = [&](int i, bool is_k) -> const bf16* {
            if (i > NWT) return (is_k ? kb : vb) + (int64_t)(i - NWT - 1) * tstride;
            if (i == NWT && open_c) return (is_k ? kb : vb) + (int64_t)tail_row * (int64_t)ldkv;
            return (is_k ? k : v) + win0 + (int64_t)i * tstride;
        };
        auto rows_of = [&](int i, bool is_k, int& ld, int& nv) -> const bf16* {
            size_t off, ld64;
            bool cp;
            tile_src(i, off, ld64, nv, cp);
            ld = (int)ld64;
            return (is_k ? (cp ? kb : k) : (cp ? vb : v)) + off;
        };
        // the V buffer of tile first-1 holds zeros: the first value product
        // reads it (with zero probabilities); the prologue's parked prefix
        // there has been read (barrier after its use above)
        {
            bf16* vz = vbuf(first - 1);
            for (int x = tid; x < kVTile / 8; x += 64 * NW) st_bf8(vz + 8 * x, zero_bf8());
        }
        bf16x8 pb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) pb[ks] = zero_bf8();
        // lane offsets of this wave's staging instructions (pieces wave,
        // wave + 8 and, for K, wave + 16 when it exists)
        const unsigned ld2 = 2u * (unsigned)ldkv;
        unsigned kpo[3], vpo[2];
#pragma unroll
        for (int x = 0; x < 3; ++x) kpo[x] = k_piece_off(min(wave + 2 * HB * x, kKPieces - 1), ld2);
#pragma unroll
        for (int x = 0; x < 2; ++x) vpo[x] = v_piece_off(wave + 2 * HB * x, ld2);
        // K of first+1 (V of first and K of first are in place; a tile index
        // past the last one stages the last one again, unused)
        {
            int ld, nv;
            const bf16* src = rows_of(min(first + 1, ntile - 1), true, ld, nv);
            stage_k_share_u<2 * HB>(src, ld, nv, lds0 + 2u * ((first + 1) & 1) * kKTile, wave);
        }
        qk(first, sc);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        lds_barrier();
        // One iteration: tile s's logits in sc and tile s-1's probabilities in
        // pb; leaves tile s+1's logits in sn and tile s's probabilities in pn.
        // Two calls per loop turn with the roles swapped keep every value in
        // place (no copies).
        // The first query half, which the SIMD's issue order favours, reaches
        // the iteration's barrier at the end of its stream; the second half
        // (late != 0) reaches it after step 11 and runs its last value
        // products (of tile s-1, whose V buffer stays intact until iteration
        // s+2) beyond it, so the two halves arrive together.  Both issue their
        // staging in steps 1-5, well before either barrier point.
        auto iteration = [&](int s, f32x16 (&sc)[2], bf16x8 (&pb)[4], f32x16 (&sn)[2], bf16x8 (&pn)[4])
                             __attribute__((always_inline)) {
            // One stream of 16 steps pinned by scheduling barriers.  Steps 0-7
            // take the logits of tile s+1 (two products each: keys 0-31 and
            // 32-63), steps 8-15 the value product of tile s-1 (two each);
            // every step does the exps of two elements of tile s and issues
            // the operand reads of the step two ahead; some steps issue a
            // staging instruction.  The reads of the first two steps go out
            // before the iteration's scalar set-up, which runs under them.
            const bf16* kt = kbuf(s + 1) + col * kKS + 8 * hf;
            // V buffers of tiles s (staged now) and s-1 (read now), as scalars
            const int vcur = __builtin_amdgcn_readfirstlane(s % 3);
            const int vprv = __builtin_amdgcn_readfirstlane((s + 2) % 3);
            const bf16* vt = smem + 2 * kKTile + vprv * kVTile;
            bf16x8 a0[16], a1[16];
            auto operands = [&](int st) __attribute__((always_inline)) {
                if (st < 8) {
                    a0[st] = ld_bf8(kt + 16 * st);
                    a1[st] = ld_bf8(kt + 32 * kKS + 16 * st);
                } else {
                    const int x = 2 * (st - 8);
                    a0[st] = vt_frag(vt, voff, x & 3, x >> 2);
                    a1[st] = vt_frag(vt, voff, (x + 1) & 3, (x + 1) >> 2);
                }
            };
            operands(0);
            operands(1);
            __builtin_amdgcn_sched_barrier(0);
            // softmax of tile s: masking (edge tiles only), then the exps
            // against the current reference m2 in the stream below; their
            // sums (ls - ls0) are checked after it
            softmax_mask(s, sc);
            const float ls0 = ls;
            // staging destinations and sources: K of s+2 (or the last tile
            // again), V of s
            const bf16* ksrc = tile_ptr(min(s + 2, ntile - 1), true);
            const bf16* vsrc = tile_ptr(s, false);
            const unsigned kdst = lds0 + 2u * (s & 1) * kKTile;
            const unsigned vdst = lds0 + 2u * (2 * kKTile + vcur * kVTile);
            sn[0] = zero16();
            sn[1] = zero16();
            const float nm = -m2;
            float pt[8];
#pragma unroll
            for (int st = 0; st < 16; ++st) {
                if (st + 2 < 16) operands(st + 2);
                if (st < 8) {
                    sn[0] = mfma32(a0[st], qf[0][st], sn[0]);
                    sn[1] = mfma32(a1[st], qf[0][st], sn[1]);
                } else {
                    const int x = 2 * (st - 8);
                    o[x & 3] = mfma32(a0[st], pb[x >> 2], o[x & 3]);
                    o[(x + 1) & 3] = mfma32(a1[st], pb[(x + 1) >> 2], o[(x + 1) & 3]);
                }
#pragma unroll
                for (int e = 2 * st; e < 2 * st + 2; ++e) {
                    // the logits stay in sc (the overflow check may need them)
                    pt[e & 7] = __builtin_amdgcn_exp2f(fmaf(sc[e >> 4][e & 15], cl2, nm));
                    // the empty asm needs the result here, which keeps the exp in
                    // this step (otherwise the exps of the first of two unrolled
                    // iterations sink below its products, into one block of their own)
                    __asm__ volatile("" ::"v"(pt[e & 7]));
                }
                if ((st & 3) == 3) {
                    // the normaliser sums the same bf16 probabilities the value
                    // product uses (two per dot instruction)
                    bf16x8 pk;
#pragma unroll
                    for (int j = 0; j < 8; ++j) pk[j] = (bf16)pt[j];
                    pn[st >> 2] = pk;
                    const bf16x2 one2 = {(bf16)1.f, (bf16)1.f};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bf16x2 pr = {pk[2 * j], pk[2 * j + 1]};
                        ls = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, ls, false);
                    }
                    // keeps the pack and the sums in this step (as for the exps)
                    __asm__ volatile("" ::"v"(pk), "v"(ls));
                }
                if (st == 1 || st == 3 || st == 5) {
                    const int x = st / 2;  // the third piece (16) is wave 0's alone
                    dma16_sbase_if(ksrc, kpo[x], kdst + 1024u * (wave + 2 * HB * x),
                                   x < 2 || wave + 2 * HB * x < kKPieces);
                }
                if (st == 2 || st == 4) {
                    const int x = st / 2 - 1;
                    dma16_sbase_if(vsrc, vpo[x], vdst + 1024u * (wave + 2 * HB * x), 1);
                }
                if (st == 11) staged_barrier_if(qh);
                // within the step: both products first, then the operand
                // reads, then the vector instructions (measured 1% faster
                // than leaving the order to the scheduler, which splits them)
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 30, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            staged_barrier_if(qh ^ 1);
            // Reference point.  The exps above were taken against m2, which
            // starts at the linear terms' reference 0 and is kept unless a
            // tile's exps come out too large: when some lane's sum for this
            // tile reaches 2^64 (or is not finite), m2 moves up to the next
            // integer at or above the tile's maximum, O and the normaliser
            // scale by al (a power of two, so exactly) and the tile's
            // probabilities are formed again from its logits.  Weights below
            // 2^64 keep their relative precision in fp32 and bf16, so no
            // running maximum is needed on the common path.
            // A query without linear mass takes this path at each tile until
            // the first one with a key it can see, whose maximum becomes its
            // reference (earlier tiles summed nothing: O and ls are 0).
            if (__any(!(ls - ls0 < 0x1p64f) || nola)) {
                // a rare path: keep the compiler from speculating it into every tile
                __asm__ volatile("");
                float mx = kNegInf;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int vv = 0; vv < 16; ++vv) mx = vmax(mx, sc[kt][vv]);
                const float pm = half_pair_max(mx) * cl2;
                float mn = ceilf(fmaxf(m2, pm));
                float al = __builtin_amdgcn_exp2f(m2 - mn);
                if (nola && pm > kNegInf) {
                    mn = ceilf(pm);
                    al = 0.f;
                    nola = false;
                }
                m2 = mn;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int vv = 0; vv < 16; ++vv) o[dt][vv] *= al;
                ls = ls0 * al;
                const bf16x2 one2 = {(bf16)1.f, (bf16)1.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        pn[ks][j] = (bf16)__builtin_amdgcn_exp2f(fmaf(sc[ks >> 1][8 * (ks & 1) + j], cl2, -mn));
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bf16x2 pr = {pn[ks][2 * j], pn[ks][2 * j + 1]};
                        ls = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, ls, false);
                    }
                }
            }
        };
        f32x16 sc2[2];
        bf16x8 pb2[4];
        int s = first;
        for (; s + 1 < ntile; s += 2) {
            iteration(s, sc, pb, sc2, pb2);
            iteration(s + 1, sc2, pb2, sc, pb);
        }
        if (s < ntile) {
            iteration(s, sc, pb, sc2, pb2);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) pb[ks] = pb2[ks];
        }
        {
            // value product of the last tile
            const bf16* vt = vbuf(ntile - 1);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) o[dt] = mfma32(vt_frag(vt, voff, dt, ks), pb[ks], o[dt]);
        }
    } else {
        // The first query half runs [logits, softmax, values] of tile i; the
        // second runs [softmax, values] of tile i-1 and then the logits of
        // tile i, so on each SIMD one wave's exp arithmetic meets the other's
        // products.  Tile i+1 is staged during step i.
        for (int i = first; i <= ntile; ++i) {
            if (i + 1 < ntile) stage(i + 1, true, true);
#pragma unroll 1
            for (int ph = 0; ph < 2; ++ph) {
                if (ph == qh && i < ntile) qk(i, sc);
                if (ph == 0) {
                    const int j = i - qh;
                    if (j >= first && j < ntile) {
                        softmax(j, sc);
                        const bf16* vt = vbuf(j);
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks) {
                            const bf16x8 pa = pack_acc(sc[ks >> 1], ks & 1);
#pragma unroll
                            for (int dt = 0; dt < 4; ++dt) o[dt] = mfma32(vt_frag(vt, voff, dt, ks), pa, o[dt]);
                        }
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile i+1 landed
            __syncthreads();
        }
    }

    if constexpr (STATS) {
        // statistics of the lane's query: D = dout . O / l over the lane's 64
        // dims (32 dt + acc_row(..)) plus the other half's
        const float lsum = ls + xor32(ls);
        const int tq = min(t0 + oq, D.N - 1);
        const size_t qo = ((size_t)b * D.N + tq) * D.Hq + h;
        const bf16* dr = dout + qo * kD;
        float dp = 0.f;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const bf16x4 d4 = *reinterpret_cast<const bf16x4*>(dr + 32 * dt + acc_row(4 * v4, hf));
#pragma unroll
                for (int j = 0; j < 4; ++j) dp = fmaf(o[dt][4 * v4 + j], (float)d4[j], dp);
            }
        dp = (dp + xor32(dp)) / lsum;
        if (hf == 0 && t0 + oq < D.N) {
            constexpr float kLn2 = 0.6931471805599453f;
            f32x4 st;
            st[0] = m2 * kLn2;
            st[1] = lsum;
            st[2] = dp;
            st[3] = lamass ? __builtin_amdgcn_exp2f(-m2) / lsum : 0.f;
            *reinterpret_cast<f32x4*>(stat + qo * 4) = st;
        }
        // tile staging issued by the loop's last steps lands before the wave ends
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        return;
    }
    // epilogue: normalise, stage each wave's 32 x 128 tile in LDS, write rows
    const float lsum = ls + xor32(ls);
    const float il = 1.f / lsum;
    if (stat && hf == 0 && t0 + oq < D.N) {
        // the statistics a backward can start from: reference m (natural
        // units), normaliser l, 0 in place of dout . out, c = exp(-m) / l
        // for a query with linear terms (else 0)
        constexpr float kLn2 = 0.6931471805599453f;
        f32x4 st;
        st[0] = m2 * kLn2;
        st[1] = lsum;
        st[2] = 0.f;
        st[3] = lamass ? __builtin_amdgcn_exp2f(-m2) / lsum : 0.f;
        *reinterpret_cast<f32x4*>(stat + (((size_t)b * D.N + t0 + oq) * D.Hq + h) * 4) = st;
    }
    bf16* ot = reinterpret_cast<bf16*>(sts) + wave * (32 * kKS);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            // dims 32 dt + acc_row(4 v4 .. 4 v4 + 3) are consecutive
            bf16x4 t4;
#pragma unroll
            for (int j = 0; j < 4; ++j) t4[j] = (bf16)(o[dt][4 * v4 + j] * il);
            *reinterpret_cast<bf16x4*>(ot + col * kKS + 32 * dt + acc_row(4 * v4, hf)) = t4;
        }
    __syncthreads();
    const int nq = min(32, D.N - t0 - 32 * qh);
    for (int x = lane; x < 32 * 16; x += kWave) {
        const int row = x >> 4, piece = x & 15;
        if (row < nq)
            st_bf8(out + (((size_t)b * D.N + t0 + 32 * qh + row) * D.Hq + h) * kD + 8 * piece,
                   ld_bf8(ot + row * kKS + 8 * piece));
    }
}

// ---------------------------------------------------------------------------
// Backward pass on the matrix cores (routing held fixed)
// ---------------------------------------------------------------------------
// Compact K / V lists of a given selection: selw [B, Hkv, n_full, lam] holds
// each complete chunk's selected positions ascending and -1 padded.  Chunk c
// of (b, g) gets rows off[c] .. off[c] + n_c - 1 (n_c its valid entries,
// off the exclusive prefix), laid out like the forward's lists; block
// c = n_full writes the total and the open chunk's 64-row copy (rows past N
// repeat token N-1; zeros when the last chunk is complete).  The first
// chunk's blocks of sequence 0 also split the NP-Map projections.
__global__ __launch_bounds__(256) void bwd_lists_kernel(const int32_t* __restrict__ selw,
                                                        const bf16* __restrict__ k,
                                                        const bf16* __restrict__ v,
                                                        bf16* __restrict__ ksel, bf16* __restrict__ vsel,
                                                        int* __restrict__ list_off,
                                                        const float* __restrict__ wq,
                                                        const float* __restrict__ wk,
                                                        bf16* __restrict__ wsplit, Dims D) {
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const size_t bg = (size_t)b * D.Hkv + g;
    const int32_t* sw = selw + bg * D.n_full * D.lam;
    __shared__ int red[256];
    int cnt = 0;
    for (int i = tid; i < c * D.lam; i += 256) cnt += sw[i] >= 0;
    red[tid] = cnt;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    const int off = red[0];
    if (tid == 0) list_off[bg * (D.n_full + 1) + c] = off;
    const size_t ldkv = (size_t)D.Hkv * kD;
    const size_t list0 = ((size_t)b * sel_list_rows(D) * D.Hkv + g) * kD;
    if (c < D.n_full) {
        for (int x = tid; x < D.lam * 16; x += 256) {
            const int i = x >> 4, piece = x & 15;
            const int pos = sw[c * D.lam + i];  // valid entries come first
            if (pos >= 0) {
                const size_t src = (((size_t)b * D.N + pos) * D.Hkv + g) * kD + 8 * piece;
                const size_t dst = list0 + (size_t)(off + i) * ldkv + 8 * piece;
                st_bf8(ksel + dst, ld_bf8(k + src));
                st_bf8(vsel + dst, ld_bf8(v + src));
            }
        }
    } else {
        const bool open = D.T > D.n_full;
        const int t0 = D.n_full * kC;
        for (int x = tid; x < kC * 16; x += 256) {
            const int p = x >> 4, piece = x & 15;
            const size_t src = (((size_t)b * D.N + min(t0 + p, D.N - 1)) * D.Hkv + g) * kD + 8 * piece;
            const size_t dst = list0 + (size_t)(off + p) * ldkv + 8 * piece;
            st_bf8(ksel + dst, open ? ld_bf8(k + src) : zero_bf8());
            st_bf8(vsel + dst, open ? ld_bf8(v + src) : zero_bf8());
        }
    }
    if (c == 0 && b == 0) split_projections(wq, wk, wsplit, D.Hkv, g, 256);
}

// The same lists when chunks span CT = C / 64 > 1 tiles, indexed by tile so
// that the kernels after it work in 64-token tiles (D: chunk dimensions, DT:
// tile dimensions, DT.lam = min(lam, 64)).  Block tau takes tile tau: its
// selected tokens are a run of its chunk's entries of selw (ascending, valid
// entries first), which it writes to selw_t [B, Hkv, N / 64, DT.lam] (-1
// padded) and gathers to list rows off .. off + n - 1, off = loff[tau] = the
// valid entries at positions below 64 tau.  Block tau = N / 64 writes the
// total and the copy of an incomplete last tile (zeros when N is a multiple
// of 64).  Tile 0's blocks of sequence 0 also split the NP-Map projections.
__global__ __launch_bounds__(256) void bwd_lists_tiles_kernel(const int32_t* __restrict__ selw,
                                                              const bf16* __restrict__ k,
                                                              const bf16* __restrict__ v,
                                                              int32_t* __restrict__ selw_t,
                                                              bf16* __restrict__ ksel, bf16* __restrict__ vsel,
                                                              int* __restrict__ list_off,
                                                              const float* __restrict__ wq,
                                                              const float* __restrict__ wk,
                                                              bf16* __restrict__ wsplit, Dims D, Dims DT) {
    const int tau = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const size_t bg = (size_t)b * D.Hkv + g;
    const int ct = D.C / kC, cc = tau / ct, p0 = tau * kC;
    const int32_t* sw = selw + bg * D.n_full * D.lam;
    // valid entries of the earlier chunks, of chunk cc below p0, and of chunk
    // cc inside the tile
    __shared__ int red[3][256];
    int prev = 0, below = 0, in = 0;
    for (int i = tid; i < min(cc, D.n_full) * D.lam; i += 256) prev += sw[i] >= 0;
    if (cc < D.n_full)
        for (int i = tid; i < D.lam; i += 256) {
            const int p = sw[cc * D.lam + i];
            below += p >= 0 && p < p0;
            in += p >= p0 && p < p0 + kC;
        }
    red[0][tid] = prev;
    red[1][tid] = below;
    red[2][tid] = in;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) {
            red[0][tid] += red[0][tid + w];
            red[1][tid] += red[1][tid + w];
            red[2][tid] += red[2][tid + w];
        }
        __syncthreads();
    }
    below = red[1][0];
    in = red[2][0];
    const int off = red[0][0] + below;
    if (tid == 0) list_off[bg * (DT.n_full + 1) + tau] = off;
    const size_t ldkv = (size_t)D.Hkv * kD;
    const size_t list0 = ((size_t)b * sel_list_rows(DT) * D.Hkv + g) * kD;
    if (tau < DT.n_full) {
        int32_t* st = selw_t + (bg * DT.n_full + tau) * DT.lam;
        for (int i = tid; i < DT.lam; i += 256) st[i] = i < in ? sw[cc * D.lam + below + i] : -1;
        for (int x = tid; x < in * 16; x += 256) {
            const int i = x >> 4, piece = x & 15;
            const int pos = sw[cc * D.lam + below + i];
            const size_t src = (((size_t)b * D.N + pos) * D.Hkv + g) * kD + 8 * piece;
            const size_t dst = list0 + (size_t)(off + i) * ldkv + 8 * piece;
            st_bf8(ksel + dst, ld_bf8(k + src));
            st_bf8(vsel + dst, ld_bf8(v + src));
        }
    } else {
        const bool open = DT.T > DT.n_full;
        const int t0 = DT.n_full * kC;
        for (int x = tid; x < kC * 16; x += 256) {
            const int p = x >> 4, piece = x & 15;
            const size_t src = (((size_t)b * D.N + min(t0 + p, D.N - 1)) * D.Hkv + g) * kD + 8 * piece;
            const size_t dst = list0 + (size_t)(off + p) * ldkv + 8 * piece;
            st_bf8(ksel + dst, open ? ld_bf8(k + src) : zero_bf8());
            st_bf8(vsel + dst, open ? ld_bf8(v + src) : zero_bf8());
        }
    }
    if (tau == 0 && b == 0) split_projections(wq, wk, wsplit, D.Hkv, g, 256);
}

}  // namespace

bool mfma_fwd_supported(const Dims& D) {
    return D.bf16 && D.d == kD && D.fd == kD && (D.W == kC || D.W == 2 * kC || D.W == 4 * kC) &&
           (D.C == kC || D.C == 2 * kC || D.C == 4 * kC) && D.W >= D.C &&
           (D.G == 1 || D.G == 2 || D.G == 4 || D.G == 8);
}

hipError_t launch_win_select(const Dims& D, const void* q, const void* k, const void* v,
                             float* scores, int32_t* sel_idx, uint8_t* route, void* ksel,
                             void* vsel, const float* wphi_q, const float* wphi_k, void* wsplit,
                             int chunk, hipStream_t s) {
    dim3 grid(D.T, D.Hkv, D.B);
    const bf16* qq = reinterpret_cast<const bf16*>(q);
    const bf16* kk = reinterpret_cast<const bf16*>(k);
    const bf16* vv = reinterpret_cast<const bf16*>(v);
    bf16* ks = reinterpret_cast<bf16*>(ksel);
    bf16* vs = reinterpret_cast<bf16*>(vsel);
#define STILL_WS(NW, NWT)                                                                          \
    hipLaunchKernelGGL((win_select_kernel<NW, NWT>), grid, dim3(64 * NW), 0, s, qq, kk, vv, scores, \
                       sel_idx, route, ks, vs, wphi_q, wphi_k, reinterpret_cast<bf16*>(wsplit),     \
                       chunk, D)
    const int nwt = D.W / kC;
#define STILL_WS_NWT(NW)          \
    do {                          \
        if (nwt == 1)             \
            STILL_WS(NW, 1);      \
        else if (nwt == 2)        \
            STILL_WS(NW, 2);      \
        else                      \
            STILL_WS(NW, 4);      \
    } while (0)
    if (D.G >= 4) STILL_WS_NWT(4);
    else if (D.G == 2) STILL_WS_NWT(2);
    else STILL_WS_NWT(1);
#undef STILL_WS_NWT
#undef STILL_WS
    return hipGetLastError();
}

hipError_t launch_chunk_select(const Dims& D, const float* scores, const void* k, const void* v,
                               int32_t* sel_idx, uint8_t* route, void* ksel, void* vsel, int* loff,
                               int list_rows, hipStream_t s) {
    dim3 grid(D.T, D.Hkv, D.B);
    const bf16* kk = reinterpret_cast<const bf16*>(k);
    const bf16* vv = reinterpret_cast<const bf16*>(v);
    bf16* ks = reinterpret_cast<bf16*>(ksel);
    bf16* vs = reinterpret_cast<bf16*>(vsel);
    if (D.C == 2 * kC)
        hipLaunchKernelGGL(chunk_select_kernel<2>, grid, dim3(256), 0, s, scores, kk, vv, sel_idx, route, ks, vs,
                           loff, list_rows, D);
    else if (D.C == 4 * kC)
        hipLaunchKernelGGL(chunk_select_kernel<4>, grid, dim3(256), 0, s, scores, kk, vv, sel_idx, route, ks, vs,
                           loff, list_rows, D);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_la_state(const Dims& D, const void* k, const void* v, const void* wsplit,
                           const uint8_t* route, void* phik, const LinBufs& L, int cap_chunk,
                           hipStream_t s) {
    if (D.n_full == 0) return hipSuccess;
    const int n = D.Hkv * (kD / 2) * kD;
    const bf16* wkh = reinterpret_cast<const bf16*>(wsplit) + 2 * (size_t)n;
    const bf16* wkl = wkh + n;
    dim3 grid((D.n_full + D.ng - 1) / D.ng, D.Hkv, D.B);
    hipLaunchKernelGGL(la_state_kernel, grid, dim3(256), 0, s, reinterpret_cast<const bf16*>(k),
                       reinterpret_cast<const bf16*>(v), wkh, wkl, route, reinterpret_cast<bf16*>(phik),
                       L, cap_chunk, D);
    return hipGetLastError();
}

hipError_t launch_la_group_scan(const Dims& D, const LinBufs& L, int cap_chunk, float* cap_S,
                                float* cap_z, hipStream_t s) {
    constexpr int E1 = (kD + 1) * kD;
    const int ngroups = D.n_full == 0 ? 0 : (D.n_full + D.ng - 1) / D.ng;
    dim3 grid((E1 + 255) / 256, D.Hkv, D.B);
    hipLaunchKernelGGL(la_group_scan_kernel, grid, dim3(256), 0, s, L, ngroups, cap_chunk, cap_S, cap_z,
                       D);
    return hipGetLastError();
}

hipError_t launch_hybrid_main(const Dims& D, const void* q, const void* k, const void* v,
                              const void* wsplit, const void* phik, const uint8_t* route,
                              const void* ksel, const void* vsel, const LinBufs& L,
                              const float* gate, const int* list_off, void* out, float* stats,
                              hipStream_t s) {
    const int n = D.Hkv * (kD / 2) * kD;
    const bf16* wqh = reinterpret_cast<const bf16*>(wsplit);
    const bf16* wql = wqh + n;
    const int HB = D.G >= 4 ? 4 : D.G;  // query heads per block, two waves each
    const unsigned nblk = (unsigned)D.T * D.B * D.Hkv * (D.G / HB);
    const int nwt = D.W / kC;
#define STILL_MAIN1(H, NWT)                                                                      \
    hipLaunchKernelGGL((hybrid_main_kernel<H, NWT>), dim3(nblk), dim3(128 * H), 0, s,           \
                       reinterpret_cast<const bf16*>(q), reinterpret_cast<const bf16*>(k),      \
                       reinterpret_cast<const bf16*>(v), wqh, wql,                                \
                       reinterpret_cast<const bf16*>(phik), route,                              \
                       reinterpret_cast<const bf16*>(ksel), reinterpret_cast<const bf16*>(vsel), \
                       L, gate, reinterpret_cast<bf16*>(out), list_off, nullptr, stats, nullptr, D)
#define STILL_MAIN(H)              \
    do {                           \
        if (nwt == 1)              \
            STILL_MAIN1(H, 1);     \
        else if (nwt == 2)         \
            STILL_MAIN1(H, 2);     \
        else                       \
            STILL_MAIN1(H, 4);     \
    } while (0)
    if (HB == 4) STILL_MAIN(4);
    else if (HB == 2) STILL_MAIN(2);
    else STILL_MAIN(1);
#undef STILL_MAIN
#undef STILL_MAIN1
    return hipGetLastError();
}

bool mfma_bwd_supported(const Dims& D) { return mfma_fwd_supported(D); }

hipError_t launch_bwd_lists(const Dims& D, const int32_t* selw, const void* k, const void* v,
                            void* ksel, void* vsel, int* list_off, const float* wq, const float* wk,
                            void* wsplit, hipStream_t s) {
    dim3 grid(D.n_full + 1, D.Hkv, D.B);
    hipLaunchKernelGGL(bwd_lists_kernel, grid, dim3(256), 0, s, selw, reinterpret_cast<const bf16*>(k),
                       reinterpret_cast<const bf16*>(v), reinterpret_cast<bf16*>(ksel),
                       reinterpret_cast<bf16*>(vsel), list_off, wq, wk, reinterpret_cast<bf16*>(wsplit), D);
    return hipGetLastError();
}

hipError_t launch_bwd_lists_tiles(const Dims& D, const Dims& DT, const int32_t* selw, const void* k,
                                  const void* v, int32_t* selw_t, void* ksel, void* vsel, int* list_off,
                                  const float* wq, const float* wk, void* wsplit, hipStream_t s) {
    dim3 grid(DT.n_full + 1, D.Hkv, D.B);
    hipLaunchKernelGGL(bwd_lists_tiles_kernel, grid, dim3(256), 0, s, selw, reinterpret_cast<const bf16*>(k),
                       reinterpret_cast<const bf16*>(v), selw_t, reinterpret_cast<bf16*>(ksel),
                       reinterpret_cast<bf16*>(vsel), list_off, wq, wk, reinterpret_cast<bf16*>(wsplit), D, DT);
    return hipGetLastError();
}

hipError_t launch_hybrid_stats(const Dims& D, const void* q, const void* k, const void* v,
                               const void* wsplit, const void* phik, const uint8_t* route,
                               const void* ksel, const void* vsel, const LinBufs& L,
                               const float* gate, const int* list_off, const void* dout,
                               float* stat, void* phiq, hipStream_t s) {
    const int n = D.Hkv * (kD / 2) * kD;
    const bf16* wqh = reinterpret_cast<const bf16*>(wsplit);
    const bf16* wql = wqh + n;
    const int HB = D.G >= 4 ? 4 : D.G;
    const unsigned nblk = (unsigned)D.T * D.B * D.Hkv * (D.G / HB);
    const int nwt = D.W / kC;
#define STILL_STATS1(H, NWT)                                                                     \
    hipLaunchKernelGGL((hybrid_main_kernel<H, NWT, true>), dim3(nblk), dim3(128 * H), 0, s,     \
                       reinterpret_cast<const bf16*>(q), reinterpret_cast<const bf16*>(k),      \
                       reinterpret_cast<const bf16*>(v), wqh, wql,                                \
                       reinterpret_cast<const bf16*>(phik), route,                              \
                       reinterpret_cast<const bf16*>(ksel), reinterpret_cast<const bf16*>(vsel), \
                       L, gate, nullptr, list_off, reinterpret_cast<const bf16*>(dout), stat,       \
                       reinterpret_cast<bf16*>(phiq), D)
#define STILL_STATS(H)             \
    do {                           \
        if (nwt == 1)              \
            STILL_STATS1(H, 1);    \
        else if (nwt == 2)         \
            STILL_STATS1(H, 2);    \
        else                       \
            STILL_STATS1(H, 4);    \
    } while (0)
    if (HB == 4) STILL_STATS(4);
    else if (HB == 2) STILL_STATS(2);
    else STILL_STATS(1);
#undef STILL_STATS
#undef STILL_STATS1
    return hipGetLastError();
}


}  // namespace still
