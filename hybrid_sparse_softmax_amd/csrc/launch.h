// Internal launch interface between the C-ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace still {

// Validated problem dimensions.
struct Dims {
    int B, N, Hq, Hkv, G, d, fd;  // fd = NP-Map feature size d'
    int W, C, lam;                // lam = min(topk, C)
    int T;                        // ceil(N / C)
    int n_full;                   // N / C complete chunks
    int ng;                       // chunks per run of the MFMA path's linear-state kernel
    int route;                    // routing criterion (kRoute*)
    float eps, tau;
    bool bf16;
};

// Rows per (sequence) of the MFMA path's compact selected K / V lists, laid
// out [B, rows, Hkv, d] like k and v: every complete chunk's lam selected
// rows in order, then 64 rows holding the last chunk's tokens when it is
// incomplete (later rows repeat the last token) and zeros otherwise, so any
// 64-row window a key tile stages lies inside the list.
__host__ __device__ inline int sel_list_rows(const Dims& D) { return D.n_full * D.lam + 64; }

// Cache pointers as the kernels see them.
struct CacheView {
    void *win_k, *win_v;
    uint8_t* win_route;
    float* pend;
    void *sel_k, *sel_v;
    int32_t* sel_count;
    int32_t cap;
    float *lin_S, *lin_z;
    int64_t pos;
    int64_t* pos_dev;  // [B] per-sequence positions (ragged decode step) or nullptr
};

// ---- general kernels (any supported shape, f32 or bf16 storage) ----------
// phi[tok, h, :] = NP-Map of x[tok, h, :] with projection P[h / heads_per_proj]
// gate: logits [B, N, H] whose sigmoid scales each phi row (queries with a
// gate), or nullptr
hipError_t launch_phi(const Dims& D, const void* x, int H, int heads_per_proj, const float* P,
                      const float* gate, float* phi, hipStream_t s);
// per-query-head Self-Saliency hs[b, h, t]
hipError_t launch_head_scores(const Dims& D, const void* q, const void* k, float* hs, hipStream_t s);
// group mean, per-chunk top-k, route flags, selected positions
hipError_t launch_select(const Dims& D, const float* hs, float* scores, int32_t* sel_idx,
                         uint8_t* route, const void* k, hipStream_t s);
// per-chunk linear-attention sums (S then z, fd*(d+1) floats per chunk), then
// in-place inclusive prefix over chunks; optional fp32 copy of chunk `cap_chunk`
hipError_t launch_la_chunks(const Dims& D, const float* phik, const void* v, const uint8_t* route,
                            float* lin, hipStream_t s);
hipError_t launch_la_scan(const Dims& D, float* lin, int cap_chunk, float* cap_S, float* cap_z,
                          hipStream_t s);
// hybrid output, one wave per (b, t, h); stats (optional) [B, N, Hq, 4] gets
// each query's (m, l, 0, c) for a backward
hipError_t launch_main_general(const Dims& D, const void* q, const void* k, const void* v,
                               const float* phiq, const float* phik, const uint8_t* route,
                               const int32_t* sel_idx, const float* lin, void* out, float* stats,
                               hipStream_t s);
// prefill -> decode cache hand-off (after the scan wrote chunk cap_chunk into lin_S / lin_z)
hipError_t launch_handoff(const Dims& D, const void* k, const void* v, const float* wphi_k,
                          const float* scores, const int32_t* sel_idx, const uint8_t* route,
                          int cap_chunk, const CacheView& c, hipStream_t s);

// ---- gfx950 MFMA forward (bf16, d = d' = 128, W in {64, 128, 256}, C in
// {64, 128, 256} with C <= W, any topk) ----
// The kernels below the selection work in 64-token tiles: for C > 64 they take
// the tile dimensions (C = 64, T and n_full counted in tiles, lam per chunk of
// the true C) and a per-tile list offset table.
bool mfma_fwd_supported(const Dims& D);
// scores, top-k, route flags, compact selected K/V lists [B, sel_list_rows,
// Hkv, d], and the NP-Map projections as bf16 high/low parts:
// wsplit = [wq hi, wq lo, wk hi, wk lo], each Hkv * (d'/2) * d elements.
// chunk: the true chunk length; above 64 only the scores and wsplit (D in tiles)
hipError_t launch_win_select(const Dims& D, const void* q, const void* k, const void* v,
                             float* scores, int32_t* sel_idx, uint8_t* route, void* ksel,
                             void* vsel, const float* wphi_q, const float* wphi_k, void* wsplit,
                             int chunk, hipStream_t s);
// chunks of C = 128 or 256 (D in chunks): top-lam per chunk from the scores,
// sel_idx, route flags, compact lists (list_rows rows per sequence) and the
// per-tile offsets loff [B, Hkv, N / 64 + 1] (rows at positions below 64 tau)
hipError_t launch_chunk_select(const Dims& D, const float* scores, const void* k, const void* v,
                               int32_t* sel_idx, uint8_t* route, void* ksel, void* vsel, int* loff,
                               int list_rows, hipStream_t s);
// Linear-attention prefixes of the MFMA path.  A state is S^T [d][d'] plus
// z [d'] (features in kperm order), E1 = (d + 1) d' entries in fp32 form.
// ngroups = ceil(n_full / ng) runs of ng chunks.
struct LinBufs {
    void* sh;     // [B, Hkv, n_full, d, d'] bf16: within-run prefix of each chunk, S^T rows
    float* lz;    // [B, Hkv, n_full, d']    its z
    float* ltot;  // [B, Hkv, ngroups, E1]   fp32 within-run prefix at each run's last chunk
    float* lcap;  // [B, Hkv, E1]            fp32 within-run prefix at the hand-off chunk
    void* gh;     // [B, Hkv, ngroups, d, d'] bf16: exclusive prefix over the earlier runs, S^T rows
    float* gz;    // [B, Hkv, ngroups, d']    its z
};
// phi_k rows [B, Hkv, N, d'] (bf16, features in kperm order) and the
// within-run prefixes (L.sh, L.lz, L.ltot; L.lcap when cap_chunk >= 0)
hipError_t launch_la_state(const Dims& D, const void* k, const void* v, const void* wsplit,
                           const uint8_t* route, void* phik, const LinBufs& L, int cap_chunk,
                           hipStream_t s);
// exclusive prefix over runs (L.gh, L.gz) and the decode hand-off state
hipError_t launch_la_group_scan(const Dims& D, const LinBufs& L, int cap_chunk, float* cap_S,
                                float* cap_z, hipStream_t s);
hipError_t launch_hybrid_main(const Dims& D, const void* q, const void* k, const void* v,
                              const void* wsplit, const void* phik, const uint8_t* route,
                              const void* ksel, const void* vsel, const LinBufs& L,
                              const float* gate, const int* list_off, void* out, float* stats,
                              hipStream_t s);

// ---- backward on the matrix cores (bf16, d = 128, W = 64 / 128 / 256, C = 64 / 128 / 256, C <= W) ----
bool mfma_bwd_supported(const Dims& D);
// compact K / V lists of the selection selw (ascending, -1 padded per chunk):
// chunk c's rows start at list_off[(b Hkv + g) (n_full + 1) + c]; also the
// NP-Map projection split (wsplit, as for the forward)
hipError_t launch_bwd_lists(const Dims& D, const int32_t* selw, const void* k, const void* v,
                            void* ksel, void* vsel, int* list_off, const float* wq, const float* wk,
                            void* wsplit, hipStream_t s);
// the same for chunks of C > 64 (D in chunks, DT in tiles): lists, per-tile
// offsets list_off [B, Hkv, N / 64 + 1] and the selection by tile selw_t
// [B, Hkv, N / 64, DT.lam] (-1 padded), so the later kernels run on DT
hipError_t launch_bwd_lists_tiles(const Dims& D, const Dims& DT, const int32_t* selw, const void* k,
                                  const void* v, int32_t* selw_t, void* ksel, void* vsel, int* list_off,
                                  const float* wq, const float* wk, void* wsplit, hipStream_t s);
// the forward's main kernel writing (m, l, D = dout . out, c) per query head
// to stat [B, N, Hq, 4] instead of the output, and the gated NP-Map features
// of the queries to phiq [B, N, Hq, d'] (bf16, feature order)
hipError_t launch_hybrid_stats(const Dims& D, const void* q, const void* k, const void* v,
                               const void* wsplit, const void* phik, const uint8_t* route,
                               const void* ksel, const void* vsel, const LinBufs& L,
                               const float* gate, const int* list_off, const void* dout,
                               float* stat, void* phiq, hipStream_t s);
// softmax part of dk and dv: phase 0 the window keys (dk and dv added
// to), phase 1 the selected keys over the compact rows (both added to; part:
// bwd_kv_part_floats(D) floats of segment sums, then merged)
size_t bwd_kv_part_floats(const Dims& D);
hipError_t launch_bwd_kv(const Dims& D, const void* q, const void* k, const void* v, const void* dout,
                         const uint8_t* route, const void* ksel, const void* vsel,
                         const int32_t* selw, const int* list_off, const float* stat, float* dk,
                         float* dv, float* part, int phase, hipStream_t s);
// linear terms of the keys on the matrix cores: phase 0 the chunk sums
// ust [B, Hkv, T, d' (d + 1)] (fp32, [i][e] then u; the suffix kernel turns
// them into suffix sums, U in bf16 in ust16), phase 1 dv (written: the linear part) and, through
// the keys' NP-Map backward (projections from wsplit), dk (written: the
// NP-Map part; the softmax kernels add theirs) and du16 (bf16 [Hkv, B N,
// d'/2]) for the projection gradient
hipError_t launch_bwd_key_lin(const Dims& D, const void* v, const void* dout, const void* phiq,
                              const void* phik16, const uint8_t* route, const float* stat, float* ust,
                              const void* ust16, float* dv, const void* k, const void* wsplit, float* dk,
                              void* du16, int phase, hipStream_t s);
// partial projection gradients of one side over nslice row slices:
// part [nslice, Hkv, d/2, d] (summed by the reduce kernel)
hipError_t launch_dw_mfma(const Dims& D, const void* x, int side, const void* du16, float* part,
                          int nslice, hipStream_t s);
// dq (fp32, overwritten): the softmax part, then the linear terms' gradient
// w.r.t. the queries' NP-Map features carried through the NP-Map backward
// (P^T du and the norm term), with du (bf16 [Hkv, B N G, d'/2], rows token G
// + head offset) for the projection gradient, and with a gate dgate.
// stat_in (with the forward's out):
// the forward's (m, l, -, c); the kernel then writes stat (with D = dout .
// out) and phiq (gated features, from the projection split wsplit) itself
// instead of reading what the first pass wrote there
hipError_t launch_bwd_dq(const Dims& D, const void* q, const void* k, const void* v, const void* dout,
                         const uint8_t* route, const void* ksel, const void* vsel,
                         const int* list_off, float* stat, const void* phik16, const LinBufs& L,
                         const float* gate, void* phiq, float* dq, void* du, float* dgate,
                         const float* stat_in, const void* out, const void* wsplit, hipStream_t s);

// ---- decode step ------------------------------------------------------------
struct DecodeWork {
    float* la;      // [B, Hq, d + 1]   linear numerator, denominator
    float* win;     // [B, Hq, d + 2]   window partial (m, l, acc)
    float* part;    // [B, Hq, splits, d + 2] selected-list partials
    int splits;
    int rows_per_split;
};
hipError_t launch_decode_prep(const Dims& D, const void* q, const void* k, const void* v,
                              const float* wphi_q, const float* wphi_k, const float* gate,
                              const CacheView& c, const DecodeWork& w, hipStream_t s);
hipError_t launch_decode_sel(const Dims& D, const void* q, const CacheView& c, const DecodeWork& w,
                             hipStream_t s);
// advances pos_dev[b] by one when pos_dev is not null (ragged decode step)
hipError_t launch_decode_combine(const Dims& D, const DecodeWork& w, void* out, int64_t* pos_dev,
                                 hipStream_t s);

// ---- fast decode step (bf16, d = d' = 128, window 1..256, G in {1,2,4,8}) -------
bool fast_decode_supported(const Dims& D);
int fast_decode_splits(int cap);                     // stream splits of 1024 selected rows
size_t fast_decode_floats(const Dims& D, int nsplit);  // workspace, in floats
hipError_t launch_fast_decode(const Dims& D, const void* q, const void* k, const void* v,
                              const float* wq, const float* wk, const float* gate,
                              const CacheView& c, float* ws, int nsplit, void* out, int phase,
                              hipStream_t s);  // phase 0, then 1

// ---- backward (general kernels; routing held fixed) ----------------------
struct BwdArgs {
    const void *q, *k, *v, *dout;       // dtype, layouts of the forward
    const float *wq, *wk;               // [Hkv, fd/2, d]
    const int32_t* sel_idx;             // [B, Hkv, n_full, lam] the forward's selection
    float *dq, *dk, *dv, *dwq, *dwk;    // fp32 gradients, overwritten
    const float* gate;                  // [B, N, Hq] gate logits, or nullptr
    float* dgate;                       // [B, N, Hq] fp32, written when gate and dgate are set
    // the forward's output and statistics (m, l, 0, c) per query head, or
    // both nullptr: with them the matrix-core path skips its first pass
    const void* out;
    const float* stats;
};
struct BwdWork {
    float *phiq, *phik;   // [B, N, Hq | Hkv, fd] (fp32; the matrix-core path keeps phiq in bf16)
    float* lin;           // [B, Hkv, T, fd (d + 1)] LA prefix states
    float* stat;          // [B, N, Hq, 4] m, l, D_t, exp(-m) / l
    float *dphiq, *dphik; // [B, N, Hq | Hkv, fd]
    float* ust;           // [B, Hkv, T, fd (d + 1)] suffix sums of c phi_q dout^T, c D phi_q
    void* ust16;          // matrix-core path: the U part of the suffix sums in bf16 [B, Hkv, T, fd d]
    float *duq, *duk;     // [B, N, Hq | Hkv, fd / 2]
    float* dwpart;        // [nslice, Hkv, fd / 2, d]
    uint8_t* route;       // [B, Hkv, N]
    int32_t* selw;        // [B, Hkv, n_full, lam] ascending, -1 padded
    int nslice;
    // matrix-core path (mfma): the softmax part of dq and the statistics on
    // the matrix cores, over compact lists of the given selection
    bool mfma;
    void *ksel, *vsel;    // [B, sel_list_rows, Hkv, d] bf16
    int* list_off;        // [B, Hkv, n_full + 1]
    void* phik16;         // [B, Hkv, N, d'] bf16 (kperm features)
    void* wsplit;         // NP-Map projections as bf16 high / low parts
    LinBufs lin16;        // linear prefixes of the matrix-core path
    bool lin_given;       // phik16 and lin16 are the forward's (not recomputed)
    float* kvpart;        // segment sums of the selected keys' dk, dv
    // the matrix-core kernels after the lists work in 64-token tiles: tile
    // holds those dimensions (C = 64, lam = min(lam, 64), T and n_full in
    // tiles; the chunk dimensions themselves when C = 64) and selw_t the
    // selection by tile (selw itself when C = 64); list_off, ust and the
    // buffers above count tiles
    Dims tile;
    int32_t* selw_t;
};
// called before each launch with the kernel's name (per-launch events)
struct BwdMark {
    hipError_t (*fn)(void* ctx, const char* name);
    void* ctx;
};
int bwd_launch_count(bool mfma);  // at most this many launches
hipError_t launch_bwd(const Dims& D, const BwdArgs& a, const BwdWork& w, hipStream_t s, BwdMark mark);
hipError_t launch_zero(float* p, int n, hipStream_t s);

// ---- future-KV-utility diagnostic (general kernels) ----------------------
// stat [B, N, Hq, 2] fp32 scratch; util [B, Hkv, N] fp32, written
hipError_t launch_future_utility(const Dims& D, const void* q, const void* k, float* stat,
                                 float* util, hipStream_t s);

}  // namespace still
