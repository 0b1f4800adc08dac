// C-ABI layer of libstill: host-side validation, workspace carving and the
// launch sequence of each entry point.  Declarations and contracts are in
// include/still.h.
#include "still.h"

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "launch.h"

namespace still {

// ---------------------------------------------------------------------------
// validation
// ---------------------------------------------------------------------------
static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

static int check_shape(const still_shape* sh, bool decode) {
    if (!sh) return STILL_ERR_INVALID_ARG;
    if (sh->batch < 0 || sh->seqlen < 0) return STILL_ERR_INVALID_ARG;
    if (sh->n_q_heads < 1 || sh->n_kv_heads < 1) return STILL_ERR_INVALID_ARG;
    if (sh->n_q_heads % sh->n_kv_heads) return STILL_ERR_INVALID_ARG;
    if (sh->window < 0 || sh->chunk < 1 || sh->topk < 0) return STILL_ERR_INVALID_ARG;
    if (sh->window == 0 && sh->topk > 0) return STILL_ERR_INVALID_ARG;
    if (sh->topk > 0 && sh->window < sh->chunk) return STILL_ERR_INVALID_ARG;
    if (!(sh->eps > 0.f) || !std::isfinite(sh->eps)) return STILL_ERR_INVALID_ARG;
    if (!(sh->softmax_scale >= 0.f) || !std::isfinite(sh->softmax_scale)) return STILL_ERR_INVALID_ARG;
    if (sh->dtype != STILL_F32 && sh->dtype != STILL_BF16) return STILL_ERR_INVALID_ARG;
    if (sh->head_dim < 1 || sh->feat_dim < 2 || (sh->feat_dim & 1)) return STILL_ERR_INVALID_ARG;
    if (sh->flags & ~(STILL_FLAG_GENERAL_KERNELS | STILL_ROUTE_MASK)) return STILL_ERR_INVALID_ARG;
    if (((sh->flags & STILL_ROUTE_MASK) >> STILL_ROUTE_SHIFT) > STILL_ROUTE_RANDOM) return STILL_ERR_INVALID_ARG;
    // built variants
    if (sh->head_dim != 64 && sh->head_dim != 128) return STILL_ERR_UNSUPPORTED;
    if (sh->feat_dim != sh->head_dim) return STILL_ERR_UNSUPPORTED;
    if (sh->n_q_heads / sh->n_kv_heads > 8) return STILL_ERR_UNSUPPORTED;
    if (sh->window > 1024 || sh->chunk > 1024) return STILL_ERR_UNSUPPORTED;
    (void)decode;
    return STILL_OK;
}

// runs of consecutive chunks for the MFMA path's linear-state kernel: about
// one block per compute unit, at most 16 chunks per run
static int runs_of(const Dims& D) {
    const int64_t chunks = (int64_t)D.B * D.Hkv * D.n_full;
    const int64_t ng = chunks / 256;
    return ng < 1 ? 1 : (ng > 16 ? 16 : (int)ng);
}

// The MFMA kernels after the selection work in 64-token tiles: the same
// dimensions counted in tiles (lam stays per chunk of the true C).
static Dims tile_dims(const Dims& D) {
    Dims T = D;
    T.C = 64;
    T.T = (D.N + 63) / 64;
    T.n_full = D.N / 64;
    T.ng = runs_of(T);
    return T;
}

static Dims make_dims(const still_shape* sh, int seqlen) {
    Dims D;
    D.B = sh->batch;
    D.N = seqlen;
    D.Hq = sh->n_q_heads;
    D.Hkv = sh->n_kv_heads;
    D.G = D.Hq / D.Hkv;
    D.d = sh->head_dim;
    D.fd = sh->feat_dim;
    D.W = sh->window;
    D.C = sh->chunk;
    D.lam = sh->topk < sh->chunk ? sh->topk : sh->chunk;
    D.T = (seqlen + D.C - 1) / D.C;
    D.n_full = seqlen / D.C;
    D.ng = runs_of(D);
    D.route = (int)((sh->flags & STILL_ROUTE_MASK) >> STILL_ROUTE_SHIFT);
    D.eps = sh->eps;
    D.tau = sh->softmax_scale > 0.f ? sh->softmax_scale : 1.0f / std::sqrt((float)D.d);
    D.bf16 = sh->dtype == STILL_BF16;
    return D;
}

static size_t elem_size(const Dims& D) { return D.bf16 ? 2 : 4; }

// Bump allocator over the caller's workspace; 256-byte aligned pieces.
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* p) : base(static_cast<char*>(p)) {}
    template <typename X> X* take(size_t count) {
        off = (off + 255) & ~size_t(255);
        X* p = base ? reinterpret_cast<X*>(base + off) : nullptr;
        off += count * sizeof(X);
        return p;
    }
};

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
struct FwdBuffers {
    float *phiq, *phik, *hs, *scores, *lin;
    int32_t* sel;
    uint8_t* route;
};

static FwdBuffers carve_fwd(const Dims& D, Carver& cv) {
    FwdBuffers f;
    const size_t BN = (size_t)D.B * D.N;
    f.phiq = cv.take<float>(BN * D.Hq * D.fd);
    f.phik = cv.take<float>(BN * D.Hkv * D.fd);
    f.hs = cv.take<float>((size_t)D.B * D.Hq * D.N);
    f.scores = cv.take<float>((size_t)D.B * D.Hkv * D.N);
    f.sel = cv.take<int32_t>((size_t)D.B * D.Hkv * D.n_full * D.lam);
    f.route = cv.take<uint8_t>((size_t)D.B * D.Hkv * D.N);
    f.lin = cv.take<float>((size_t)D.B * D.Hkv * D.T * D.fd * (D.d + 1));
    return f;
}

struct MfmaBuffers {
    float* scores;
    int32_t* sel;
    uint8_t* route;
    void *ksel, *vsel, *phik, *wsplit;
    int* loff;  // per-tile list offsets (chunks of more than 64 tokens)
    LinBufs lin;
};

// D: the true dimensions; the lists and linear states are sized in tiles
static MfmaBuffers carve_mfma(const Dims& Dc, Carver& cv) {
    MfmaBuffers f;
    const Dims D = tile_dims(Dc);
    const size_t BG = (size_t)D.B * D.Hkv;
    const size_t nsel = BG * Dc.n_full * Dc.lam;
    f.scores = cv.take<float>(BG * D.N);
    f.sel = cv.take<int32_t>(nsel);
    f.route = cv.take<uint8_t>(BG * D.N);
    f.loff = cv.take<int>(BG * (size_t)(D.n_full + 1));
    const size_t nlist = BG * (size_t)sel_list_rows(D);
    f.ksel = cv.take<uint16_t>(nlist * D.d);
    f.vsel = cv.take<uint16_t>(nlist * D.d);
    f.phik = cv.take<uint16_t>(BG * D.N * D.fd);
    const size_t ngroups = D.n_full == 0 ? 0 : (size_t)(D.n_full + D.ng - 1) / D.ng;
    const size_t E1 = (size_t)(D.d + 1) * D.fd;
    f.lin.sh = cv.take<uint16_t>(BG * D.n_full * (size_t)D.d * D.fd);
    f.lin.lz = cv.take<float>(BG * D.n_full * (size_t)D.fd);
    f.lin.ltot = cv.take<float>(BG * ngroups * E1);
    f.lin.lcap = cv.take<float>(BG * E1);
    f.lin.gh = cv.take<uint16_t>(BG * ngroups * (size_t)D.d * D.fd);
    f.lin.gz = cv.take<float>(BG * ngroups * (size_t)D.fd);
    f.wsplit = cv.take<uint16_t>((size_t)4 * D.Hkv * (D.fd / 2) * D.d);
    return f;
}

static bool use_mfma(const Dims& D, const still_shape* sh) {
    return !(sh->flags & STILL_FLAG_GENERAL_KERNELS) && mfma_fwd_supported(D);
}

static size_t fwd_bytes(const Dims& D, const still_shape* sh) {
    Carver cv(nullptr);
    if (use_mfma(D, sh)) carve_mfma(D, cv);
    else carve_fwd(D, cv);
    return cv.off + 256;
}

// pos >= 0: cache->pos must equal it; pos == -1: any cache->pos >= 0;
// pos == -2: cache->pos is not used (ragged decode step)
static int check_cache(const Dims& D, const still_cache* c, int64_t pos, int64_t need_sel) {
    if (!c) return STILL_ERR_INVALID_ARG;
    if (c->pos != pos && pos >= 0) return STILL_ERR_INVALID_ARG;
    if (c->pos < 0 && pos != -2) return STILL_ERR_INVALID_ARG;
    if (!c->lin_S || !c->lin_z) return STILL_ERR_INVALID_ARG;
    if (D.W > 0 && (!c->win_k || !c->win_v || !c->win_route || !c->pend_score))
        return STILL_ERR_INVALID_ARG;
    if (D.W > 0 && (!aligned16(c->win_k) || !aligned16(c->win_v))) return STILL_ERR_INVALID_ARG;
    if (D.lam > 0) {
        if (!c->sel_k || !c->sel_v || !c->sel_count || c->sel_cap < 0) return STILL_ERR_INVALID_ARG;
        if (!aligned16(c->sel_k) || !aligned16(c->sel_v)) return STILL_ERR_INVALID_ARG;
        if (need_sel > c->sel_cap) return STILL_ERR_CAPACITY;
    }
    return STILL_OK;
}

static CacheView view_of(const still_cache* c) {
    CacheView v;
    v.win_k = c->win_k;
    v.win_v = c->win_v;
    v.win_route = c->win_route;
    v.pend = c->pend_score;
    v.sel_k = c->sel_k;
    v.sel_v = c->sel_v;
    v.sel_count = c->sel_count;
    v.cap = c->sel_cap;
    v.lin_S = c->lin_S;
    v.lin_z = c->lin_z;
    v.pos = c->pos;
    v.pos_dev = nullptr;
    return v;
}

static int64_t ceil_div(int64_t a, int64_t b) { return a <= 0 ? 0 : (a + b - 1) / b; }

#define STILL_TRY(expr)                                \
    do {                                               \
        if ((expr) != hipSuccess) return STILL_ERR_HIP; \
    } while (0)

// Optional per-launch events (the *_timed entry points).
struct Timeline {
    hipEvent_t* ev = nullptr;
    int max_ev = 0;
    int n = 0;
    const char** names = nullptr;
    hipError_t mark(hipStream_t s, const char* name) {
        if (ev) {
            if (names) names[n] = name;
            hipError_t e = hipEventRecord(ev[n], s);
            ++n;
            return e;
        }
        ++n;
        return hipSuccess;
    }
    hipError_t end(hipStream_t s) { return ev ? hipEventRecord(ev[n], s) : hipSuccess; }
};
#define STILL_LAUNCH(tl, s, name, expr)       \
    do {                                      \
        STILL_TRY((tl).mark((s), (name)));    \
        STILL_TRY(expr);                      \
    } while (0)

static int fwd_launches(const Dims& D, const still_shape* sh, bool with_cache) {
    if (use_mfma(D, sh)) return 4 + (D.C > 64 ? 1 : 0) + (with_cache ? 1 : 0);
    return 6 + (D.W > 0 ? 1 : 0) + (with_cache ? 1 : 0);
}

static int fwd(const still_shape* sh, const void* q, const void* k, const void* v,
               const float* wq, const float* wk, const float* gate, void* out, float* scores_opt,
               int32_t* sel_idx_opt, float* stats_opt, still_cache* cache, void* ws, size_t ws_bytes,
               hipStream_t s, Timeline& tl) {
    int st = check_shape(sh, false);
    if (st) return st;
    const Dims D = make_dims(sh, sh->seqlen);
    if (D.B == 0 || D.N == 0) return STILL_OK;  // nothing to compute; pointers unused
    if (!q || !k || !v || !wq || !wk || !out) return STILL_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(wq) ||
        !aligned16(wk) || !aligned4(gate) || !aligned16(stats_opt))
        return STILL_ERR_INVALID_ARG;
    if (cache) {
        const int64_t need = D.lam * ceil_div((int64_t)D.N - D.W, D.C);
        st = check_cache(D, cache, D.N, need);
        if (st) return st;
    }
    const size_t need_ws = fwd_bytes(D, sh);
    if (!ws || ws_bytes < need_ws) return STILL_ERR_WORKSPACE;
    if (tl.ev && tl.max_ev < fwd_launches(D, sh, cache != nullptr) + 1) return STILL_ERR_INVALID_ARG;

    void* wsa = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
    Carver cv(wsa);
    // the hand-off's linear state covers tokens j <= N-1-W: chunks below
    // floor((N-W)/C) in full, captured by the scan
    const int cap_chunk = cache ? (D.N > D.W ? D.N - D.W : 0) / D.C - 1 : -1;
    if (use_mfma(D, sh)) {
        MfmaBuffers f = carve_mfma(D, cv);
        float* scores = scores_opt ? scores_opt : f.scores;
        int32_t* sel = sel_idx_opt ? sel_idx_opt : f.sel;
        // chunks of C > 64: scores per 64-token tile, selection per chunk,
        // everything after it in tiles (cap_tile: the last tile of chunk cap_chunk)
        const bool wide = D.C > 64;
        const Dims DT = tile_dims(D);
        const int ct = D.C / 64;
        const int cap_tile = cap_chunk < 0 ? -1 : (cap_chunk + 1) * ct - 1;
        STILL_LAUNCH(tl, s, "win_select",
                     launch_win_select(DT, q, k, v, scores, sel, f.route, f.ksel, f.vsel, wq, wk, f.wsplit,
                                       D.C, s));
        if (wide)
            STILL_LAUNCH(tl, s, "chunk_select",
                         launch_chunk_select(D, scores, k, v, sel, f.route, f.ksel, f.vsel, f.loff,
                                             sel_list_rows(DT), s));
        STILL_LAUNCH(tl, s, "la_state",
                     launch_la_state(DT, k, v, f.wsplit, f.route, f.phik, f.lin, cap_tile, s));
        STILL_LAUNCH(tl, s, "la_scan",
                     launch_la_group_scan(DT, f.lin, cap_tile, cache ? cache->lin_S : nullptr,
                                          cache ? cache->lin_z : nullptr, s));
        STILL_LAUNCH(tl, s, "hybrid_main",
                     launch_hybrid_main(DT, q, k, v, f.wsplit, f.phik, f.route, f.ksel, f.vsel, f.lin, gate,
                                        wide ? f.loff : nullptr, out, stats_opt, s));
        if (cache)
            STILL_LAUNCH(tl, s, "handoff",
                         launch_handoff(D, k, v, wk, scores, sel, f.route, cap_chunk, view_of(cache), s));
        STILL_TRY(tl.end(s));
        return STILL_OK;
    }
    FwdBuffers f = carve_fwd(D, cv);
    float* scores = scores_opt ? scores_opt : f.scores;
    int32_t* sel = sel_idx_opt ? sel_idx_opt : f.sel;

    STILL_LAUNCH(tl, s, "phi_q", launch_phi(D, q, D.Hq, D.G, wq, gate, f.phiq, s));
    STILL_LAUNCH(tl, s, "phi_k", launch_phi(D, k, D.Hkv, 1, wk, nullptr, f.phik, s));
    if (D.W > 0) STILL_LAUNCH(tl, s, "head_scores", launch_head_scores(D, q, k, f.hs, s));
    STILL_LAUNCH(tl, s, "select", launch_select(D, f.hs, scores, sel, f.route, k, s));
    STILL_LAUNCH(tl, s, "la_chunk", launch_la_chunks(D, f.phik, v, f.route, f.lin, s));
    STILL_LAUNCH(tl, s, "la_scan", launch_la_scan(D, f.lin, cap_chunk, cache ? cache->lin_S : nullptr,
                                                  cache ? cache->lin_z : nullptr, s));
    STILL_LAUNCH(tl, s, "main_general",
                 launch_main_general(D, q, k, v, f.phiq, f.phik, f.route, sel, f.lin, out, stats_opt, s));
    if (cache)
        STILL_LAUNCH(tl, s, "handoff",
                     launch_handoff(D, k, v, wk, scores, sel, f.route, cap_chunk, view_of(cache), s));
    STILL_TRY(tl.end(s));
    return STILL_OK;
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------
static constexpr int kRowsPerSplit = 256;

static DecodeWork carve_decode(const Dims& D, int cap, Carver& cv) {
    DecodeWork w;
    w.rows_per_split = kRowsPerSplit;
    w.splits = D.lam > 0 ? (int)ceil_div(cap, kRowsPerSplit) : 0;
    w.la = cv.take<float>((size_t)D.B * D.Hq * (D.d + 1));
    w.win = cv.take<float>((size_t)D.B * D.Hq * (D.d + 2));
    w.part = cv.take<float>((size_t)D.B * D.Hq * (w.splits > 0 ? w.splits : 1) * (D.d + 2));
    return w;
}

static bool use_fast_decode(const Dims& D, const still_shape* sh) {
    return !(sh->flags & STILL_FLAG_GENERAL_KERNELS) && fast_decode_supported(D);
}

static size_t decode_bytes(const Dims& D, const still_shape* sh, int cap) {
    if (use_fast_decode(D, sh)) return fast_decode_floats(D, fast_decode_splits(cap)) * sizeof(float) + 256;
    Carver cv(nullptr);
    carve_decode(D, cap, cv);
    return cv.off + 256;
}

// Scratch of still_hybrid_attn_decode_step_noalloc: one array per GPU, part
// of the library's device code, so it exists wherever that code is loaded.
// Host code never uses the array's name as an address: the device address is
// looked up once per GPU (with that GPU current) and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[STILL_DECODE_SCRATCH_BYTES];

static constexpr int kMaxDevices = 64;
static std::mutex scratch_mu;
static void* scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's scratch (looked up on first use).
static int current_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return STILL_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return STILL_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return STILL_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return STILL_OK;
}

// pos_dev == nullptr: one position for the batch, cache->pos (advanced here).
// Otherwise the ragged form: pos_dev [B] device positions, advanced by the
// step's last kernel, and max_pos >= every one of them for the capacity check.
// use_scratch: ws is ignored; after every check (with ws_bytes =
// STILL_DECODE_SCRATCH_BYTES) the current GPU's scratch array serves instead.
static int decode(const still_shape* sh, const void* q, const void* k, const void* v,
                  const float* wq, const float* wk, const float* gate, still_cache* cache,
                  void* out, void* ws,
                  size_t ws_bytes, hipStream_t s, Timeline& tl, int64_t* pos_dev = nullptr,
                  int64_t max_pos = 0, bool use_scratch = false) {
    if (use_scratch) ws_bytes = STILL_DECODE_SCRATCH_BYTES;
    int st = check_shape(sh, true);
    if (st) return st;
    const Dims D = make_dims(sh, 1);
    if (!cache) return STILL_ERR_INVALID_ARG;
    const bool ragged = pos_dev != nullptr;
    if (ragged && max_pos < 0) return STILL_ERR_INVALID_ARG;
    if (D.B == 0) {  // nothing to compute; the batch's position still advances
        if (ragged) return STILL_OK;
        if (cache->pos < 0) return STILL_ERR_INVALID_ARG;
        cache->pos += 1;
        return STILL_OK;
    }
    if (!q || !k || !v || !wq || !wk || !out) return STILL_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(wq) ||
        !aligned16(wk) || !aligned4(gate))
        return STILL_ERR_INVALID_ARG;
    if (ragged && (reinterpret_cast<uintptr_t>(pos_dev) & 7u)) return STILL_ERR_INVALID_ARG;
    const int64_t t = ragged ? max_pos : cache->pos;
    const int64_t need = D.lam * ceil_div(t + 1 - D.W, D.C);
    st = check_cache(D, cache, ragged ? -2 : -1, need);
    if (st) return st;
    if (D.lam > 0 && cache->sel_cap < 1) return STILL_ERR_CAPACITY;
    const size_t need_ws = decode_bytes(D, sh, cache->sel_cap);
    if ((!ws && !use_scratch) || ws_bytes < need_ws) return STILL_ERR_WORKSPACE;
    if (tl.ev && tl.max_ev < 4) return STILL_ERR_INVALID_ARG;
    if (use_scratch) {
        st = current_scratch(&ws);
        if (st) return st;
    }
    void* wsa = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
    if (use_fast_decode(D, sh)) {
        CacheView cvw = view_of(cache);
        cvw.pos_dev = pos_dev;
        const int nsplit = fast_decode_splits(cache->sel_cap);
        float* fw = static_cast<float*>(wsa);
        STILL_LAUNCH(tl, s, "dec_stream", launch_fast_decode(D, q, k, v, wq, wk, gate, cvw, fw, nsplit, out, 0, s));
        STILL_LAUNCH(tl, s, "dec_combine", launch_fast_decode(D, q, k, v, wq, wk, gate, cvw, fw, nsplit, out, 1, s));
        STILL_TRY(tl.end(s));
        if (!ragged) cache->pos = t + 1;
        return STILL_OK;
    }
    Carver cv(wsa);
    DecodeWork w = carve_decode(D, cache->sel_cap, cv);
    CacheView cvw = view_of(cache);
    cvw.pos_dev = pos_dev;
    STILL_LAUNCH(tl, s, "decode_prep", launch_decode_prep(D, q, k, v, wq, wk, gate, cvw, w, s));
    STILL_LAUNCH(tl, s, "decode_sel", launch_decode_sel(D, q, cvw, w, s));
    STILL_LAUNCH(tl, s, "decode_combine", launch_decode_combine(D, w, out, pos_dev, s));
    STILL_TRY(tl.end(s));
    if (!ragged) cache->pos = t + 1;
    return STILL_OK;
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------
static int bwd_slices(const Dims& D, bool mfma) {
    // token slices of the projection-gradient sums: about 2048 blocks in all
    // (512 on the matrix cores, whose blocks take 64-row tiles: 256 leaves the
    // query side latency-bound, 1024 makes the slice sum cost more than it saves)
    const int64_t ntok = (int64_t)D.B * D.N;
    int64_t n = ((mfma ? 512 : 2048) + D.Hkv - 1) / D.Hkv;
    if (n > ntok) n = ntok;
    return n < 1 ? 1 : (int)n;
}

static bool use_mfma_bwd(const Dims& D, const still_shape* sh) {
    return !(sh->flags & STILL_FLAG_GENERAL_KERNELS) && mfma_bwd_supported(D);
}

static BwdWork carve_bwd(const Dims& D, Carver& cv, bool mfma) {
    BwdWork w;
    const size_t BN = (size_t)D.B * D.N, BG = (size_t)D.B * D.Hkv;
    const size_t E1 = (size_t)D.fd * (D.d + 1);
    // the matrix-core kernels after the lists count 64-token tiles
    Dims DT = D;
    if (mfma) {
        DT = tile_dims(D);
        DT.lam = D.lam < 64 ? D.lam : 64;
    }
    w.tile = DT;
    w.nslice = bwd_slices(D, mfma);
    w.phiq = cv.take<float>(BN * D.Hq * D.fd);
    w.phik = cv.take<float>(BN * D.Hkv * D.fd);
    w.lin = cv.take<float>(BG * D.T * E1);
    w.stat = cv.take<float>(BN * D.Hq * 4);
    w.dphiq = cv.take<float>(BN * D.Hq * D.fd);
    w.dphik = cv.take<float>(BN * D.Hkv * D.fd);
    w.ust = cv.take<float>(BG * DT.T * E1);
    w.duq = cv.take<float>(BN * D.Hq * (D.fd / 2));
    w.duk = cv.take<float>(BN * D.Hkv * (D.fd / 2));
    w.dwpart = cv.take<float>((size_t)w.nslice * D.Hkv * (D.fd / 2) * D.d);
    w.route = cv.take<uint8_t>(BG * D.N);
    w.selw = cv.take<int32_t>(BG * D.n_full * D.lam);
    w.selw_t = D.C > 64 && mfma ? cv.take<int32_t>(BG * DT.n_full * DT.lam) : w.selw;
    w.mfma = mfma;
    w.ksel = w.vsel = w.phik16 = w.wsplit = nullptr;
    w.kvpart = nullptr;
    w.ust16 = nullptr;
    w.list_off = nullptr;
    w.lin16 = LinBufs{};
    if (mfma) {
        const size_t nlist = BG * (size_t)sel_list_rows(DT);
        w.ksel = cv.take<uint16_t>(nlist * D.d);
        w.vsel = cv.take<uint16_t>(nlist * D.d);
        w.list_off = cv.take<int>(BG * (DT.n_full + 1));
        w.phik16 = cv.take<uint16_t>(BG * D.N * D.fd);
        const size_t ngroups = DT.n_full == 0 ? 0 : (size_t)(DT.n_full + DT.ng - 1) / DT.ng;
        w.lin16.sh = cv.take<uint16_t>(BG * DT.n_full * (size_t)D.d * D.fd);
        w.lin16.lz = cv.take<float>(BG * DT.n_full * (size_t)D.fd);
        w.lin16.ltot = cv.take<float>(BG * ngroups * E1);
        w.lin16.lcap = cv.take<float>(BG * E1);
        w.lin16.gh = cv.take<uint16_t>(BG * ngroups * (size_t)D.d * D.fd);
        w.lin16.gz = cv.take<float>(BG * ngroups * (size_t)D.fd);
        w.wsplit = cv.take<uint16_t>((size_t)4 * D.Hkv * (D.fd / 2) * D.d);
        w.kvpart = cv.take<float>(bwd_kv_part_floats(DT));
        w.ust16 = cv.take<uint16_t>(BG * DT.T * (size_t)D.fd * D.d);
    }
    return w;
}

static size_t bwd_bytes(const Dims& D, const still_shape* sh) {
    Carver cv(nullptr);
    carve_bwd(D, cv, use_mfma_bwd(D, sh));
    return cv.off + 256;
}

struct MarkCtx {
    Timeline* tl;
    hipStream_t s;
};
static hipError_t mark_launch(void* ctx, const char* name) {
    MarkCtx* m = static_cast<MarkCtx*>(ctx);
    return m->tl->mark(m->s, name);
}

static int bwd(const still_shape* sh, const void* q, const void* k, const void* v,
               const float* wq, const float* wk, const float* gate, const int32_t* sel_idx,
               const void* dout, const void* out_opt, const float* stats_opt, const void* fws,
               size_t fws_bytes, float* dq, float* dk, float* dv, float* dwq, float* dwk, float* dgate,
               void* ws, size_t ws_bytes, hipStream_t s, Timeline& tl) {
    int st = check_shape(sh, false);
    if (st) return st;
    const Dims D = make_dims(sh, sh->seqlen);
    const int nw = D.Hkv * (D.fd / 2) * D.d;
    if (D.B == 0 || D.N == 0) {  // no tokens: the projections get zero gradient
        if (dwq) STILL_TRY(launch_zero(dwq, nw, s));
        if (dwk) STILL_TRY(launch_zero(dwk, nw, s));
        return STILL_OK;
    }
    if (!q || !k || !v || !wq || !wk || !dout || !dq || !dk || !dv || !dwq || !dwk)
        return STILL_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, wq, wk, dout, dq, dk, dv, dwq, dwk};
    for (const void* p : ptrs)
        if (!aligned16(p)) return STILL_ERR_INVALID_ARG;
    if (!aligned4(gate) || !aligned4(dgate)) return STILL_ERR_INVALID_ARG;
    // the forward's output and statistics come together or not at all
    if ((out_opt == nullptr) != (stats_opt == nullptr) || !aligned16(out_opt) || !aligned16(stats_opt))
        return STILL_ERR_INVALID_ARG;
    if (D.lam > 0 && D.n_full > 0 && (!sel_idx || (reinterpret_cast<uintptr_t>(sel_idx) & 3u)))
        return STILL_ERR_INVALID_ARG;
    if (!ws || ws_bytes < bwd_bytes(D, sh)) return STILL_ERR_WORKSPACE;
    const bool mfma = use_mfma_bwd(D, sh);
    if (tl.ev && tl.max_ev < bwd_launch_count(mfma) + 1) return STILL_ERR_INVALID_ARG;
    // the forward's workspace: its keys' NP-Map features and linear prefixes
    // (the matrix-core forward leaves them there; same carving as the forward)
    if (fws && mfma && fws_bytes < fwd_bytes(D, sh)) return STILL_ERR_WORKSPACE;
    void* wsa = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
    Carver cv(wsa);
    BwdWork w = carve_bwd(D, cv, mfma);
    w.lin_given = false;
    if (fws && mfma) {
        Carver cf(reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(fws) + 255) & ~uintptr_t(255)));
        const MfmaBuffers f = carve_mfma(D, cf);
        w.phik16 = f.phik;
        w.lin16 = f.lin;
        w.lin_given = true;
    }
    BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.wq = wq;
    a.wk = wk;
    a.sel_idx = sel_idx;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dwq = dwq;
    a.dwk = dwk;
    a.gate = gate;
    a.dgate = gate ? dgate : nullptr;
    a.out = out_opt;
    a.stats = stats_opt;
    MarkCtx mc{&tl, s};
    STILL_TRY(launch_bwd(D, a, w, s, BwdMark{mark_launch, &mc}));
    STILL_TRY(tl.end(s));
    return STILL_OK;
}

// ---------------------------------------------------------------------------
// future-KV-utility diagnostic
// ---------------------------------------------------------------------------
static size_t util_bytes(const Dims& D) { return (size_t)D.B * D.N * D.Hq * 2 * sizeof(float) + 256; }

static int future_utility(const still_shape* sh, const void* q, const void* k, float* util,
                          void* ws, size_t ws_bytes, hipStream_t s) {
    int st = check_shape(sh, false);
    if (st) return st;
    const Dims D = make_dims(sh, sh->seqlen);
    if (D.B == 0 || D.N == 0) return STILL_OK;
    if (!q || !k || !util) return STILL_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || (reinterpret_cast<uintptr_t>(util) & 3u)) return STILL_ERR_INVALID_ARG;
    if (!ws || ws_bytes < util_bytes(D)) return STILL_ERR_WORKSPACE;
    float* stat = reinterpret_cast<float*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
    STILL_TRY(launch_future_utility(D, q, k, stat, util, s));
    return STILL_OK;
}

}  // namespace still

// ---------------------------------------------------------------------------
// exported C symbols
// ---------------------------------------------------------------------------
extern "C" {

int32_t still_abi_version(void) { return STILL_ABI_VERSION; }

const char* still_status_str(int status) {
    switch (status) {
        case STILL_OK: return "ok";
        case STILL_ERR_INVALID_ARG: return "invalid argument";
        case STILL_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case STILL_ERR_WORKSPACE: return "workspace too small";
        case STILL_ERR_CAPACITY: return "selected-token cache capacity exceeded";
        case STILL_ERR_HIP: return "HIP launch failure";
        default: return "unknown status";
    }
}

int32_t still_topk_for_budget(int32_t m, int32_t window, int32_t chunk, int64_t n_max) {
    if (chunk < 1 || n_max < 1 || m < window || window < 0) return -1;
    const int64_t t_max = (n_max + chunk - 1) / chunk;
    return (int32_t)((int64_t)(m - window) / t_max);
}

int still_fwd_workspace_size(const still_shape* shape, size_t* bytes) {
    if (!bytes) return STILL_ERR_INVALID_ARG;
    const int st = still::check_shape(shape, false);
    if (st) return st;
    *bytes = still::fwd_bytes(still::make_dims(shape, shape->seqlen), shape);
    return STILL_OK;
}

int still_hybrid_attn_fwd(const still_shape* shape, const void* q, const void* k, const void* v,
                          const float* wphi_q, const float* wphi_k, const float* gate_opt,
                          void* out, float* scores_opt, int32_t* sel_idx_opt, float* stats_opt,
                          still_cache* cache_opt, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    still::Timeline tl;
    return still::fwd(shape, q, k, v, wphi_q, wphi_k, gate_opt, out, scores_opt, sel_idx_opt,
                      stats_opt, cache_opt, workspace, workspace_bytes, stream, tl);
}

int still_hybrid_attn_fwd_timed(const still_shape* shape, const void* q, const void* k,
                                const void* v, const float* wphi_q, const float* wphi_k,
                                const float* gate_opt, void* out, float* scores_opt,
                                int32_t* sel_idx_opt, float* stats_opt,
                                still_cache* cache_opt, void* workspace, size_t workspace_bytes,
                                hipStream_t stream, hipEvent_t* events, int32_t max_events,
                                int32_t* n_launches, const char** kernel_names_opt) {
    if (!events || !n_launches || max_events < 1) return STILL_ERR_INVALID_ARG;
    still::Timeline tl;
    tl.ev = events;
    tl.max_ev = max_events;
    tl.names = kernel_names_opt;
    const int st = still::fwd(shape, q, k, v, wphi_q, wphi_k, gate_opt, out, scores_opt,
                              sel_idx_opt, stats_opt, cache_opt, workspace, workspace_bytes, stream, tl);
    *n_launches = tl.n;
    return st;
}

int still_decode_workspace_size(const still_shape* shape, int32_t sel_cap, size_t* bytes) {
    if (!bytes || sel_cap < 0) return STILL_ERR_INVALID_ARG;
    const int st = still::check_shape(shape, true);
    if (st) return st;
    *bytes = still::decode_bytes(still::make_dims(shape, 1), shape, sel_cap);
    return STILL_OK;
}

int still_hybrid_attn_decode_step(const still_shape* shape, const void* q, const void* k,
                                  const void* v, const float* wphi_q, const float* wphi_k,
                                  const float* gate_opt, still_cache* cache, void* out,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
    still::Timeline tl;
    return still::decode(shape, q, k, v, wphi_q, wphi_k, gate_opt, cache, out, workspace,
                         workspace_bytes, stream, tl);
}

int still_hybrid_attn_decode_step_timed(const still_shape* shape, const void* q, const void* k,
                                        const void* v, const float* wphi_q,
                                        const float* wphi_k, const float* gate_opt,
                                        still_cache* cache, void* out,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream, hipEvent_t* events,
                                        int32_t max_events, int32_t* n_launches,
                                        const char** kernel_names_opt) {
    if (!events || !n_launches || max_events < 1) return STILL_ERR_INVALID_ARG;
    still::Timeline tl;
    tl.ev = events;
    tl.max_ev = max_events;
    tl.names = kernel_names_opt;
    const int st = still::decode(shape, q, k, v, wphi_q, wphi_k, gate_opt, cache, out,
                                 workspace, workspace_bytes, stream, tl);
    *n_launches = tl.n;
    return st;
}

int still_hybrid_attn_decode_step_noalloc(const still_shape* shape, const void* q, const void* k,
                                          const void* v, const float* wphi_q,
                                          const float* wphi_k, const float* gate_opt,
                                          still_cache* cache, void* out, hipStream_t stream) {
    still::Timeline tl;
    return still::decode(shape, q, k, v, wphi_q, wphi_k, gate_opt, cache, out, nullptr, 0, stream,
                         tl, nullptr, 0, true);
}

int still_hybrid_attn_decode_step_ragged(const still_shape* shape, const void* q, const void* k,
                                         const void* v, const float* wphi_q, const float* wphi_k,
                                         const float* gate_opt, still_cache* cache,
                                         int64_t* pos_dev, int64_t max_pos, void* out,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
    if (!pos_dev) return STILL_ERR_INVALID_ARG;
    still::Timeline tl;
    return still::decode(shape, q, k, v, wphi_q, wphi_k, gate_opt, cache, out, workspace,
                         workspace_bytes, stream, tl, pos_dev, max_pos);
}

int still_bwd_workspace_size(const still_shape* shape, size_t* bytes) {
    if (!bytes) return STILL_ERR_INVALID_ARG;
    const int st = still::check_shape(shape, false);
    if (st) return st;
    *bytes = still::bwd_bytes(still::make_dims(shape, shape->seqlen), shape);
    return STILL_OK;
}

int still_hybrid_attn_bwd(const still_shape* shape, const void* q, const void* k, const void* v,
                          const float* wphi_q, const float* wphi_k, const float* gate_opt,
                          const int32_t* sel_idx, const void* dout, const void* out_opt,
                          const float* stats_opt, const void* fwd_workspace_opt,
                          size_t fwd_workspace_bytes, float* dq, float* dk,
                          float* dv, float* dwphi_q, float* dwphi_k, float* dgate_opt,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
    still::Timeline tl;
    return still::bwd(shape, q, k, v, wphi_q, wphi_k, gate_opt, sel_idx, dout, out_opt, stats_opt,
                      fwd_workspace_opt, fwd_workspace_bytes, dq, dk, dv, dwphi_q, dwphi_k, dgate_opt,
                      workspace, workspace_bytes, stream, tl);
}

int still_hybrid_attn_bwd_timed(const still_shape* shape, const void* q, const void* k,
                                const void* v, const float* wphi_q, const float* wphi_k,
                                const float* gate_opt, const int32_t* sel_idx, const void* dout,
                                const void* out_opt, const float* stats_opt,
                                const void* fwd_workspace_opt, size_t fwd_workspace_bytes,
                                float* dq, float* dk, float* dv, float* dwphi_q, float* dwphi_k,
                                float* dgate_opt, void* workspace,
                                size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
                                int32_t max_events, int32_t* n_launches,
                                const char** kernel_names_opt) {
    if (!events || !n_launches || max_events < 1) return STILL_ERR_INVALID_ARG;
    still::Timeline tl;
    tl.ev = events;
    tl.max_ev = max_events;
    tl.names = kernel_names_opt;
    const int st = still::bwd(shape, q, k, v, wphi_q, wphi_k, gate_opt, sel_idx, dout, out_opt,
                              stats_opt, fwd_workspace_opt, fwd_workspace_bytes, dq, dk, dv, dwphi_q,
                              dwphi_k, dgate_opt, workspace, workspace_bytes, stream, tl);
    *n_launches = tl.n;
    return st;
}

int still_future_kv_utility_workspace_size(const still_shape* shape, size_t* bytes) {
    if (!bytes) return STILL_ERR_INVALID_ARG;
    const int st = still::check_shape(shape, false);
    if (st) return st;
    *bytes = still::util_bytes(still::make_dims(shape, shape->seqlen));
    return STILL_OK;
}

int still_future_kv_utility(const still_shape* shape, const void* q, const void* k, float* util,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return still::future_utility(shape, q, k, util, workspace, workspace_bytes, stream);
}

}  // extern "C"
