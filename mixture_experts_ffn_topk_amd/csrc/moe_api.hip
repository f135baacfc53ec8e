// moe_api.hip -- host implementation of the C ABI declared in include/moe.h:
// argument validation, the workspace plan, kernel selection and launch
// sequence of the fused layer, and optional per-kernel event timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "moe_kernels.h"

using namespace moe;

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

moe_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return MOE_OK;
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// Per-kernel timing
// ---------------------------------------------------------------------------
enum Stage {
    ST_TOPK = 0,
    ST_ALIGN,
    ST_QUANT_X,
    ST_GEMM1,
    ST_GEMM1_REDUCE,
    ST_QUANT_ACT,
    ST_GEMM2,
    ST_COMBINE,
    ST_PREPACK,
    ST_ALIGN_PUBLIC,
    ST_QUANT_PUBLIC,
    ST_DEQUANT,
    ST_ROUTE_ALIGN,
    ST_COUNT
};
const char* kStageNames[ST_COUNT] = {"topk",      "align",   "quant_x",  "gemm1",
                                     "gemm1_splitk_reduce", "quant_act", "gemm2",
                                     "combine",   "prepack", "align_block_size",
                                     "quant_int8_rows", "dequant_fp8", "topk_align"};

struct Rec {
    int stage;
    hipEvent_t e0, e1;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<Rec> g_prof;

// Set for the duration of a call that must not create HIP objects (the
// no-allocation entry point): per-kernel events are skipped there.
thread_local bool g_prof_suppressed = false;

template <class F>
hipError_t timed(int stage, hipStream_t st, F&& launch) {
    bool on;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        on = g_prof_on;
    }
    if (!on || g_prof_suppressed) return launch();
    hipEvent_t e0, e1;
    hipError_t err = hipEventCreate(&e0);
    if (err != hipSuccess) return err;
    err = hipEventCreate(&e1);
    if (err != hipSuccess) return err;
    (void)hipEventRecord(e0, st);
    err = launch();
    (void)hipEventRecord(e1, st);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof.push_back({stage, e0, e1});
    return err;
}

// ---------------------------------------------------------------------------
// The fused layer's plan: kernel family, tiling, split-K and workspace layout
// ---------------------------------------------------------------------------
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Plan {
    int wtype, T, H, I, E, k, shared;
    int P, P_tot, E_tot;
    int path;  // MOE_PATH_DECODE / MOE_PATH_PREFILL
    int MB, chunk_rows, max_chunks;
    int64_t cap;   // slots of sorted_ids
    int64_t rows;  // rows of the per-row buffers: at most this many slots survive the padding
    int splits1, kbps1, splits2, kbps2, groups1, groups2;
    int act8;        // FP8 tile path with FP8 activations
    int kbp1, kbp2;  // act8: scale bytes per row of the GEMM1 / GEMM2 inputs
    size_t off_sorted, off_meta, off_chunks, off_sched, off_blkcnt, off_xq, off_xs, off_act,
        off_actq, off_acts, off_partial, off_y, total;
};

constexpr int kAlignB = 16;
static_assert(sizeof(Chunk) == sizeof(moe_chunk) && offsetof(moe_chunk, row_start) == offsetof(Chunk, row_start) &&
                  offsetof(moe_chunk, nrows) == offsetof(Chunk, nrows),
              "moe_chunk describes the chunk list the kernels write");
constexpr double kPrefillRowsPerExpert = 8.0;  // AUTO: above this many expected rows -> MFMA tiles
constexpr int kDecodeTargetWaves = 1536;      // streaming waves the K split aims for (measured: fewer,
                                              // longer splits beat more waves once the split-K
                                              // reduction and combine are counted)

Plan make_plan(int wtype, int T, int H, int I, int E, int k, int shared, const moe_options* opt) {
    Plan p{};
    p.wtype = wtype;
    p.T = T;
    p.H = H;
    p.I = I;
    p.E = E;
    p.k = k;
    p.shared = shared;
    p.P = T * k;
    p.P_tot = p.P + (shared ? T : 0);
    p.E_tot = E + (shared ? 1 : 0);
    const double rbar = (double)T * k / E;
    int path = opt ? opt->path : MOE_PATH_AUTO;
    if (path != MOE_PATH_DECODE && path != MOE_PATH_PREFILL) {
        path = rbar > kPrefillRowsPerExpert ? MOE_PATH_PREFILL : MOE_PATH_DECODE;
        if (wtype == W_FP8 && std::max(H, I) > kPrefillFp8MaxK) path = MOE_PATH_DECODE;
        if (wtype == W_INT4) path = MOE_PATH_DECODE;  // weight-only INT4: decode kernels only
        // the decode kernels address activations with 32-bit buffer offsets
        const int64_t rows16 = (int64_t)p.P_tot + (int64_t)std::min(p.E_tot, p.P_tot) * (kAlignB - 1);
        if (path == MOE_PATH_DECODE && std::max((int64_t)T * H, rows16 * I) * 2 >= 0x7fffffff)
            path = MOE_PATH_PREFILL;
    }
    p.path = path;
    if (path == MOE_PATH_DECODE) {
        p.MB = rbar <= 2.0 ? 1 : (rbar <= 4.0 ? 2 : 4);
        p.chunk_rows = 16 * p.MB;
    } else {
        p.MB = wtype == W_FP8 ? kPrefillF8MB : kPrefillMB;
        p.chunk_rows = 16 * p.MB;
    }
    p.cap = (int64_t)p.P_tot + (int64_t)p.E_tot * (kAlignB - 1);
    const int used = std::min(p.E_tot, p.P_tot);
    // npp = sum over experts of count rounded up to 16 <= P_tot + 15 * (experts with a pair)
    p.rows = std::min(p.cap, (int64_t)p.P_tot + (int64_t)used * (kAlignB - 1));
    p.max_chunks = used + (int)((p.P_tot + (int64_t)(kAlignB - 1) * used) / p.chunk_rows) + 1;

    const int nkb1 = H / 128, nkb2 = I / 128;
    if (path == MOE_PATH_DECODE) {
        p.groups1 = (I / 16 + kDecodeWavesPerWG - 1) / kDecodeWavesPerWG;
        const int g2t = decode_g2_tiles(wtype);
        p.groups2 = (H / 16 + kDecodeWavesPerWG * g2t - 1) / (kDecodeWavesPerWG * g2t);
        const int est = std::min(E, p.P) + (shared ? 1 : 0);
        int s1 = (int)std::max<int64_t>(1, (kDecodeTargetWaves + (int64_t)est * (I / 16) - 1) /
                                               ((int64_t)est * (I / 16)));
        s1 = std::min(s1, std::min(nkb1, 16));
        // INT8 tiny batches: no split (GEMM2's prologue quantises the rows;
        // measured faster than two or more splits at T = 1 and 4, equal at 2)
        if (wtype == W_INT8 && T <= kTinyMaxT && !(opt && opt->tiny_fusion != 0)) s1 = 1;
        if (opt && opt->split_k > 0) s1 = std::min(opt->split_k, nkb1);
        p.kbps1 = (nkb1 + s1 - 1) / s1;
        p.splits1 = (nkb1 + p.kbps1 - 1) / p.kbps1;
        const int64_t w2 = (int64_t)est * (H / 16 / g2t);
        int s2 = (int)std::max<int64_t>(1, (kDecodeTargetWaves + w2 - 1) / w2);
        s2 = std::min(s2, std::min(nkb2, 8));
        p.kbps2 = (nkb2 + s2 - 1) / s2;
        p.splits2 = (nkb2 + p.kbps2 - 1) / p.kbps2;
    } else if (wtype == W_FP8) {
        p.groups1 = 2 * I / kPrefillF8Cols;  // I is a multiple of 128
        p.groups2 = (H + kPrefillF8Cols - 1) / kPrefillF8Cols;
        p.splits1 = p.splits2 = 1;
        p.kbps1 = nkb1;
        p.kbps2 = nkb2;
    } else {
        const int cols = prefill_cols(wtype);  // H, I are multiples of 128
        p.groups1 = (2 * I + cols - 1) / cols;
        p.groups2 = (H + cols - 1) / cols;
        p.splits1 = p.splits2 = 1;
        p.kbps1 = nkb1;
        p.kbps2 = nkb2;
    }

    size_t o = 0;
    auto seg = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes, 256);
        return at;
    };
    p.off_sorted = seg(sizeof(int32_t) * (size_t)p.cap);
    p.off_meta = seg(64);
    // padded to a multiple of 8 slots: the prefill kernels read their slot
    // before comparing its index with the chunk count
    p.off_chunks = seg(sizeof(Chunk) * (size_t)((p.max_chunks + 7) / 8 * 8));
    // the tile kernels' schedule: the same chunks, largest first
    p.off_sched = seg(path == MOE_PATH_PREFILL ? sizeof(Chunk) * (size_t)((p.max_chunks + 7) / 8 * 8) : 0);
    // per-block expert counts of the many-workgroup alignment
    p.off_blkcnt = seg(p.P_tot >= kAlignMultiMin ? sizeof(int32_t) * (size_t)align_blocks(p.P_tot) * p.E_tot : 0);
    // activations as the GEMMs read them: INT8 codes + row scales, or for the
    // FP8 tile path E4M3 hi/lo records (2 bytes per element) + row scales
    const bool i8 = wtype == W_INT8;
    const bool f8t = wtype == W_FP8 && path == MOE_PATH_PREFILL;
    // FP8 activations: 1-byte codes and a per (row, 128-element block) scale
    // byte, rows of the table padded to whole 16-byte requests
    p.act8 = f8t && opt && opt->fp8_activations ? 1 : 0;
    p.kbp1 = p.act8 ? (int)align_up((size_t)nkb1, 16) : 0;
    p.kbp2 = p.act8 ? (int)align_up((size_t)nkb2, 16) : 0;
    const size_t f8e = p.act8 ? 1 : 2;  // activation bytes per element on the FP8 tile path
    const size_t xq_row = i8 ? (size_t)H : (f8t ? f8e * H : 0);
    const size_t aq_row = i8 ? (size_t)I : (f8t ? f8e * I : 0);
    p.off_xq = seg((size_t)T * xq_row);
    p.off_xs = seg(p.act8 ? (size_t)T * p.kbp1 : (xq_row ? sizeof(float) * (size_t)T : 0));
    // (FP8 activations: GEMM1 writes the down GEMM's codes itself, no bf16 rows)
    p.off_act = seg(p.act8 ? 0 : sizeof(uint16_t) * (size_t)p.rows * I);
    p.off_actq = seg((size_t)p.rows * aq_row);
    p.off_acts = seg(p.act8 ? (size_t)p.rows * p.kbp2 : (aq_row ? sizeof(float) * (size_t)p.rows : 0));
    p.off_partial =
        seg(p.splits1 > 1 ? sizeof(float) * (size_t)p.splits1 * p.rows * 2 * (size_t)I : 0);
    const size_t ybytes = path == MOE_PATH_DECODE
                              ? sizeof(float) * (size_t)p.splits2 * p.P_tot * H
                              : sizeof(uint16_t) * (size_t)p.P_tot * H;
    p.off_y = seg(ybytes);
    p.total = o;
    return p;
}

int elem_bytes(int wtype) { return wtype == MOE_W_BF16 ? 2 : 1; }
// stored bytes of an E x K x N weight stack (INT4: two codes per byte)
size_t weight_bytes(int wtype, int E, int K, int N) {
    const size_t n = (size_t)E * K * N;
    return wtype == MOE_W_INT4 ? n / 2 : n * elem_bytes(wtype);
}

moe_status check_fused_args(int wtype, const void* x, const void* w13, const float* s13,
                            const void* w2, const float* s2, const float* tw, const int32_t* ti,
                            int T, int H, int I, int E, int k, const moe_dense_expert* sh,
                            const void* ws, const void* out) {
    if (wtype < MOE_W_BF16 || wtype > MOE_W_INT4) return fail(MOE_ERR_ARG, "bad weight dtype %d", wtype);
    if (T < 0) return fail(MOE_ERR_ARG, "T=%d < 0", T);
    if (E < 1 || E > 1023) return fail(MOE_ERR_ARG, "E=%d outside [1, 1023]", E);
    if (k < 1 || k > E || k > 32) return fail(MOE_ERR_ARG, "k=%d outside [1, min(E, 32)]", k);
    if (H < 128 || I < 128 || H % 128 || I % 128)
        return fail(MOE_ERR_ARG, "H=%d and I=%d must be positive multiples of 128", H, I);
    if ((int64_t)T * k > (1 << 24)) return fail(MOE_ERR_ARG, "T*k=%lld exceeds 2^24", (long long)T * k);
    if (!x || !w13 || !w2 || !tw || !ti || !out || !ws)
        return fail(MOE_ERR_ARG, "null tensor pointer");
    if (wtype != MOE_W_BF16 && (!s13 || !s2)) return fail(MOE_ERR_ARG, "scales required for FP8/INT8");
    if (sh) {
        if (!sh->w13 || !sh->w2) return fail(MOE_ERR_ARG, "shared expert with null weights");
        if (wtype != MOE_W_BF16 && (!sh->w13_scale || !sh->w2_scale))
            return fail(MOE_ERR_ARG, "shared expert without scales");
        if (sh->inter != I)
            return fail(MOE_ERR_UNSUPPORTED, "shared expert intermediate %d != I=%d", sh->inter, I);
    }
    return MOE_OK;
}

// The decode kernels' tiny-batch form (launch_decode_gemm1_tiny): at most
// kTinyMaxT tokens, so every expert's pairs fit one 16-row block -- the
// router's ids are distinct per token; caller ids may repeat an expert, so
// those need T*k <= 16.  INT8 also keeps the token rows in registers and one
// split's K range of them in LDS.
bool tiny_fits(const Plan& p, bool routed, const moe_options* opt) {
    if (opt && opt->tiny_fusion != 0) return false;
    if (p.path != MOE_PATH_DECODE || p.MB != 1 || p.chunk_rows != 16 || p.T > kTinyMaxT) return false;
    if (p.P_tot > kTinyMaxPairs || p.E > kTinyMaxE || p.k > kTinyMaxPairs) return false;
    if (!routed && p.P > 16) return false;
    if (p.wtype == W_INT8 && ((int64_t)p.T * p.H > kTinyMaxElems ||
                              (int64_t)(p.T + 1) * p.kbps1 * 128 > kTinyMaxLds))
        return false;
    return true;
}

// route != nullptr: the top-k of route->logits is computed here too, into
// tw / ti (see fused_moe_routed).
moe_status run_fused(int wtype, const uint16_t* x, const void* w13, const float* s13,
                     const void* w2, const float* s2, const float* tw, const int32_t* ti, int T,
                     int H, int I, int E, int k, const moe_dense_expert* sh, void* ws,
                     size_t ws_bytes, uint16_t* out, const moe_options* opt, hipStream_t st,
                     const RouteArgs* route = nullptr) {
    moe_status rc = check_fused_args(wtype, x, w13, s13, w2, s2, tw, ti, T, H, I, E, k, sh, ws, out);
    if (rc != MOE_OK) return rc;
    if (route && !route->logits) return fail(MOE_ERR_ARG, "null logits");
    if (route && route->score != MOE_SCORE_SOFTMAX && route->score != MOE_SCORE_SIGMOID)
        return fail(MOE_ERR_ARG, "bad score function %d", route->score);
    if (opt && opt->prefill_span < 0) return fail(MOE_ERR_ARG, "negative prefill_span %d", opt->prefill_span);
    if (T == 0) return MOE_OK;
    const Plan p = make_plan(wtype, T, H, I, E, k, sh != nullptr, opt);
    if (p.path == MOE_PATH_PREFILL && wtype == W_FP8 && std::max(H, I) > kPrefillFp8MaxK)
        return fail(MOE_ERR_UNSUPPORTED, "FP8 prefill path needs H, I <= %d", kPrefillFp8MaxK);
    if (p.path == MOE_PATH_PREFILL && wtype == W_INT4)
        return fail(MOE_ERR_UNSUPPORTED, "INT4 weights run on the decode kernels only");
    if (p.path == MOE_PATH_DECODE && std::max((int64_t)T * H, p.rows * (int64_t)I) * 2 >= 0x7fffffff)
        return fail(MOE_ERR_UNSUPPORTED, "decode path: activation tensors must stay below 2 GiB "
                                         "(T*H and rows*I elements); use the prefill path");
    if (ws_bytes < p.total)
        return fail(MOE_ERR_WORKSPACE, "workspace %zu B < required %zu B", ws_bytes, p.total);
    char* base = (char*)ws;
    int32_t* sorted = (int32_t*)(base + p.off_sorted);
    int32_t* meta = (int32_t*)(base + p.off_meta);
    Chunk* chunks = (Chunk*)(base + p.off_chunks);
    // tile kernels: chunks in the schedule order (largest first)
    Chunk* sched = p.path == MOE_PATH_PREFILL ? (Chunk*)(base + p.off_sched) : nullptr;
    int8_t* xq = (int8_t*)(base + p.off_xq);
    float* xs = (float*)(base + p.off_xs);
    uint16_t* act = (uint16_t*)(base + p.off_act);
    int8_t* actq = (int8_t*)(base + p.off_actq);
    float* acts = (float*)(base + p.off_acts);
    float* partial = (float*)(base + p.off_partial);
    void* y = base + p.off_y;

    hipError_t e;
    // Tiny batches: routing, alignment and the INT8 token quantisation run
    // in the first GEMM's prologue (no launches of their own)
    const bool tiny = tiny_fits(p, route != nullptr, opt);
    // few-row decode with a split first GEMM: its reduction runs in GEMM2's
    // prologue (no launch of its own)
    bool red2 = false;
    if (p.path == MOE_PATH_DECODE && (p.splits1 > 1 || (tiny && wtype == W_INT8)) && p.MB == 1 &&
        I <= kSplitQuantMaxI && !(opt && opt->tiny_fusion != 0)) {
        GemmArgs probe{};
        probe.P_tot = p.P_tot;
        probe.kb_per_split = p.kbps2;
        red2 = gemm2_red_lds(wtype, probe) <= (size_t)kGemm2RedMaxLds;
    }
    // 1. alignment
    AlignArgs al{};
    al.ids = ti;
    al.P = p.P;
    al.n_shared = sh ? T : 0;
    al.E = E;
    al.B = kAlignB;
    al.cap = p.cap;
    al.sorted_ids = sorted;
    al.expert_ids = nullptr;
    al.npp = meta;
    al.meta = meta;
    al.chunks = chunks;
    al.sched = sched;
    al.chunk_rows = p.chunk_rows;
    al.skip_tail = 1;  // every kernel below stops at npp = meta[0]
    al.blk_cnt = p.P_tot >= kAlignMultiMin ? (int32_t*)(base + p.off_blkcnt) : nullptr;
    // 2. INT8: the token rows are quantised once, by extra blocks of the
    // alignment launch (independent work)
    if (wtype == W_INT8) {
        al.qx = x;
        al.q_rows = T;
        al.q_cols = H;
        al.qq = xq;
        al.qs = xs;
    }
    if (tiny) {
        // (step 3 below)
    } else if (route && route_align_fits(T, E, k)) {
        // 0+1. top-k and alignment in one workgroup
        e = timed(ST_ROUTE_ALIGN, st, [&] { return launch_route_align(al, *route, st); });
        if (e != hipSuccess) return hip_status(e, "top-k + align launch");
    } else {
        if (route) {  // 0. top-k
            e = timed(ST_TOPK, st, [&] {
                return launch_topk(route->logits, T, E, k, route->score, route->renorm,
                                   route->w_out, route->id_out, st);
            });
            if (e != hipSuccess) return hip_status(e, "topk launch");
        }
        e = timed(ST_ALIGN, st, [&] { return launch_align(al, st); });
        if (e != hipSuccess) return hip_status(e, "align launch");
    }

    // 2'. FP8 tile path: token rows -> E4M3 hi/lo records
    const bool f8t = wtype == W_FP8 && p.path == MOE_PATH_PREFILL;
    if (f8t) {
        SplitArgs q{};
        q.x = x;
        q.rows = T;
        q.K = H;
        q.out = (uint8_t*)xq;
        q.rscale = xs;
        q.act8 = p.act8;
        q.exps = (uint8_t*)xs;
        q.exp_stride = p.kbp1;
        e = timed(ST_QUANT_X, st, [&] { return launch_split_rows(q, st); });
        if (e != hipSuccess) return hip_status(e, "split launch");
    }

    // 3. GEMM1 + SiLU(C1)*C2 (INT8 with split K: the reduction also quantises
    // the intermediate rows; with red2 the reduction runs in GEMM2's prologue)
    const bool fused_quant = wtype == W_INT8 && p.path == MOE_PATH_DECODE && p.splits1 > 1 &&
                             I <= kSplitQuantMaxI;
    GemmArgs g{};
    g.A = (wtype == W_INT8 || f8t) ? (const void*)xq : (const void*)x;
    g.a_bytes = (int64_t)T * H * (wtype == W_INT8 ? 1 : 2);
    g.a_scale = xs;
    g.W = (const uint8_t*)w13;
    g.w_scale = s13;
    g.W_sh = sh ? (const uint8_t*)sh->w13 : nullptr;
    g.w_scale_sh = sh ? sh->w13_scale : nullptr;
    g.sorted_ids = sorted;
    g.chunks = sched ? sched : chunks;
    g.meta = meta;
    g.K = H;
    g.N = 2 * I;
    g.E = E;
    g.topk = k;
    g.P = p.P;
    g.P_tot = p.P_tot;
    g.cap = p.rows;  // row stride of the split-K partials; grid of the row kernels
    g.act8 = p.act8;
    g.a_exp = (const uint8_t*)xs;
    g.exp_stride = p.kbp1;
    g.out_codes = (uint8_t*)actq;
    g.out_exps = (uint8_t*)acts;
    g.out_exp_stride = p.kbp2;
    g.out = act;
    if (p.path == MOE_PATH_DECODE) {
        g.n_groups = p.groups1;
        g.splits = p.splits1;
        g.kb_per_split = p.kbps1;
        g.partial = partial;
        g.topk_ids = ti;
        if (tiny) {
            TinyRoute tr{};
            tr.logits = route ? route->logits : nullptr;
            tr.ids = ti;
            tr.T = T;
            tr.k = k;
            tr.score = route ? route->score : 0;
            tr.renorm = route ? route->renorm : 0;
            tr.w_out = route ? route->w_out : nullptr;
            tr.id_out = route ? route->id_out : nullptr;
            tr.x = x;
            tr.xq_out = xq;
            tr.xs_out = xs;
            tr.sorted_ids = sorted;
            tr.meta = meta;
            tr.chunks = chunks;
            const int slots = std::min(E, p.P) + (sh ? 1 : 0);
            e = timed(ST_GEMM1, st, [&] { return launch_decode_gemm1_tiny(wtype, g, tr, slots, st); });
        } else {
            e = timed(ST_GEMM1, st, [&] { return launch_decode_gemm1(wtype, p.MB, g, p.max_chunks, st); });
        }
        if (e == hipSuccess && p.splits1 > 1 && !red2) {
            if (fused_quant) {
                g.act_q = actq;
                g.act_s = acts;
                e = timed(ST_GEMM1_REDUCE, st, [&] { return launch_splitk_silu_quant(g, st); });
            } else {
                e = timed(ST_GEMM1_REDUCE, st, [&] { return launch_splitk_silu(wtype, g, st); });
            }
        }
    } else {
        g.n_groups = p.groups1;
        g.group_span = opt ? opt->prefill_span : 0;
        g.splits = 1;
        g.kb_per_split = H / 128;
        e = timed(ST_GEMM1, st, [&] { return launch_prefill_gemm1(wtype, g, p.max_chunks, st); });
    }
    if (e != hipSuccess) return hip_status(e, "gemm1 launch");

    // 4. INT8: quantise the intermediate rows
    if (wtype == W_INT8 && !fused_quant && !red2) {
        QuantArgs q{};
        q.x = act;
        q.rows = p.rows;
        q.cols = I;
        q.q = actq;
        q.scale = acts;
        q.row_ids = sorted;
        q.meta = meta;
        q.sentinel = p.P_tot;
        e = timed(ST_QUANT_ACT, st, [&] { return launch_quant_rows(q, st); });
        if (e != hipSuccess) return hip_status(e, "quant launch");
    } else if (f8t && !p.act8) {
        // FP8 tile path: intermediate rows -> E4M3 hi/lo records (with FP8
        // activations GEMM1 wrote the codes and scale bytes already)
        SplitArgs q{};
        q.x = act;
        q.rows = p.rows;
        q.K = I;
        q.out = (uint8_t*)actq;
        q.rscale = acts;
        q.row_ids = sorted;
        q.meta = meta;
        q.sentinel = p.P_tot;
        q.act8 = p.act8;
        q.exps = (uint8_t*)acts;
        q.exp_stride = p.kbp2;
        e = timed(ST_QUANT_ACT, st, [&] { return launch_split_rows(q, st); });
        if (e != hipSuccess) return hip_status(e, "split launch");
    }

    // 6's arguments (the fused GEMM2 of tiny INT8 batches takes them too)
    CombineArgs c{};
    c.y = y;
    c.topk_w = tw;
    c.topk_ids = ti;
    c.T = T;
    c.k = k;
    c.H = H;
    c.E = E;
    c.P = p.P;
    c.has_shared = sh != nullptr;
    c.out = out;

    // 5. GEMM2
    bool comb = false;  // GEMM2 and the combine in one launch
    GemmArgs g2 = g;
    g2.A = (wtype == W_INT8 || f8t) ? (const void*)actq : (const void*)act;
    g2.a_bytes = p.rows * (int64_t)I * (wtype == W_INT8 ? 1 : 2);
    g2.a_scale = acts;
    g2.a_exp = (const uint8_t*)acts;
    g2.exp_stride = p.kbp2;
    g2.W = (const uint8_t*)w2;
    g2.w_scale = s2;
    g2.W_sh = sh ? (const uint8_t*)sh->w2 : nullptr;
    g2.w_scale_sh = sh ? sh->w2_scale : nullptr;
    g2.K = I;
    g2.N = H;
    g2.out = y;
    g2.partial = nullptr;
    if (p.path == MOE_PATH_DECODE) {
        g2.n_groups = p.groups2;
        g2.splits = p.splits2;
        g2.kb_per_split = p.kbps2;
        g2.y_bf16 = 0;
        if (red2) {
            SplitRed rd{};
            rd.partial = partial;
            rd.splits = p.splits1 > 1 ? p.splits1 : 0;
            rd.act = act;
            rd.cap = p.rows;
            rd.chunk_cap = p.max_chunks;
            rd.x_scale = xs;
            rd.w1_scale = s13;
            rd.w1_scale_sh = sh ? sh->w13_scale : nullptr;
            // INT8 tiny batches of a few pairs: the combine's sums inside
            // GEMM2 (one wave per chunk, one column tile per workgroup)
            comb = tiny && wtype == W_INT8 && rd.splits == 0 && p.splits2 == 1 && p.P_tot <= kCombMaxPairs &&
                   T * decode_g2_tiles(W_INT8) * 16 <= 64 * kCombMaxPairs && gemm2_comb_lds(g2) <= (size_t)kGemm2RedMaxLds;
            if (comb)
                e = timed(ST_GEMM2, st, [&] { return launch_decode_gemm2_comb(g2, rd, c, st); });
            else
                e = timed(ST_GEMM2, st, [&] { return launch_decode_gemm2_red(wtype, g2, rd, p.max_chunks, st); });
        } else {
            e = timed(ST_GEMM2, st, [&] { return launch_decode_gemm2(wtype, p.MB, g2, p.max_chunks, st); });
        }
    } else {
        g2.n_groups = p.groups2;
        g2.splits = 1;
        g2.kb_per_split = I / 128;
        g2.y_bf16 = 1;
        e = timed(ST_GEMM2, st, [&] { return launch_prefill_gemm2(wtype, g2, p.max_chunks, st); });
    }
    if (e != hipSuccess) return hip_status(e, "gemm2 launch");

    // 6. combine (done inside the fused GEMM2)
    if (comb) return MOE_OK;
    c.y_bf16 = g2.y_bf16;
    c.splits = g2.splits;
    e = timed(ST_COMBINE, st, [&] { return launch_combine(c, st); });
    if (e != hipSuccess) return hip_status(e, "combine launch");
    return MOE_OK;
}

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

}  // namespace

// ---------------------------------------------------------------------------
// Workspace for callers that cannot allocate (fused_moe_routed_noalloc): one
// file-scope device array per GPU, held until the process ends.  Host code
// never uses the array's name as a device address: its address on each
// device comes from hipGetSymbolAddress, taken once per device on the first
// call made with that device current.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status scratch_of_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MOE_OK;
}

struct ProfSuppress {
    ProfSuppress() { g_prof_suppressed = true; }
    ~ProfSuppress() { g_prof_suppressed = false; }
};

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int moe_version(void) { return 100; }

moe_status moe_topk(const float* logits, int T, int E, int k, moe_score score, int renormalize,
                    float* topk_weights, int32_t* topk_ids, hipStream_t stream) {
    if (T < 0) return fail(MOE_ERR_ARG, "T=%d < 0", T);
    if (E < 1 || E > 1024) return fail(MOE_ERR_ARG, "E=%d outside [1, 1024]", E);
    if (k < 1 || k > E || k > 32) return fail(MOE_ERR_ARG, "k=%d outside [1, min(E, 32)]", k);
    if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID)
        return fail(MOE_ERR_ARG, "bad score function %d", (int)score);
    if (T == 0) return MOE_OK;
    if (!logits || !topk_weights || !topk_ids) return fail(MOE_ERR_ARG, "null pointer");
    hipError_t e = timed(ST_TOPK, stream, [&] {
        return launch_topk(logits, T, E, k, (int)score, renormalize ? 1 : 0, topk_weights,
                           topk_ids, stream);
    });
    return hip_status(e, "topk launch");
}

int64_t moe_align_capacity(int64_t P, int E, int block_size) {
    if (P < 0 || E < 1 || block_size < 1) return -1;
    return P + (int64_t)E * (block_size - 1);
}

moe_status moe_align_block_size(const int32_t* topk_ids, int T, int k, int E, int block_size,
                                int32_t* sorted_ids, int32_t* expert_ids,
                                int32_t* num_tokens_post_pad, hipStream_t stream) {
    if (T < 0 || k < 1) return fail(MOE_ERR_ARG, "T=%d k=%d", T, k);
    if (E < 1 || E > 1024) return fail(MOE_ERR_ARG, "E=%d outside [1, 1024]", E);
    if (!is_pow2(block_size) || block_size > 256)
        return fail(MOE_ERR_ARG, "block_size=%d is not a power of two in [1, 256]", block_size);
    if ((int64_t)T * k > (1 << 24)) return fail(MOE_ERR_ARG, "T*k exceeds 2^24");
    if (!sorted_ids || !expert_ids || !num_tokens_post_pad || (T > 0 && !topk_ids))
        return fail(MOE_ERR_ARG, "null pointer");
    AlignArgs a{};
    a.ids = topk_ids;
    a.P = T * k;
    a.n_shared = 0;
    a.E = E;
    a.B = block_size;
    a.cap = moe_align_capacity(a.P, E, block_size);
    a.sorted_ids = sorted_ids;
    a.expert_ids = expert_ids;
    a.npp = num_tokens_post_pad;
    a.meta = nullptr;
    a.chunks = nullptr;
    a.chunk_rows = block_size;
    hipError_t e = timed(ST_ALIGN_PUBLIC, stream, [&] { return launch_align(a, stream); });
    return hip_status(e, "align launch");
}

moe_status moe_quant_int8_rows(const uint16_t* x_bf16, int rows, int cols, int8_t* q,
                               float* scale, hipStream_t stream) {
    if (rows < 0 || cols < 1 || cols % 8) return fail(MOE_ERR_ARG, "rows=%d cols=%d", rows, cols);
    if (rows == 0) return MOE_OK;
    if (!x_bf16 || !q || !scale) return fail(MOE_ERR_ARG, "null pointer");
    QuantArgs a{};
    a.x = x_bf16;
    a.rows = rows;
    a.cols = cols;
    a.q = q;
    a.scale = scale;
    hipError_t e = timed(ST_QUANT_PUBLIC, stream, [&] { return launch_quant_rows(a, stream); });
    return hip_status(e, "quant launch");
}

size_t moe_packed_bytes(moe_wdtype wdtype, int E, int K, int N) {
    if (E < 1 || K < 1 || N < 1) return 0;
    if (wdtype < MOE_W_BF16 || wdtype > MOE_W_INT4) return 0;
    return weight_bytes((int)wdtype, E, K, N);
}

moe_status moe_prepack(moe_wdtype wdtype, const void* w_logical, int E, int K, int N, int is_w13,
                       void* w_packed, hipStream_t stream) {
    if (wdtype < MOE_W_BF16 || wdtype > MOE_W_INT4) return fail(MOE_ERR_ARG, "bad dtype");
    if (E < 1 || K < 64 || K % 64 || N < 16 || N % 16 || (is_w13 && (N / 2) % 16))
        return fail(MOE_ERR_ARG, "prepack shape E=%d K=%d N=%d is_w13=%d", E, K, N, is_w13);
    if (wdtype == MOE_W_INT4 && K % 128)
        return fail(MOE_ERR_ARG, "INT4 prepack needs K %% 128 == 0 (K=%d)", K);
    if (!w_logical || !w_packed) return fail(MOE_ERR_ARG, "null pointer");
    if (w_logical == w_packed) return fail(MOE_ERR_ARG, "prepack cannot run in place");
    hipError_t e = timed(ST_PREPACK, stream, [&] {
        return launch_prepack(elem_bytes(wdtype), (int)wdtype, w_logical, E, K, N, is_w13 ? 1 : 0,
                              w_packed, stream);
    });
    return hip_status(e, "prepack launch");
}

moe_status moe_prepack_bf16(const uint16_t* w, int E, int K, int N, int is_w13, uint16_t* packed,
                            hipStream_t stream) {
    return moe_prepack(MOE_W_BF16, w, E, K, N, is_w13, packed, stream);
}
moe_status moe_prepack_fp8(const uint8_t* w, int E, int K, int N, int is_w13, uint8_t* packed,
                           hipStream_t stream) {
    return moe_prepack(MOE_W_FP8, w, E, K, N, is_w13, packed, stream);
}
moe_status moe_prepack_int8(const int8_t* w, int E, int K, int N, int is_w13, int8_t* packed,
                            hipStream_t stream) {
    return moe_prepack(MOE_W_INT8, w, E, K, N, is_w13, packed, stream);
}

moe_status moe_dequant_fp8(const uint8_t* codes, const float* scale, int K, int N, int mode,
                           float* out, hipStream_t stream) {
    if (K < 1 || N < 1 || (K * (int64_t)N) % 4) return fail(MOE_ERR_ARG, "K*N must be a multiple of 4");
    if (scale && (K % 128 || N % 128)) return fail(MOE_ERR_ARG, "scaled shape must tile by 128");
    if (mode != 0 && mode != 1) return fail(MOE_ERR_ARG, "mode");
    if (!codes || !out) return fail(MOE_ERR_ARG, "null pointer");
    hipError_t e = timed(ST_DEQUANT, stream,
                         [&] { return launch_dequant_fp8(codes, scale, K, N, mode, out, stream); });
    return hip_status(e, "dequant launch");
}

size_t fused_moe_workspace_bytes_ex(moe_wdtype wdtype, int T, int H, int I, int E, int k,
                                    int has_shared, const moe_options* opt) {
    if (T < 1 || H < 128 || I < 128 || E < 1 || k < 1 || k > E) return 0;
    return make_plan((int)wdtype, T, H, I, E, k, has_shared ? 1 : 0, opt).total;
}

size_t fused_moe_workspace_bytes(moe_wdtype wdtype, int T, int H, int I, int E, int k,
                                 int has_shared) {
    moe_options d{}, pf{};
    d.path = MOE_PATH_DECODE;
    pf.path = MOE_PATH_PREFILL;
    return std::max(fused_moe_workspace_bytes_ex(wdtype, T, H, I, E, k, has_shared, &d),
                    fused_moe_workspace_bytes_ex(wdtype, T, H, I, E, k, has_shared, &pf));
}

moe_status fused_moe_workspace_layout(moe_wdtype wdtype, int T, int H, int I, int E, int k,
                                      int has_shared, const moe_options* opt,
                                      moe_workspace_layout* layout) {
    if (!layout) return fail(MOE_ERR_ARG, "null layout");
    if (wdtype < MOE_W_BF16 || wdtype > MOE_W_INT4) return fail(MOE_ERR_ARG, "bad weight dtype %d", (int)wdtype);
    if (T < 1 || E < 1 || E > 1023 || k < 1 || k > E || k > 32 || H < 128 || I < 128 || H % 128 ||
        I % 128 || (int64_t)T * k > (1 << 24))
        return fail(MOE_ERR_ARG, "layout shape T=%d H=%d I=%d E=%d k=%d", T, H, I, E, k);
    const Plan p = make_plan((int)wdtype, T, H, I, E, k, has_shared ? 1 : 0, opt);
    layout->path = p.path;
    layout->block_size = kAlignB;
    layout->chunk_rows = p.chunk_rows;
    layout->max_chunks = p.max_chunks;
    layout->cap = p.cap;
    layout->rows = p.rows;
    layout->sorted_ids = p.off_sorted;
    layout->meta = p.off_meta;
    layout->chunks = p.off_chunks;
    layout->xq = p.off_xq;
    layout->xs = p.off_xs;
    layout->xs_stride = p.kbp1;
    layout->total = p.total;
    layout->sched = p.path == MOE_PATH_PREFILL ? p.off_sched : SIZE_MAX;
    return MOE_OK;
}

moe_status fused_moe_ex(moe_wdtype wdtype, const uint16_t* x, const void* w13,
                        const float* w13_scale, const void* w2, const float* w2_scale,
                        const float* topk_weights, const int32_t* topk_ids, int T, int H, int I,
                        int E, int k, const moe_dense_expert* shared, void* ws, size_t ws_bytes,
                        uint16_t* out, const moe_options* opt, hipStream_t stream) {
    return run_fused((int)wdtype, x, w13, w13_scale, w2, w2_scale, topk_weights, topk_ids, T, H,
                     I, E, k, shared, ws, ws_bytes, out, opt, stream);
}

moe_status fused_moe_routed(moe_wdtype wdtype, const float* logits, moe_score score,
                            int renormalize, const uint16_t* x, const void* w13,
                            const float* w13_scale, const void* w2, const float* w2_scale,
                            float* topk_weights, int32_t* topk_ids, int T, int H, int I, int E,
                            int k, const moe_dense_expert* shared, void* ws, size_t ws_bytes,
                            uint16_t* out, const moe_options* opt, hipStream_t stream) {
    RouteArgs r{};
    r.logits = logits;
    r.k = k;
    r.score = (int)score;
    r.renorm = renormalize ? 1 : 0;
    r.w_out = topk_weights;
    r.id_out = topk_ids;
    return run_fused((int)wdtype, x, w13, w13_scale, w2, w2_scale, topk_weights, topk_ids, T, H,
                     I, E, k, shared, ws, ws_bytes, out, opt, stream, &r);
}

moe_status fused_moe_routed_noalloc(moe_wdtype wdtype, const float* logits, moe_score score,
                                    int renormalize, const uint16_t* x, const void* w13,
                                    const float* w13_scale, const void* w2, const float* w2_scale,
                                    float* topk_weights, int32_t* topk_ids, int T, int H, int I,
                                    int E, int k, const moe_dense_expert* shared, uint16_t* out,
                                    const moe_options* opt, hipStream_t stream) {
    // (the workspace is the static scratch: any non-null stand-in passes the check)
    moe_status rc = check_fused_args((int)wdtype, x, w13, w13_scale, w2, w2_scale, topk_weights,
                                     topk_ids, T, H, I, E, k, shared, (const void*)1, out);
    if (rc == MOE_OK && !logits) rc = fail(MOE_ERR_ARG, "null logits");
    if (rc != MOE_OK) return rc;
    if (T == 0) return MOE_OK;
    // the size check needs no device: a batch over the limit is refused first
    const size_t need = make_plan((int)wdtype, T, H, I, E, k, shared != nullptr, opt).total;
    if (need > kNoAllocScratchBytes)
        return fail(MOE_ERR_UNSUPPORTED,
                    "fused_moe_routed_noalloc: this batch needs %zu bytes of scratch, the static "
                    "maximum is %zu (use fused_moe_routed with a caller workspace)",
                    need, kNoAllocScratchBytes);
    void* ws = nullptr;
    rc = scratch_of_current_device(&ws);
    if (rc != MOE_OK) return rc;
    ProfSuppress quiet;
    return fused_moe_routed(wdtype, logits, score, renormalize, x, w13, w13_scale, w2, w2_scale,
                            topk_weights, topk_ids, T, H, I, E, k, shared, ws,
                            kNoAllocScratchBytes, out, opt, stream);
}

moe_status fused_moe_bf16(const uint16_t* x, const uint16_t* w13, const uint16_t* w2,
                          const float* topk_weights, const int32_t* topk_ids, int T, int H, int I,
                          int E, int k, const moe_dense_expert* shared, void* ws, size_t ws_bytes,
                          uint16_t* out, hipStream_t stream) {
    return run_fused(MOE_W_BF16, x, w13, nullptr, w2, nullptr, topk_weights, topk_ids, T, H, I,
                     E, k, shared, ws, ws_bytes, out, nullptr, stream);
}

moe_status fused_moe_fp8(const uint16_t* x, const uint8_t* w13, const float* w13_scale,
                         const uint8_t* w2, const float* w2_scale, const float* topk_weights,
                         const int32_t* topk_ids, int T, int H, int I, int E, int k,
                         const moe_dense_expert* shared, void* ws, size_t ws_bytes, uint16_t* out,
                         hipStream_t stream) {
    return run_fused(MOE_W_FP8, x, w13, w13_scale, w2, w2_scale, topk_weights, topk_ids, T, H, I,
                     E, k, shared, ws, ws_bytes, out, nullptr, stream);
}

moe_status fused_moe_int4(const uint16_t* x, const uint8_t* w13, const float* w13_scale,
                          const uint8_t* w2, const float* w2_scale, const float* topk_weights,
                          const int32_t* topk_ids, int T, int H, int I, int E, int k,
                          const moe_dense_expert* shared, void* ws, size_t ws_bytes,
                          uint16_t* out, hipStream_t stream) {
    return run_fused(MOE_W_INT4, x, w13, w13_scale, w2, w2_scale, topk_weights, topk_ids, T, H, I,
                     E, k, shared, ws, ws_bytes, out, nullptr, stream);
}

moe_status moe_prepack_int4(const uint8_t* w, int E, int K, int N, int is_w13, uint8_t* packed,
                            hipStream_t stream) {
    return moe_prepack(MOE_W_INT4, w, E, K, N, is_w13, packed, stream);
}

moe_status fused_moe_int8(const uint16_t* x, const int8_t* w13, const float* w13_scale,
                          const int8_t* w2, const float* w2_scale, const float* topk_weights,
                          const int32_t* topk_ids, int T, int H, int I, int E, int k,
                          const moe_dense_expert* shared, void* ws, size_t ws_bytes,
                          uint16_t* out, hipStream_t stream) {
    return run_fused(MOE_W_INT8, x, w13, w13_scale, w2, w2_scale, topk_weights, topk_ids, T, H, I,
                     E, k, shared, ws, ws_bytes, out, nullptr, stream);
}

moe_status moe_profile_enable(int on) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on = on != 0;
    return MOE_OK;
}

int moe_profile_collect(double* total_ms, int64_t* launches, int max_stages) {
    std::vector<Rec> recs;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        recs.swap(g_prof);
    }
    for (int i = 0; i < max_stages && i < ST_COUNT; ++i) {
        if (total_ms) total_ms[i] = 0.0;
        if (launches) launches[i] = 0;
    }
    for (const Rec& r : recs) {
        (void)hipEventSynchronize(r.e1);
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, r.e0, r.e1) == hipSuccess && r.stage < max_stages) {
            if (total_ms) total_ms[r.stage] += ms;
            if (launches) launches[r.stage] += 1;
        }
        (void)hipEventDestroy(r.e0);
        (void)hipEventDestroy(r.e1);
    }
    return ST_COUNT;
}

const char* moe_profile_stage_name(int stage) {
    return (stage >= 0 && stage < ST_COUNT) ? kStageNames[stage] : "";
}

}  // extern "C"
