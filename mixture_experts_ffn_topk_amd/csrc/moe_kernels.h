// moe_kernels.h -- argument blocks and host launchers of the libmoe kernels.
// Internal header: the public boundary is include/moe.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"

namespace moe {

struct AlignArgs {
    const int32_t* ids;   // [P]
    int P;                // routed pairs
    int n_shared;         // shared-expert pairs appended (one per token), 0 = none
    int E;                // routed experts (the shared expert gets index E)
    int B;                // block size
    int64_t cap;          // length of sorted_ids
    int32_t* sorted_ids;  // [cap]
    int32_t* expert_ids;  // [ceil(cap/B)] or nullptr
    int32_t* npp;         // [1]
    int32_t* meta;        // [2] (npp, n_chunks) or nullptr
    Chunk* chunks;        // or nullptr
    Chunk* sched;         // or nullptr: the chunk list again, largest chunks first
                          // (the order the tile kernels take them in)
    int chunk_rows;       // rows per chunk (multiple of B)
    int skip_tail;        // 1: leave sorted_ids[npp..cap) / expert_ids past npp/B unwritten
                          //    (readers that stop at npp do not need them)
    int32_t* blk_cnt;     // [align_blocks(P_tot)][E_tot] workspace of the many-workgroup
                          // alignment (used from kAlignMultiMin pairs), or nullptr
    // optional INT8 quantisation of token rows in the same launch (qx == nullptr: none)
    const uint16_t* qx;   // bf16 [q_rows, q_cols]
    int64_t q_rows;
    int q_cols;
    int8_t* qq;           // [q_rows, q_cols]
    float* qs;            // [q_rows]
};

// FP8 tile path: bf16 rows -> E4M3 hi/lo records (see moe_prefill_f8.hip).
struct SplitArgs {
    const uint16_t* x;       // bf16 [rows, K]
    int64_t rows;
    int K;                   // multiple of 64
    uint8_t* out;            // [rows, K/64, 128 B]
    float* rscale;           // [rows]: 2^-e, the row was multiplied by 2^e before splitting
    const int32_t* row_ids;  // optional row filter (sorted_ids): rows >= meta[0] or whose
    const int32_t* meta;     // id >= sentinel are skipped
    int sentinel;
    // FP8-activation variant: out = E4M3 codes [rows, K/64, 64 B] and exps =
    // per (row, 128-element block) MFMA scale bytes [rows, exp_stride]
    int act8;
    uint8_t* exps;
    int exp_stride;
};

struct QuantArgs {
    const uint16_t* x;       // bf16 [rows, cols]
    int64_t rows;
    int cols;
    int8_t* q;               // [rows, cols]
    float* scale;            // [rows]
    const int32_t* row_ids;  // optional row filter (sorted_ids), see kernel
    const int32_t* meta;     // meta[0] = valid row count when row_ids != nullptr
    int sentinel;
};

// Grouped GEMM over the row chunks of the alignment (both kernel families).
struct GemmArgs {
    const void* A;            // GEMM1: x bf16 / xq int8 [T, K]; GEMM2: act bf16 / actq int8 [cap, K]
                              // (FP8 tile path: E4M3 hi/lo records [rows, K/64, 128 B])
    int64_t a_bytes;          // bytes of the A tensor (decode kernels: < 2^31)
    const float* a_scale;     // per-row activation scale ([T] for GEMM1, [cap] for GEMM2):
                              // INT8 quantisation scale / FP8 tile path 2^-e
    const uint8_t* W;         // packed routed weights (E experts)
    const float* w_scale;     // FP8 block scales / INT8 channel scales of the routed experts
    const uint8_t* W_sh;      // packed shared expert (expert index E) or nullptr
    const float* w_scale_sh;
    const int32_t* sorted_ids;
    const Chunk* chunks;
    const int32_t* meta;      // meta[1] = number of chunks
    int K, N;                 // logical GEMM shape: GEMM1 K=H, N=2I; GEMM2 K=I, N=H
    int E, topk, P, P_tot;    // routed experts, k, routed pairs, pairs incl. shared
    int n_groups;             // column groups per chunk (prefill kernels: workgroups
                              // per chunk at launch, each running group_span groups)
    int group_span;           // BF16 / INT8 prefill: column groups per workgroup, 0 = auto
    int col_groups;           // set by the prefill launcher: column groups per chunk
    int splits;               // K splits (decode family)
    int kb_per_split;         // 128-row K blocks per split
    float* partial;           // GEMM1 decode split-K partials [splits][cap][N]
    const int32_t* topk_ids;  // [P] (split-K reduction: expert of each pair)
    int64_t cap;
    void* out;                // GEMM1: act bf16 [cap, N/2]; GEMM2: y (see kernels)
    int y_bf16;               // GEMM2: 1 -> y bf16 [P_tot, N], 0 -> fp32 [splits, P_tot, N]
    int8_t* act_q;            // INT8 split-K reduction: quantised rows [cap, N/2] ...
    float* act_s;             // ... and their scales [cap] (the bf16 rows are not written)
    // FP8 tile path with FP8 activations: A holds E4M3 codes [rows, K/64, 64 B]
    // and a_exp the per (row, 128-element K block) MFMA scale bytes
    int act8;
    const uint8_t* a_exp;     // [rows, exp_stride]
    int exp_stride;           // bytes per row: K/128 rounded up to 16
    // ... and GEMM1 then writes the down GEMM's input that way itself:
    uint8_t* out_codes;       // [cap rows, N/2 / 64, 64 B]
    uint8_t* out_exps;        // [cap rows, out_exp_stride]
    int out_exp_stride;
};

struct CombineArgs {
    const void* y;            // fp32 [splits, P_tot, H] or bf16 [P_tot, H]
    int y_bf16;
    int splits;
    const float* topk_w;      // [T, k]
    const int32_t* topk_ids;  // [T, k]
    int T, k, H, E, P, has_shared;
    uint16_t* out;            // bf16 [T, H]
};

hipError_t launch_topk(const float* logits, int T, int E, int k, int score, int renorm, float* w,
                       int32_t* ids, hipStream_t st);
// Router arguments of the fused top-k + alignment launch.
struct RouteArgs {
    const float* logits;  // fp32 [T, E]
    int k, score, renorm;
    float* w_out;         // [T, k]
    int32_t* id_out;      // [T, k]
};
constexpr int kRouteAlignMaxTokens = 16;  // top-k + alignment in one workgroup up to this T
bool route_align_fits(int T, int E, int k);
hipError_t launch_route_align(const AlignArgs& a, const RouteArgs& r, hipStream_t st);
int align_waves(int E_tot, int P_tot);
// From kAlignMultiMin pairs (and with a blk_cnt workspace) the alignment runs
// over many workgroups: blocks of align_blk_pairs() consecutive pairs, at
// most 256 blocks.
constexpr int kAlignMultiMin = 8192;
inline int align_blk_pairs(int64_t P_tot) {
    int bp = 2048;
    while ((P_tot + bp - 1) / bp > 256) bp *= 2;
    return bp;
}
inline int align_blocks(int64_t P_tot) { return (int)((P_tot + align_blk_pairs(P_tot) - 1) / align_blk_pairs(P_tot)); }
size_t align_lds_bytes(int E_tot, int P_tot);
hipError_t launch_align(const AlignArgs& a, hipStream_t st);
hipError_t launch_quant_rows(const QuantArgs& a, hipStream_t st);
hipError_t launch_prepack(int elem_bytes, int wtype, const void* w, int E, int K, int N,
                          int is_w13, void* out, hipStream_t st);
hipError_t launch_dequant_fp8(const uint8_t* codes, const float* scale, int K, int N, int mode,
                              float* out, hipStream_t st);

// Decode family: weight streaming, MB 16-row blocks per chunk (1, 2 or 4).
hipError_t launch_decode_gemm1(int wtype, int MB, const GemmArgs& a, int max_chunks,
                               hipStream_t st);
hipError_t launch_decode_gemm2(int wtype, int MB, const GemmArgs& a, int max_chunks,
                               hipStream_t st);
// Tiny batches (T <= kTinyMaxT tokens) on the decode kernels: GEMM1 runs the
// router top-k (or reads the given ids), the alignment and, for INT8, the
// token rows' quantisation in every workgroup's prologue (see
// moe_decode.hip); workgroup 0 publishes what the later kernels and the
// caller read.  The grid covers `slots` possible experts (min(E, T*k) plus
// the shared one); workgroups past the distinct experts exit.
struct TinyRoute {
    const float* logits;     // fp32 [T, E], or nullptr: the ids come from `ids`
    const int32_t* ids;      // [T, k] when logits == nullptr
    int T, k, score, renorm;
    float* w_out;            // [T, k] router weights (logits only)
    int32_t* id_out;         // [T, k] router ids (logits only)
    const uint16_t* x;       // INT8: bf16 token rows [T, K]
    int8_t* xq_out;          // INT8: their codes [T, K] ...
    float* xs_out;           // ... and scales [T]
    int32_t* sorted_ids;     // alignment: slots [0, npp) ...
    int32_t* meta;           // ... npp and the chunk count ...
    Chunk* chunks;           // ... and the chunk list
    int tiles_per_wg;        // set by the launcher: pair tiles per workgroup (<= 4 waves)
};
constexpr int kTinyMaxT = 4;
constexpr int kTinyMaxPairs = 64;      // T*k plus T shared pairs: one per lane
constexpr int kTinyMaxE = 256;         // router experts (four logits per lane)
constexpr int kTinyMaxElems = 16384;   // INT8: T*H token elements held in registers
constexpr int kTinyMaxLds = 65536;     // INT8: (T + 1) rows of one split's K range
hipError_t launch_decode_gemm1_tiny(int wtype, const GemmArgs& a, const TinyRoute& r, int slots,
                                    hipStream_t st);
// Sum GEMM1 split-K partials in split order and apply SiLU(C1)*C2 -> act.
// INT8 split-K reduction fused with the row quantisation of the intermediate
// (N/2 <= kSplitQuantMaxI); writes a.act_q / a.act_s.
constexpr int kSplitQuantMaxI = 4096;
hipError_t launch_splitk_silu_quant(const GemmArgs& a, hipStream_t st);
hipError_t launch_splitk_silu(int wtype, const GemmArgs& a, hipStream_t st);
// GEMM2 with GEMM1's split-K reduction (and, INT8, the intermediate rows'
// quantisation; INT8 without a split: the quantisation only) in its
// prologue: one 16-row block per chunk, I <= kSplitQuantMaxI, and the
// chunk's live rows of one K split in LDS.
struct SplitRed {
    const void* partial;      // GEMM1 split partials [splits][cap][2I] (int32 INT8, else fp32)
    int splits;               // 0 (INT8 only): no split; the rows are GEMM1's bf16 `act`
    const uint16_t* act;      // [cap][I] when splits == 0
    int64_t cap;
    int chunk_cap;            // entries of the chunk list (a.chunks)
    const float* x_scale;     // INT8: token scales [T]
    const float* w1_scale;    // INT8: GEMM1 channel scales [E][2I] ...
    const float* w1_scale_sh; // ... and the shared expert's [2I]
};
constexpr int kGemm2RedMaxLds = 65536;
size_t gemm2_red_lds(int wtype, const GemmArgs& a);
// INT8 tiny batches of at most kCombMaxPairs pairs, GEMM1 unsplit: GEMM2 and
// the combine in one launch (one wave per chunk, one column tile per
// workgroup); CombineArgs as for launch_combine.
constexpr int kCombMaxPairs = 8;
size_t gemm2_comb_lds(const GemmArgs& a);
hipError_t launch_decode_gemm2_comb(const GemmArgs& a, const SplitRed& rd, const CombineArgs& c, hipStream_t st);
hipError_t launch_decode_gemm2_red(int wtype, const GemmArgs& a, const SplitRed& rd, int max_chunks,
                                   hipStream_t st);
// Prefill family: MFMA tiles through LDS; BF16 / INT8: producer/consumer waves,
// 192-row chunks; FP8 weights: 160-row chunks (below).
hipError_t launch_prefill_gemm1(int wtype, const GemmArgs& a, int max_chunks, hipStream_t st);
hipError_t launch_prefill_gemm2(int wtype, const GemmArgs& a, int max_chunks, hipStream_t st);
// FP8 weights on the tile path (dispatched from the two above): activations
// as E4M3 hi/lo records, native FP8 MFMA, 256 weight columns per workgroup.
hipError_t launch_prefill_f8_gemm1(const GemmArgs& a, int max_chunks, hipStream_t st);
hipError_t launch_prefill_f8_gemm2(const GemmArgs& a, int max_chunks, hipStream_t st);
hipError_t launch_split_rows(const SplitArgs& a, hipStream_t st);
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);

// Column-group geometry shared by host and device.
constexpr int kDecodeWavesPerWG = 4;   // one pair tile (GEMM1) / decode_g2_tiles tiles (GEMM2) per wave
// decode GEMM2: 16-column tiles per wave (INT8: one, measured faster at five
// waves per SIMD; FP8 / BF16: two)
// (INT4: two as well; four measured slower, 67 vs 47 us at the DeepSeek-R1
// decode shape, from two waves per SIMD)
constexpr int decode_g2_tiles(int wtype) { return wtype == W_INT8 ? 1 : 2; }
constexpr int kPrefillMB = 12;         // 16-row blocks per prefill chunk (192 rows; BF16 / INT8)
constexpr int kPrefillF8MB = 10;       // 16-row blocks per prefill chunk (160 rows; FP8)
// weight columns per prefill workgroup (BF16: 128; INT8: 256)
constexpr int prefill_cols(int wtype) { return wtype == W_INT8 ? 256 : 128; }
constexpr int kPrefillF8Cols = 256;    // weight columns per prefill workgroup (FP8)
constexpr int kPrefillFp8MaxK = 16384; // FP8 prefill: block scales held in two registers per tile

}  // namespace moe
