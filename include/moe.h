/*
 * moe.h -- C ABI of libmoe, the MI355X (gfx950) fused Mixture-of-Experts FFN
 * layer:  router top-k -> alignment of topk_ids into expert-blocked
 * sorted_ids -> grouped gate/up GEMM with SiLU(C1)*C2 fused -> down GEMM ->
 * top-k-weighted combine, on BF16, FP8-E4M3FN (128x128 block scales) or INT8
 * (per-output-channel scales, dynamic per-row activation quantisation) weights.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless a comment says "host".
 *  - The caller allocates and owns every buffer.  The library never allocates
 *    device memory; fused_moe_* take a caller workspace whose size
 *    fused_moe_workspace_bytes() reports.
 *  - Work is enqueued on `stream` and the call returns without waiting.
 *    Arguments are validated on the host before anything is enqueued: an
 *    invalid call returns MOE_ERR_ARG / MOE_ERR_UNSUPPORTED /
 *    MOE_ERR_WORKSPACE and launches nothing.  A launch failure returns
 *    MOE_ERR_HIP.  moe_last_error() gives a one-line reason for the last
 *    non-OK status of the calling thread.  No exception crosses the ABI.
 *  - Matrices are row-major with the last index contiguous.  bf16 tensors are
 *    passed as uint16_t bit patterns, FP8 as uint8_t E4M3FN codes (OCP
 *    variant: bias 7, max 448, subnormals, no infinities).
 *  - Notation: T tokens, H hidden size, I intermediate size, E routed experts,
 *    k experts per token, P = T*k (token, slot) pairs with flat pair index
 *    i = t*k + j.
 *
 * Sources are cited by page title and section:
 *  [blog]  Intel PyTorch team blog on SGLang's Xeon 6 CPU backend.
 *  [notes] The author's own write-up of the same backend.
 *  [osdi]  Summary of the OSDI'26 local-MoE inference paper (CPU-GPU hybrid).
 *  [lmsys] News rewrite of the LMSYS large-scale expert-parallel blog.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t, hipEvent_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_ARG = 1,         /* invalid argument (null pointer, bad size, k > E, ...) */
    MOE_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels implement */
    MOE_ERR_WORKSPACE = 3,   /* workspace smaller than fused_moe_workspace_bytes() */
    MOE_ERR_HIP = 4          /* a HIP call or kernel launch failed */
} moe_status;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;

/* MOE_W_INT4: weight-only 4-bit (see fused_moe_int4), decode kernels only. */
typedef enum { MOE_W_BF16 = 0, MOE_W_FP8 = 1, MOE_W_INT8 = 2, MOE_W_INT4 = 3 } moe_wdtype;

/* Kernel family for the grouped GEMMs.  AUTO picks from the expected rows per
 * expert T*k/E: few rows -> the weight-streaming decode kernels, many rows ->
 * the MFMA tile kernels.  The others force one family (both are exact
 * implementations of the same layer; forcing is for tests and A/B timing).
 * The FP8 tile kernels take H, I <= 16384 (AUTO falls back to the decode
 * kernels above that; forcing PREFILL returns MOE_ERR_UNSUPPORTED). */
typedef enum { MOE_PATH_AUTO = 0, MOE_PATH_DECODE = 1, MOE_PATH_PREFILL = 2 } moe_path;

/* Static description; host pointer to a string that lives forever. */
const char* moe_status_str(moe_status s);
/* Host string describing the last non-OK status returned on this thread. */
const char* moe_last_error(void);
/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int moe_version(void);

/* ---------------------------------------------------------------------------
 * Router top-k  ([blog] section "MoE": topk_ids per token feed the argsort;
 * score functions per the workload list: softmax, or sigmoid + renormalise).
 *
 * logits        fp32 [T, E], finite values.
 * topk_weights  fp32 [T, k]  out: score of each chosen expert; with
 *               renormalize != 0 divided by the sum of the k chosen scores.
 *               Scores: softmax over all E logits, or 1 / (1 + exp(-logit)).
 * topk_ids      int32 [T, k] out: the k largest logits of the row in
 *               descending order, ties to the lower expert id (selection on
 *               logits is exact and matches selection on either score).
 * Limits: 1 <= E <= 1024, 1 <= k <= min(E, 32), T >= 0 (T == 0 is a no-op).
 * ------------------------------------------------------------------------- */
moe_status moe_topk(const float* logits, int T, int E, int k, moe_score score, int renormalize,
                    float* topk_weights, int32_t* topk_ids, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Alignment of topk_ids into expert-blocked sorted_ids
 * ([blog] "MoE": argsort of topk_ids, indices kept in sorted_ids grouped by
 * expert id; [notes] 03 (3): moe_align_index, blocking of sorted_ids with
 * each block's expert id recorded; only the per-expert set matters).
 *
 * Host helper: capacity of sorted_ids = P + E*(block_size-1).
 * ------------------------------------------------------------------------- */
int64_t moe_align_capacity(int64_t P, int E, int block_size);

/* topk_ids            int32 [T, k], values in [0, E).  An id outside [0, E)
 *                     is dropped (it appears in no block).
 * sorted_ids          int32 [cap] out.  For e = 0..E-1 in order, the flat
 *                     indices i with topk_ids.flat[i] == e in ascending i,
 *                     padded with the sentinel P to a multiple of
 *                     block_size; experts with no pair get no block.
 *                     Slots from num_tokens_post_pad to cap hold P.
 * expert_ids          int32 [ceil(cap / block_size)] out: expert of each
 *                     block; -1 after the last used block.
 * num_tokens_post_pad int32 [1] out: total padded length (a multiple of
 *                     block_size).
 * Deterministic: positions come from prefix sums, never from atomics, so
 * the output is bit-identical on every run.
 * Limits: 1 <= E <= 1024, block_size a power of two in [1, 256],
 *         P = T*k <= 2^24.
 * ------------------------------------------------------------------------- */
moe_status moe_align_block_size(const int32_t* topk_ids, int T, int k, int E, int block_size,
                                int32_t* sorted_ids, int32_t* expert_ids,
                                int32_t* num_tokens_post_pad, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Dynamic symmetric INT8 quantisation of bf16 rows ([blog] "MoE": dynamic
 * activation quantisation fused with the fetch; [notes] 02: per-channel INT8).
 * Per row, in binary32: s = amax / 127; q = clamp(rint(x / s), -127, 127),
 * ties to even; an all-zero row gives s = 0, q = 0.
 * x_bf16 [rows, cols] -> q int8 [rows, cols], scale fp32 [rows].
 * Limits: rows >= 0, 1 <= cols, cols % 8 == 0.
 * ------------------------------------------------------------------------- */
moe_status moe_quant_int8_rows(const uint16_t* x_bf16, int rows, int cols, int8_t* q,
                               float* scale, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Weight prepack (one-time, not part of the timed layer).
 *
 * Converts logical weights [E, K, N] (w13: K = H, N = 2I with gate columns
 * [0, I) and up columns [I, 2I) -- [blog] "MoE": A x [B1, B2], SiLU on the
 * left half, multiply by the right; w2: K = I, N = H) into the MFMA-operand
 * order the fused kernels stream: 16-column x 64-row tiles of
 * 64 lanes x 16 elements, contiguous along K, with w13's gate and up tiles of
 * the same intermediate column interleaved.  Same bytes, no rescaling; scale
 * arrays are NOT repacked (pass them to fused_moe_* unchanged).
 *
 * is_w13   1 for w13 (interleave gate/up), 0 for w2.
 * Limits: K % 64 == 0, N % 16 == 0 (w13: N/2 % 16 == 0); E >= 1.
 * moe_packed_bytes() gives the size of the packed buffer (equal to the
 * logical size).
 * ------------------------------------------------------------------------- */
size_t moe_packed_bytes(moe_wdtype wdtype, int E, int K, int N);
moe_status moe_prepack(moe_wdtype wdtype, const void* w_logical, int E, int K, int N, int is_w13,
                       void* w_packed, hipStream_t stream);
moe_status moe_prepack_bf16(const uint16_t* w, int E, int K, int N, int is_w13, uint16_t* packed,
                            hipStream_t stream);
moe_status moe_prepack_fp8(const uint8_t* w, int E, int K, int N, int is_w13, uint8_t* packed,
                           hipStream_t stream);
moe_status moe_prepack_int8(const int8_t* w, int E, int K, int N, int is_w13, int8_t* packed,
                            hipStream_t stream);
/* INT4: w logical [E, K, N/2] bytes (column 2j in the low nibble of byte j,
 * two's complement codes); packed into per (16-column tile, 128-row K block)
 * blocks of 1 KiB, the same E*K*N/2 bytes.  K % 128 == 0. */
moe_status moe_prepack_int4(const uint8_t* w, int E, int K, int N, int is_w13, uint8_t* packed,
                            hipStream_t stream);

/* ---------------------------------------------------------------------------
 * The fused layer.
 *
 * out[t] = bf16( sum_j topk_weights[t,j] * FFN_{topk_ids[t,j]}(x[t])
 *                + FFN_shared(x[t]) )
 * FFN_e(v) = ( SiLU(v W13_e[:, :I]) * (v W13_e[:, I:]) ) W2_e
 *   ([blog] "MoE": GEMM-SiLU-GEMM per expert with SiLU(C1)*C2 fused into the
 *   first GEMM; [notes] 03 (3): experts computed in parallel over blocks of
 *   sorted_ids; [osdi] "CPU decode backend": FP8 E4M3FN weights whose
 *   128-element block scale is applied after the block's partial dot product;
 *   [blog] "FP8 inference": FP8 is weight-only against BF16 activations;
 *   [blog] "MoE" + [notes] 02: INT8 weights per output channel with dynamic
 *   8-bit activations.)
 *
 * x             bf16 [T, H]
 * w13, w2       PACKED weights (moe_prepack_*) of logical [E, H, 2I], [E, I, H]
 * w13_scale     FP8: fp32 [E, H/128, 2I/128]; INT8: fp32 [E, 2I]; INT4: fp32
 *               [E, H/128, 2I]; BF16: NULL
 * w2_scale      FP8: fp32 [E, I/128, H/128];  INT8: fp32 [E, H];  INT4: fp32
 *               [E, I/128, H]; BF16: NULL
 * topk_weights  fp32 [T, k], topk_ids int32 [T, k] (as moe_topk writes them;
 *               ids must lie in [0, E) -- out-of-range slots are dropped)
 * shared        host pointer, NULL for none: a dense expert of the same format
 *               and intermediate size, weight 1, applied to every token
 *               (DeepSeek-R1-style shared expert).  Its w13/w2 are packed
 *               with E = 1; scales as above without the E axis.
 * ws, ws_bytes  device workspace of at least fused_moe_workspace_bytes().
 *               Contents on entry are ignored; clobbered on exit.
 * out           bf16 [T, H]
 * Limits: T >= 0 (T == 0 is a no-op), 1 <= E <= 1023, 1 <= k <= min(E, 32),
 *   H and I positive multiples of 128 (all weight types), T*k <= 2^24.
 * Results: every routed pair is computed exactly once; the combine sums the k
 *   slots in ascending j (then the shared expert) in fp32, so repeated calls
 *   are bit-identical.
 * ------------------------------------------------------------------------- */
typedef struct {
    const void* w13;       /* packed [1, H, 2I] */
    const float* w13_scale;
    const void* w2;        /* packed [1, I, H] */
    const float* w2_scale;
    int inter;             /* must equal I */
} moe_dense_expert;

typedef struct {
    int path;       /* moe_path; MOE_PATH_DECODE needs T*H*2 and cap*I*2 bytes below
                       2 GiB (cap = moe_align_capacity(T*k + shared T, E + shared, 16)),
                       else MOE_ERR_UNSUPPORTED; AUTO picks decode only for few
                       rows per expert (T*k/E <= 8) */
    int split_k;    /* decode kernels: K splits of the first GEMM, 0 = auto */
    int prefill_span; /* BF16 / INT8 prefill kernels: column groups (BF16: 128
                       weight columns, INT8: 256) that one workgroup runs back
                       to back, 0 = auto; larger values are clamped to the
                       number of groups and to 8 (INT8) or 64 (BF16);
                       negative ones are an argument error.  Results do not
                       depend on it. */
    int fp8_activations; /* FP8 weights on the MFMA tile kernels (prefill), opt in:
                       1 quantises both GEMM inputs (the token rows, the
                       intermediate rows) to E4M3FN with one power-of-two scale
                       per row and 128-element K block ([lmsys] "DeepGEMM集成":
                       FP8 grouped GEMMs), and each product is one FP8 MFMA at
                       the FP8 rate.  Results are then those of 3-bit-mantissa
                       activations (a few percent relative L2 error against the
                       bf16-activation layer), not within the 1e-2 gate.  0
                       (default): bf16 activations kept exact (each product is
                       a hi/lo pair of FP8 MFMAs).  Ignored by the decode
                       kernels, which stream the weights against bf16
                       activations either way, and for BF16 / INT8 weights. */
    int tiny_fusion; /* decode kernels, T <= 4 tokens (and T*k <= 16 when the
                       ids come from the caller): 0 (default) runs the router
                       top-k, the alignment and the INT8 token quantisation
                       inside the first GEMM's launch (each of its workgroups
                       rebuilds the one-block-per-expert layout from the T*k
                       ids; [lmsys] "DeepGEMM集成": the masked layout of a
                       fixed block per expert for decode).  Also, whenever
                       the decode kernels split the first GEMM's K range and
                       every chunk is one 16-row block, the split-K
                       reduction (SiLU(C1)*C2, INT8: the intermediate rows'
                       quantisation) runs in the second GEMM's prologue;
                       INT8 batches of at most 4 tokens then do not split
                       that K range at all and the second GEMM's prologue
                       quantises the first one's rows; with at most 8 pairs
                       (and the second GEMM unsplit) its launch also takes
                       the combine.  1 keeps all of these
                       as launches of their own (and the usual split, so the
                       workspace size depends on this field:
                       fused_moe_workspace_bytes_ex).  Results, the workspace
                       contents listed by moe_workspace_layout (the chunks'
                       reserved field aside) and the top-k outputs are the
                       same bit for bit either way (INT8 partial sums are
                       exact integers). */
    int reserved[3];
} moe_options;

/* Workspace that fused_moe_{bf16,fp8,int8} (and fused_moe_ex with default
 * options, either kernel family) need; 0 for invalid shapes.
 * The size depends on T, and not monotonically on the decode kernels: a
 * batch that touches few experts splits the first GEMM's K range more ways
 * and keeps more fp32 partial sums than a slightly larger batch.  A caller
 * that reuses one workspace for several batch sizes allocates the largest
 * of their sizes.  The per-row buffers hold P' + 15 * min(E', P') rows
 * (P' = T*k plus T with a shared expert, E' = E plus one with a shared
 * expert): at most that many rows survive the 16-row padding. */
size_t fused_moe_workspace_bytes(moe_wdtype wdtype, int T, int H, int I, int E, int k,
                                 int has_shared);
/* Workspace for fused_moe_ex with the given options. */
size_t fused_moe_workspace_bytes_ex(moe_wdtype wdtype, int T, int H, int I, int E, int k,
                                    int has_shared, const moe_options* opt);

/* One chunk of the row table the alignment step writes for the grouped GEMMs:
 * `nrows` consecutive slots of sorted_ids from `row_start` (a multiple of 16),
 * all routed to expert `expert` (== E for the shared expert).  Chunks follow
 * the experts in ascending order; an expert's padded group is cut into
 * chunks of `chunk_rows` slots, the last one shorter. */
typedef struct {
    int32_t expert;
    int32_t row_start;
    int32_t nrows;
    int32_t reserved;  /* internal use (the decode path's tiny batches: the
                          chunk's live rows, which come first) */
} moe_chunk;

/* Where a fused_moe_* call keeps its alignment inside the workspace, so a
 * caller (a test, a tool) can read it back after the call has finished.
 * The fused layer aligns with block size 16 on the pairs topk_ids plus, with
 * a shared expert, one pair (t, shared) per token appended after the routed
 * ones as expert E: pair P + t.  Its sentinel is that pair count P'.
 * Offsets are in bytes from the workspace start. */
typedef struct {
    int path;              /* kernel family the call runs (MOE_PATH_DECODE / _PREFILL) */
    int block_size;        /* alignment block: 16 */
    int chunk_rows;        /* slots per chunk (a multiple of 16) */
    int max_chunks;        /* capacity of the chunk list */
    int64_t cap;           /* slots of sorted_ids: P' + E' * 15 */
    int64_t rows;          /* rows of the per-row buffers: P' + 15 * min(E', P') */
    size_t sorted_ids;     /* int32 [cap]; slots [0, npp) are written by every call */
    size_t meta;           /* int32 [2]: npp (padded total), number of chunks */
    size_t chunks;         /* moe_chunk [max_chunks]; the first meta[1] are written */
    size_t xq;             /* INT8 weights: the token rows' codes int8 [T, H];
                              FP8 with fp8_activations on the tile kernels: their
                              E4M3 codes as records [T, H/64, 64 bytes], record
                              part p holding k = 64 s + 8p .. +7 and 64 s + 32 + 8p
                              .. +7 of stage s (other cases: internal use) */
    size_t xs;             /* INT8 weights: their scales fp32 [T], as
                              moe_quant_int8_rows writes them; FP8 with
                              fp8_activations: per (token, 128-element block b)
                              the byte 127 - e_b, [T, xs_stride], the codes being
                              E4M3(x * 2^e_b) */
    int xs_stride;         /* bytes per token of that table (0 otherwise) */
    size_t total;          /* == fused_moe_workspace_bytes_ex() */
    size_t sched;          /* tile kernels (MOE_PATH_PREFILL): the same meta[1]
                              chunks again, moe_chunk [max_chunks], in order of
                              non-increasing nrows -- the order the workgroups
                              take them in, so the largest start first (chunks
                              of one size in no fixed order); SIZE_MAX on the
                              decode path, which has no such list */
} moe_workspace_layout;

/* Host-only: fills *layout for the call fused_moe_ex(wdtype, ..., T, H, I, E,
 * k, shared ? ... : NULL, ..., opt) would make.  MOE_ERR_ARG for a shape the
 * fused layer rejects or a NULL layout. */
moe_status fused_moe_workspace_layout(moe_wdtype wdtype, int T, int H, int I, int E, int k,
                                      int has_shared, const moe_options* opt,
                                      moe_workspace_layout* layout);

moe_status fused_moe_bf16(const uint16_t* x, const uint16_t* w13, const uint16_t* w2,
                          const float* topk_weights, const int32_t* topk_ids, int T, int H, int I,
                          int E, int k, const moe_dense_expert* shared, void* ws, size_t ws_bytes,
                          uint16_t* out, hipStream_t stream);

moe_status fused_moe_fp8(const uint16_t* x, const uint8_t* w13, const float* w13_scale,
                         const uint8_t* w2, const float* w2_scale, const float* topk_weights,
                         const int32_t* topk_ids, int T, int H, int I, int E, int k,
                         const moe_dense_expert* shared, void* ws, size_t ws_bytes, uint16_t* out,
                         hipStream_t stream);

moe_status fused_moe_int8(const uint16_t* x, const int8_t* w13, const float* w13_scale,
                          const int8_t* w2, const float* w2_scale, const float* topk_weights,
                          const int32_t* topk_ids, int T, int H, int I, int E, int k,
                          const moe_dense_expert* shared, void* ws, size_t ws_bytes,
                          uint16_t* out, hipStream_t stream);

/* INT4 weight-only layer ([osdi] "CPU 解码后端" and [notes] 06 后续工作: INT4
 * weights for decode; the pages fix no layout).  Codes are signed 4-bit,
 * w13 logical [E, H, I] bytes and w2 [E, I, H/2] bytes (two codes per byte
 * along N, packed with moe_prepack_int4); scales fp32 per output column and
 * 128-row K group: w13_scale [E, H/128, 2I], w2_scale [E, I/128, H]; the
 * weight is code * scale, activations stay bf16.  Runs on the decode
 * (weight-streaming) kernels whatever T is: forcing MOE_PATH_PREFILL returns
 * MOE_ERR_UNSUPPORTED. */
moe_status fused_moe_int4(const uint16_t* x, const uint8_t* w13, const float* w13_scale,
                          const uint8_t* w2, const float* w2_scale, const float* topk_weights,
                          const int32_t* topk_ids, int T, int H, int I, int E, int k,
                          const moe_dense_expert* shared, void* ws, size_t ws_bytes,
                          uint16_t* out, hipStream_t stream);

/* Same layer with an explicit dtype and options (opt may be NULL = defaults). */
moe_status fused_moe_ex(moe_wdtype wdtype, const uint16_t* x, const void* w13,
                        const float* w13_scale, const void* w2, const float* w2_scale,
                        const float* topk_weights, const int32_t* topk_ids, int T, int H, int I,
                        int E, int k, const moe_dense_expert* shared, void* ws, size_t ws_bytes,
                        uint16_t* out, const moe_options* opt, hipStream_t stream);

/* Router and fused layer in one call: the same results as moe_topk(logits,
 * T, E, k, score, renormalize, topk_weights, topk_ids) followed by
 * fused_moe_ex(wdtype, x, ..., topk_weights, topk_ids, ...) -- topk_weights
 * and topk_ids are written exactly as moe_topk writes them, out exactly as
 * fused_moe_ex writes it -- on the same workspace
 * (fused_moe_workspace_bytes_ex).  For T <= 16 the top-k and the expert
 * alignment run in one workgroup that keeps the ids in shared memory, so
 * they do not make a round trip through device memory between two kernels;
 * larger T run the two steps as separate kernels.  ([blog] "MoE": the gating
 * top-k is the input of the per-expert grouping.)
 * logits fp32 [T, E]; score and renormalize as for moe_topk; every other
 * argument and limit as for fused_moe_ex (E <= 1023). */
moe_status fused_moe_routed(moe_wdtype wdtype, const float* logits, moe_score score,
                            int renormalize, const uint16_t* x, const void* w13,
                            const float* w13_scale, const void* w2, const float* w2_scale,
                            float* topk_weights, int32_t* topk_ids, int T, int H, int I, int E,
                            int k, const moe_dense_expert* shared, void* ws, size_t ws_bytes,
                            uint16_t* out, const moe_options* opt, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * The same routed layer for callers that cannot allocate device memory at
 * all (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): no workspace argument.  The workspace is a file-scope
 * device array of MOE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU,
 * held until the process ends; its address on the current device is looked
 * up once (hipGetSymbolAddress) on the first call made with that device
 * current.  The call itself allocates nothing and creates no HIP objects
 * (per-kernel profiling events are skipped).
 * Every other argument, limit and result is that of fused_moe_routed (the
 * outputs are bit-identical to it).  The stream must belong to the current
 * device.  A batch whose workspace (fused_moe_workspace_bytes_ex with the
 * same options) exceeds MOE_NOALLOC_SCRATCH_BYTES returns
 * MOE_ERR_UNSUPPORTED before anything is enqueued; 64 MiB covers the
 * decode-sized batches (e.g. T <= 64 at hidden 7168, 256 experts, top-8).
 * All calls on one GPU share its array: calls whose work overlaps on that
 * GPU (other streams, other threads) race on it and must be serialised by
 * the caller.  Nothing in the array needs to start at zero.
 * ------------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status fused_moe_routed_noalloc(moe_wdtype wdtype, const float* logits, moe_score score,
                                    int renormalize, const uint16_t* x, const void* w13,
                                    const float* w13_scale, const void* w2, const float* w2_scale,
                                    float* topk_weights, int32_t* topk_ids, int T, int H, int I,
                                    int E, int k, const moe_dense_expert* shared, uint16_t* out,
                                    const moe_options* opt, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * FP8 block dequantisation with the library's own converters ([osdi] "CPU
 * decode backend": E4M3FN codes with 128-element-block scales).
 * codes uint8 [K, N] E4M3FN; scale fp32 [K/128, N/128] or NULL (= 1);
 * out fp32 [K, N].
 *   mode 0: value(code) * scale, code widened exactly (the converter the
 *           decode kernels use; the scale multiply is done here in fp32);
 *   mode 1: bf16(value(code) * scale), rounded once to nearest even (a
 *           dequantise-to-bf16 converter; no fused kernel uses it: the FP8
 *           tile kernels multiply the raw codes on the FP8 matrix cores).
 * Limits: K*N % 4 == 0; with scales, K and N multiples of 128.
 * ------------------------------------------------------------------------- */
moe_status moe_dequant_fp8(const uint8_t* codes, const float* scale, int K, int N, int mode,
                           float* out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Per-kernel timing (measurement support, off by default).
 * While enabled, every kernel the library launches is bracketed by hipEvents
 * recorded on its stream.  moe_profile_collect() waits for those events,
 * adds each kernel's elapsed time to per-stage totals (host arrays of
 * length max_stages: total ms and launch count) and forgets them; it returns
 * the number of stages.  moe_profile_stage_name(i) names stage i (host).
 * ------------------------------------------------------------------------- */
moe_status moe_profile_enable(int on);
int moe_profile_collect(double* total_ms, int64_t* launches, int max_stages);
const char* moe_profile_stage_name(int stage);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
