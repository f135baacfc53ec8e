// moe_decode.hip -- weight-streaming grouped GEMMs for few rows per expert
// (decode), and the top-k-weighted combine.
//
// Each wave owns one column block of one expert (GEMM1: a gate tile and the
// matching up tile, so SiLU(C1)*C2 is lane-local; GEMM2: one output tile for
// INT8, two otherwise) and streams that block's packed weights over its K
// range with 16-byte coalesced loads, one 128-row K block ahead.  The
// activations of the chunk's rows (<= 16*MB) come straight from L2 through
// buffer loads; a padding row's lanes use an offset past the end of the
// tensor, which returns zeros without a memory access.  FP8 codes are
// widened to bf16 in registers (exact) and each 128x128 block's scale is
// applied to the block's partial sums after the MFMAs (post-scaling).  INT8
// runs the i8 MFMA with int32 accumulation and applies activation and channel
// scales once at the end.  INT4 (weight-only) streams one 16-byte load per
// lane per 128-row K block (half of FP8's bytes), turns the biased codes into
// bf16 fragments of 136 + q with one AND-OR per pair, removes the 136 with one
// product per K block against a constant fragment (shared by the wave's
// tiles) and applies the per-column group scales to each block's sums.
//
// GEMM1 may split K across workgroups (when few experts are active); the
// splits' raw partial sums go to the workspace and a small reduction kernel
// adds them in split order and runs the SiLU epilogue.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

template <int WT>
struct WT_ {
    static constexpr int EB = WT == W_BF16 ? 2 : 1;   // weight element bytes (INT4: see packed_i4_offset)
    static constexpr int BV = WT == W_BF16 ? 2 : 1;   // u32x4 per lane per k-tile (weights; INT4: per K block)
    static constexpr int AEB = WT == W_INT8 ? 1 : 2;  // activation element bytes
    static constexpr int AV = WT == W_INT8 ? 1 : 2;   // u32x4 per lane per k-tile (activations)
    typedef typename std::conditional<WT == W_INT8, i32x4, f32x4>::type Acc;
};

// One k-tile (64 rows of K) contribution of a weight fragment `b` and an
// activation fragment `av` to accumulator `c`.
template <int WT>
__device__ inline void mma_ktile(const u32x4 (&av)[WT_<WT>::AV], const bf16x8& b0,
                                 const bf16x8& b1, const u32x4& bi8,
                                 typename WT_<WT>::Acc& c) {
    if constexpr (WT == W_INT8) {
        c = mfma_i8(av[0], bi8, c);
    } else {
        c = mfma_bf16(__builtin_bit_cast(bf16x8, av[0]), b0, c);
        c = mfma_bf16(__builtin_bit_cast(bf16x8, av[1]), b1, c);
    }
}

// Turn a raw weight fragment (one k-tile) into MFMA B operands.
template <int WT>
__device__ inline void b_frags(const u32x4 (&raw)[WT_<WT>::BV], bf16x8& b0, bf16x8& b1) {
    if constexpr (WT == W_FP8) {
        fp8x16_to_frags(raw[0], b0, b1);
    } else if constexpr (WT == W_BF16) {
        b0 = __builtin_bit_cast(bf16x8, raw[0]);
        b1 = __builtin_bit_cast(bf16x8, raw[1]);
    }
}

// Weight-ring depth: K blocks of weights in flight per wave (D-1 ahead of the
// one being multiplied).  Two stages for every type (tiny INT8 batches: see
// tiny_depth): once every stage issues
// the same loads (so the waits are exact), a third stage only cost occupancy
// (fewer resident waves), which measured slower for FP8 and for INT8; INT4,
// whose stage is half as many bytes, measured the same with three stages
// and slower with four.
template <int WT, int MB>
struct Depth {
    static constexpr int D = 2;
};

// The INT8 kernels of tiny batches (top-k in GEMM1's prologue) run so few
// waves -- at T = 1 one per SIMD or less -- that occupancy costs nothing and
// the weight bytes each wave keeps in flight set the stream's rate: four
// stages there (at T = 1, 38.0 -> 36.7 us per layer; the same depth for the
// larger INT8 decode batches, many waves per SIMD, was slower).
template <int WT>
constexpr int tiny_depth() { return WT == W_INT8 ? 4 : Depth<WT, 1>::D; }
// The fused GEMM2 + combine of INT8 tiny batches: its prologue (the rows'
// quantisation) takes longer than a weight round trip, so eight stages go
// out before it (T = 1: 35.3 -> 34.9 us per layer; thirteen, a whole
// 1536-deep tile, no better)
constexpr int kCombDepth = 8;

template <int WT, int MB, int NT, int DD = Depth<WT, MB>::D>
struct DecodeTile {
    using T = WT_<WT>;
    using Acc = typename T::Acc;
    static constexpr int D = DD;
    static constexpr int KT = WT == W_INT4 ? 1 : 2;  // weight loads per K block (INT4: both k-tiles in one)
    u32x4 bq[D][NT][KT][T::BV];    // weights [stage][tile][k-tile][vec]
    float sq[D][NT];               // FP8 block scales / INT4 per-lane column scales of the staged blocks
    u32x4 aq[2][MB][2][T::AV];     // activations (from L2, one block ahead) [stage][row block][k-tile][vec]
    Acc acc[MB][NT];
};

// A padding row's byte offset into the activation tensor: past its end, so a
// buffer load returns zeros without touching memory (a_bytes < 2^31 is
// checked on the host).
constexpr uint32_t kAPastEnd = 0x7fffffffu;

// One weight stage: K block kb of the NT tiles into ring slot buf.  A weight
// block's FP8 / INT4 scales are loaded with it (scalar loads: not in the
// vector-memory queue, so waiting for them never waits for the weight blocks
// issued after them).
template <int WT, int MB, int NT, int DD, typename ScaleFn>
__device__ inline void stream_load_b(DecodeTile<WT, MB, NT, DD>& st, const uint8_t* const (&bptr)[NT], int kb,
                                     int buf, ScaleFn& scale) {
    using T = WT_<WT>;
    constexpr size_t kt_bytes = 64 * 16 * T::EB;
    if constexpr (WT == W_INT4) {
#pragma unroll
        for (int n = 0; n < NT; ++n) st.bq[buf][n][0][0] = ldg16_nt(bptr[n] + (size_t)kb * 1024);
    } else {
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int v = 0; v < T::BV; ++v)
                    st.bq[buf][n][kt][v] = ldg16_nt(bptr[n] + (size_t)(kb * 2 + kt) * kt_bytes + v * 16);
    }
    if constexpr (WT == W_FP8 || WT == W_INT4) {
#pragma unroll
        for (int n = 0; n < NT; ++n) st.sq[buf][n] = scale(n, kb);
    }
}

// The first D-1 weight stages of decode_stream<..., PRE = true>, issued
// early (before a prologue that does not touch the ring).  Every stage is
// requested, past the range as the range's last block again (never used):
// with a fixed number of loads in flight the prologue's own waits count
// exactly, instead of waiting for every load.
template <int WT, int MB, int NT, int DD, typename ScaleFn>
__device__ inline void stream_prefetch(DecodeTile<WT, MB, NT, DD>& st, const uint8_t* const (&bptr)[NT], int kb0,
                                       int kb1, ScaleFn scale) {
    constexpr int D = DD;
#pragma unroll
    for (int d = 0; d < D - 1; ++d) stream_load_b<WT, MB, NT>(st, bptr, max(min(kb0 + d, kb1 - 1), 0), d, scale);
}

// Streams K blocks [kb0, kb1) of NT column tiles for MB row blocks: weights
// through a ring of D stages (the loads of block kb+D-1 go out before block kb
// is multiplied), activation rows one block ahead.
//   bptr[n]  : this lane's byte pointer into tile n at k-tile 0
//   aoff[rb] : this lane's byte offset of its activation row (plus its
//              16-byte column piece) in abase; kAPastEnd = padding row
//   abase, a_bytes : the whole activation tensor (a_bytes < 2^31), or with
//              ALDS an LDS array holding K blocks [kb0, kb1) of every row
//              (rows of (kb1 - kb0) * 128 elements), padding rows pointing at
//              a zero row
//   scale(n, kb) : FP8 block scale of tile n at K block kb
//   PRE          : the first D-1 weight stages were issued by stream_prefetch
// FP8 partial sums of a 128-row block are scaled once.
template <int WT, int MB, int NT, bool ALDS, bool PRE, int DD, typename ScaleFn>
__device__ inline void decode_stream(DecodeTile<WT, MB, NT, DD>& st, const uint8_t* const (&bptr)[NT],
                                     const uint32_t (&aoff)[MB], const char* abase,
                                     int64_t a_bytes, int kb0, int kb1, ScaleFn scale) {
    using T = WT_<WT>;
    using Acc = typename T::Acc;
    constexpr int D = DD;
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int n = 0; n < NT; ++n) st.acc[rb][n] = Acc{0, 0, 0, 0};

    // Every stage of the steady loop issues the same loads, unconditionally:
    // the compiler then knows exactly how many loads are younger than the
    // ones a multiply needs and waits for those only (a load that may or may
    // not have been issued forces it to wait for everything).  Activation
    // rows are read with buffer loads over the A tensor: a padding lane's
    // offset lies past the tensor, so its load returns zeros without any
    // memory traffic (most rows of a decode chunk are padding).
    const __amdgpu_buffer_rsrc_t arsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)abase, (short)0, (int)a_bytes, 0x00020000);

    auto load_b = [&](int kb, int buf) { stream_load_b<WT, MB, NT>(st, bptr, kb, buf, scale); };
    auto load_a = [&](int kb, int buf) {
#pragma unroll
        for (int rb = 0; rb < MB; ++rb)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int v = 0; v < T::AV; ++v) {
                    if constexpr (ALDS) {
                        st.aq[buf][rb][kt][v] = *reinterpret_cast<const u32x4*>(
                            abase + aoff[rb] + (uint32_t)(((kb - kb0) * 128 + kt * 64) * T::AEB) +
                            (WT == W_INT8 ? 0u : (uint32_t)(v * 64)));
                    } else {
                        const uint32_t off = (uint32_t)((kb * 128 + kt * 64) * T::AEB) +
                                             (WT == W_INT8 ? 0u : (uint32_t)(v * 64));
                        st.aq[buf][rb][kt][v] = __builtin_bit_cast(
                            u32x4, __builtin_amdgcn_raw_buffer_load_b128(arsrc, aoff[rb] + off, 0, 0));
                    }
                }
    };

    auto compute = [&](int kb, int buf, int abuf) {
        (void)kb;
        // all weight fragments of the block are widened first, then the MFMAs
        // issue back to back (VALU and MFMA of one wave do not overlap)
        bf16x8 b0[NT][2], b1[NT][2];
        if constexpr (WT == W_INT4) {
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const u32x4 w = st.bq[buf][n][0][0];
                b0[n][0] = int4x8_to_frag_biased(w.x);
                b1[n][0] = int4x8_to_frag_biased(w.y);
                b0[n][1] = int4x8_to_frag_biased(w.z);
                b1[n][1] = int4x8_to_frag_biased(w.w);
            }
        } else if constexpr (WT != W_INT8) {
#pragma unroll
            for (int n = 0; n < NT; ++n)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) b_frags<WT>(st.bq[buf][n][kt], b0[n][kt], b1[n][kt]);
        }
        // every row block is multiplied, live or not: no branch between the
        // MFMAs (a branch there made the compiler move accumulators between
        // register files at block edges, and one such copy read an MFMA result
        // before its latency had passed).  Row blocks past the chunk hold a
        // valid row's data and their sums are never stored.
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) {
            // INT4: the rows' sums against -136 (every column alike), once per
            // K block; each tile's sums start from it
            f32x4 corr = {0, 0, 0, 0};
            if constexpr (WT == W_INT4) {
                const bf16x8 cneg = __builtin_bit_cast(
                    bf16x8, u32x4{kBf16Minus136x2, kBf16Minus136x2, kBf16Minus136x2, kBf16Minus136x2});
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    corr = mfma_bf16(__builtin_bit_cast(bf16x8, st.aq[abuf][rb][kt][0]), cneg, corr);
                    corr = mfma_bf16(__builtin_bit_cast(bf16x8, st.aq[abuf][rb][kt][1]), cneg, corr);
                }
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                if constexpr (WT == W_INT4) {
                    f32x4 tmp = corr;
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt) {
                        tmp = mfma_bf16(__builtin_bit_cast(bf16x8, st.aq[abuf][rb][kt][0]), b0[n][kt], tmp);
                        tmp = mfma_bf16(__builtin_bit_cast(bf16x8, st.aq[abuf][rb][kt][1]), b1[n][kt], tmp);
                    }
                    st.acc[rb][n] += st.sq[buf][n] * tmp;
                } else if constexpr (WT == W_FP8) {
                    f32x4 tmp = {0, 0, 0, 0};
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
                        mma_ktile<WT>(st.aq[abuf][rb][kt], b0[n][kt], b1[n][kt],
                                      st.bq[buf][n][kt][0], tmp);
                    st.acc[rb][n] += st.sq[buf][n] * tmp;
                } else {
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
                        mma_ktile<WT>(st.aq[abuf][rb][kt], b0[n][kt], b1[n][kt],
                                      st.bq[buf][n][kt][0], st.acc[rb][n]);
                }
            }
        }
    };

    // Loads of a stage go out activations first: VMEM loads complete in
    // order, so waiting for a stage's activations then does not also wait for
    // the weight blocks issued after them.
    if (kb0 >= kb1) return;
    constexpr int UF = D % 2 == 0 ? D : 2 * D;  // unroll: both ring indices static
    load_a(kb0, 0);
    if constexpr (!PRE) {
#pragma unroll
        for (int d = 0; d < D - 1; ++d)
            if (kb0 + d < kb1) load_b(kb0 + d, d);
    }
    int kb = kb0;
    // steady state: stage k issues A(k+1) and B(k+D-1), both inside [kb0, kb1)
    const int steady_end = kb1 - (D - 1);
    for (; kb + UF <= steady_end; kb += UF) {
#pragma unroll
        for (int d = 0; d < UF; ++d) {
            const int k = kb + d;
            load_a(k + 1, (d + 1) % 2);
            load_b(k + D - 1, (d + D - 1) % D);
            compute(k, d % D, d % 2);
        }
    }
    // the last stages (fewer than UF + D - 1): loads only while in range
    for (; kb < kb1; kb += UF) {
#pragma unroll
        for (int d = 0; d < UF; ++d) {
            const int k = kb + d;
            if (k >= kb1) break;
            if (k + 1 < kb1) load_a(k + 1, (d + 1) % 2);
            if (k + D - 1 < kb1) load_b(k + D - 1, (d + D - 1) % D);
            compute(k, d % D, d % 2);
        }
    }
}

__device__ inline int pair_token(int pid, int P, int topk) { return pid < P ? pid / topk : pid - P; }

// ---------------------------------------------------------------------------
// GEMM1: act[row, :] = SiLU(A W13[:, gate]) * (A W13[:, up]), one pair tile per wave
// ---------------------------------------------------------------------------
// INT4 with one row block: four waves per SIMD (its registers fit 128 with
// the compiler asked to; left alone it took 136 and three waves)
template <int WT, int MB>
constexpr int dec_waves_per_eu() { return WT == W_INT4 && MB == 1 ? 4 : 1; }

// One wave's GEMM1 work on chunk `ch` (pair tile pt, split `split`) once the
// chunk's rows are known: stream the K range, then publish the split's raw
// partial sums or the SiLU(gate) * up rows.
//   pid_of(r)   : pair of row r of the chunk (>= P_tot: padding row)
//   aoff_of(pid): the row's activation offset for decode_stream (padding:
//                 kAPastEnd, or the zero row with ALDS)
//   xscale_of(t): INT8 scale of token t
//   prologue()  : runs after the weight setup; with PRE the first weight
//                 stages are already in flight while it runs (the row
//                 accessors are called only after it)
template <int WT, int MB, bool ALDS, bool PRE, int DD, typename PidFn, typename AoffFn, typename XsFn,
          typename ProFn>
__device__ inline void gemm1_tile(const GemmArgs& a, const Chunk& ch, int pt, int split, int lane,
                                  const char* abase, PidFn pid_of, AoffFn aoff_of, XsFn xscale_of,
                                  ProFn prologue) {
    using T = WT_<WT>;
    const int g = lane >> 4, c16 = lane & 15;
    const int I = a.N >> 1;
    const bool sh = ch.expert >= a.E;
    const size_t wbytes = WT == W_INT4 ? (size_t)a.K * a.N / 2 : (size_t)a.K * a.N * T::EB;
    const uint8_t* W = sh ? a.W_sh : a.W + (size_t)ch.expert * wbytes;
    const int nsc = WT == W_FP8 ? (a.K / 128) * (a.N / 128) : (WT == W_INT4 ? (a.K / 128) * a.N : a.N);
    const float* ws = sh ? a.w_scale_sh : (a.w_scale ? a.w_scale + (size_t)ch.expert * nsc : nullptr);

    const uint8_t* bptr[2];
    if constexpr (WT == W_INT4) {
        bptr[0] = W + packed_i4_offset(a.K, 2 * pt, 0) + lane * 16;
        bptr[1] = W + packed_i4_offset(a.K, 2 * pt + 1, 0) + lane * 16;
    } else {
        bptr[0] = W + packed_tile_offset(T::EB, a.K, 2 * pt, 0) + lane * 16 * T::EB;
        bptr[1] = W + packed_tile_offset(T::EB, a.K, 2 * pt + 1, 0) + lane * 16 * T::EB;
    }
    const int nrb = ch.nrows >> 4;
    const int nkb = a.K / 128;
    const int kb0 = split * a.kb_per_split;
    const int kb1 = min(nkb, kb0 + a.kb_per_split);
    const int nb_g = (pt * 16) / 128, nb_u = (I + pt * 16) / 128, nbw = a.N / 128;
    auto scale = [&](int n, int kb) {
        if constexpr (WT == W_INT4)  // this lane's column of the gate (n = 0) or up tile
            return ws[(size_t)kb * a.N + (n ? I : 0) + pt * 16 + c16];
        else
            return ws[kb * nbw + (n ? nb_u : nb_g)];
    };
    DecodeTile<WT, MB, 2, DD> st;
    if constexpr (PRE) stream_prefetch<WT, MB, 2>(st, bptr, kb0, kb1, scale);
    prologue();
    uint32_t aoff[MB];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) aoff[rb] = aoff_of(rb < nrb ? pid_of(rb * 16 + c16) : a.P_tot);
    decode_stream<WT, MB, 2, ALDS, PRE>(st, bptr, aoff, abase, a.a_bytes, kb0, kb1, scale);

    if (a.splits > 1) {
        // publish this split's raw partial sums (fp32, or int32 for INT8); the
        // split-reduce kernel adds the splits in split order and runs the SiLU
        // epilogue (no cross-workgroup synchronisation inside this kernel)
        using Elem = typename std::conditional<WT == W_INT8, int, float>::type;
        Elem* part = reinterpret_cast<Elem*>(a.partial);
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) {
            if (rb < nrb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = ch.row_start + rb * 16 + 4 * g + i;
                    Elem* p = part + ((size_t)split * a.cap + row) * a.N;
                    const Elem gv = st.acc[rb][0][i];
                    const Elem uv = st.acc[rb][1][i];
                    p[pt * 16 + c16] = gv;
                    p[I + pt * 16 + c16] = uv;
                }
            }
        }
        return;
    }

    uint16_t* act = (uint16_t*)a.out;
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
        if (rb < nrb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = ch.row_start + rb * 16 + 4 * g + i;
                const int pid = pid_of(rb * 16 + 4 * g + i);
                if (pid >= a.P_tot) continue;
                float gv, uv;
                if constexpr (WT == W_INT8) {
                    const float sx = xscale_of(pair_token(pid, a.P, a.topk));
                    gv = (float)st.acc[rb][0][i] * sx * ws[pt * 16 + c16];
                    uv = (float)st.acc[rb][1][i] * sx * ws[I + pt * 16 + c16];
                } else {
                    gv = st.acc[rb][0][i];
                    uv = st.acc[rb][1][i];
                }
                act[(size_t)row * I + pt * 16 + c16] = f32_to_bf16_bits(silu(gv) * uv);
            }
        }
    }
}

template <int WT, int MB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(dec_waves_per_eu<WT, MB>())))
void decode_gemm1_kernel(GemmArgs a) {
    using T = WT_<WT>;
    // the wave index is uniform: from readfirstlane the compiler knows it, so
    // per-wave addresses (weight tiles, block scales) stay scalar
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int bid = blockIdx.x;
    const int split = bid % a.splits;
    bid /= a.splits;
    const int grp = bid % a.n_groups;
    const int ci = bid / a.n_groups;
    // slot and chunk count in one round trip (ci < the list's capacity)
    const int nchunks = a.meta[1];
    const Chunk ch = a.chunks[ci];
    if (ci >= nchunks) return;
    const int pt = grp * kDecodeWavesPerWG + wv;
    if (pt >= (a.N >> 1) / 16) return;
    const uint32_t g16 = (uint32_t)((lane >> 4) * 16);
    gemm1_tile<WT, MB, false, false, Depth<WT, MB>::D>(
        a, ch, pt, split, lane, (const char*)a.A,
        [&](int r) { return a.sorted_ids[ch.row_start + r]; },
        [&](int pid) {
            return pid < a.P_tot ? (uint32_t)pair_token(pid, a.P, a.topk) * (uint32_t)(a.K * T::AEB) + g16
                                 : kAPastEnd;
        },
        [&](int t) { return a.a_scale[t]; }, [] {});
}

// ---------------------------------------------------------------------------
// GEMM1 for tiny batches, with the routing in its prologue.
//
// With at most kTinyMaxT tokens an expert holds at most that many pairs, so
// the alignment is one 16-row block per routed expert -- a fixed-capacity
// block per expert with a mask of live rows -- and every workgroup can build
// it from the T*k ids in a few wave operations instead of reading it from a
// separate alignment launch.  Every workgroup therefore:
//   1. runs the router top-k of the T tokens (wave t takes token t; or reads
//      the given ids) and, for INT8, quantises the token rows: the row
//      maxima over all four waves, then the codes of its split's K range into
//      LDS (the same arithmetic as quant_row, so the same codes);
//   2. ranks the distinct experts (ascending id, the shared expert E last):
//      lane l holds pair l, lanes of one expert are found with a ballot per id
//      bit, an expert's rank is the number of distinct smaller ids, and a
//      pair's row inside its block the number of earlier pairs of its expert;
//   3. takes block ci = its slot, exits if there is none, and streams that
//      expert's weights exactly as decode_gemm1_kernel does.
// Workgroup 0 also publishes everything later kernels and the caller read:
// the top-k weights and ids, sorted_ids[0, npp), meta and the chunk list
// (the values the alignment kernel writes: chunk c = block c, 16 rows) and,
// for INT8, every token code and scale.
// ---------------------------------------------------------------------------
template <int WT, int VPL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(dec_waves_per_eu<WT, 1>())))
void decode_gemm1_tiny_kernel(GemmArgs a, TinyRoute r) {
    using T = WT_<WT>;
    extern __shared__ __attribute__((aligned(16))) char xq_l[];  // INT8: (T + 1) rows of the split's codes
    __shared__ int ids_l[kTinyMaxPairs];
    __shared__ int pid_l[16];
    __shared__ int exp_l[kTinyMaxPairs], cnt_l[kTinyMaxPairs];
    __shared__ uint32_t bm_l[kTinyMaxE / 32 + 1];  // experts present (E_tot <= kTinyMaxE + 1 bits)
    __shared__ int blk_l[2];                       // this slot's expert (-1: none), distinct experts
    __shared__ float amax_l[kDecodeWavesPerWG][kTinyMaxT];
    __shared__ float xs_l[kTinyMaxT];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bid = blockIdx.x;
    const int split = bid % a.splits;
    bid /= a.splits;
    const int grp = bid % a.n_groups;
    const int ci = bid / a.n_groups;
    const bool pub = blockIdx.x == 0;
    const int nT = r.T, K = a.K;
    const int kb0 = split * a.kb_per_split;
    const int kb1 = min(K / 128, kb0 + a.kb_per_split);
    const int span = (kb1 - kb0) * 128;  // INT8 codes per row held in LDS
    if (tid <= kTinyMaxE / 32) bm_l[tid] = 0u;

    // 1. INT8: the token rows' loads go out first (piece j = 8 elements of
    // the [T, K] rows; thread tid takes j = tid + 256 i)
    constexpr int NPC = WT == W_INT8 ? kTinyMaxElems / 8 / 256 : 1;
    const int pieces = nT * (K / 8);
    u32x4 xv[NPC];
    if constexpr (WT == W_INT8) {
#pragma unroll
        for (int i = 0; i < NPC; ++i) {
            const int j = tid + 256 * i;
            xv[i] = j < pieces ? ldg16(r.x + (size_t)j * 8) : u32x4{0, 0, 0, 0};
        }
    }
    if (wv < nT) {
        if constexpr (VPL > 0)
            topk_token<VPL>(r.logits, wv, a.E, r.k, r.score, r.renorm, pub ? r.w_out : nullptr,
                            pub ? r.id_out : nullptr, ids_l, lane);
        else if (lane < r.k)
            ids_l[wv * r.k + lane] = r.ids[wv * r.k + lane];
    }
    if constexpr (WT == W_INT8) {
        float am[kTinyMaxT];
#pragma unroll
        for (int t = 0; t < kTinyMaxT; ++t) am[t] = 0.f;
#pragma unroll
        for (int i = 0; i < NPC; ++i) {
            const int j = tid + 256 * i;
            float m = 0.f;
            const uint32_t w4[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                m = fmaxf(m, fabsf(bf16_bits_to_f32((uint16_t)(w4[q] & 0xffff))));
                m = fmaxf(m, fabsf(bf16_bits_to_f32((uint16_t)(w4[q] >> 16))));
            }
            const int t = j / (K / 8);  // >= T past the rows: matches no token
#pragma unroll
            for (int tt = 0; tt < kTinyMaxT; ++tt) am[tt] = t == tt ? fmaxf(am[tt], m) : am[tt];
        }
#pragma unroll
        for (int tt = 0; tt < kTinyMaxT; ++tt) {
            if (tt < nT) {  // uniform
                const float v = wave_max(am[tt]);
                if (lane == 0) amax_l[wv][tt] = v;
            }
        }
    }
    __syncthreads();  // ids_l, amax_l, bm_l

    // 2. the alignment, by wave 0: lane l holds pair l.  An expert's rank is
    // the number of distinct smaller ids (a bitmap of the experts present,
    // counted below the id), a pair's row the number of earlier pairs of its
    // expert (lanes holding the same id: one ballot per id bit).
    const int P = a.P, P_tot = a.P_tot, E = a.E;
    if (wv == 0) {
        int e = -1;
        if (lane < P_tot) e = lane < P ? ids_l[lane] : E;
        const bool valid = lane < P_tot && (lane >= P || (e >= 0 && e < E));
        if (valid) atomicOr(&bm_l[e >> 5], 1u << (e & 31));
        const uint64_t peers = match_any(e, valid, 32 - __clz(E));
        const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
        const bool first = valid && (peers & below) == 0;
        const int row = __popcll(peers & below);
        int rank = 0, nd = 0;
        const int ew = valid ? e >> 5 : -1;
#pragma unroll
        for (int w = 0; w <= kTinyMaxE / 32; ++w) {
            const uint32_t word = bm_l[w];
            nd += __popc(word);
            rank += w < ew ? __popc(word) : (w == ew ? __popc(word & ((1u << (e & 31)) - 1u)) : 0);
        }
        const bool mine = valid && rank == ci;
        if (lane < 16) pid_l[lane] = P_tot;  // padding rows, then the block's pairs
        if (lane == 0) {
            blk_l[0] = -1;
            blk_l[1] = nd;
        }
        if (mine) pid_l[row] = lane;
        if (mine && row == 0) blk_l[0] = e;
        if (pub) {
            if (first) {
                exp_l[rank] = e;
                cnt_l[rank] = __popcll(peers);
            }
            if (valid) r.sorted_ids[16 * rank + row] = lane;
            for (int p = lane; p < 16 * nd; p += 64)
                if ((p & 15) >= cnt_l[p >> 4]) r.sorted_ids[p] = P_tot;
            if (lane < nd) r.chunks[lane] = Chunk{exp_l[lane], 16 * lane, 16, cnt_l[lane]};  // pad: live rows
            if (lane == 0) {
                r.meta[0] = 16 * nd;
                r.meta[1] = nd;
            }
        }
    }
    __syncthreads();  // pid_l, blk_l
    const int expert = blk_l[0];
    // INT8: the token codes of this split's K range to LDS (and, workgroup 0,
    // every code and scale to the workspace); run while the first weight
    // stage is in flight
    auto quant_rows = [&]() {
        if constexpr (WT == W_INT8) {
            float sc[kTinyMaxT], rc[kTinyMaxT];
#pragma unroll
            for (int tt = 0; tt < kTinyMaxT; ++tt) {
                sc[tt] = __fdiv_rn(fmaxf(fmaxf(amax_l[0][tt], amax_l[1][tt]), fmaxf(amax_l[2][tt], amax_l[3][tt])),
                                   127.0f);
                rc[tt] = quant_recip(sc[tt]);
            }
            if (tid < nT) {
                float v = sc[0];
#pragma unroll
                for (int tt = 1; tt < kTinyMaxT; ++tt) v = tid == tt ? sc[tt] : v;
                xs_l[tid] = v;
                if (pub) r.xs_out[tid] = v;
            }
            const int lo = kb0 * 128, hi = kb1 * 128;
#pragma unroll
            for (int i = 0; i < NPC; ++i) {
                const int j = tid + 256 * i;
                if (j < pieces) {
                    const int t = j / (K / 8), c = (j % (K / 8)) * 8;
                    float s = sc[0], rs = rc[0];
#pragma unroll
                    for (int tt = 1; tt < kTinyMaxT; ++tt) {
                        s = t == tt ? sc[tt] : s;
                        rs = t == tt ? rc[tt] : rs;
                    }
                    const bool in = c >= lo && c < hi;
                    if (in || pub) {
                        const uint2 q = quant8(xv[i], s, rs);
                        if (in) *reinterpret_cast<uint2*>(xq_l + t * span + (c - lo)) = q;
                        if (pub) *reinterpret_cast<uint2*>(r.xq_out + (size_t)j * 8) = q;
                    }
                }
                // one piece's divisions at a time (interleaving them all spills)
                __builtin_amdgcn_sched_barrier(0);
            }
            for (int o = tid * 16; o < span; o += 256 * 16)  // the zero row of padding lanes
                *reinterpret_cast<u32x4*>(xq_l + nT * span + o) = u32x4{0, 0, 0, 0};
            __syncthreads();  // xq_l, xs_l
        }
    };
    if (expert < 0) {  // no expert for this slot (uniform)
        if (pub) quant_rows();
        return;
    }
    const Chunk ch{expert, 16 * ci, 16, 0};

    // 3. the block's GEMM1 tile (waves past tiles_per_wg stream nothing)
    const int tpw = r.tiles_per_wg;
    const int pt = wv < tpw ? grp * tpw + wv : (a.N >> 1) / 16;
    const uint32_t g16 = (uint32_t)((lane >> 4) * 16);
    auto pid_of = [&](int rr) { return pid_l[rr]; };
    auto xscale_of = [&](int t) { return xs_l[t]; };
    if constexpr (WT == W_INT8) {
        if (pt >= (a.N >> 1) / 16) {  // no columns for this wave: its share of the codes only
            quant_rows();
            return;
        }
        gemm1_tile<WT, 1, true, true, tiny_depth<WT>()>(
            a, ch, pt, split, lane, xq_l, pid_of,
            [&](int pid) {
                return (uint32_t)((pid < P_tot ? pair_token(pid, P, a.topk) : nT) * span) + g16;
            },
            xscale_of, quant_rows);
    } else {
        if (pt >= (a.N >> 1) / 16) return;
        gemm1_tile<WT, 1, false, false, Depth<WT, 1>::D>(
            a, ch, pt, split, lane, (const char*)a.A, pid_of,
            [&](int pid) {
                return pid < P_tot ? (uint32_t)pair_token(pid, P, a.topk) * (uint32_t)(K * T::AEB) + g16
                                   : kAPastEnd;
            },
            xscale_of, [] {});
    }
}

// ---------------------------------------------------------------------------
// Split-K reduction of GEMM1: act[row, c] = SiLU(sum_s gate_s) * sum_s up_s,
// splits added in split order (deterministic); INT8 partials are exact int32
// sums, scaled once by the token's activation scale and the channel scales.
// Grid: one block per (row of the sorted table, 1024-column slab).
// ---------------------------------------------------------------------------
template <int WT>
__global__ __launch_bounds__(256) void splitk_silu_kernel(GemmArgs a, int col_blocks) {
    const int row = blockIdx.x / col_blocks;
    if (row >= a.meta[0]) return;
    const int pid = a.sorted_ids[row];
    if (pid >= a.P_tot) return;
    const int I = a.N >> 1;
    const int c = ((blockIdx.x % col_blocks) * blockDim.x + threadIdx.x) * 4;
    if (c >= I) return;
    // the row's expert: needed for the INT8 channel scales
    float sx = 1.f;
    const float* ws = nullptr;
    if constexpr (WT == W_INT8) {
        const int t = pid < a.P ? pid / a.topk : pid - a.P;
        const int e = pid < a.P ? a.topk_ids[pid] : a.E;
        sx = a.a_scale[t];
        ws = e < a.E ? a.w_scale + (size_t)e * a.N : a.w_scale_sh;
    }
    using Elem = typename std::conditional<WT == W_INT8, int, float>::type;
    const Elem* part = reinterpret_cast<const Elem*>(a.partial);
    Elem gs[4] = {0, 0, 0, 0}, us[4] = {0, 0, 0, 0};
    for (int s = 0; s < a.splits; ++s) {
        const Elem* p = part + ((size_t)s * a.cap + row) * a.N;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            gs[q] += p[c + q];
            us[q] += p[I + c + q];
        }
    }
    float o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float gv, uv;
        if constexpr (WT == W_INT8) {
            gv = (float)gs[q] * sx * ws[c + q];
            uv = (float)us[q] * sx * ws[I + c + q];
        } else {
            gv = gs[q];
            uv = us[q];
        }
        o[q] = silu(gv) * uv;
    }
    *reinterpret_cast<uint2*>((uint16_t*)a.out + (size_t)row * I + c) =
        make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
}

// ---------------------------------------------------------------------------
// INT8 split-K reduction fused with the dynamic row quantisation of the
// intermediate: one workgroup per row of the sorted table.  The int32 split
// partials are exact, the scales and SiLU(gate)*up follow the unsplit
// epilogue, the row is rounded to bf16 (as the unsplit path stores it) and
// then quantised like quant_row: s = amax/127, q = clamp(rint(v/s), +-127).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void splitk_silu_quant_kernel(GemmArgs a) {
    constexpr int MAXJ = kSplitQuantMaxI / 1024;  // 4-column groups per thread
    __shared__ float red[4];
    const int row = blockIdx.x;
    if (row >= a.meta[0]) return;
    const int pid = a.sorted_ids[row];
    if (pid >= a.P_tot) return;  // padding row (the whole block exits)
    const int I = a.N >> 1, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int t = pid < a.P ? pid / a.topk : pid - a.P;
    const int e = pid < a.P ? a.topk_ids[pid] : a.E;
    const float sx = a.a_scale[t];
    const float* ws = e < a.E ? a.w_scale + (size_t)e * a.N : a.w_scale_sh;
    const int* part = reinterpret_cast<const int*>(a.partial);
    float v[MAXJ][4];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
        const int c = (j * 256 + threadIdx.x) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[j][q] = 0.f;
        if (c < I) {
            i32x4 gs = {0, 0, 0, 0}, us = {0, 0, 0, 0};
            for (int s = 0; s < a.splits; ++s) {
                const int* p = part + ((size_t)s * a.cap + row) * a.N;
                gs += *reinterpret_cast<const i32x4*>(p + c);
                us += *reinterpret_cast<const i32x4*>(p + I + c);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float gv = (float)gs[q] * sx * ws[c + q];
                const float uv = (float)us[q] * sx * ws[I + c + q];
                v[j][q] = bf16_bits_to_f32(f32_to_bf16_bits(silu(gv) * uv));
                amax = fmaxf(amax, fabsf(v[j][q]));
            }
        }
    }
    amax = wave_max(amax);
    if (lane == 0) red[w] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = __fdiv_rn(amax, 127.0f), r = quant_recip(s);
    if (threadIdx.x == 0) a.act_s[row] = s;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
        const int c = (j * 256 + threadIdx.x) * 4;
        if (c < I) {
            int q[4];
            quant_codes<4>(v[j], s, r, q);
            *reinterpret_cast<uint32_t*>(a.act_q + (size_t)row * I + c) = pack_codes4(q);
        }
    }
}

// ---------------------------------------------------------------------------
// GEMM2: y[pair, :] = act[row, :] W2, two output tiles per wave
// ---------------------------------------------------------------------------
// One wave's GEMM2 work on chunk `ch` (column tiles nt0 .. nt0+NT-1, split
// `split`) once the chunk's rows are known.
//   pid_of(r)    : pair of row r of the chunk (>= P_tot: padding row)
//   aoff_of(r)   : row r's activation offset for decode_stream
//   ascale_of(r) : INT8 scale of row r's activation codes
//   prologue()   : runs after the weight setup; with PRE the first weight
//                  stages are already in flight while it runs (the row
//                  accessors are called only after it)
// store(pid, split, col, v) receives each y value (y_store: to a.out)
template <int WT, int MB, bool ALDS, bool PRE, int DD, typename PidFn, typename AoffFn, typename AsFn,
          typename ProFn, typename StoreFn>
__device__ inline void gemm2_tile(const GemmArgs& a, const Chunk& ch, int nt0, int split, int lane,
                                  const char* abase, PidFn pid_of, AoffFn aoff_of, AsFn ascale_of,
                                  ProFn prologue, StoreFn store) {
    using T = WT_<WT>;
    constexpr int NT = decode_g2_tiles(WT);
    const int g = lane >> 4, c16 = lane & 15;
    const bool sh = ch.expert >= a.E;
    const size_t wbytes = WT == W_INT4 ? (size_t)a.K * a.N / 2 : (size_t)a.K * a.N * T::EB;
    const uint8_t* W = sh ? a.W_sh : a.W + (size_t)ch.expert * wbytes;
    const int nsc = WT == W_FP8 ? (a.K / 128) * (a.N / 128) : (WT == W_INT4 ? (a.K / 128) * a.N : a.N);
    const float* ws = sh ? a.w_scale_sh : (a.w_scale ? a.w_scale + (size_t)ch.expert * nsc : nullptr);

    const uint8_t* bptr[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int nt = min(nt0 + n, a.N / 16 - 1);  // N % 32 may leave a lone tile: recompute it
        if constexpr (WT == W_INT4)
            bptr[n] = W + packed_i4_offset(a.K, nt, 0) + lane * 16;
        else
            bptr[n] = W + packed_tile_offset(T::EB, a.K, nt, 0) + lane * 16 * T::EB;
    }
    const int nrb = ch.nrows >> 4;
    const int nkb = a.K / 128;
    const int kb0 = split * a.kb_per_split;
    const int kb1 = min(nkb, kb0 + a.kb_per_split);
    const int nbw = a.N / 128;
    auto scale = [&](int n, int kb) {
        if constexpr (WT == W_INT4)  // this lane's column of tile n
            return ws[(size_t)kb * a.N + min(nt0 + n, a.N / 16 - 1) * 16 + c16];
        else
            return ws[kb * nbw + (min(nt0 + n, a.N / 16 - 1) * 16) / 128];
    };
    DecodeTile<WT, MB, NT, DD> st;
    if constexpr (PRE) stream_prefetch<WT, MB, NT>(st, bptr, kb0, kb1, scale);
    prologue();
    uint32_t aoff[MB];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) aoff[rb] = rb < nrb ? aoff_of(rb * 16 + c16) : (ALDS ? aoff_of(-1) : kAPastEnd);
    decode_stream<WT, MB, NT, ALDS, PRE>(st, bptr, aoff, abase, a.a_bytes, kb0, kb1, scale);

#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
        if (rb < nrb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rb * 16 + 4 * g + i;
                const int pid = pid_of(r);
                if (pid >= a.P_tot) continue;
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    if (nt0 + n >= a.N / 16) continue;
                    const int col = (nt0 + n) * 16 + c16;
                    float v;
                    if constexpr (WT == W_INT8)
                        v = (float)st.acc[rb][n][i] * ascale_of(r) * ws[col];
                    else
                        v = st.acc[rb][n][i];
                    store(pid, split, col, v);
                }
            }
        }
    }
}

// y in memory: bf16 [P_tot, N], or fp32 [splits, P_tot, N]
__device__ inline auto y_store(const GemmArgs& a) {
    return [&a](int pid, int split, int col, float v) {
        if (a.y_bf16)
            ((uint16_t*)a.out)[(size_t)pid * a.N + col] = f32_to_bf16_bits(v);
        else
            ((float*)a.out)[((size_t)split * a.P_tot + pid) * a.N + col] = v;
    };
}

template <int WT, int MB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(dec_waves_per_eu<WT, MB>())))
void decode_gemm2_kernel(GemmArgs a) {
    using T = WT_<WT>;
    constexpr int NT = decode_g2_tiles(WT);
    // the wave index is uniform: from readfirstlane the compiler knows it, so
    // per-wave addresses (weight tiles, block scales) stay scalar
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int bid = blockIdx.x;
    const int split = bid % a.splits;
    bid /= a.splits;
    const int grp = bid % a.n_groups;
    const int ci = bid / a.n_groups;
    // slot and chunk count in one round trip (ci < the list's capacity)
    const int nchunks = a.meta[1];
    const Chunk ch = a.chunks[ci];
    if (ci >= nchunks) return;
    const int nt0 = (grp * kDecodeWavesPerWG + wv) * NT;
    if (nt0 >= a.N / 16) return;
    const uint32_t g16 = (uint32_t)((lane >> 4) * 16);
    gemm2_tile<WT, MB, false, false, Depth<WT, MB>::D>(
        a, ch, nt0, split, lane, (const char*)a.A, [&](int r) { return a.sorted_ids[ch.row_start + r]; },
        [&](int r) {
            const int row = ch.row_start + r;
            return a.sorted_ids[row] < a.P_tot ? (uint32_t)row * (uint32_t)(a.K * T::AEB) + g16 : kAPastEnd;
        },
        [&](int r) { return a.a_scale[ch.row_start + r]; }, [] {}, y_store(a));
}

// ---------------------------------------------------------------------------
// GEMM2 with the split-K reduction of GEMM1 in its prologue (one 16-row block
// per chunk); for INT8 without a split, the same prologue only quantises
// GEMM1's bf16 rows (rd.splits == 0, rd.act).  Each workgroup rebuilds the intermediate rows of its own chunk
// from GEMM1's split partial sums, exactly as the split-reduce kernels do --
// splits added in split order, the channel and token scales (INT8), SiLU(gate)
// * up rounded to bf16, then for INT8 the row's dynamic quantisation -- and
// keeps this split's K range of them in LDS (the chunk's live rows, then a
// zero row for the padding rows).  The reduction kernel's launch, and the
// round trip of the intermediate through memory, disappear; every workgroup
// of a chunk repeats the (small) reduction, reading the partials from L2.
// ---------------------------------------------------------------------------
template <int WT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(dec_waves_per_eu<WT, 1>())))
void decode_gemm2_red_kernel(GemmArgs a, SplitRed rd) {
    using T = WT_<WT>;
    constexpr int NT = decode_g2_tiles(WT);
    constexpr int MAXJ = kSplitQuantMaxI / 1024;  // 4-column groups per thread
    extern __shared__ __attribute__((aligned(16))) char a_l[];
    __shared__ int pid_l[16], slot_l[16];
    __shared__ float sc_l[16];
    __shared__ float red_l[2][kDecodeWavesPerWG];
    __shared__ int nlive_l;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bid = blockIdx.x;
    const int split = bid % a.splits;
    bid /= a.splits;
    const int grp = bid % a.n_groups;
    const int ci = bid / a.n_groups;
    const int nchunks = a.meta[1];
    const Chunk ch = a.chunks[ci];
    if (ci >= nchunks) return;  // uniform
    const int I = a.K, P_tot = a.P_tot;
    const int kb0 = split * a.kb_per_split;
    const int kb1 = min(I / 128, kb0 + a.kb_per_split);
    const int lo = kb0 * 128, span = (kb1 - kb0) * 128;
    // the intermediate rows of this chunk, rebuilt into LDS (every wave takes
    // part; the first weight stages are already in flight meanwhile)
    auto prologue = [&]() {
        if (wv == 0) {
            const int pid = lane < 16 ? a.sorted_ids[ch.row_start + lane] : P_tot;
            const bool live = lane < 16 && pid < P_tot;
            const uint64_t lm = __ballot(live);
            const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
            if (lane < 16) {
                pid_l[lane] = pid;
                slot_l[lane] = live ? __popcll(lm & below) : -1;
            }
            if (lane == 0) nlive_l = __popcll(lm);
        }
        __syncthreads();
        const int nlive = nlive_l;
        using Elem = typename std::conditional<WT == W_INT8, int, float>::type;
        const Elem* part = reinterpret_cast<const Elem*>(rd.partial);
        for (int r = 0; r < 16; ++r) {
            const int slot = slot_l[r];  // uniform
            if (slot < 0) continue;
            const int row = ch.row_start + r, pid = pid_l[r];
            float sx = 1.f;
            const float* ws1 = nullptr;
            if constexpr (WT == W_INT8) {
                const int t = pid < a.P ? pid / a.topk : pid - a.P;
                sx = rd.x_scale[t];  // (every row of the chunk is the chunk's expert's)
                ws1 = ch.expert < a.E ? rd.w1_scale + (size_t)ch.expert * 2 * I : rd.w1_scale_sh;
            }
            float v[MAXJ][4];
            float amax = 0.f;
#pragma unroll
            for (int j = 0; j < MAXJ; ++j) {
                const int c = (j * 256 + tid) * 4;
#pragma unroll
                for (int q = 0; q < 4; ++q) v[j][q] = 0.f;
                if (c < I && rd.splits == 0) {
                    // GEMM1 did not split K: its bf16 rows, to be quantised here
                    const uint2 b = *reinterpret_cast<const uint2*>(rd.act + (size_t)row * I + c);
                    const uint32_t w2[2] = {b.x, b.y};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        v[j][q] = bf16_bits_to_f32((uint16_t)(w2[q >> 1] >> ((q & 1) * 16)));
                        amax = fmaxf(amax, fabsf(v[j][q]));
                    }
                } else if (c < I) {
                    // 16-byte loads (c is a multiple of 4, rows of 2I elements)
                    using V4 = typename std::conditional<WT == W_INT8, i32x4, f32x4>::type;
                    V4 gs = {0, 0, 0, 0}, us = {0, 0, 0, 0};
                    for (int sp = 0; sp < rd.splits; ++sp) {
                        const Elem* p = part + ((size_t)sp * rd.cap + row) * 2 * I;
                        gs += *reinterpret_cast<const V4*>(p + c);
                        us += *reinterpret_cast<const V4*>(p + I + c);
                    }
                    f32x4 wg = {1.f, 1.f, 1.f, 1.f}, wu = {1.f, 1.f, 1.f, 1.f};
                    if constexpr (WT == W_INT8) {
                        wg = *reinterpret_cast<const f32x4*>(ws1 + c);
                        wu = *reinterpret_cast<const f32x4*>(ws1 + I + c);
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float gv, uv;
                        if constexpr (WT == W_INT8) {
                            gv = (float)gs[q] * sx * wg[q];
                            uv = (float)us[q] * sx * wu[q];
                        } else {
                            gv = gs[q];
                            uv = us[q];
                        }
                        v[j][q] = bf16_bits_to_f32(f32_to_bf16_bits(silu(gv) * uv));
                        amax = fmaxf(amax, fabsf(v[j][q]));
                    }
                }
            }
            char* dst = a_l + (size_t)slot * span * T::AEB;
            if constexpr (WT == W_INT8) {
                amax = wave_max(amax);
                if (lane == 0) red_l[slot & 1][wv] = amax;
                __syncthreads();  // (red_l alternates between rows: one barrier per row)
                amax = fmaxf(fmaxf(red_l[slot & 1][0], red_l[slot & 1][1]),
                             fmaxf(red_l[slot & 1][2], red_l[slot & 1][3]));
                const float sq = __fdiv_rn(amax, 127.0f), rq = quant_recip(sq);
                if (tid == 0) sc_l[slot] = sq;
#pragma unroll
                for (int j = 0; j < MAXJ; ++j) {
                    const int c = (j * 256 + tid) * 4;
                    if (c >= lo && c < lo + span) {
                        int q[4];
                        quant_codes<4>(v[j], sq, rq, q);
                        *reinterpret_cast<uint32_t*>(dst + (c - lo)) = pack_codes4(q);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < MAXJ; ++j) {
                    const int c = (j * 256 + tid) * 4;
                    if (c >= lo && c < lo + span)
                        *reinterpret_cast<uint2*>(dst + (size_t)(c - lo) * 2) =
                            make_uint2(pack_bf16x2(v[j][0], v[j][1]), pack_bf16x2(v[j][2], v[j][3]));
                }
            }
        }
        for (int o = tid * 16; o < span * T::AEB; o += 256 * 16)  // the zero row of the padding rows
            *reinterpret_cast<u32x4*>(a_l + (size_t)nlive * span * T::AEB + o) = u32x4{0, 0, 0, 0};
        __syncthreads();
    };
    const int nt0 = (grp * kDecodeWavesPerWG + wv) * NT;
    if (nt0 >= a.N / 16) {  // no columns for this wave: the prologue's barriers only
        prologue();
        return;
    }
    const uint32_t g16 = (uint32_t)((lane >> 4) * 16);
    const uint32_t rowb = (uint32_t)(span * T::AEB);
    gemm2_tile<WT, 1, true, true, tiny_depth<WT>()>(
        a, ch, nt0, split, lane, a_l, [&](int r) { return pid_l[r]; },
        [&](int r) {
            const int sl = r >= 0 ? slot_l[r] : -1;
            return (uint32_t)(sl >= 0 ? sl : nlive_l) * rowb + g16;
        },
        [&](int r) { return sc_l[slot_l[r]]; }, prologue, y_store(a));
}

// ---------------------------------------------------------------------------
// INT8 tiny batches of at most kCombMaxPairs pairs whose GEMM1 ran unsplit:
// GEMM2 and the combine in one launch.  A workgroup takes one INT8 column
// tile of every chunk of the batch -- wave w the chunk w (one 16-row block per
// expert) -- so a token's weighted sum over its slots stays inside the
// workgroup.  Each wave quantises its chunk's live rows (GEMM1's bf16 rows:
// the row's amax, codes, as decode_gemm2_red_kernel does) into LDS, the
// chunks' rows one after another, while its first weight stages are in
// flight, streams its expert's tile, and leaves the y values in LDS; after a
// barrier the workgroup sums them exactly as combine_kernel does (fp32, the
// slots in order, then the shared expert) and stores its output columns.
// The combine launch and the round trip of y through memory disappear.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64 * kCombMaxPairs) void decode_gemm2_comb_kernel(GemmArgs a, SplitRed rd,
                                                                                CombineArgs c) {
    constexpr int NT = decode_g2_tiles(W_INT8);
    constexpr int W = NT * 16;  // output columns per workgroup
    extern __shared__ __attribute__((aligned(16))) char a_l[];  // codes [P_tot + 1][I]: live rows by slot; the last: zeros
    __shared__ float sc_l[kCombMaxPairs];
    __shared__ int pid_l[kCombMaxPairs][16];
    __shared__ float ys_l[kCombMaxPairs][W];
    __shared__ float cw_l[kCombMaxPairs];  // the routed slots' weights ...
    __shared__ int cok_l[kCombMaxPairs];   // ... and whether their ids are in range
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int I = a.K, P_tot = a.P_tot;
    const int nt0 = blockIdx.x * NT;
    // the slots' ids and weights, read now (to LDS before the combine)
    int slot_e = -1;
    float slot_w = 0.f;
    if (tid < c.P) {
        slot_e = c.topk_ids[tid];
        slot_w = c.topk_w[tid];
    }
    // Everything the prologue reads goes out at once, before the chunk count
    // is known: this wave's chunk, the live-row counts of the chunks before
    // it, its sorted ids and its first row.  The chunks of a tiny batch are
    // one 16-row block per present expert (chunk w from row 16 w) with their
    // live-row counts in the fourth field, live rows first; a wave without a
    // chunk reads clamped, in-range entries and uses none of them.
    constexpr int MAXJ = kSplitQuantMaxI / 256;  // 4-element groups per lane
    const int rows = (int)rd.cap;
    const Chunk ch = a.chunks[min(wv, rd.chunk_cap - 1)];
    int base = 0;  // this wave's rows go to LDS slots base .. base + nlive - 1
#pragma unroll
    for (int w2 = 0; w2 < kCombMaxPairs - 1; ++w2) {  // every count requested at once
        const int pad = a.chunks[min(w2, rd.chunk_cap - 1)].pad;
        base += w2 < wv ? pad : 0;
    }
    const int row0 = min(16 * wv, rows - 1);
    const int pid = lane < 16 ? a.sorted_ids[min(row0 + lane, rows - 1)] : P_tot;
    // the row's pieces past its end re-read its last piece and count as zeros
    auto load_row = [&](int row, uint2 (&b)[MAXJ]) {
        const uint16_t* src = rd.act + (size_t)row * I;
#pragma unroll
        for (int j = 0; j < MAXJ; ++j)
            b[j] = *reinterpret_cast<const uint2*>(src + min((j * 64 + lane) * 4, I - 4));
    };
    uint2 b0[MAXJ];
    load_row(row0, b0);
    const int nchunks = a.meta[1];  // at most kCombMaxPairs (one chunk per present expert)
    if (wv < nchunks) {
        const int nlive = ch.pad;
        // one row's codes and scale to LDS slot `slot`
        auto quant_row = [&](const uint2 (&b)[MAXJ], int slot) {
            float v[MAXJ][4];
            float amax = 0.f;
#pragma unroll
            for (int j = 0; j < MAXJ; ++j) {
                const int col = (j * 64 + lane) * 4;
                const uint32_t w2[2] = {b[j].x, b[j].y};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v[j][q] = col < I ? bf16_bits_to_f32((uint16_t)(w2[q >> 1] >> ((q & 1) * 16))) : 0.f;
                    amax = fmaxf(amax, fabsf(v[j][q]));
                }
            }
            amax = wave_max(amax);
            const float sq = __fdiv_rn(amax, 127.0f), rq = quant_recip(sq);
            if (lane == 0) sc_l[slot] = sq;
            char* dst = a_l + (size_t)slot * I;
#pragma unroll
            for (int j = 0; j < MAXJ; ++j) {
                const int col = (j * 64 + lane) * 4;
                if (col < I) {
                    int q[4];
                    quant_codes<4>(v[j], sq, rq, q);
                    *reinterpret_cast<uint32_t*>(dst + col) = pack_codes4(q);
                }
            }
        };
        // this wave's chunk rows into LDS (wave-local: written and read by
        // this wave only), the zero row of the padding rows, then the
        // workgroup's first barrier (the zero row is shared)
        auto prologue = [&]() {
            // the first row from the loads issued at the start (older than
            // the weight stages: waiting for it leaves them in flight)
            quant_row(b0, base);
            for (int r = 1; r < nlive; ++r) {
                uint2 b[MAXJ];
                load_row(ch.row_start + r, b);
                quant_row(b, base + r);
            }
            for (int o = lane * 16; o < I; o += 64 * 16)
                *reinterpret_cast<u32x4*>(a_l + (size_t)P_tot * I + o) = u32x4{0, 0, 0, 0};
            if (lane < 16) pid_l[wv][lane] = pid;
            __syncthreads();
        };
        const uint32_t g16 = (uint32_t)((lane >> 4) * 16);
        gemm2_tile<W_INT8, 1, true, true, kCombDepth>(
            a, ch, nt0, 0, lane, a_l, [&](int r) { return pid_l[wv][r]; },
            [&](int r) { return (uint32_t)(r >= 0 && r < nlive ? base + r : P_tot) * (uint32_t)I + g16; },
            [&](int r) { return sc_l[base + r]; }, prologue,
            [&](int pid, int, int col, float v) { ys_l[pid][col - nt0 * 16] = v; });
    } else {
        // A use of the early loads on this path too, behind a test that
        // never passes (a chunk count is never negative): with uses on both
        // paths the compiler keeps the loads ahead of the branch instead of
        // sinking them behind the chunk count's round trip.
        if (nchunks < 0) {
            uint32_t h = (uint32_t)pid;
#pragma unroll
            for (int j = 0; j < MAXJ; ++j) h ^= b0[j].x ^ b0[j].y;
            sc_l[0] = __uint_as_float(h);
        }
        __syncthreads();  // the prologue's barrier
    }
    if (tid < c.P) {
        cw_l[tid] = slot_w;
        cok_l[tid] = slot_e >= 0 && slot_e < c.E;  // dropped slots contribute nothing
    }
    __syncthreads();  // every wave's y values are in LDS
    // combine_kernel's sums for this workgroup's columns
    if (tid < c.T * W) {
        const int t = tid / W, cc = tid % W, col = nt0 * 16 + cc;
        if (col < c.H) {
            const int nslots = c.k + (c.has_shared ? 1 : 0);  // the shared expert is the last slot
            float acc = 0.f;
            for (int j = 0; j < nslots; ++j) {
                bool ok;
                float wt;
                int pid;
                if (j < c.k) {
                    pid = t * c.k + j;
                    ok = cok_l[pid] != 0;
                    wt = cw_l[pid];
                } else {
                    ok = true;
                    wt = 1.0f;
                    pid = c.P + t;
                }
                if (ok) {
                    float ys = 0.f;  // (one split, summed as the combine sums splits)
                    ys += ys_l[pid][cc];
                    ys += 0.f;
                    acc += wt * ys;
                }
            }
            c.out[(size_t)t * c.H + col] = f32_to_bf16_bits(acc);
        }
    }
}

// ---------------------------------------------------------------------------
// Combine: out[t] = bf16( sum_j w[t,j] * y[t*k+j] + y_shared[t] ), fp32 sums in
// ascending j, then the shared expert; split partials summed in split order.
// ---------------------------------------------------------------------------
// YB: y in bf16 (one split), the rows of SB = 8 slots in flight together and
// summed straight from the loaded registers (few registers: high occupancy);
// otherwise fp32 per split, SB = 4 slots.  Same sums in the same order.
template <bool YB, int SB>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int per_row = a.H / 8;
    if (gid >= (int64_t)a.T * per_row) return;
    const int t = (int)(gid / per_row);
    const int n = (int)(gid % per_row) * 8;
    const int P_tot = a.P + (a.has_shared ? a.T : 0);
    const int nslots = a.k + (a.has_shared ? 1 : 0);  // the shared expert is the last slot
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // slots are summed in order (j = 0..k-1, then the shared expert), splits
    // in order inside each slot.  A slot's y row (pair t*k+j, or P+t for the
    // shared expert) does not depend on its id, so the rows of up to 4 slots
    // (and 2 splits) are loaded together with the slots' ids and weights; a
    // dropped slot's row (never written) is discarded by the id check, not
    // multiplied.
    for (int j0 = 0; j0 < nslots; j0 += SB) {
        int pid[SB];
        bool in[SB];
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            const int j = j0 + u;
            in[u] = j < nslots;
            pid[u] = j < a.k ? t * a.k + j : a.P + t;
        }
        int ev[SB];
        float wv[SB];
#pragma unroll
        for (int u = 0; u < SB; ++u) {  // straight-line loads (index clamped into the row)
            const int jj = min(j0 + u, a.k - 1);
            ev[u] = a.topk_ids[(size_t)t * a.k + jj];
            wv[u] = a.topk_w[(size_t)t * a.k + jj];
        }
        bool ok[SB];
        float wt[SB];
        auto slot_weights = [&]() {
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                const int j = j0 + u;
                if (j < a.k) {
                    ok[u] = ev[u] >= 0 && ev[u] < a.E;  // dropped slots contribute nothing
                    wt[u] = wv[u];
                } else {
                    ok[u] = in[u];  // the shared expert
                    wt[u] = 1.0f;
                }
            }
        };
        if constexpr (YB) {
            u32x4 v[SB];
#pragma unroll
            for (int u = 0; u < SB; ++u)
                v[u] = in[u] ? ldg16((const uint16_t*)a.y + (size_t)pid[u] * a.H + n) : u32x4{0, 0, 0, 0};
            slot_weights();
#pragma unroll
            for (int u = 0; u < SB; ++u)
                if (ok[u]) {
                    const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[2 * i] += wt[u] * bf16_bits_to_f32((uint16_t)(w4[i] & 0xffff));
                        acc[2 * i + 1] += wt[u] * bf16_bits_to_f32((uint16_t)(w4[i] >> 16));
                    }
                }
        } else {
            float ys[SB][8];
#pragma unroll
            for (int u = 0; u < SB; ++u)
#pragma unroll
                for (int i = 0; i < 8; ++i) ys[u][i] = 0.f;
            for (int s0 = 0; s0 < a.splits; s0 += 2) {
                f32x4 v[2][SB][2];
#pragma unroll
                for (int ds = 0; ds < 2; ++ds)
#pragma unroll
                    for (int u = 0; u < SB; ++u) {
                        const bool ld = in[u] && s0 + ds < a.splits;
                        const float* p = (const float*)a.y + ((size_t)(s0 + ds) * P_tot + pid[u]) * a.H + n;
                        v[ds][u][0] = ld ? *reinterpret_cast<const f32x4*>(p) : f32x4{0, 0, 0, 0};
                        v[ds][u][1] = ld ? *reinterpret_cast<const f32x4*>(p + 4) : f32x4{0, 0, 0, 0};
                    }
#pragma unroll
                for (int ds = 0; ds < 2; ++ds)
#pragma unroll
                    for (int u = 0; u < SB; ++u)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            ys[u][i] += v[ds][u][0][i];
                            ys[u][4 + i] += v[ds][u][1][i];
                        }
            }
            slot_weights();
#pragma unroll
            for (int u = 0; u < SB; ++u)
                if (ok[u])
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] += wt[u] * ys[u][i];
        }
    }
    u32x4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<u32x4*>(a.out + (size_t)t * a.H + n) = o;
}

template <int WT>
static hipError_t dec1(int MB, const GemmArgs& a, dim3 grid, hipStream_t st) {
    if (MB == 1)
        decode_gemm1_kernel<WT, 1><<<grid, 256, 0, st>>>(a);
    else if (MB == 2)
        decode_gemm1_kernel<WT, 2><<<grid, 256, 0, st>>>(a);
    else
        decode_gemm1_kernel<WT, 4><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
}
template <int WT>
static hipError_t dec2(int MB, const GemmArgs& a, dim3 grid, hipStream_t st) {
    if (MB == 1)
        decode_gemm2_kernel<WT, 1><<<grid, 256, 0, st>>>(a);
    else if (MB == 2)
        decode_gemm2_kernel<WT, 2><<<grid, 256, 0, st>>>(a);
    else
        decode_gemm2_kernel<WT, 4><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_decode_gemm1(int wtype, int MB, const GemmArgs& a, int max_chunks,
                               hipStream_t st) {
    if (a.a_bytes <= 0 || a.a_bytes >= 0x7fffffff) return hipErrorInvalidValue;  // buffer-load range
    dim3 grid((unsigned)((size_t)max_chunks * a.n_groups * a.splits));
    if (wtype == W_FP8) return dec1<W_FP8>(MB, a, grid, st);
    if (wtype == W_INT8) return dec1<W_INT8>(MB, a, grid, st);
    if (wtype == W_INT4) return dec1<W_INT4>(MB, a, grid, st);
    return dec1<W_BF16>(MB, a, grid, st);
}

template <int WT>
static hipError_t tiny1(int vpl, const GemmArgs& a, const TinyRoute& r, dim3 grid, size_t lds, hipStream_t st) {
    if (vpl == 0)
        decode_gemm1_tiny_kernel<WT, 0><<<grid, 256, lds, st>>>(a, r);
    else if (vpl == 1)
        decode_gemm1_tiny_kernel<WT, 1><<<grid, 256, lds, st>>>(a, r);
    else if (vpl == 2)
        decode_gemm1_tiny_kernel<WT, 2><<<grid, 256, lds, st>>>(a, r);
    else
        decode_gemm1_tiny_kernel<WT, 4><<<grid, 256, lds, st>>>(a, r);
    return hipGetLastError();
}

hipError_t launch_decode_gemm1_tiny(int wtype, const GemmArgs& a, const TinyRoute& r, int slots,
                                    hipStream_t st) {
    if (a.a_bytes <= 0 || a.a_bytes >= 0x7fffffff) return hipErrorInvalidValue;  // buffer-load range
    if (r.T < 1 || r.T > kTinyMaxT || a.P_tot > kTinyMaxPairs || a.E > kTinyMaxE || a.E < 1 ||
        a.P != r.T * r.k || slots < 1)
        return hipErrorInvalidValue;
    if (!r.logits && !r.ids) return hipErrorInvalidValue;
    size_t lds = 0;
    if (wtype == W_INT8) {
        lds = (size_t)(r.T + 1) * a.kb_per_split * 128;
        if ((int64_t)r.T * a.K > kTinyMaxElems || a.K % 128 || lds > (size_t)kTinyMaxLds || !r.x || !r.xq_out ||
            !r.xs_out)
            return hipErrorInvalidValue;
    }
    const int vpl = r.logits ? (a.E + 63) / 64 : 0;
    const int v = vpl <= 0 ? 0 : (vpl == 1 ? 1 : (vpl == 2 ? 2 : 4));
    // INT8 (unsplit) with fewer workgroups than CUs at four pair tiles each:
    // three per workgroup when that still fits one workgroup per CU (the
    // Qwen3-shaped T = 1 layer: 192 -> 256 workgroups, GEMM1 24.1 -> 23.6 us)
    GemmArgs b = a;
    TinyRoute rt = r;
    rt.tiles_per_wg = kDecodeWavesPerWG;
    const int tiles = (a.N >> 1) / 16;
    if (wtype == W_INT8 && a.splits == 1) {
        static const int cus = [] {
            int dev = 0, n = 0;
            if (hipGetDevice(&dev) != hipSuccess ||
                hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
                n = 256;
            return n;
        }();
        const int64_t wg4 = (int64_t)slots * ((tiles + 3) / 4), wg3 = (int64_t)slots * ((tiles + 2) / 3);
        if (wg4 < cus && wg3 <= cus) {
            rt.tiles_per_wg = 3;
            b.n_groups = (tiles + 2) / 3;
        }
    }
    if (b.n_groups * rt.tiles_per_wg < tiles) return hipErrorInvalidValue;
    dim3 grid((unsigned)((size_t)slots * b.n_groups * b.splits));
    if (wtype == W_FP8) return tiny1<W_FP8>(v, b, rt, grid, lds, st);
    if (wtype == W_INT8) return tiny1<W_INT8>(v, b, rt, grid, lds, st);
    if (wtype == W_INT4) return tiny1<W_INT4>(v, b, rt, grid, lds, st);
    return tiny1<W_BF16>(v, b, rt, grid, lds, st);
}

hipError_t launch_splitk_silu(int wtype, const GemmArgs& a, hipStream_t st) {
    const int I = a.N / 2;
    const int cb = (I / 4 + 255) / 256;
    dim3 grid((unsigned)(cb * a.cap)), block(256);
    if (wtype == W_FP8 || wtype == W_INT4)  // fp32 partials, scales already applied
        splitk_silu_kernel<W_FP8><<<grid, block, 0, st>>>(a, cb);
    else if (wtype == W_INT8)
        splitk_silu_kernel<W_INT8><<<grid, block, 0, st>>>(a, cb);
    else
        splitk_silu_kernel<W_BF16><<<grid, block, 0, st>>>(a, cb);
    return hipGetLastError();
}

hipError_t launch_splitk_silu_quant(const GemmArgs& a, hipStream_t st) {
    if ((a.N >> 1) > kSplitQuantMaxI || a.splits < 1) return hipErrorInvalidValue;
    splitk_silu_quant_kernel<<<(unsigned)a.cap, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_decode_gemm2(int wtype, int MB, const GemmArgs& a, int max_chunks,
                               hipStream_t st) {
    if (a.a_bytes <= 0 || a.a_bytes >= 0x7fffffff) return hipErrorInvalidValue;  // buffer-load range
    dim3 grid((unsigned)((size_t)max_chunks * a.n_groups * a.splits));
    if (wtype == W_FP8) return dec2<W_FP8>(MB, a, grid, st);
    if (wtype == W_INT8) return dec2<W_INT8>(MB, a, grid, st);
    if (wtype == W_INT4) return dec2<W_INT4>(MB, a, grid, st);
    return dec2<W_BF16>(MB, a, grid, st);
}

size_t gemm2_red_lds(int wtype, const GemmArgs& a) {
    const int live = a.P_tot < 16 ? a.P_tot : 16;
    return (size_t)(live + 1) * a.kb_per_split * 128 * (wtype == W_INT8 ? 1 : 2);
}

size_t gemm2_comb_lds(const GemmArgs& a) { return (size_t)(a.P_tot + 1) * a.K; }

hipError_t launch_decode_gemm2_comb(const GemmArgs& a, const SplitRed& rd, const CombineArgs& c, hipStream_t st) {
    if (a.P_tot < 1 || a.P_tot > kCombMaxPairs || a.splits != 1 || rd.splits != 0 || !rd.act || rd.cap < 16 ||
        rd.cap > INT32_MAX || rd.chunk_cap < 1)
        return hipErrorInvalidValue;
    if (a.K > kSplitQuantMaxI || a.K % 128 || a.N % 16 || c.H != a.N || c.T * decode_g2_tiles(W_INT8) * 16 > 64 * kCombMaxPairs)
        return hipErrorInvalidValue;
    const size_t lds = gemm2_comb_lds(a);
    if (lds > (size_t)kGemm2RedMaxLds) return hipErrorInvalidValue;
    const int tiles = a.N / 16, NT = decode_g2_tiles(W_INT8);
    dim3 grid((unsigned)((tiles + NT - 1) / NT));
    decode_gemm2_comb_kernel<<<grid, 64 * kCombMaxPairs, lds, st>>>(a, rd, c);
    return hipGetLastError();
}

hipError_t launch_decode_gemm2_red(int wtype, const GemmArgs& a, const SplitRed& rd, int max_chunks,
                                   hipStream_t st) {
    if (a.a_bytes <= 0 || a.a_bytes >= 0x7fffffff) return hipErrorInvalidValue;
    if (a.K > kSplitQuantMaxI || a.K % 128 || rd.splits < 0) return hipErrorInvalidValue;
    if (rd.splits == 0 ? (wtype != W_INT8 || !rd.act) : !rd.partial) return hipErrorInvalidValue;
    if (wtype == W_INT8 && (!rd.x_scale || !rd.w1_scale)) return hipErrorInvalidValue;
    const size_t lds = gemm2_red_lds(wtype, a);
    if (lds > (size_t)kGemm2RedMaxLds) return hipErrorInvalidValue;
    dim3 grid((unsigned)((size_t)max_chunks * a.n_groups * a.splits));
    if (wtype == W_FP8)
        decode_gemm2_red_kernel<W_FP8><<<grid, 256, lds, st>>>(a, rd);
    else if (wtype == W_INT8)
        decode_gemm2_red_kernel<W_INT8><<<grid, 256, lds, st>>>(a, rd);
    else if (wtype == W_INT4)
        decode_gemm2_red_kernel<W_INT4><<<grid, 256, lds, st>>>(a, rd);
    else
        decode_gemm2_red_kernel<W_BF16><<<grid, 256, lds, st>>>(a, rd);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
    const int64_t n = (int64_t)a.T * (a.H / 8);
    if (n == 0) return hipSuccess;
    if (a.y_bf16)
        combine_kernel<true, 8><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(a);
    else
        combine_kernel<false, 4><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace moe
