// moe_prefill.hip -- MFMA tile grouped GEMMs for many rows per expert, BF16
// and INT8 weights (FP8 weights: moe_prefill_f8.hip).
//
// A workgroup owns one chunk of up to 192 sorted rows of one expert and one
// or more consecutive column groups of weight columns (MFMA column tiles of
// 16: for GEMM1 gate tiles interleaved with the matching up tiles, so
// SiLU(C1)*C2 stays lane-local), each over the full K range, so each weight
// byte of a column group is fetched from HBM once per chunk and needs no
// cross-workgroup reduction.  K advances in 64-deep stages; the stages of
// the workgroup's groups follow each other through the same rings, and each
// group's results are stored from registers after its last stage.  BF16:
// 128 columns per group, 8 waves; INT8: 256 columns, 12 waves (wave roles:
// PF below).
//
// The waves specialise:
//   producers (the waves after the consumers) only load: direct global->LDS
//     loads (global_load_lds_dwordx4: lane l's 16 bytes land at slot +
//     16*l) into an activation ring (the chunk's rows, gathered through
//     sorted_ids for GEMM1, mostly L2 hits) and, for BF16, a weight ring (the
//     HBM stream, several stages ahead); INT8's weight waves keep five
//     stages in flight as ordinary loads into registers and write each to a
//     two-slot LDS ring just before it is published (faster than the
//     direct-to-LDS stream here);
//   consumers (the first waves: 4 for BF16, one per SIMD; 8 for INT8) run
//     bf16 MFMA 16x16x32 (i8 MFMA 16x16x64 for INT8), software-pipelined
//     with explicit ds_read_b128 so LDS latency stays off the critical path:
//     consumer (h, c) owns row blocks h, h+2, ... and column tiles 4c..4c+3,
//     and reads all fragments of stage j+1 while the MFMAs of stage j run
//     from registers.
// Barrier j publishes stage j+1: producers have waited (explicit vmcnt) for
// its loads before arriving, consumers have drained their reads of the slots
// the producers refill after it.  No wave both loads into LDS through the DMA
// path and reads it with the compiler's LDS accesses: LDS reads in the main
// loops are explicit ds_read with explicit waits, so the compiler adds no
// vmcnt(0) drains before them.
// Workgroup ids are dealt round-robin to the 8 XCDs; consecutive ids of one
// XCD take the column groups of one chunk, so the chunk's activation rows
// are shared through that XCD's L2 while its weights stream from HBM once.
#include <algorithm>

#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int kRows = 16 * kPrefillMB;  // rows per chunk (12 row blocks)
constexpr int kRBC = kPrefillMB / 2;    // row blocks per consumer wave (at most)
constexpr int kTPC = 4;                 // 16-column tiles per consumer wave

template <int WT>
struct PF {
    // Wave roles.  Consumers: row-block parity x column group of kTPC tiles.
    // INT8 (HBM-bound): 8 consumers over 256 columns, so each activation
    // byte staged through a CU serves twice the weight bytes of a 128-column
    // tile (the activation rows otherwise compete with the weight stream for
    // the CU's load path), with two activation and two weight producers:
    // 12 waves.  BF16: 4 consumers over 128 columns, three activation
    // producers and one weight producer: 8 waves.
    static constexpr int NCONS = WT == W_INT8 ? 8 : 4;
    static constexpr int NAW = WT == W_INT8 ? 2 : 3;   // activation producer waves
    static constexpr int NBW = WT == W_INT8 ? 2 : 1;   // weight producer waves
    static constexpr int NWAVES = NCONS + NAW + NBW;
    static constexpr int TILES = NCONS / 2 * kTPC;      // 16-column tiles per workgroup
    static constexpr int EB = WT == W_BF16 ? 2 : 1;    // weight element bytes
    static constexpr int AEB = WT == W_INT8 ? 1 : 2;   // activation element bytes
    static constexpr int A_ROW = 64 * AEB;             // bytes per row per K stage
    // K stages per activation slot: INT8 rows are staged 128 bytes (two
    // stages) at a time, so every row piece a load requests is a whole
    // 128-byte line (64-byte pieces fetched each line twice, once per stage)
    static constexpr int AD = WT == W_INT8 ? 2 : 1;
    static constexpr int A_ROWB = A_ROW * AD;          // bytes per row in a slot (128)
    static constexpr int A_PARTS = A_ROWB / 16;        // 16-byte parts per row in a slot (8)
    // rows whose same-numbered part must fall in distinct LDS banks: the
    // 16 rows of an MFMA fragment, read by one 16-lane group
    static constexpr int SWZ_SHIFT = A_PARTS == 8 ? 1 : 2;
    static constexpr int A_SLOT = kRows * A_ROWB;
    // activation slots in the ring.  AD = 1: slot s % 3 holds stage s, which
    // is requested two stages before it is published.  AD = 2: slot D % 3
    // holds stages 2D and 2D+1, requested four stages before stage 2D is
    // published (the rows come from L2 or the MALL with high latency under
    // the weight stream)
    static constexpr int A_SLOTS = 3;
    static constexpr int B_TILE = 64 * 16 * EB;        // one packed k-tile of one column tile
    static constexpr int B_SLOT = TILES * B_TILE;
    // weight stages requested ahead of the stage being published (DMA: =
    // ring slots); a weight wave keeps B_AHEAD - 1 stages counted in vmcnt
    // (6 bits).  INT8 instead stages the weights through the weight waves'
    // registers (REG_W): RS stages in flight as ordinary 16-byte loads, each
    // written to a two-slot LDS ring two stages before it is published --
    // 3.5 % faster than the direct-to-LDS stream on the Qwen3-235B-shaped
    // layer at T=2048 (GEMM1 320 -> 309 us; 2-4 register stages 312-314 us,
    // 6 spills).  BF16's weight stage (16 KiB per wave) would not fit the
    // registers.
    // Deeper rings measured no faster (INT8 at T=2048 with column-group spans:
    // activation 3-4 x weights 4-6 stages within 1%, 3 x 4 the fastest)
    static constexpr int B_AHEAD = 4;
    static constexpr bool REG_W = WT == W_INT8;
    static constexpr int RS = 5;                       // REG_W: register stages
    static constexpr int B_SLOTS = REG_W ? 2 : B_AHEAD;
    // direct-to-LDS instructions per stage (1 KiB each): the weight waves
    // split the weight stage, the activation waves share the activation rows
    // in rounds of NAW instructions
    static constexpr int B_INSTR = B_SLOT / 1024;
    static constexpr int BIW = B_INSTR / NBW;                          // per weight wave
    static constexpr int ROWS_PER_INSTR = 1024 / A_ROWB;
    static constexpr int A_ROUND = NAW * ROWS_PER_INSTR;               // rows per round
    static constexpr int A_INSTR = (kRows + A_ROUND - 1) / A_ROUND;    // rounds for a full chunk
    static_assert(B_INSTR % NBW == 0, "weight stage split");
    static_assert((B_AHEAD - 1) * BIW < 64, "weight wave vmcnt range");
    // shared-memory layout
    static constexpr int A_OFF = 0;
    static constexpr int B_OFF = A_OFF + A_SLOTS * A_SLOT;
    // row table: source row, pair id and activation row scale per chunk row
    static constexpr int R_OFF = B_OFF + B_SLOTS * B_SLOT;
    // INT8 channel scales of the workgroup's column groups (up to MAX_SPAN
    // groups of TILES*16 columns)
    static constexpr int MAX_SPAN = WT == W_INT8 ? 8 : 64;
    static constexpr int S_OFF = R_OFF + kRows * 12;
    // per consumer wave a staging tile for the epilogue: 16 rows of its
    // columns (GEMM1: 32 act columns, GEMM2: 64 y columns) as bf16, rows
    // padded by 32 bytes so the four rows a store instruction writes fall in
    // distinct banks
    static constexpr int E_ROW1 = kTPC * 8 * 2 + 32, E_ROW2 = kTPC * 16 * 2 + 32;
    static constexpr int E_WAVE = 16 * E_ROW2;
    static constexpr int E_OFF = S_OFF + (WT == W_INT8 ? MAX_SPAN * TILES * 16 * 4 : 0);
    static constexpr int SMEM = E_OFF + NCONS * E_WAVE;
    // output columns of one column group: act columns for GEMM1, y for GEMM2
    static constexpr int TILE_W1 = TILES * 16 / 2, TILE_W2 = TILES * 16;
    static_assert(SMEM <= 160 * 1024, "LDS budget");
    static_assert(B_AHEAD >= 3, "in-order load completion argument needs 3 stages");
    typedef typename std::conditional<WT == W_INT8, i32x4, f32x4>::type Acc;
};

// byte offset of (row, logical 16-byte part) in an activation slot
template <int WT>
__device__ inline int a_off(int row, int part) {
    using T = PF<WT>;
    return row * T::A_ROWB + ((part ^ ((row >> T::SWZ_SHIFT) & (T::A_PARTS - 1))) << 4);
}

// ----------------------------------------------------------------------------
// BF16 / INT8 consumer main loop for NRB row blocks per wave (1..6), fully
// unrolled over row blocks so every LDS wait count is exact.  It runs the
// ns = groups * nkt stages of the workgroup's column groups back to back; in
// the last K stage of each group it calls epi(group, NRB) right after the
// MFMAs (epi stores the group's results and clears the accumulators) and
// only then reads the next stage's fragments, so those registers are free
// during the epilogue.  One barrier per stage, as the producers count them.
// ----------------------------------------------------------------------------
template <int WT, int NRB, class EPI>
__device__ __attribute__((always_inline)) inline void consume(char* smem, int nkt, int ns, int h, int cgrp,
                                                              int lane, typename PF<WT>::Acc (&acc)[kRBC][kTPC],
                                                              EPI&& epi) {
    using T = PF<WT>;
    const int g = lane >> 4, c16 = lane & 15;
    // rows of row block i: (2i + h)*16 + c16; the swizzle term depends on c16 only
    const int row = h * 16 + c16;
    const uint32_t a_base = lds_addr(smem + T::A_OFF);
    constexpr int RB_STRIDE = 32 * T::A_ROWB;  // bytes between this wave's row blocks
    // B fragment addresses (stage slot added per stage)
    const uint32_t b_base =
        lds_addr(smem + T::B_OFF) + cgrp * 4 * T::B_TILE + lane * (WT == W_BF16 ? 32 : 16);
    auto b_slot = [&](int s) -> uint32_t { return (uint32_t)((s % T::B_SLOTS) * T::B_SLOT); };

    if constexpr (WT == W_INT8) {
        // stage s: slot (s / 2) % A_SLOTS, bytes 64 * (s % 2) .. of each row
        static_assert(T::AD == 2, "INT8 activation slots hold two stages");
        // (arithmetic, not a select of the two: a select of references
        // becomes a pointer to stack copies)
        const uint32_t a_ev = a_base + a_off<WT>(row, g);
        const uint32_t d_od = a_off<WT>(row, 4 + g) - a_off<WT>(row, g);
        auto a_at = [&](int s) -> uint32_t {
            return a_ev + (uint32_t)(s & 1) * d_od + ((s >> 1) % T::A_SLOTS) * T::A_SLOT;
        };
        u32x4 af[NRB], bA[4], bB[4];
        auto ldA = [&](uint32_t ab, auto I) {
            constexpr int i = decltype(I)::value;
            af[i] = ds_read16<i * RB_STRIDE>(ab);
        };
        auto ldB = [&](uint32_t bb, u32x4 (&b)[4]) {
            b[0] = ds_read16<0>(bb);
            b[1] = ds_read16<1024>(bb);
            b[2] = ds_read16<2048>(bb);
            b[3] = ds_read16<3072>(bb);
        };
        auto sync = [&](u32x4 (&b)[4]) {
            lgkm_wait0();
            static_for<NRB>([&](auto I) { tie(af[decltype(I)::value]); });
#pragma unroll
            for (int n = 0; n < 4; ++n) tie(b[n]);
        };
        stage_barrier();
        static_for<NRB>([&](auto I) { ldA(a_ev, I); });
        ldB(b_base + b_slot(0), bA);
        auto stage = [&](int j, u32x4 (&b)[4], u32x4 (&nb)[4]) {
            sync(b);
            stage_barrier();  // stage j+1 published
            ldB(b_base + b_slot(j + 1), nb);
            const uint32_t ab = a_at(j + 1);
            static_for<NRB>([&](auto I) {
                constexpr int i = decltype(I)::value;
#pragma unroll
                for (int n = 0; n < 4; ++n) acc[i][n] = mfma_i8(af[i], b[n], acc[i][n]);
                __builtin_amdgcn_sched_barrier(0);
                ldA(ab, I);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        // a group's last stage: MFMAs, the group's epilogue, then (unless it
        // is the workgroup's last stage) the reads of the next stage
        auto stage_last = [&](int j, u32x4 (&b)[4], u32x4 (&nb)[4], int gi) {
            sync(b);
            stage_barrier();  // stage j+1 published
            static_for<NRB>([&](auto I) {
                constexpr int i = decltype(I)::value;
#pragma unroll
                for (int n = 0; n < 4; ++n) acc[i][n] = mfma_i8(af[i], b[n], acc[i][n]);
            });
            epi(gi, std::integral_constant<int, NRB>{});
            if (j + 1 < ns) {
                ldB(b_base + b_slot(j + 1), nb);
                const uint32_t ab = a_at(j + 1);
                static_for<NRB>([&](auto I) { ldA(ab, I); });
            }
        };
        for (int gi = 0, j = 0; j < ns; ++gi) {
            for (int kk = 0; kk < nkt - 2; kk += 2, j += 2) {
                stage(j, bA, bB);
                stage(j + 1, bB, bA);
            }
            stage(j, bA, bB);
            stage_last(j + 1, bB, bA, gi);
            j += 2;
        }
    } else {
        const uint32_t a_lo = a_base + a_off<WT>(row, g);
        const uint32_t a_hi = a_base + a_off<WT>(row, 4 + g);
        u32x4 af[NRB][2], bA[4][2], bB[4][2];
        auto ldA = [&](uint32_t lo, uint32_t hi, auto I) {
            constexpr int i = decltype(I)::value;
            af[i][0] = ds_read16<i * RB_STRIDE>(lo);
            af[i][1] = ds_read16<i * RB_STRIDE>(hi);
        };
        auto ldB = [&](uint32_t bb, u32x4 (&b)[4][2]) {  // packed bf16 tile: [lane][32 B]
            b[0][0] = ds_read16<0>(bb);
            b[0][1] = ds_read16<16>(bb);
            b[1][0] = ds_read16<2048>(bb);
            b[1][1] = ds_read16<2064>(bb);
            b[2][0] = ds_read16<4096>(bb);
            b[2][1] = ds_read16<4112>(bb);
            b[3][0] = ds_read16<6144>(bb);
            b[3][1] = ds_read16<6160>(bb);
        };
        auto sync = [&](u32x4 (&b)[4][2]) {
            lgkm_wait0();
            static_for<NRB>([&](auto I) {
                tie(af[decltype(I)::value][0]);
                tie(af[decltype(I)::value][1]);
            });
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                tie(b[n][0]);
                tie(b[n][1]);
            }
        };
        stage_barrier();
        static_for<NRB>([&](auto I) { ldA(a_lo, a_hi, I); });
        ldB(b_base + b_slot(0), bA);
        auto mma = [&](u32x4 (&b)[4][2], auto I) {
            constexpr int i = decltype(I)::value;
            const bf16x8 a0 = __builtin_bit_cast(bf16x8, af[i][0]);
            const bf16x8 a1 = __builtin_bit_cast(bf16x8, af[i][1]);
#pragma unroll
            for (int n = 0; n < 4; ++n)
                acc[i][n] = mfma_bf16(a0, __builtin_bit_cast(bf16x8, b[n][0]), acc[i][n]);
#pragma unroll
            for (int n = 0; n < 4; ++n)
                acc[i][n] = mfma_bf16(a1, __builtin_bit_cast(bf16x8, b[n][1]), acc[i][n]);
        };
        auto stage = [&](int j, u32x4 (&b)[4][2], u32x4 (&nb)[4][2]) {
            sync(b);
            stage_barrier();  // stage j+1 published
            ldB(b_base + b_slot(j + 1), nb);
            const uint32_t so = ((j + 1) % T::A_SLOTS) * T::A_SLOT;
            const uint32_t lo = a_lo + so, hi = a_hi + so;
            static_for<NRB>([&](auto I) {
                mma(b, I);
                __builtin_amdgcn_sched_barrier(0);
                ldA(lo, hi, I);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        // a group's last stage: MFMAs, the group's epilogue, then (unless it
        // is the workgroup's last stage) the reads of the next stage
        auto stage_last = [&](int j, u32x4 (&b)[4][2], u32x4 (&nb)[4][2], int gi) {
            sync(b);
            stage_barrier();  // stage j+1 published
            static_for<NRB>([&](auto I) { mma(b, I); });
            epi(gi, std::integral_constant<int, NRB>{});
            if (j + 1 < ns) {
                ldB(b_base + b_slot(j + 1), nb);
                const uint32_t so = ((j + 1) % T::A_SLOTS) * T::A_SLOT;
                static_for<NRB>([&](auto I) { ldA(a_lo + so, a_hi + so, I); });
            }
        };
        for (int gi = 0, j = 0; j < ns; ++gi) {
            for (int kk = 0; kk < nkt - 2; kk += 2, j += 2) {
                stage(j, bA, bB);
                stage(j + 1, bB, bA);
            }
            stage(j, bA, bB);
            stage_last(j + 1, bB, bA, gi);
            j += 2;
        }
    }
}

}  // namespace

template <int WT, int GEMM>
__global__ __launch_bounds__(PF<WT>::NWAVES * 64, 1) void prefill_kernel(GemmArgs a) {
    using T = PF<WT>;
    using Acc = typename T::Acc;
    __shared__ __attribute__((aligned(1024))) char smem[T::SMEM];
    int* row_src = reinterpret_cast<int*>(smem + T::R_OFF);
    int* row_pid = row_src + kRows;
    float* row_rs = reinterpret_cast<float*>(row_pid + kRows);

    const int tid = threadIdx.x;
    // wave index as a scalar: role and row-block branches are wave-uniform
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int ci = (slot / a.n_groups) * 8 + xcd;
    const int grp = slot % a.n_groups;
    // the chunk slot is read together with the chunk count (one round trip):
    // the chunk list is padded to a multiple of 8 slots, so ci is in bounds
    const int nchunks = a.meta[1];
    const Chunk ch = a.chunks[ci];
    if (ci >= nchunks) return;  // uniform for the whole workgroup
    const int nrows = ch.nrows;
    const int nrb = nrows >> 4;

    const bool sh = ch.expert >= a.E;
    const size_t wbytes = (size_t)a.K * a.N * T::EB;
    const uint8_t* W = sh ? a.W_sh : a.W + (size_t)ch.expert * wbytes;
    static_assert(WT != W_FP8, "FP8 weights use prefill_f8_kernel");
    const int nsc = a.N;  // INT8: one scale per output channel
    const float* ws = sh ? a.w_scale_sh : (a.w_scale ? a.w_scale + (size_t)ch.expert * nsc : nullptr);
    const int nkt = a.K / 64;  // even: K is a multiple of 128
    // column groups gfirst .. gfirst+ng-1 of the chunk, one after the other:
    // stage s of the workgroup is K stage s % nkt of group gfirst + s / nkt
    const int gfirst = grp * a.group_span;
    const int ng = min(a.group_span, a.col_groups - gfirst);
    const int ns = ng * nkt;

    // logical first column of packed tile nt (group gc owns tiles
    // gc*TILES .. gc*TILES+TILES-1)
    auto col_of = [&](int nt) { return GEMM == 1 ? (nt & 1) * (a.N / 2) + (nt >> 1) * 16 : nt * 16; };

    // the weight waves need no row table: their first stages go out before
    // the table's barrier, so their HBM latency overlaps the table set-up.
    // Weight wave wb issues 1 KiB pieces wb*BIW .. wb*BIW+BIW-1 of each
    // stage; tiles past the last one (a partial last column group) re-read
    // it, and stages past the last one re-read that stage.  (bs, bg, bk): the
    // next stage to issue, its group and its K stage.
    const int wb = wv - (T::NCONS + T::NAW);
    const int ntiles = a.N / 16;
    int bs = 0, bg = 0, bk = 0;
    auto issue_b = [&]() {
        const size_t off = (size_t)bk * T::B_TILE;
        char* dst = smem + T::B_OFF + (bs % T::B_SLOTS) * T::B_SLOT;
#pragma unroll
        for (int q = 0; q < T::BIW; ++q) {
            const int i = wb * T::BIW + q;
            // 1 KiB piece i of the slot: tile i*1024/B_TILE, offset i*1024%B_TILE
            const int tile = min((gfirst + bg) * T::TILES + i * 1024 / T::B_TILE, ntiles - 1);
            const int within = i * 1024 % T::B_TILE;
            lds_dma16_stream(W + packed_tile_offset(T::EB, a.K, tile, 0) + lane * 16 + within + off,
                             dst + i * 1024);
        }
        if (++bs < ns && ++bk == nkt) {
            bk = 0;
            ++bg;
        }
    };
    if constexpr (T::REG_W) {
        if (wb >= 0) {
            // A weight wave's whole life: its first RS stages go out before
            // the row table's barrier (their HBM latency overlaps the table
            // set-up; branching off here keeps the register ring out of the
            // other waves' code).
            // stage s travels in registers rr[s % RS] and is written to LDS
            // slot s % 2 right after the barrier that frees that slot (the
            // one publishing stage s-1); the loads' waits are the compiler's
            // (every steady-state stage issues the same loads, so they are
            // exact)
            u32x4 rr[T::RS][T::BIW];
            auto load_b = [&](u32x4(&r)[T::BIW]) {
                const size_t off = (size_t)bk * T::B_TILE;
#pragma unroll
                for (int q = 0; q < T::BIW; ++q) {
                    const int i = wb * T::BIW + q;
                    const int tile = min((gfirst + bg) * T::TILES + i * 1024 / T::B_TILE, ntiles - 1);
                    const int within = i * 1024 % T::B_TILE;
                    r[q] = ldg16_nt(W + packed_tile_offset(T::EB, a.K, tile, 0) + lane * 16 + within + off);
                }
                if (++bs < ns && ++bk == nkt) {
                    bk = 0;
                    ++bg;
                }
            };
            auto store_b = [&](const u32x4(&r)[T::BIW], int slot) {
                char* dst = smem + T::B_OFF + slot * T::B_SLOT;
#pragma unroll
                for (int q = 0; q < T::BIW; ++q)
                    *reinterpret_cast<u32x4*>(dst + (wb * T::BIW + q) * 1024 + lane * 16) = r[q];
            };
#pragma unroll
            for (int s = 0; s < T::RS; ++s) load_b(rr[s]);
            __syncthreads();  // the row table's barrier (no part of the table is this wave's)
            store_b(rr[0], 0);
            store_b(rr[1], 1);
            load_b(rr[0]);  // stage RS
            load_b(rr[1]);  // stage RS + 1
            lgkm_wait0();
            stage_barrier();  // publishes stage 0
            constexpr int U = T::RS % 2 == 0 ? T::RS : 2 * T::RS;  // static register and LDS slots
            int j0 = 0;
            for (; j0 + U <= ns; j0 += U) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    stage_barrier();                      // publishes stage j+1; slot j % 2 is free
                    store_b(rr[(u + 2) % T::RS], u % 2);  // stage j+2
                    load_b(rr[(u + 2) % T::RS]);          // stage j+2+RS
                    lgkm_wait0();
                }
            }
            // the last stages: stage s is loaded by iteration s - 2 - RS, so
            // these iterations keep loading (past the last stage they re-read
            // it) for the later ones of their own
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (j0 + u < ns) {
                    stage_barrier();
                    store_b(rr[(u + 2) % T::RS], u % 2);
                    load_b(rr[(u + 2) % T::RS]);
                    lgkm_wait0();
                }
            }
            wait_vm<0>();  // no load may land after the workgroup ends
            return;
        }
    }
    if constexpr (!T::REG_W) {
        if (wb >= 0)
            for (int s = 0; s < T::B_AHEAD; ++s) issue_b();
    }

    if (tid < kRows) {
        int src = -1, pid = a.P_tot;
        float rs = 1.f;
        if (tid < nrows) {
            pid = a.sorted_ids[ch.row_start + tid];
            if (pid < a.P_tot) {
                if (GEMM == 1)
                    src = pid < a.P ? pid / a.topk : pid - a.P;
                else
                    src = ch.row_start + tid;
                if constexpr (WT == W_INT8) rs = a.a_scale[src];
            }
        }
        row_src[tid] = src;
        row_pid[tid] = pid;
        row_rs[tid] = rs;
    }
    if constexpr (WT == W_INT8) {
        // channel scales of the span (column c of packed tile t is channel
        // col_of(t) + c), loaded by the consumer waves: the weight waves'
        // first stages are in flight and must not be waited for here
        float* sc = reinterpret_cast<float*>(smem + T::S_OFF);
        for (int idx = tid; idx < ng * T::TILES * 16 && tid < T::NCONS * 64; idx += T::NCONS * 64) {
            const int t = min(gfirst * T::TILES + (idx >> 4), ntiles - 1);
            sc[idx] = ws[col_of(t) + (idx & 15)];
        }
    }
    __syncthreads();

    if (wv >= T::NCONS) {
        // ------------------------------ producer ------------------------------
        // NAW waves load activation rows, NBW waves load weights, so each
        // wave's vmcnt counts only its own stream: a weight wave keeps
        // B_AHEAD stages in flight while an activation wave waits for its own
        // rows only (loads retire in issue order within a wave).  Every stage
        // issues the same loads, so the wait counts are constants.
        const int pw = wv - T::NCONS;
        if (wb >= 0) {  // its first B_AHEAD stages are already requested
            wait_vm<(T::B_AHEAD - 1) * T::BIW>();  // stage 0
            stage_barrier();                         // publishes stage 0
            wait_vm<(T::B_AHEAD - 2) * T::BIW>();  // stage 1
            for (int j = 0; j < ns; ++j) {
                stage_barrier();  // publishes stage j+1; stage j's slot is free
                issue_b();        // stage j + B_AHEAD
                wait_vm<(T::B_AHEAD - 2) * T::BIW>();  // stage j+2 landed
            }
            wait_vm<0>();  // no load may land after the workgroup ends
        } else {
        // activation waves: rows are loaded in rounds of A_ROUND rows
        // (instruction i of wave pw takes rows (NAW*i + pw) * ROWS_PER_INSTR ..),
        // only as many rounds as the chunk needs; rows of the last round past
        // the chunk re-read its first row (never stored back).  Every group
        // re-reads the same rows over K (from L2).
        auto produce = [&](auto NIc) {
            constexpr int NI = decltype(NIc)::value;  // instructions per stage
            // (compile-time loops: a runtime-indexed pointer array would live
            // in scratch, whose accesses the in-order vmcnt waits would
            // serialise with the row loads)
            const char* a_src[NI];
            const int src0 = row_src[0];  // the first row of a chunk is always a real pair
            static_for<NI>([&](auto Ic) {
                constexpr int i = decltype(Ic)::value;
                const int row0 = (T::NAW * i + pw) * T::ROWS_PER_INSTR;
                const int row = row0 + lane / T::A_PARTS;
                const int q = lane % T::A_PARTS;  // LDS part slot of this lane
                const int part = q ^ ((row >> T::SWZ_SHIFT) & (T::A_PARTS - 1));  // logical part it holds
                int src = row < nrows ? row_src[row] : -1;
                if (src < 0) src = src0;
                a_src[i] = (const char*)a.A + (size_t)src * a.K * T::AEB + part * 16;
            });
            // slots of AD stages: the next to issue and its K position (in
            // slots) within the group; past the last one the last is re-read
            const int nsl = ns / T::AD, nkl = nkt / T::AD;  // nkt is even
            int as = 0, ak = 0;
            auto issue_a = [&]() {
                const size_t off = (size_t)ak * T::A_ROWB;
                char* dst = smem + T::A_OFF + (as % T::A_SLOTS) * T::A_SLOT;
                static_for<NI>([&](auto Ic) {  // rows (NAW*i + pw) * ROWS_PER_INSTR ..
                    constexpr int i = decltype(Ic)::value;
                    lds_dma16(a_src[i] + off, dst + (T::NAW * i + pw) * T::ROWS_PER_INSTR * T::A_ROWB);
                });
                if (++as < nsl && ++ak == nkl) ak = 0;
            };
            for (int s = 0; s < T::A_SLOTS; ++s) issue_a();
            wait_vm<(T::A_SLOTS - 1) * NI>();  // slot 0 (stage 0)
            stage_barrier();                     // publishes stage 0
            if constexpr (T::AD == 1) {
                wait_vm<(T::A_SLOTS - 2) * NI>();  // stage 1
                for (int j = 0; j < ns; ++j) {
                    stage_barrier();  // publishes stage j+1; the slot of stage j is free
                    issue_a();        // stage j + 3
                    wait_vm<NI>();    // stage j+2 landed; stage j+3 may stay in flight
                }
            } else {
                // barrier s publishes stage s; after an even one (s = 2m) the
                // slot of stages 2m-2, 2m-1 is free and takes slot
                // m-1+A_SLOTS; after an odd one (s = 2m+1) slot m+1 must land
                // before barrier 2m+2 publishes its first stage (the later
                // ones may stay in flight)
                for (int j = 0; j < ns; j += 2) {
                    stage_barrier();  // publishes stage j+1 (odd)
                    wait_vm<(T::A_SLOTS - 2) * NI>();
                    stage_barrier();  // publishes stage j+2 (even)
                    issue_a();
                }
            }
            wait_vm<0>();
        };
        // rounds the chunk needs: at most A_INSTR (A_INSTR rounds cover kRows);
        // every case runs the full barrier sequence
        constexpr int M = T::A_INSTR;
        switch ((nrows + T::A_ROUND - 1) / T::A_ROUND) {
            case 1: produce(std::integral_constant<int, 1>{}); break;
            case 2: produce(std::integral_constant<int, (2 < M ? 2 : M)>{}); break;
            case 3: produce(std::integral_constant<int, (3 < M ? 3 : M)>{}); break;
            case 4: produce(std::integral_constant<int, (4 < M ? 4 : M)>{}); break;
            case 5: produce(std::integral_constant<int, (5 < M ? 5 : M)>{}); break;
            case 6: produce(std::integral_constant<int, (6 < M ? 6 : M)>{}); break;
            case 7: produce(std::integral_constant<int, (7 < M ? 7 : M)>{}); break;
            case 8: produce(std::integral_constant<int, (8 < M ? 8 : M)>{}); break;
            case 9: produce(std::integral_constant<int, (9 < M ? 9 : M)>{}); break;
            case 10: produce(std::integral_constant<int, (10 < M ? 10 : M)>{}); break;
            case 11: produce(std::integral_constant<int, (11 < M ? 11 : M)>{}); break;
            default: produce(std::integral_constant<int, M>{}); break;
        }
        }
        return;
    }

    // ------------------------------- consumer -------------------------------
    // consumer (h, cgrp): row blocks h, h+2, ... and column tiles
    // cgrp*kTPC .. cgrp*kTPC+kTPC-1 of each group
    const int h = wv & 1, cgrp = wv >> 1;
    const int my_nrb = (nrb - h + 1) >> 1;  // row blocks 2*i + h, i < my_nrb
    Acc acc[kRBC][kTPC];
#pragma unroll
    for (int i = 0; i < kRBC; ++i)
#pragma unroll
        for (int n = 0; n < kTPC; ++n) acc[i][n] = Acc{0, 0, 0, 0};

    // Epilogue of group gi: lane (g, c16) holds rows 4g..4g+3 of each of its
    // row blocks in column c16 of each tile.  Per row block the wave writes
    // its 16 rows of bf16 results (GEMM1: SiLU(gate)*up of act columns; GEMM2:
    // y columns) to its staging tile in LDS and reads them back as 16-byte
    // row pieces (lane l: row l/4, pieces l%4 and l%4 + 4), which go to memory
    // whole: an eighth of the store instructions of 2-byte stores from the
    // accumulator layout (measured: those stores took a quarter of GEMM2 on
    // the Qwen3-235B-shaped INT8 layer at T=2048).  The rings keep streaming
    // the next group meanwhile.  The lane index passes through an empty asm
    // statement so that per-row addresses are formed here, not hoisted out of
    // the stage loop (where they would occupy registers for the whole loop).
    auto epi = [&](int gi, auto NRBc) {
        constexpr int NRB = decltype(NRBc)::value;
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int eg = ln >> 4, ec = ln & 15;
        const int pr = ln >> 2, pq = ln & 3;  // read-back: row and first piece
        const int gc = gfirst + gi;
        uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
        constexpr int ER = GEMM == 1 ? T::E_ROW1 : T::E_ROW2;  // staging row stride (bytes)
        constexpr int NP = GEMM == 1 ? 1 : 2;                   // 16-byte pieces per lane per row block
        char* et = smem + T::E_OFF + wv * T::E_WAVE;
        float wsc[kTPC];  // INT8 channel scales of this lane's columns
#pragma unroll
        for (int n = 0; n < kTPC; ++n) {
            wsc[n] = 1.f;
            if constexpr (WT == W_INT8)
                wsc[n] = reinterpret_cast<const float*>(smem + T::S_OFF)[(gi * T::TILES + cgrp * kTPC + n) * 16 + ec];
        }
#pragma unroll
        for (int i = 0; i < NRB; ++i) {
            const int r0 = (2 * i + h) * 16 + 4 * eg;  // this lane's rows r0 .. r0+3
            f32x4 rs4 = {1.f, 1.f, 1.f, 1.f};
            if constexpr (WT == W_INT8) rs4 = *reinterpret_cast<const f32x4*>(row_rs + r0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[kTPC];
#pragma unroll
                for (int n = 0; n < kTPC; ++n) {
                    if constexpr (WT == W_INT8)
                        v[n] = (float)acc[i][n][q] * rs4[q] * wsc[n];
                    else
                        v[n] = acc[i][n][q];
                }
                uint16_t* e = reinterpret_cast<uint16_t*>(et + (4 * eg + q) * ER) + ec;
                if constexpr (GEMM == 1) {
                    // tiles 2pp (gate) and 2pp+1 (up): staging column pp*16 + c16
#pragma unroll
                    for (int pp = 0; pp < kTPC / 2; ++pp) e[pp * 16] = f32_to_bf16_bits(silu(v[2 * pp]) * v[2 * pp + 1]);
                } else {
#pragma unroll
                    for (int n = 0; n < kTPC; ++n) e[n * 16] = f32_to_bf16_bits(v[n]);
                }
                __builtin_amdgcn_sched_barrier(0);  // one row at a time (registers)
            }
            // (the wave's own LDS writes complete before its reads: in order)
            const int rr = (2 * i + h) * 16 + pr;  // chunk row of this lane's pieces
            const int pid = row_pid[rr];
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int pc = pq + 4 * p;  // piece: columns 8*pc .. 8*pc+7 of the wave's
                const u32x4 v8 = *reinterpret_cast<const u32x4*>(et + pr * ER + pc * 16);
                if (pid < a.P_tot) {
                    if constexpr (GEMM == 1) {
                        // non-temporal: the intermediate is read by the next
                        // kernel only, so it need not take L2 lines from the
                        // chunk's activations (Qwen3-shaped T = 2048 layer,
                        // same box: GEMM1 295 -> 283 us, the layer 572 -> 565)
                        __builtin_nontemporal_store(
                            v8, reinterpret_cast<u32x4*>(out + (size_t)(ch.row_start + rr) * (a.N / 2) +
                                                         gc * T::TILE_W1 + cgrp * kTPC * 8 + pc * 8));
                    } else {
                        const int col = gc * T::TILE_W2 + cgrp * kTPC * 16 + pc * 8;
                        if (col < a.N) *reinterpret_cast<u32x4*>(out + (size_t)pid * a.N + col) = v8;
                    }
                }
            }
#pragma unroll
            for (int n = 0; n < kTPC; ++n) acc[i][n] = Acc{0, 0, 0, 0};
            __builtin_amdgcn_sched_barrier(0);  // one row block at a time (registers)
        }
    };

    switch (my_nrb) {
        case 1: consume<WT, 1>(smem, nkt, ns, h, cgrp, lane, acc, epi); break;
        case 2: consume<WT, 2>(smem, nkt, ns, h, cgrp, lane, acc, epi); break;
        case 3: consume<WT, 3>(smem, nkt, ns, h, cgrp, lane, acc, epi); break;
        case 4: consume<WT, 4>(smem, nkt, ns, h, cgrp, lane, acc, epi); break;
        case 5: consume<WT, 5>(smem, nkt, ns, h, cgrp, lane, acc, epi); break;
        case 6: consume<WT, 6>(smem, nkt, ns, h, cgrp, lane, acc, epi); break;
        default:  // no rows for this wave: keep the workgroup's barrier count
            for (int j = 0; j <= ns; ++j) stage_barrier();
            break;
    }
}

// Column groups per workgroup when the caller leaves it open: the widest
// span up to kMaxSpan that divides the chunk's groups evenly (equal
// workgroups) and still gives every CU at least two workgroups for the
// expected chunk count (one chunk per touched expert, more for experts beyond
// a chunk's rows).  A wider span streams the weights of several groups
// through the same rings, so the workgroup's set-up and its pipeline fill and
// drain are paid once per span instead of once per group (Qwen3-sized INT8
// layer, T=2048: GEMM1 330 -> 316 us at span 3, GEMM2 231 -> 221 us at span
// 4; an uneven span 3 over GEMM2's 16 groups measured slower than span 2).
constexpr int kMaxSpan = 4;
static int prefill_group_span(const GemmArgs& a) {
    static const int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
            n = 256;
        return n;
    }();
    const int64_t e_tot = a.E + (a.W_sh ? 1 : 0);
    const int64_t est = std::max<int64_t>(std::min<int64_t>(e_tot, a.P_tot), a.P_tot / kRows);
    int span = 1;
    for (int g = 2; g <= kMaxSpan; ++g)
        if (a.n_groups % g == 0 && est * (a.n_groups / g) >= 2 * (int64_t)cus) span = g;
    return span;
}

static_assert(PF<W_INT8>::TILES * 16 == prefill_cols(W_INT8) && PF<W_BF16>::TILES * 16 == prefill_cols(W_BF16),
              "the host plans column groups of the kernels' width");

// a.n_groups: column groups of a chunk (prefill_cols(wtype) weight columns
// each); a.group_span: groups per workgroup (0: chosen here).  The launch
// runs ceil(n_groups / span) workgroups per chunk slot.
template <int GEMM>
static hipError_t launch_prefill(int wtype, const GemmArgs& a, int max_chunks, hipStream_t st) {
    if (a.K % 128 != 0) return hipErrorInvalidValue;  // two stages per pipelined loop trip
    const int tiles = wtype == W_INT8 ? PF<W_INT8>::TILES : PF<W_BF16>::TILES;
    if (a.n_groups < 1 || (size_t)a.n_groups * tiles * 16 < (size_t)a.N) return hipErrorInvalidValue;
    GemmArgs b = a;
    b.col_groups = a.n_groups;
    b.group_span = a.group_span > 0 ? std::min(a.group_span, a.n_groups) : prefill_group_span(a);
    b.group_span = std::min(b.group_span, wtype == W_INT8 ? PF<W_INT8>::MAX_SPAN : PF<W_BF16>::MAX_SPAN);
    b.n_groups = (a.n_groups + b.group_span - 1) / b.group_span;
    const int slots_per_xcd = (max_chunks + 7) / 8;
    dim3 grid((unsigned)(8 * (size_t)slots_per_xcd * b.n_groups));
    if (wtype == W_INT8)
        prefill_kernel<W_INT8, GEMM><<<grid, PF<W_INT8>::NWAVES * 64, 0, st>>>(b);
    else
        prefill_kernel<W_BF16, GEMM><<<grid, PF<W_BF16>::NWAVES * 64, 0, st>>>(b);
    return hipGetLastError();
}

hipError_t launch_prefill_gemm1(int wtype, const GemmArgs& a, int max_chunks, hipStream_t st) {
    if (wtype == W_FP8) return launch_prefill_f8_gemm1(a, max_chunks, st);
    return launch_prefill<1>(wtype, a, max_chunks, st);
}
hipError_t launch_prefill_gemm2(int wtype, const GemmArgs& a, int max_chunks, hipStream_t st) {
    if (wtype == W_FP8) return launch_prefill_f8_gemm2(a, max_chunks, st);
    return launch_prefill<2>(wtype, a, max_chunks, st);
}

}  // namespace moe
