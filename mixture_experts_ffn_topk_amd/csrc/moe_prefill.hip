// moe_prefill.hip -- MFMA tile grouped GEMMs for many rows per expert, BF16
// and INT8 weights (FP8 weights: moe_prefill_f8.hip).
//
// A workgroup owns one chunk of up to 192 sorted rows of one expert and a
// column group of weight columns (MFMA column tiles of 16: for GEMM1 gate
// tiles interleaved with the matching up tiles, so SiLU(C1)*C2 stays
// lane-local) over the full K range, so each weight byte of a column group is
// fetched from HBM once per chunk and needs no cross-workgroup reduction.
// K advances in 64-deep stages.  BF16: 128 columns, 8 waves; INT8: 256
// columns, 12 waves (wave roles: PF below).
//
// The waves specialise:
//   producers (the waves after the consumers) only issue direct global->LDS loads
//     (global_load_lds_dwordx4: lane l's 16 bytes land at slot + 16*l) into
//     an activation ring (the chunk's rows, gathered through sorted_ids for
//     GEMM1, mostly L2 hits) and a weight ring (the HBM stream, several
//     stages ahead);
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
    static constexpr int A_PARTS = A_ROW / 16;         // 16-byte parts per row (8 or 4)
    // rows whose same-numbered part must fall in distinct LDS banks: the
    // 16 rows of an MFMA fragment, read by one 16-lane group
    static constexpr int SWZ_SHIFT = A_PARTS == 8 ? 1 : 2;
    static constexpr int A_SLOT = kRows * A_ROW;
    // activation stages requested ahead of the stage being published (the
    // rows come from L2 with high latency under the weight stream)
    static constexpr int A_AHEAD = WT == W_INT8 ? 4 : 3;
    static constexpr int A_SLOTS = A_AHEAD;
    static constexpr int B_TILE = 64 * 16 * EB;        // one packed k-tile of one column tile
    static constexpr int B_SLOT = TILES * B_TILE;
    // weight stages requested ahead of the stage being published (= ring
    // slots); a weight wave keeps B_AHEAD - 1 stages counted in vmcnt (6 bits)
    static constexpr int B_AHEAD = WT == W_BF16 ? 4 : 6;
    static constexpr int B_SLOTS = B_AHEAD;
    // direct-to-LDS instructions per stage (1 KiB each): the weight waves
    // split the weight stage, the activation waves share the activation rows
    // in rounds of NAW instructions
    static constexpr int B_INSTR = B_SLOT / 1024;
    static constexpr int BIW = B_INSTR / NBW;                          // per weight wave
    static constexpr int ROWS_PER_INSTR = 1024 / A_ROW;
    static constexpr int A_ROUND = NAW * ROWS_PER_INSTR;               // rows per round
    static constexpr int A_INSTR = (kRows + A_ROUND - 1) / A_ROUND;    // rounds for a full chunk
    static_assert(B_INSTR % NBW == 0, "weight stage split");
    static_assert((B_AHEAD - 1) * BIW < 64, "weight wave vmcnt range");
    // shared-memory layout
    static constexpr int A_OFF = 0;
    static constexpr int B_OFF = A_OFF + A_SLOTS * A_SLOT;
    // row table: source row, pair id and activation row scale per chunk row
    static constexpr int R_OFF = B_OFF + B_SLOTS * B_SLOT;
    static constexpr int SMEM = R_OFF + kRows * 12;
    // epilogue: the bf16 output tile (act columns for GEMM1, TILES tiles of y
    // for GEMM2) is staged in the rings, free after the main loop
    static constexpr int TILE_W1 = TILES * 16 / 2, TILE_W2 = TILES * 16;
    static_assert(kRows * TILE_W2 * 2 <= R_OFF, "epilogue tile fits the rings");
    static_assert(SMEM <= 160 * 1024, "LDS budget");
    static_assert(B_AHEAD >= 3, "in-order load completion argument needs 3 stages");
    typedef typename std::conditional<WT == W_INT8, i32x4, f32x4>::type Acc;
};

// byte offset of (row, logical 16-byte part) in an activation slot
template <int WT>
__device__ inline int a_off(int row, int part) {
    using T = PF<WT>;
    return row * T::A_ROW + ((part ^ ((row >> T::SWZ_SHIFT) & (T::A_PARTS - 1))) << 4);
}

// ----------------------------------------------------------------------------
// BF16 / INT8 consumer main loop for NRB row blocks per wave (1..6), fully
// unrolled over row blocks so every LDS wait count is exact.
// ----------------------------------------------------------------------------
template <int WT, int NRB>
__device__ __attribute__((always_inline)) inline void consume(char* smem, int nkt, int h, int cgrp, int lane,
                               typename PF<WT>::Acc (&acc)[kRBC][kTPC]) {
    using T = PF<WT>;
    const int g = lane >> 4, c16 = lane & 15;
    // rows of row block i: (2i + h)*16 + c16; the swizzle term depends on c16 only
    const int row = h * 16 + c16;
    const uint32_t a_base = lds_addr(smem + T::A_OFF);
    constexpr int RB_STRIDE = 32 * T::A_ROW;  // bytes between this wave's row blocks
    // B fragment addresses (stage slot added per stage)
    const uint32_t b_base =
        lds_addr(smem + T::B_OFF) + cgrp * 4 * T::B_TILE + lane * (WT == W_BF16 ? 32 : 16);
    auto b_slot = [&](int s) -> uint32_t { return (uint32_t)((s % T::B_SLOTS) * T::B_SLOT); };

    if constexpr (WT == W_INT8) {
        const uint32_t a_lo = a_base + a_off<WT>(row, g);
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
        static_for<NRB>([&](auto I) { ldA(a_lo, I); });
        ldB(b_base + b_slot(0), bA);
        auto stage = [&](int j, u32x4 (&b)[4], u32x4 (&nb)[4]) {
            sync(b);
            stage_barrier();  // stage j+1 published
            ldB(b_base + b_slot(j + 1), nb);
            const uint32_t ab = a_lo + ((j + 1) % T::A_SLOTS) * T::A_SLOT;
            static_for<NRB>([&](auto I) {
                constexpr int i = decltype(I)::value;
#pragma unroll
                for (int n = 0; n < 4; ++n) acc[i][n] = mfma_i8(af[i], b[n], acc[i][n]);
                __builtin_amdgcn_sched_barrier(0);
                ldA(ab, I);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        for (int j = 0; j < nkt; j += 2) {
            stage(j, bA, bB);
            stage(j + 1, bB, bA);
        }
        sync(bA);
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
        auto stage = [&](int j, u32x4 (&b)[4][2], u32x4 (&nb)[4][2]) {
            sync(b);
            stage_barrier();  // stage j+1 published
            ldB(b_base + b_slot(j + 1), nb);
            const uint32_t so = ((j + 1) % T::A_SLOTS) * T::A_SLOT;
            const uint32_t lo = a_lo + so, hi = a_hi + so;
            static_for<NRB>([&](auto I) {
                constexpr int i = decltype(I)::value;
                const bf16x8 a0 = __builtin_bit_cast(bf16x8, af[i][0]);
                const bf16x8 a1 = __builtin_bit_cast(bf16x8, af[i][1]);
#pragma unroll
                for (int n = 0; n < 4; ++n)
                    acc[i][n] = mfma_bf16(a0, __builtin_bit_cast(bf16x8, b[n][0]), acc[i][n]);
#pragma unroll
                for (int n = 0; n < 4; ++n)
                    acc[i][n] = mfma_bf16(a1, __builtin_bit_cast(bf16x8, b[n][1]), acc[i][n]);
                __builtin_amdgcn_sched_barrier(0);
                ldA(lo, hi, I);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        for (int j = 0; j < nkt; j += 2) {
            stage(j, bA, bB);
            stage(j + 1, bB, bA);
        }
        sync(bA);
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
    const int lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int ci = (slot / a.n_groups) * 8 + xcd;
    const int grp = slot % a.n_groups;
    if (ci >= a.meta[1]) return;  // uniform for the whole workgroup
    const Chunk ch = a.chunks[ci];
    const int nrows = ch.nrows;
    const int nrb = nrows >> 4;

    const bool sh = ch.expert >= a.E;
    const size_t wbytes = (size_t)a.K * a.N * T::EB;
    const uint8_t* W = sh ? a.W_sh : a.W + (size_t)ch.expert * wbytes;
    static_assert(WT != W_FP8, "FP8 weights use prefill_f8_kernel");
    const int nsc = a.N;  // INT8: one scale per output channel
    const float* ws = sh ? a.w_scale_sh : (a.w_scale ? a.w_scale + (size_t)ch.expert * nsc : nullptr);
    const int nkt = a.K / 64;  // even: K is a multiple of 128

    // logical first column of packed tile nt (this workgroup owns tiles
    // grp*TILES .. grp*TILES+TILES-1)
    auto col_of = [&](int nt) { return GEMM == 1 ? (nt & 1) * (a.N / 2) + (nt >> 1) * 16 : nt * 16; };

    // the weight waves need no row table: their first stages go out before
    // the table's barrier, so their HBM latency overlaps the table set-up.
    // Weight wave wb issues 1 KiB pieces wb*BIW .. wb*BIW+BIW-1 of each
    // stage; tiles past the last one (a partial last column group) re-read it
    const int wb = wv - (T::NCONS + T::NAW);
    const int ntiles = a.N / 16;
    auto issue_b = [&](int s) {
        const size_t off = (size_t)min(s, nkt - 1) * T::B_TILE;
        char* dst = smem + T::B_OFF + (s % T::B_SLOTS) * T::B_SLOT;
#pragma unroll
        for (int q = 0; q < T::BIW; ++q) {
            const int i = wb * T::BIW + q;
            // 1 KiB piece i of the slot: tile i*1024/B_TILE, offset i*1024%B_TILE
            const int tile = min(grp * T::TILES + i * 1024 / T::B_TILE, ntiles - 1);
            const int within = i * 1024 % T::B_TILE;
            lds_dma16_stream(W + packed_tile_offset(T::EB, a.K, tile, 0) + lane * 16 + within + off,
                             dst + i * 1024);
        }
    };
    if (wb >= 0)
        for (int s = 0; s < T::B_AHEAD; ++s) issue_b(s);

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
    __syncthreads();

    Acc acc[kRBC][kTPC];
    int col0[kTPC];
    const int h = wv & 1, cgrp = wv >> 1;  // consumer: row-block parity, column group
    bool has_rows = false;

    if (wv >= T::NCONS) {
        // ------------------------------ producer ------------------------------
        // NAW waves load activation rows, NBW waves load weights, so each
        // wave's vmcnt counts only its own stream: a weight wave keeps
        // B_AHEAD stages in flight while an activation wave waits for its own
        // rows only (loads retire in issue order within a wave).  Every stage
        // issues the same loads, so the wait counts are constants; K stages
        // past the end re-read the last stage.
        const int pw = wv - T::NCONS;
        if (wb >= 0) {  // its first B_AHEAD stages are already requested
            wait_vm<(T::B_AHEAD - 1) * T::BIW>();  // stage 0
            stage_barrier();                         // publishes stage 0
            wait_vm<(T::B_AHEAD - 2) * T::BIW>();  // stage 1
            for (int j = 0; j < nkt; ++j) {
                stage_barrier();  // publishes stage j+1; stage j's slot is free
                issue_b(j + T::B_AHEAD);
                wait_vm<(T::B_AHEAD - 2) * T::BIW>();  // stage j+2 landed
            }
            wait_vm<0>();  // no load may land after the rings are reused
        } else {
        // activation waves: rows are loaded in rounds of A_ROUND rows
        // (instruction i of wave pw takes rows (NAW*i + pw) * ROWS_PER_INSTR ..),
        // only as many rounds as the chunk needs; rows of the last round past
        // the chunk re-read its first row (never stored back)
        auto produce = [&](auto NIc) {
            constexpr int NI = decltype(NIc)::value;  // instructions per stage
            const char* a_src[NI];
            int a_lds[NI];
            const int src0 = row_src[0];  // the first row of a chunk is always a real pair
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int row0 = (T::NAW * i + pw) * T::ROWS_PER_INSTR;
                const int row = row0 + lane / T::A_PARTS;
                const int q = lane % T::A_PARTS;  // LDS part slot of this lane
                const int part = q ^ ((row >> T::SWZ_SHIFT) & (T::A_PARTS - 1));  // logical part it holds
                int src = row < nrows ? row_src[row] : -1;
                if (src < 0) src = src0;
                a_src[i] = (const char*)a.A + (size_t)src * a.K * T::AEB + part * 16;
                a_lds[i] = row0 * T::A_ROW;
            }
            auto issue_a = [&](int s) {
                const size_t off = (size_t)min(s, nkt - 1) * T::A_ROW;
                char* dst = smem + T::A_OFF + (s % T::A_SLOTS) * T::A_SLOT;
#pragma unroll
                for (int i = 0; i < NI; ++i) lds_dma16(a_src[i] + off, dst + a_lds[i]);
            };
            for (int s = 0; s < T::A_AHEAD; ++s) issue_a(s);
            wait_vm<(T::A_AHEAD - 1) * NI>();  // stage 0
            stage_barrier();                     // publishes stage 0
            wait_vm<(T::A_AHEAD - 2) * NI>();  // stage 1
            for (int j = 0; j < nkt; ++j) {
                stage_barrier();  // publishes stage j+1; the slots consumers released are free
                issue_a(j + T::A_AHEAD);
                wait_vm<(T::A_AHEAD - 2) * NI>();  // stage j+2 landed; later stages may stay in flight
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
            default: produce(std::integral_constant<int, M>{}); break;
        }
        }
    } else {
    // ------------------------------- consumer -------------------------------
    const int my_nrb = (nrb - h + 1) >> 1;  // row blocks 2*i + h, i < my_nrb
    has_rows = my_nrb > 0;
#pragma unroll
    for (int i = 0; i < kRBC; ++i)
#pragma unroll
        for (int n = 0; n < kTPC; ++n) acc[i][n] = Acc{0, 0, 0, 0};
#pragma unroll
    for (int n = 0; n < kTPC; ++n) col0[n] = col_of(min(grp * T::TILES + cgrp * kTPC + n, ntiles - 1));

    switch (my_nrb) {
        case 1: consume<WT, 1>(smem, nkt, h, cgrp, lane, acc); break;
        case 2: consume<WT, 2>(smem, nkt, h, cgrp, lane, acc); break;
        case 3: consume<WT, 3>(smem, nkt, h, cgrp, lane, acc); break;
        case 4: consume<WT, 4>(smem, nkt, h, cgrp, lane, acc); break;
        case 5: consume<WT, 5>(smem, nkt, h, cgrp, lane, acc); break;
        case 6: consume<WT, 6>(smem, nkt, h, cgrp, lane, acc); break;
        default:  // no rows for this wave: keep the workgroup's barrier count
            for (int j = 0; j <= nkt; ++j) stage_barrier();
            break;
    }
    }

    // ---- epilogue: consumers stage bf16 results in the (now free) rings,
    // then every thread writes whole rows with 16-byte stores; pair ids and
    // row scales come from the row table ----
    constexpr int TW = GEMM == 1 ? T::TILE_W1 : T::TILE_W2;
    uint16_t* tile = reinterpret_cast<uint16_t*>(smem + T::A_OFF);
    __syncthreads();  // every load has landed and every ring read is done
    if (has_rows) {
        float wsc[kTPC];
#pragma unroll
        for (int n = 0; n < kTPC; ++n) wsc[n] = 1.f;
        if constexpr (WT == W_INT8) {
#pragma unroll
            for (int n = 0; n < kTPC; ++n) wsc[n] = ws[col0[n] + c16];
        }
#pragma unroll
        for (int i = 0; i < kRBC; ++i) {
            const int rbk = 2 * i + h;
            if (rbk >= nrb) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = rbk * 16 + 4 * g + q;
                const float rs = row_rs[r];
                float v[kTPC];
#pragma unroll
                for (int n = 0; n < kTPC; ++n) {
                    if constexpr (WT == W_INT8)
                        v[n] = (float)acc[i][n][q] * rs * wsc[n];
                    else
                        v[n] = acc[i][n][q];
                }
                if constexpr (GEMM == 1) {
                    // tiles 2pp (gate) and 2pp+1 (up) of this consumer: act
                    // columns cgrp*kTPC*8 + pp*16 + c16 of the workgroup's TW
#pragma unroll
                    for (int pp = 0; pp < kTPC / 2; ++pp)
                        tile[r * TW + cgrp * kTPC * 8 + pp * 16 + c16] =
                            f32_to_bf16_bits(silu(v[2 * pp]) * v[2 * pp + 1]);
                } else {
#pragma unroll
                    for (int n = 0; n < kTPC; ++n)
                        tile[r * TW + (cgrp * kTPC + n) * 16 + c16] = f32_to_bf16_bits(v[n]);
                }
            }
        }
    }
    __syncthreads();
    constexpr int CPR = TW / 8;  // 16-byte pieces per row
    // output columns of this group (a last group may be partial: its tiles
    // past the end computed a copy of the last tile, which is not stored)
    const int ncol = min(TW, (GEMM == 1 ? a.N / 2 : a.N) - grp * TW);
    for (int idx = tid; idx < nrows * CPR; idx += blockDim.x) {
        const int r = idx / CPR, c8 = (idx % CPR) * 8;
        const int pid = row_pid[r];
        if (pid >= a.P_tot || c8 >= ncol) continue;
        const u32x4 v = *reinterpret_cast<const u32x4*>(tile + r * TW + c8);
        if constexpr (GEMM == 1)
            *reinterpret_cast<u32x4*>((uint16_t*)a.out + (size_t)(ch.row_start + r) * (a.N / 2) + grp * TW + c8) = v;
        else
            *reinterpret_cast<u32x4*>((uint16_t*)a.out + (size_t)pid * a.N + grp * TW + c8) = v;
    }
}

template <int GEMM>
static hipError_t launch_prefill(int wtype, const GemmArgs& a, int max_chunks, hipStream_t st) {
    if (a.K % 128 != 0) return hipErrorInvalidValue;  // two stages per pipelined loop trip
    const int slots_per_xcd = (max_chunks + 7) / 8;
    dim3 grid((unsigned)(8 * (size_t)slots_per_xcd * a.n_groups));
    if (wtype == W_INT8) {
        using T = PF<W_INT8>;
        if ((size_t)a.n_groups * T::TILES * 16 < (size_t)a.N) return hipErrorInvalidValue;
        prefill_kernel<W_INT8, GEMM><<<grid, T::NWAVES * 64, 0, st>>>(a);
    } else {
        using T = PF<W_BF16>;
        if ((size_t)a.n_groups * T::TILES * 16 < (size_t)a.N) return hipErrorInvalidValue;
        prefill_kernel<W_BF16, GEMM><<<grid, T::NWAVES * 64, 0, st>>>(a);
    }
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
