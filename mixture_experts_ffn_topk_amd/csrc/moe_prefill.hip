// moe_prefill.hip -- MFMA tile grouped GEMMs for many rows per expert.
//
// A workgroup owns one chunk of up to 192 sorted rows of one expert and 128
// weight columns (8 MFMA column tiles: for GEMM1 four gate tiles interleaved
// with the four matching up tiles, so SiLU(C1)*C2 stays lane-local) over the
// full K range, so each weight byte of a column block is fetched from HBM
// once per chunk and needs no cross-workgroup reduction.
//
// The 8 waves specialise:
//   producers (waves 4..7) only issue direct global->LDS loads
//     (global_load_lds_dwordx4: each lane's 16 bytes land at slot + 16*lane)
//     into two LDS rings: the 8 packed weight tiles of a 64-row K stage
//     (HBM stream, 64 KiB in flight per workgroup) and the chunk's activation
//     rows (gathered through sorted_ids for GEMM1, mostly L2 hits, two stages
//     in flight).  Before the barrier that publishes stage kt a producer
//     waits (explicit vmcnt) until its own loads of stage kt have landed;
//   consumers (waves 0..3, one per SIMD) read their fragments from LDS,
//     widen FP8 weight codes to bf16 with the 128x128 block scale folded in
//     (dequantise-then-GEMM) and run bf16 MFMA 16x16x32 (i8 MFMA 16x16x64
//     for INT8); consumer (h, c) owns row blocks h, h+2, ... and 4 of the 8
//     column tiles.
// No wave both loads into LDS and reads it, so neither role carries waits
// for the other's traffic; one barrier per K stage orders the rings.
// Workgroup ids are dealt round-robin to the 8 XCDs; consecutive ids of one
// XCD take the column groups of one chunk, so the chunk's activation rows
// are shared through that XCD's L2 while its weights stream from HBM once.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int kRows = 16 * kPrefillMB;     // rows per chunk (12 row blocks)
constexpr int kRBC = kPrefillMB / 2;       // row blocks per consumer wave
constexpr int kTiles = 8;                  // 16-column tiles per workgroup
constexpr int kAStages = 2;                // activation stages in flight
constexpr int kBBytes = 64 * 1024;         // weight bytes in flight per workgroup

template <int WT>
struct PF {
    static constexpr int EB = WT == W_BF16 ? 2 : 1;    // weight element bytes
    static constexpr int AEB = WT == W_INT8 ? 1 : 2;   // activation element bytes
    static constexpr int A_ROW = 64 * AEB;             // bytes per row per K stage
    static constexpr int A_PARTS = A_ROW / 16;         // 16-byte parts per row
    static constexpr int A_SLOT = kRows * A_ROW;
    static constexpr int A_SLOTS = kAStages + 1;
    static constexpr int B_TILE = 64 * 16 * EB;        // one packed k-tile of one column tile
    static constexpr int B_SLOT = kTiles * B_TILE;
    static constexpr int B_STAGES = kBBytes / B_SLOT;  // 8 (8-bit weights) or 4 (bf16)
    static constexpr int B_SLOTS = B_STAGES + 1;
    // direct-to-LDS instructions per producer wave per stage (1 KiB each)
    static constexpr int A_INSTR = A_SLOT / 1024 / 4;
    static constexpr int B_INSTR = B_SLOT / 1024 / 4;
    static constexpr int ROWS_PER_INSTR = 1024 / A_ROW;
    typedef typename std::conditional<WT == W_INT8, i32x4, f32x4>::type Acc;
};

// Barrier that orders LDS traffic only (used by the consumers).
__device__ inline void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// XOR swizzle of a row's 16-byte parts: consecutive rows reading the same
// logical part hit different LDS banks.  (row, logical part) -> byte offset.
__device__ inline int a_off(int row, int part, int parts) {
    return row * parts * 16 + ((part ^ (row & (parts - 1))) << 4);
}

// Producer wait: at most N of this wave's vector-memory operations (its
// direct-to-LDS loads) may still be outstanding.
template <int N>
__device__ inline void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if constexpr (N == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else if constexpr (N == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if constexpr (N == 10) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    else static_assert(N == 0, "add this vmcnt value");
}

}  // namespace

template <int WT, int GEMM>
__global__ __launch_bounds__(512, 1) void prefill_kernel(GemmArgs a) {
    using T = PF<WT>;
    using Acc = typename T::Acc;
    __shared__ __attribute__((aligned(1024))) char lds_a[T::A_SLOTS][T::A_SLOT];
    __shared__ __attribute__((aligned(1024))) char lds_b[T::B_SLOTS][T::B_SLOT];
    __shared__ int row_src[kRows];

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
    const int nsc = WT == W_FP8 ? (a.K / 128) * (a.N / 128) : a.N;
    const float* ws = sh ? a.w_scale_sh : (a.w_scale ? a.w_scale + (size_t)ch.expert * nsc : nullptr);
    const int nkt = a.K / 64;

    // logical first column of packed tile nt (this workgroup owns tiles grp*8 .. grp*8+7)
    auto col_of = [&](int nt) { return GEMM == 1 ? (nt & 1) * (a.N / 2) + (nt >> 1) * 16 : nt * 16; };

    if (tid < kRows) {
        int src = -1;
        if (tid < nrows) {
            const int pid = a.sorted_ids[ch.row_start + tid];
            if (pid < a.P_tot) {
                if (GEMM == 1)
                    src = pid < a.P ? pid / a.topk : pid - a.P;
                else
                    src = ch.row_start + tid;
            }
        }
        row_src[tid] = src;
    }
    __syncthreads();

    if (wv >= 4) {
        // ------------------------------ producer ------------------------------
        // Every stage issues the same loads, so the wait count is a constant:
        // rows past the chunk re-read its first row (their results are never
        // read back), K stages past the end re-read the last stage.
        const int pw = wv - 4;
        const char* a_src[T::A_INSTR];
        int a_lds[T::A_INSTR];
        const int src0 = row_src[0];  // the first row of a chunk is always a real pair
#pragma unroll
        for (int i = 0; i < T::A_INSTR; ++i) {
            const int row0 = (pw * T::A_INSTR + i) * T::ROWS_PER_INSTR;
            const int row = row0 + lane / T::A_PARTS;
            const int q = lane % T::A_PARTS;                 // LDS part slot of this lane
            const int part = q ^ (row & (T::A_PARTS - 1));   // logical part it holds
            int src = row < nrows ? row_src[row] : -1;
            if (src < 0) src = src0;
            a_src[i] = (const char*)a.A + (size_t)src * a.K * T::AEB + part * 16;
            a_lds[i] = row0 * T::A_ROW;
        }
        const uint8_t* b_src[T::B_INSTR];
        int b_lds[T::B_INSTR];
#pragma unroll
        for (int i = 0; i < T::B_INSTR; ++i) {
            const int piece = pw * T::B_INSTR + i;            // 1 KiB piece of the slot
            const int tile = piece * 1024 / T::B_TILE;
            const int within = piece * 1024 % T::B_TILE;
            b_src[i] = W + packed_tile_offset(T::EB, a.K, grp * kTiles + tile, 0) + within +
                       lane * 16;
            b_lds[i] = piece * 1024;
        }
        auto issue_a = [&](int kt) {
            const size_t off = (size_t)min(kt, nkt - 1) * T::A_ROW;
            char* slot_a = lds_a[kt % T::A_SLOTS];
#pragma unroll
            for (int i = 0; i < T::A_INSTR; ++i)
                lds_dma16(a_src[i] + off, slot_a + a_lds[i]);
        };
        auto issue_b = [&](int kt) {
            const size_t off = (size_t)min(kt, nkt - 1) * T::B_TILE;
            char* slot_b = lds_b[kt % T::B_SLOTS];
#pragma unroll
            for (int i = 0; i < T::B_INSTR; ++i)
                lds_dma16(b_src[i] + off, slot_b + b_lds[i]);
        };
        // prologue: weights B_STAGES stages ahead, then activations kAStages
        for (int s = 0; s < T::B_STAGES; ++s) issue_b(s);
        for (int s = 0; s < kAStages; ++s) issue_a(s);
        for (int kt = 0; kt < nkt; ++kt) {
            // stage kt's activation loads are the oldest not yet waited for;
            // everything issued after them may stay in flight
            if (kt == 0)
                wait_vm<(kAStages - 1) * T::A_INSTR>();
            else
                wait_vm<(kAStages - 1) * (T::A_INSTR + T::B_INSTR)>();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();  // publishes stage kt; stage kt-1's slots are free
            __builtin_amdgcn_sched_barrier(0);
            issue_b(kt + T::B_STAGES);
            issue_a(kt + kAStages);
        }
        return;
    }

    // ------------------------------- consumer -------------------------------
    const int h = wv & 1, cgrp = wv >> 1;  // row-block parity, column half
    const int my_nrb = (nrb - h + 1) >> 1;  // row blocks 2*i + h, i < my_nrb
    Acc acc[kRBC][4];
#pragma unroll
    for (int i = 0; i < kRBC; ++i)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[i][n] = Acc{0, 0, 0, 0};
    const int nbw = a.N / 128;
    int col0[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) col0[n] = col_of(grp * kTiles + cgrp * 4 + n);

    auto compute = [&](int kt) {
        const char* la = lds_a[kt % T::A_SLOTS];
        const char* lb = lds_b[kt % T::B_SLOTS] + cgrp * 4 * T::B_TILE;
        if constexpr (WT == W_INT8) {
            u32x4 b[4];
#pragma unroll
            for (int n = 0; n < 4; ++n) b[n] = *reinterpret_cast<const u32x4*>(lb + n * T::B_TILE + lane * 16);
            u32x4 an = {0, 0, 0, 0};
            if (my_nrb > 0)
                an = *reinterpret_cast<const u32x4*>(la + a_off(h * 16 + c16, g, T::A_PARTS));
#pragma unroll
            for (int i = 0; i < kRBC; ++i) {
                if (i < my_nrb) {
                    const u32x4 av = an;
                    if (i + 1 < my_nrb)
                        an = *reinterpret_cast<const u32x4*>(
                            la + a_off((2 * (i + 1) + h) * 16 + c16, g, T::A_PARTS));
#pragma unroll
                    for (int n = 0; n < 4; ++n) acc[i][n] = mfma_i8(av, b[n], acc[i][n]);
                }
            }
        } else {
            bf16x8 b0[4], b1[4];
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                if constexpr (WT == W_FP8) {
                    const u32x4 raw = *reinterpret_cast<const u32x4*>(lb + n * T::B_TILE + lane * 16);
                    const float sc = ws[(kt >> 1) * nbw + col0[n] / 128];
                    fp8x16_to_frags_scaled(raw, sc, b0[n], b1[n]);
                } else {
                    const char* bt = lb + n * T::B_TILE + lane * 32;
                    b0[n] = *reinterpret_cast<const bf16x8*>(bt);
                    b1[n] = *reinterpret_cast<const bf16x8*>(bt + 16);
                }
            }
            bf16x8 a0n = {}, a1n = {};
            if (my_nrb > 0) {
                const int r = h * 16 + c16;
                a0n = *reinterpret_cast<const bf16x8*>(la + a_off(r, g, T::A_PARTS));
                a1n = *reinterpret_cast<const bf16x8*>(la + a_off(r, 4 + g, T::A_PARTS));
            }
#pragma unroll
            for (int i = 0; i < kRBC; ++i) {
                if (i < my_nrb) {
                    const bf16x8 a0 = a0n, a1 = a1n;
                    if (i + 1 < my_nrb) {  // next row block's fragments under this one's MFMAs
                        const int r = (2 * (i + 1) + h) * 16 + c16;
                        a0n = *reinterpret_cast<const bf16x8*>(la + a_off(r, g, T::A_PARTS));
                        a1n = *reinterpret_cast<const bf16x8*>(la + a_off(r, 4 + g, T::A_PARTS));
                    }
#pragma unroll
                    for (int n = 0; n < 4; ++n) acc[i][n] = mfma_bf16(a0, b0[n], acc[i][n]);
#pragma unroll
                    for (int n = 0; n < 4; ++n) acc[i][n] = mfma_bf16(a1, b1[n], acc[i][n]);
                }
            }
        }
    };

    for (int kt = 0; kt < nkt; ++kt) {
        lds_barrier();
        compute(kt);
    }

    // epilogue: this consumer's rows and its 4 column tiles
#pragma unroll
    for (int i = 0; i < kRBC; ++i) {
        const int rbk = 2 * i + h;
        if (rbk >= nrb) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int grow = ch.row_start + rbk * 16 + 4 * g + q;
            const int pid = a.sorted_ids[grow];
            if (pid >= a.P_tot) continue;
            if constexpr (GEMM == 1) {
                const int I = a.N / 2;
                float sx = 1.f;
                if constexpr (WT == W_INT8) sx = a.a_scale[pid < a.P ? pid / a.topk : pid - a.P];
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    float gv, uv;
                    if constexpr (WT == W_INT8) {
                        gv = (float)acc[i][2 * pp][q] * sx * ws[col0[2 * pp] + c16];
                        uv = (float)acc[i][2 * pp + 1][q] * sx * ws[col0[2 * pp + 1] + c16];
                    } else {
                        gv = acc[i][2 * pp][q];
                        uv = acc[i][2 * pp + 1][q];
                    }
                    ((uint16_t*)a.out)[(size_t)grow * I + col0[2 * pp] + c16] =
                        f32_to_bf16_bits(silu(gv) * uv);
                }
            } else {
                float sa = 1.f;
                if constexpr (WT == W_INT8) sa = a.a_scale[grow];
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    float v;
                    if constexpr (WT == W_INT8)
                        v = (float)acc[i][n][q] * sa * ws[col0[n] + c16];
                    else
                        v = acc[i][n][q];
                    ((uint16_t*)a.out)[(size_t)pid * a.N + col0[n] + c16] = f32_to_bf16_bits(v);
                }
            }
        }
    }
}

template <int GEMM>
static hipError_t launch_prefill(int wtype, const GemmArgs& a, int max_chunks, hipStream_t st) {
    const int slots_per_xcd = (max_chunks + 7) / 8;
    dim3 grid((unsigned)(8 * (size_t)slots_per_xcd * a.n_groups));
    if (wtype == W_FP8)
        prefill_kernel<W_FP8, GEMM><<<grid, 512, 0, st>>>(a);
    else if (wtype == W_INT8)
        prefill_kernel<W_INT8, GEMM><<<grid, 512, 0, st>>>(a);
    else
        prefill_kernel<W_BF16, GEMM><<<grid, 512, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_prefill_gemm1(int wtype, const GemmArgs& a, int max_chunks, hipStream_t st) {
    return launch_prefill<1>(wtype, a, max_chunks, st);
}
hipError_t launch_prefill_gemm2(int wtype, const GemmArgs& a, int max_chunks, hipStream_t st) {
    return launch_prefill<2>(wtype, a, max_chunks, st);
}

}  // namespace moe
