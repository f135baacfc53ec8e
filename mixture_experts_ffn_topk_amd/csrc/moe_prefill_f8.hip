// moe_prefill_f8.hip -- FP8-weight grouped GEMMs for many rows per expert:
// native FP8 MFMA (32x32x64, E4M3 x E4M3) against the raw weight codes.
//
// Activations.  A bf16 value has 8 significant bits, an E4M3 value 4.  After
// a row is multiplied by the power of two 2^e that brings its largest
// magnitude to at most 448, every element x' splits into hi = E4M3(x') and
// lo = E4M3(x' - hi), and hi + lo == x' exactly whenever lo lands on the E4M3
// grid (always for |x'| >= 1/4; below that the error is under 2^-10, against
// row maxima of at least 224).  So x.w = 2^-e (hi.w + lo.w): two FP8 MFMAs,
// which at twice the bf16 rate cost the time of one bf16 MFMA, and the weight
// codes are used as stored (no widening).  split_rows_kernel writes the
// records once per GEMM input: per row and 64-deep K stage 128 bytes, eight
// 16-byte parts; part p < 4 holds hi of k = 8p .. 8p+7 then k = 32+8p .. +7
// (the k-slots of lane group p in a packed weight k-tile), part 4+p the lo
// codes of the same k.  The FP8 MFMA pairs A and B operand bytes by lane
// half and byte position, so lane (row r, half q) reading parts 2q, 2q+1 and
// the B lane (column c, half q) reading packed lane groups 2q, 2q+1 contract
// exactly the k they share.
//
// Block scales.  A 128x128 weight block's scale s = m * 2^p (m in [1, 2))
// enters the MFMA twice: 2^p as the MFMA's own E8M0 B scale (exact), m by
// rescaling the fp32 running sums by m_prev / m at each new K block and by
// the last m at the end, so every block's partial product is weighted by its
// own scale.  E8M0 has no zero: a zero scale is applied as 2^-127 with unit
// m, exact for the all-zero code blocks an amax-based quantiser gives a zero
// scale (otherwise off by under 1e-30 absolute).
// The row's 2^-e is applied in the epilogue.
//
// Tiling.  A workgroup owns one chunk of up to 160 sorted rows of one expert
// and 256 weight columns over the full K range (each weight byte of a column
// block streams from HBM once per chunk).  8 waves, two per SIMD: wave (s, h)
// owns column pair s (for GEMM1 a 32-column gate block and the matching up
// block, so SiLU(C1)*C2 stays lane-local; for GEMM2 64 consecutive columns)
// and row blocks (32 rows) h, h+2, h+4.  The two waves of a SIMD interleave
// their MFMAs, LDS reads and rescales: a row block's rescale runs just before
// its MFMAs, while the MFMA pipe works on the other wave's row blocks.
// Every wave also issues its share of the direct global->LDS loads (its own
// activation rows and two weight k-tiles per stage) three stages ahead into
// 4-slot rings, then waits (vmcnt, in issue order) only for its own loads
// before the stage barrier, which publishes stage j+1 and frees the slot of
// stage j-1; LDS reads wait per row block (lgkmcnt, in issue order), so no
// wave drains its reads at a barrier.
// Workgroup ids are dealt round-robin to the 8 XCDs; consecutive ids of one
// XCD take the column groups of one chunk, so the chunk's activation records
// are shared through that XCD's L2.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Split one 64-deep unit (stage stg, lane group g: k = stg*64 + g*8 .. +7 and
// +32 .. +39) of a row scaled by `up` into its hi and lo E4M3 parts.
__device__ inline void split_unit(u32x4 v0, u32x4 v1, float up, uint32_t (&hi)[4], uint32_t (&lo)[4]) {
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {  // codes 4d .. 4d+3 of the part
        float xs[4];
        xs[0] = bf16_bits_to_f32((uint16_t)(w[2 * d] & 0xffff)) * up;
        xs[1] = bf16_bits_to_f32((uint16_t)(w[2 * d] >> 16)) * up;
        xs[2] = bf16_bits_to_f32((uint16_t)(w[2 * d + 1] & 0xffff)) * up;
        xs[3] = bf16_bits_to_f32((uint16_t)(w[2 * d + 1] >> 16)) * up;
        int h = __builtin_amdgcn_cvt_pk_fp8_f32(xs[0], xs[1], 0, false);
        h = __builtin_amdgcn_cvt_pk_fp8_f32(xs[2], xs[3], h, true);
        const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
        const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
        int l = __builtin_amdgcn_cvt_pk_fp8_f32(xs[0] - h01.x, xs[1] - h01.y, 0, false);
        l = __builtin_amdgcn_cvt_pk_fp8_f32(xs[2] - h23.x, xs[3] - h23.y, l, true);
        hi[d] = (uint32_t)h;
        lo[d] = (uint32_t)l;
    }
}

__device__ inline float amax8(u32x4 v, float amax) {
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32((uint16_t)(w4[i] & 0xffff))));
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32((uint16_t)(w4[i] >> 16))));
    }
    return amax;
}

// largest e with amax * 2^e <= 448 (the E4M3 maximum), clamped to +-126
__device__ inline int row_exponent(float amax) {
    int e = 0;
    if (amax > 0.f && amax <= 3.0e38f) {
        int ex;
        const float f = frexpf(amax, &ex);  // amax = f * 2^ex, f in [0.5, 1)
        e = (f <= 0.875f ? 9 : 8) - ex;     // 448 = 0.875 * 2^9
        e = min(max(e, -126), 126);
    }
    return e;
}

constexpr int kSplitRegUnits = 8;  // rows up to 8 * 1024 = 8192 values stay in registers

// ---------------------------------------------------------------------------
// bf16 rows -> E4M3 hi/lo records; one wave per row.  Lane l handles the
// units u = l, l + 64, ... (unit u: stage u/4, lane group u%4); rows of at
// most 8192 values are read once into registers (every load in flight at
// once), longer ones twice.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void split_rows_kernel(SplitArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)((blockIdx.x * (size_t)blockDim.x + threadIdx.x) >> 6);
    if (r >= a.rows) return;
    if (a.row_ids) {
        // both loads in one round trip (row_ids has a slot for every row)
        const int npp = a.meta[0];
        const int rid = a.row_ids[r];
        if (r >= npp || rid >= a.sentinel) return;
    }
    const uint16_t* x = a.x + r * (int64_t)a.K;
    uint8_t* out = a.out + r * (int64_t)a.K * 2;
    const int units = a.K / 16;  // (stage, lane group) pairs
    auto unit_k0 = [](int u) { return (u >> 2) * 64 + (u & 3) * 8; };
    if (units <= 64 * kSplitRegUnits) {
        u32x4 v0[kSplitRegUnits], v1[kSplitRegUnits];
#pragma unroll
        for (int j = 0; j < kSplitRegUnits; ++j) {
            const int u = lane + 64 * j;
            const int k0 = unit_k0(u);
            v0[j] = u < units ? ldg16(x + k0) : u32x4{0, 0, 0, 0};
            v1[j] = u < units ? ldg16(x + k0 + 32) : u32x4{0, 0, 0, 0};
        }
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < kSplitRegUnits; ++j) amax = amax8(v1[j], amax8(v0[j], amax));
        amax = wave_max(amax);
        const int e = row_exponent(amax);
        const float up = ldexpf(1.f, e);
        if (lane == 0) a.rscale[r] = ldexpf(1.f, -e);
#pragma unroll
        for (int j = 0; j < kSplitRegUnits; ++j) {
            const int u = lane + 64 * j;
            if (u < units) {
                uint32_t hi[4], lo[4];
                split_unit(v0[j], v1[j], up, hi, lo);
                uint8_t* rec = out + (size_t)(u >> 2) * 128;
                *reinterpret_cast<u32x4*>(rec + (u & 3) * 16) = u32x4{hi[0], hi[1], hi[2], hi[3]};
                *reinterpret_cast<u32x4*>(rec + 64 + (u & 3) * 16) = u32x4{lo[0], lo[1], lo[2], lo[3]};
            }
        }
        return;
    }
    float amax = 0.f;
    for (int c = lane * 8; c < a.K; c += 64 * 8) amax = amax8(ldg16(x + c), amax);
    amax = wave_max(amax);
    const int e = row_exponent(amax);
    const float up = ldexpf(1.f, e);
    if (lane == 0) a.rscale[r] = ldexpf(1.f, -e);
    for (int u = lane; u < units; u += 64) {
        const int k0 = unit_k0(u);
        uint32_t hi[4], lo[4];
        split_unit(ldg16(x + k0), ldg16(x + k0 + 32), up, hi, lo);
        uint8_t* rec = out + (size_t)(u >> 2) * 128;
        *reinterpret_cast<u32x4*>(rec + (u & 3) * 16) = u32x4{hi[0], hi[1], hi[2], hi[3]};
        *reinterpret_cast<u32x4*>(rec + 64 + (u & 3) * 16) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
}

namespace {

constexpr int kRows = 16 * kPrefillF8MB;         // rows per chunk (5 blocks of 32)
constexpr int kRec = 128;                        // record bytes per row per K stage
constexpr int kTiles = kPrefillF8Cols / 16;      // packed 16-column tiles per workgroup
constexpr int A_SLOT = kRows * kRec;             // 20 KiB
constexpr int B_SLOT = kTiles * 1024;            // 16 KiB: one 1 KiB k-tile per column tile
// ring depths: the weight stream comes from HBM and needs the most bytes in
// flight, the activation records are mostly L2 hits
// 4-slot rings for both streams, three stages ahead (a fifth weight slot,
// four stages ahead, measured 1.5-2% slower on both GEMMs)
constexpr int A_SLOTS = 4, B_SLOTS = 4;
constexpr int A_AHEAD = A_SLOTS - 1, B_AHEAD = B_SLOTS - 1;  // stages requested ahead
constexpr int A_OFF = 0, B_OFF = A_SLOTS * A_SLOT, SMEM = B_OFF + B_SLOTS * B_SLOT;
static_assert(SMEM <= 160 * 1024, "LDS budget");
static_assert(kRows % 32 == 0 && kRows / 32 <= 6, "at most three 32-row blocks per wave");

// byte offset of (row, logical 16-byte part) in an activation slot: rows are
// XOR-swizzled so the 16 rows a 16-lane group reads hit distinct banks
__device__ inline int rec_off(int row, int part) { return row * kRec + ((part ^ ((row >> 1) & 7)) << 4); }

__device__ inline i32x8 cat8(u32x4 a, u32x4 b) {
    return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// acc += A x B * 2^(sb - 127); A and B E4M3, A unscaled
__device__ inline f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

// s = m * 2^(byte - 127) with the E8M0 byte as the MFMA scale: byte = the
// biased exponent (0 for subnormals, whose m = s * 2^127 < 1 is still exact).
// A zero scale maps to byte 0 and m = 1 (2^-127, the smallest E8M0 scale); a
// non-finite one to byte 255 (the E8M0 NaN).
struct BScale {
    int byte;
    float m;
};
__device__ inline BScale split_scale(float s) {
    const uint32_t bits = __builtin_bit_cast(uint32_t, s);
    const int ex = (int)((bits >> 23) & 0xff);
    BScale r;
    if (s == 0.f) {
        r.byte = 0;
        r.m = 1.f;
    } else if (ex == 0) {
        r.byte = 0;
        r.m = s * 0x1p127f;
    } else if (ex == 255) {
        r.byte = 255;
        r.m = 1.f;
    } else {
        r.byte = ex;
        r.m = __builtin_bit_cast(float, (bits & 0x807fffffu) | 0x3f800000u);
    }
    return r;
}

// After the main loop (every wave has drained its loads and LDS reads) the
// ring memory holds the chunk's row table for the epilogue: per row its pair
// id (P_tot for padding) and its activation row scale, one thread per row.
// The thread's pair id (and for GEMM2, whose rows are the chunk's own, the
// row scale) was loaded before the main loop (RowInfo `pre`), so the
// epilogue waits for at most one round trip (GEMM1's scale, indexed by the
// pair's token).  All 8 waves call this at the same point (two barriers).
struct RowInfo {
    int pid;
    float rs;
};
template <int GEMM>
__device__ inline RowInfo prefetch_row(const GemmArgs& a, const Chunk& ch) {
    RowInfo ri{a.P_tot, 0.f};
    const int row = threadIdx.x;
    if (row < kRows && row < ch.nrows) {
        ri.pid = a.sorted_ids[ch.row_start + row];
        if constexpr (GEMM == 2) ri.rs = a.a_scale[ch.row_start + row];
    }
    return ri;
}
template <int GEMM>
__device__ inline const RowInfo* publish_rows(const GemmArgs& a, const Chunk& ch, char* smem, RowInfo pre) {
    RowInfo* t = reinterpret_cast<RowInfo*>(smem);
    __syncthreads();
    const int row = threadIdx.x;
    if (row < kRows) {
        RowInfo ri{a.P_tot, 0.f};
        if (row < ch.nrows && pre.pid < a.P_tot) {
            ri.pid = pre.pid;
            ri.rs = GEMM == 2 ? pre.rs : a.a_scale[pre.pid < a.P ? pre.pid / a.topk : pre.pid - a.P];
        }
        t[row] = ri;
    }
    __syncthreads();
    return t;
}

// Output tile staged in LDS after the row table: GEMM1 writes the chunk's
// rows of act (128 columns), GEMM2 rows of y (256 columns); the workgroup
// then copies whole rows out with 16-byte stores.
constexpr int TILE_OFF = 2048;
static_assert(TILE_OFF >= kRows * 8 && TILE_OFF + kRows * kPrefillF8Cols * 2 <= SMEM, "epilogue LDS");
template <int GEMM>
__device__ inline void store_tile(const GemmArgs& a, const Chunk& ch, int grp, const char* smem,
                                  const RowInfo* rows) {
    constexpr int TW = GEMM == 1 ? kPrefillF8Cols / 2 : kPrefillF8Cols;  // tile columns
    constexpr int CPR = TW / 8;                                         // 16-byte pieces per row
    const uint16_t* tile = reinterpret_cast<const uint16_t*>(smem + TILE_OFF);
    __syncthreads();
    for (int idx = threadIdx.x; idx < ch.nrows * CPR; idx += blockDim.x) {
        const int r = idx / CPR, c8 = (idx % CPR) * 8;
        const int pid = rows[r].pid;
        if (pid >= a.P_tot) continue;
        const u32x4 v = *reinterpret_cast<const u32x4*>(tile + r * TW + c8);
        if constexpr (GEMM == 1) {
            *reinterpret_cast<u32x4*>((uint16_t*)a.out + (size_t)(ch.row_start + r) * (a.N / 2) + grp * TW + c8) = v;
        } else {
            const int col = grp * TW + c8;
            if (col < a.N) *reinterpret_cast<u32x4*>((uint16_t*)a.out + (size_t)pid * a.N + col) = v;
        }
    }
}

// Wave (s, H) with NRW row blocks (H, H+2, ...).  All waves run nkt + 1
// barriers.
template <int GEMM, int NRW, int H>
__device__ __attribute__((always_inline)) inline void f8_wave(const GemmArgs& a, char* smem, const Chunk& ch,
                                                               int grp, int s, int lane, const uint8_t* W,
                                                               const float* ws, RowInfo pre) {
    const int w = H * 4 + s;
    const int g2 = lane >> 5, r32 = lane & 31, hb = r32 >> 4, c16 = lane & 15;
    const int nkt = a.K / 64, nkb = a.K / 128;
    const int ntiles = a.N / 16;

    // ---- direct-to-LDS loads: two weight k-tiles per stage ----
    const uint8_t* b_src[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int nt = min(grp * kTiles + 2 * w + i, ntiles - 1);  // a partial last group re-reads
        b_src[i] = W + packed_tile_offset(1, a.K, nt, 0) + lane * 16;
    }
    auto issue_b = [&](int st) {
        const int sc = min(st, nkt - 1);  // stages past the end re-read the last one
        char* bd = smem + B_OFF + (st % B_SLOTS) * B_SLOT;
#pragma unroll
        for (int i = 0; i < 2; ++i) lds_dma16_stream(b_src[i] + (size_t)sc * 1024, bd + (2 * w + i) * 1024);
    };
    // activation rows: NRW instructions of 8 rows each per stage.  GEMM1
    // looks up its rows' pair ids first: loads complete in issue order, so
    // waiting for lookups issued after the weight stages would also wait for
    // those stages.  GEMM2 reads the chunk's own rows (a padding row's
    // record is stale, and its sums are never stored), so it looks up nothing.
    int pidv[NRW > 0 ? NRW : 1], pid0 = 0;
    if constexpr (GEMM == 1) {
        pid0 = a.sorted_ids[ch.row_start];  // the first row of a chunk is always a real pair
#pragma unroll
        for (int i = 0; i < NRW; ++i) {
            const int row = (H + 2 * i) * 32 + s * 8 + (lane >> 3);
            pidv[i] = a.sorted_ids[ch.row_start + min(row, ch.nrows - 1)];
        }
    }
    // the weight stream does not depend on the chunk's rows: its first stages
    // go out while the lookups are in flight
    for (int st = 0; st < B_AHEAD; ++st) issue_b(st);
    const char* a_src[NRW > 0 ? NRW : 1];
    int a_lds[NRW > 0 ? NRW : 1];
#pragma unroll
    for (int i = 0; i < NRW; ++i) {
        const int row0 = (H + 2 * i) * 32 + s * 8;  // rows row0 .. row0+7, 16 B per lane
        const int row = row0 + (lane >> 3), q = lane & 7;
        const int part = q ^ ((row >> 1) & 7);  // logical part this lane's LDS slot holds
        int src;
        if constexpr (GEMM == 1) {
            const int pid = row < ch.nrows && pidv[i] < a.P_tot ? pidv[i] : pid0;
            src = pid < a.P ? pid / a.topk : pid - a.P;
        } else {
            src = ch.row_start + (row < ch.nrows ? row : 0);
        }
        a_src[i] = (const char*)a.A + (size_t)src * a.K * 2 + part * 16;
        a_lds[i] = row0 * kRec;
    }
    auto issue_a1 = [&](int st, int i) {  // instruction i (8 rows) of stage st
        const int sc = min(st, nkt - 1);
        lds_dma16(a_src[i] + (size_t)sc * kRec, smem + A_OFF + (st % A_SLOTS) * A_SLOT + a_lds[i]);
    };
    auto issue_a = [&](int st) {
#pragma unroll
        for (int i = 0; i < NRW; ++i) issue_a1(st, i);
    };
    auto issue_b1 = [&](int st, int i) {  // weight k-tile i of stage st
        const int sc = min(st, nkt - 1);
        lds_dma16_stream(b_src[i] + (size_t)sc * 1024, smem + B_OFF + (st % B_SLOTS) * B_SLOT + (2 * w + i) * 1024);
    };

    // Ring protocol: barrier j publishes stage j+1 and frees the slots of
    // stage j-1, whose fragments every wave has consumed; during stage j the
    // wave requests A and B of stage j+3 into them.  Prefetch
    // reads of stage j+1 may still be in flight at barrier j+1: those slots
    // are refilled only after barrier j+2.  The requests of a stage are
    // spread between its row blocks' MFMAs (a burst right after the barrier
    // would stall the waves on the memory queue), B first and A's last
    // instruction last, so when the wave waits before barrier j for stage
    // j+1 (requested during stage j-2) only stage j-1's
    // NRW + 2 requests may be outstanding.
    if constexpr (NRW == 0) {  // no rows for this wave: weight loads and barriers only
        wait_vm<2 * (B_AHEAD - 1)>();  // stage 0 landed
        stage_barrier();
        for (int j = 0; j < nkt; ++j) {
            wait_vm<2 * (B_AHEAD - 2)>();  // stage j+1 landed
            stage_barrier();
            issue_b(j + B_AHEAD);
        }
        wait_vm<0>();
        store_tile<GEMM>(a, ch, grp, smem, publish_rows<GEMM>(a, ch, smem, pre));
        return;
    } else {
        // ---- fragment addresses ----
        const int frow = H * 32 + r32;  // row block i adds 64 rows
        const uint32_t abase = lds_addr(smem + A_OFF);
        const uint32_t ah0 = abase + rec_off(frow, 2 * g2), ah1 = abase + rec_off(frow, 2 * g2 + 1);
        const uint32_t al0 = abase + rec_off(frow, 4 + 2 * g2), al1 = abase + rec_off(frow, 5 + 2 * g2);
        // B lane (column r32 of column block t, half g2) reads packed lane
        // groups 2*g2 and 2*g2+1 (256 bytes apart) of tile tA (+ t * TOFF)
        constexpr int TOFF = GEMM == 1 ? 1024 : 2048;
        const int tA = GEMM == 1 ? 4 * s + 2 * hb : 4 * s + hb;
        const uint32_t bbase = lds_addr(smem + B_OFF) + tA * 1024 + (32 * g2 + c16) * 16;

        // ---- block scales, per lane for K blocks kb = lane and lane + 64:
        // rat = m(kb-1) / m(kb), the rescale entering block kb, and pk = the
        // E8M0 byte of column block t at bit 8t ----
        int colt[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
            colt[t] = GEMM == 1 ? t * (a.N / 2) + grp * 128 + 32 * s : grp * kPrefillF8Cols + 64 * s + 32 * t;
        const int nbw = a.N / 128;
        float rat[2][2], mlast[2];
        int pk[2] = {0, 0};
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int cb = min(colt[t] / 128, nbw - 1);
            float m[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int kb = lane + 64 * hh;
                const BScale bs = split_scale(kb < nkb ? ws[kb * nbw + cb] : 1.f);
                m[hh] = bs.m;
                pk[hh] |= bs.byte << (8 * t);
            }
            const float m63 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m[0]), 63));
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                float prev = __shfl_up(m[hh], 1, 64);
                if (lane == 0) prev = hh == 0 ? 1.f : m63;
                rat[t][hh] = prev / m[hh];
            }
            const int kl = nkb - 1;
            mlast[t] = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, kl < 64 ? m[0] : m[1]), kl & 63));
        }

        f32x16 acc[NRW][2];
#pragma unroll
        for (int i = 0; i < NRW; ++i) acc[i][0] = acc[i][1] = f32x16{};
        u32x4 af[NRW][4], bA[2][2], bB[2][2];
        auto ldA = [&](uint32_t so, auto I) {
            constexpr int i = decltype(I)::value;
            constexpr int off = i * 64 * kRec;
            af[i][0] = ds_read16<off>(ah0 + so);
            af[i][1] = ds_read16<off>(ah1 + so);
            af[i][2] = ds_read16<off>(al0 + so);
            af[i][3] = ds_read16<off>(al1 + so);
        };
        auto ldB = [&](uint32_t so, u32x4 (&b)[2][2]) {
            b[0][0] = ds_read16<0>(bbase + so);
            b[0][1] = ds_read16<256>(bbase + so);
            b[1][0] = ds_read16<TOFF>(bbase + so);
            b[1][1] = ds_read16<TOFF + 256>(bbase + so);
        };

        // current block's MFMA scale bytes
        int sb[2] = {127, 127};
        auto enter_block = [&](int kb, float (&r)[2]) {
            const int l = kb & 63;
            const int p = __builtin_amdgcn_readlane(kb < 64 ? pk[0] : pk[1], l);
            sb[0] = p & 0xff;
            sb[1] = (p >> 8) & 0xff;
#pragma unroll
            for (int t = 0; t < 2; ++t)
                r[t] = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, kb < 64 ? rat[t][0] : rat[t][1]), l));
        };
        // issue order so far: B of stages 0..B_AHEAD-1, then A of stages 0..2
        for (int st = 0; st < A_AHEAD; ++st) issue_a(st);
        wait_vm<(A_AHEAD - 1) * NRW>();  // stage 0 landed
        stage_barrier();                 // publishes stage 0
        ldB(0, bA);
        static_for<NRW>([&](auto I) { ldA(0, I); });
        wait_vm<NRW>();  // stage 1 landed: only A(2) was issued after A(1); the
                         // loop's count then holds from j = 1 on

        // Barrier j sits after row block 0's MFMAs of stage j (its fragments
        // were read during stage j-1), so the MFMA pipe has work while the
        // waves meet.  After it the wave reads stage j+1's B fragments, then
        // each row block's fragments right after that block's MFMAs.  LDS
        // reads complete in issue order, so before row block 0 of a stage at
        // most 4 * (NRW - 1) later reads are outstanding (the stage's other
        // row blocks), before row block i > 0 at most 4 * NRW.
        auto stage = [&](int j, auto PARc, u32x4 (&b)[2][2], u32x4 (&nb)[2][2]) {
            constexpr int PAR = decltype(PARc)::value;  // 0: first stage of a K block
            float r[2] = {1.f, 1.f};
            if constexpr (PAR == 0) enter_block(j >> 1, r);
            const uint32_t so = ((j + 1) % A_SLOTS) * A_SLOT;
            i32x8 b0, b1;
            static_for<NRW>([&](auto I) {
                constexpr int i = decltype(I)::value;
                if constexpr (i == 0) {
                    lgkm_wait<4 * (NRW - 1)>();
                    tie(b[0][0]);
                    tie(b[0][1]);
                    tie(b[1][0]);
                    tie(b[1][1]);
                    b0 = cat8(b[0][0], b[0][1]);
                    b1 = cat8(b[1][0], b[1][1]);
                } else {
                    lgkm_wait<4 * NRW>();
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) tie(af[i][q]);
                if constexpr (PAR == 0) {
                    acc[i][0] *= r[0];
                    acc[i][1] *= r[1];
                }
                const i32x8 hi = cat8(af[i][0], af[i][1]), lo = cat8(af[i][2], af[i][3]);
                acc[i][0] = mfma_f8(hi, b0, acc[i][0], sb[0]);
                acc[i][1] = mfma_f8(hi, b1, acc[i][1], sb[1]);
                acc[i][0] = mfma_f8(lo, b0, acc[i][0], sb[0]);
                acc[i][1] = mfma_f8(lo, b1, acc[i][1], sb[1]);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (i == 0) {
                    wait_vm<NRW + 2>();  // this wave's loads of stage j+1 landed
                    stage_barrier();     // stage j+1 published; stage j-1's slots are free
                    ldB(((j + 1) % B_SLOTS) * B_SLOT, nb);
                }
                ldA(so, I);  // stage j+1's fragments of this row block
                // this row block's share of the requests for later stages:
                // NRW = 1: B0 B1 A0; 2: B0 A0 B1 A1; 3: B0 A0 B1 A1 A2
                if constexpr (NRW == 1) {
                    issue_b1(j + B_AHEAD, 0);
                    issue_b1(j + B_AHEAD, 1);
                } else if constexpr (i < 2) {
                    issue_b1(j + B_AHEAD, i);
                }
                issue_a1(j + A_AHEAD, i);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        for (int j = 0; j < nkt; j += 2) {
            stage(j, std::integral_constant<int, 0>{}, bA, bB);
            stage(j + 1, std::integral_constant<int, 1>{}, bB, bA);
        }
        lgkm_wait0();  // the last (unused) prefetch
        static_for<NRW>([&](auto I) {
#pragma unroll
            for (int q = 0; q < 4; ++q) tie(af[decltype(I)::value][q]);
        });
        tie(bA[0][0]);
        tie(bA[0][1]);
        tie(bA[1][0]);
        tie(bA[1][1]);
        wait_vm<0>();  // every load has landed before the rings are reused
        const float mc[2] = {mlast[0], mlast[1]};
        const RowInfo* rows = publish_rows<GEMM>(a, ch, smem, pre);

        // ---- epilogue: lane holds column r32 of both column blocks, rows
        // 8*(q/4) + 4*g2 + q%4 of each row block; bf16 results go to the
        // tile, whole rows go out in store_tile ----
        constexpr int TW = GEMM == 1 ? kPrefillF8Cols / 2 : kPrefillF8Cols;
        uint16_t* tile = reinterpret_cast<uint16_t*>(smem + TILE_OFF);
#pragma unroll
        for (int i = 0; i < NRW; ++i) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = (H + 2 * i) * 32 + 8 * (q >> 2) + 4 * g2 + (q & 3);
                const float rs = rows[row].rs;  // 0 for padding rows (never stored)
                if constexpr (GEMM == 1) {
                    const float gv = acc[i][0][q] * mc[0] * rs, uv = acc[i][1][q] * mc[1] * rs;
                    tile[row * TW + 32 * s + r32] = f32_to_bf16_bits(silu(gv) * uv);
                } else {
                    tile[row * TW + 64 * s + r32] = f32_to_bf16_bits(acc[i][0][q] * mc[0] * rs);
                    tile[row * TW + 64 * s + 32 + r32] = f32_to_bf16_bits(acc[i][1][q] * mc[1] * rs);
                }
            }
        }
        store_tile<GEMM>(a, ch, grp, smem, rows);
    }
}

template <int GEMM, int H>
__device__ __attribute__((always_inline)) inline void f8_dispatch(int nrw, const GemmArgs& a, char* smem,
                                                                  const Chunk& ch, int grp, int s, int lane,
                                                                  const uint8_t* W, const float* ws,
                                                                  RowInfo pre) {
    switch (nrw) {
        case 0: f8_wave<GEMM, 0, H>(a, smem, ch, grp, s, lane, W, ws, pre); break;
        case 1: f8_wave<GEMM, 1, H>(a, smem, ch, grp, s, lane, W, ws, pre); break;
        case 2: f8_wave<GEMM, 2, H>(a, smem, ch, grp, s, lane, W, ws, pre); break;
        default: f8_wave<GEMM, 3, H>(a, smem, ch, grp, s, lane, W, ws, pre); break;
    }
}

}  // namespace

template <int GEMM>
__global__ __launch_bounds__(512, 1) void prefill_f8_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];
    const int tid = threadIdx.x;
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
    const bool sh = ch.expert >= a.E;
    const size_t wbytes = (size_t)a.K * a.N;
    const uint8_t* W = sh ? a.W_sh : a.W + (size_t)ch.expert * wbytes;
    const size_t nsc = (size_t)(a.K / 128) * (a.N / 128);
    const float* ws = sh ? a.w_scale_sh : a.w_scale + (size_t)ch.expert * nsc;
    const RowInfo pre = prefetch_row<GEMM>(a, ch);  // consumed by the epilogue
    const int nrb32 = (ch.nrows + 31) >> 5;  // row blocks of 32 (at most 6)
    const int s = wv & 3, h = wv >> 2;
    const int nrw = (nrb32 - h + 1) >> 1;    // blocks h, h+2, h+4 below nrb32
    if (h == 0)
        f8_dispatch<GEMM, 0>(nrw, a, smem, ch, grp, s, lane, W, ws, pre);
    else
        f8_dispatch<GEMM, 1>(nrw, a, smem, ch, grp, s, lane, W, ws, pre);
}

hipError_t launch_split_rows(const SplitArgs& a, hipStream_t st) {
    if (a.rows == 0) return hipSuccess;
    if (a.K % 64 != 0) return hipErrorInvalidValue;
    dim3 grid((unsigned)((a.rows + 3) / 4)), block(256);
    split_rows_kernel<<<grid, block, 0, st>>>(a);
    return hipGetLastError();
}

template <int GEMM>
static hipError_t launch_prefill_f8(const GemmArgs& a, int max_chunks, hipStream_t st) {
    // two stages per loop trip; block scales of at most 128 K blocks per lane pair
    if (a.K % 128 != 0 || a.K > kPrefillFp8MaxK || a.N % 128 != 0) return hipErrorInvalidValue;
    if (a.n_groups * kPrefillF8Cols < a.N) return hipErrorInvalidValue;
    const int slots_per_xcd = (max_chunks + 7) / 8;
    dim3 grid((unsigned)(8 * (size_t)slots_per_xcd * a.n_groups));
    prefill_f8_kernel<GEMM><<<grid, 512, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_prefill_f8_gemm1(const GemmArgs& a, int max_chunks, hipStream_t st) {
    return launch_prefill_f8<1>(a, max_chunks, st);
}
hipError_t launch_prefill_f8_gemm2(const GemmArgs& a, int max_chunks, hipStream_t st) {
    return launch_prefill_f8<2>(a, max_chunks, st);
}

}  // namespace moe
