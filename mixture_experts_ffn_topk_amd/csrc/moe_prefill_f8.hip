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

// The same split with WPR waves per row (256-thread blocks holding 4 / WPR
// rows), each thread UPT units, the row maximum met in LDS: for rows of at
// most 128 units (2 waves, one unit each) and of 257 .. 512 units (4 waves,
// two each), where one wave per row leaves too few waves in flight or too
// long a chain per wave (DeepSeek-R1-shaped T = 4096 layer: the token rows'
// split 28.9 -> 26.0 us, the intermediate's 60.5 -> 54.0 us; same codes).
// Every thread reaches the barrier: rows past the end or padding rows only
// skip the stores.
template <int WPR, int UPT>
__global__ __launch_bounds__(256) void split_rows_wg_kernel(SplitArgs a) {
    constexpr int RT = 64 * WPR;  // threads per row
    __shared__ float red[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int rl = tid / RT, t = tid % RT;
    const int64_t r = (int64_t)blockIdx.x * (4 / WPR) + rl;
    bool ok = r < a.rows;
    if (ok && a.row_ids) {
        // both loads in one round trip (row_ids has a slot for every row)
        const int npp = a.meta[0];
        const int rid = a.row_ids[r];
        ok = r < npp && rid < a.sentinel;
    }
    const int units = a.K / 16;
    const uint16_t* x = a.x + (ok ? r : 0) * (int64_t)a.K;
    u32x4 v0[UPT], v1[UPT];
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
        const int u = t + RT * j;
        const int k0 = (u >> 2) * 64 + (u & 3) * 8;
        const bool in = ok && u < units;
        v0[j] = in ? ldg16(x + k0) : u32x4{0, 0, 0, 0};
        v1[j] = in ? ldg16(x + k0 + 32) : u32x4{0, 0, 0, 0};
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < UPT; ++j) amax = amax8(v1[j], amax8(v0[j], amax));
    amax = wave_max(amax);
    if (lane == 0) red[w] = amax;
    __syncthreads();
    amax = red[rl * WPR];
#pragma unroll
    for (int q = 1; q < WPR; ++q) amax = fmaxf(amax, red[rl * WPR + q]);
    if (!ok) return;
    const int e = row_exponent(amax);
    const float up = ldexpf(1.f, e);
    if (t == 0) a.rscale[r] = ldexpf(1.f, -e);
    uint8_t* out = a.out + r * (int64_t)a.K * 2;
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
        const int u = t + RT * j;
        if (u < units) {
            uint32_t hi[4], lo[4];
            split_unit(v0[j], v1[j], up, hi, lo);
            uint8_t* rec = out + (size_t)(u >> 2) * 128;
            *reinterpret_cast<u32x4*>(rec + (u & 3) * 16) = u32x4{hi[0], hi[1], hi[2], hi[3]};
            *reinterpret_cast<u32x4*>(rec + 64 + (u & 3) * 16) = u32x4{lo[0], lo[1], lo[2], lo[3]};
        }
    }
}

// ---------------------------------------------------------------------------
// FP8-activation variant: bf16 rows -> E4M3 codes with one power-of-two
// scale per row and 128-element K block b: e_b = the largest exponent with
// amax_b * 2^e_b <= 448 (as row_exponent), codes = E4M3(x * 2^e_b) rounded
// to nearest even, and the block's MFMA scale byte 127 - e_b, so that the
// value the GEMM sees is code * 2^-e_b.  One wave per row; lane l takes the
// units u = l, l + 64, ... (unit u: stage u/4, lane group u%4, i.e. k =
// 64(u/4) + 8(u%4) .. +7 and +32 .. +39), so the 8 units of a K block sit
// on 8 neighbouring lanes and meet through DPP.  Records: per row and
// 64-deep stage 64 bytes, part p holding unit (stage, p)'s codes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fp8_act_rows_kernel(SplitArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)((blockIdx.x * (size_t)blockDim.x + threadIdx.x) >> 6);
    if (r >= a.rows) return;
    if (a.row_ids) {
        const int npp = a.meta[0];
        const int rid = a.row_ids[r];
        if (r >= npp || rid >= a.sentinel) return;
    }
    const uint16_t* x = a.x + r * (int64_t)a.K;
    uint8_t* out = a.out + r * (int64_t)a.K;
    uint8_t* ex = a.exps + r * (int64_t)a.exp_stride;
    const int units = a.K / 16;  // a multiple of 8 (K is a multiple of 128)
    for (int u0 = 0; u0 < units; u0 += 64) {  // every lane runs every round (DPP below)
        const int u = u0 + lane;
        const bool ok = u < units;
        const int k0 = (u >> 2) * 64 + (u & 3) * 8;
        const u32x4 v0 = ok ? ldg16(x + k0) : u32x4{0, 0, 0, 0};
        const u32x4 v1 = ok ? ldg16(x + k0 + 32) : u32x4{0, 0, 0, 0};
        float amax = amax8(v1, amax8(v0, 0.f));
        amax = fmaxf(amax, dpp_f<kDppQuadXor1>(amax));
        amax = fmaxf(amax, dpp_f<kDppQuadXor2>(amax));
        amax = fmaxf(amax, dpp_f<kDppRowHalfMirror>(amax));  // max over the block's 8 lanes
        const int e = row_exponent(amax);
        const float up = ldexpf(1.f, e);
        if (ok) {
            const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            uint32_t c[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                int h = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_bits_to_f32((uint16_t)(w[2 * d] & 0xffff)) * up,
                                                        bf16_bits_to_f32((uint16_t)(w[2 * d] >> 16)) * up, 0, false);
                h = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_bits_to_f32((uint16_t)(w[2 * d + 1] & 0xffff)) * up,
                                                    bf16_bits_to_f32((uint16_t)(w[2 * d + 1] >> 16)) * up, h, true);
                c[d] = (uint32_t)h;
            }
            *reinterpret_cast<u32x4*>(out + (size_t)(u >> 2) * 64 + (u & 3) * 16) = u32x4{c[0], c[1], c[2], c[3]};
            if ((lane & 7) == 0) ex[u >> 3] = (uint8_t)(127 - e);
        }
    }
}

namespace {

constexpr int kRows = 16 * kPrefillF8MB;         // rows per chunk (5 blocks of 32)
constexpr int kTiles = kPrefillF8Cols / 16;      // packed 16-column tiles per workgroup
constexpr int B_SLOT = kTiles * 1024;            // 16 KiB: one 1 KiB k-tile per column tile
// ring depths: the weight stream comes from HBM and needs the most bytes in
// flight, the activation records are mostly L2 hits
// 4-slot rings for both streams, three stages ahead (a fifth weight slot,
// four stages ahead, measured 1.5-2% slower on both GEMMs)
constexpr int A_SLOTS = 4, B_SLOTS = 4;
constexpr int A_AHEAD = A_SLOTS - 1, B_AHEAD = B_SLOTS - 1;  // stages requested ahead
constexpr int kMaxExpStride = kPrefillFp8MaxK / 128;  // FP8 activations: scale bytes per row, at most
// LDS plan of each variant.  A8 = FP8 activations: 64-byte records (codes
// only), one MFMA per product, and after the rings the chunk's table of
// per (row, K block) activation scale bytes.  Otherwise hi/lo records of 128
// bytes and a per-row scale applied in the epilogue.
template <bool A8>
struct F8Lds {
    static constexpr int REC = A8 ? 64 : 128;   // record bytes per row per K stage
    static constexpr int A_SLOT = kRows * REC;  // 10 / 20 KiB
    static constexpr int A_OFF = 0, B_OFF = A_SLOTS * A_SLOT;
    static constexpr int EXP_OFF = B_OFF + B_SLOTS * B_SLOT;
    static constexpr int SMEM = EXP_OFF + (A8 ? kRows * kMaxExpStride : 0);
};
static_assert(F8Lds<false>::SMEM <= 160 * 1024 && F8Lds<true>::SMEM <= 160 * 1024, "LDS budget");
static_assert(kRows % 32 == 0 && kRows / 32 <= 6, "at most three 32-row blocks per wave");

// byte offset of (row, logical 16-byte part) in an activation slot: rows are
// XOR-swizzled so the 16 rows a 16-lane group reads hit distinct banks (the
// 64-byte records of the FP8-activation variant: the same two-rows-per-bank-
// group pattern over four parts)
template <bool A8>
__device__ inline int rec_off(int row, int part) {
    if constexpr (A8)
        return row * 64 + ((part ^ (row & 3)) << 4);
    else
        return row * 128 + ((part ^ ((row >> 1) & 7)) << 4);
}

__device__ inline void tie_u(uint32_t& v) { asm volatile("" : "+v"(v)); }

// one byte from LDS, not tracked by the compiler (waited for with lgkmcnt)
__device__ inline uint32_t ds_read_byte(uint32_t addr) {
    uint32_t r;
    asm volatile("ds_read_u8 %0, %1" : "=v"(r) : "v"(addr));
    return r;
}

__device__ inline i32x8 cat8(u32x4 a, u32x4 b) {
    return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// acc += A x B * 2^(sa - 127) * 2^(sb - 127); A and B E4M3.  sa is per lane
// (the lane's row and K half), sb per lane too but uniform here.
__device__ inline f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
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
template <int GEMM, bool A8>
__device__ inline RowInfo prefetch_row(const GemmArgs& a, const Chunk& ch) {
    RowInfo ri{a.P_tot, 0.f};
    const int row = threadIdx.x;
    if (row < kRows && row < ch.nrows) {
        ri.pid = a.sorted_ids[ch.row_start + row];
        if constexpr (GEMM == 2 && !A8) ri.rs = a.a_scale[ch.row_start + row];
    }
    return ri;
}
// (FP8 activations: the scales went into the MFMAs, every real row takes 1)
template <int GEMM, bool A8>
__device__ inline const RowInfo* publish_rows(const GemmArgs& a, const Chunk& ch, char* smem, RowInfo pre) {
    RowInfo* t = reinterpret_cast<RowInfo*>(smem);
    __syncthreads();
    const int row = threadIdx.x;
    if (row < kRows) {
        RowInfo ri{a.P_tot, 0.f};
        if (row < ch.nrows && pre.pid < a.P_tot) {
            ri.pid = pre.pid;
            if constexpr (A8)
                ri.rs = 1.f;
            else
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
static_assert(TILE_OFF >= kRows * 8 && TILE_OFF + kRows * kPrefillF8Cols * 2 <= F8Lds<true>::SMEM &&
                  TILE_OFF + kRows * kPrefillF8Cols * 2 <= F8Lds<false>::SMEM,
              "epilogue LDS");
static_assert(TILE_OFF + kRows * (kPrefillF8Cols / 2) * 4 <= F8Lds<true>::SMEM, "fp32 epilogue tile");

// FP8 activations, GEMM1: the workgroup's 128 intermediate columns of a row
// are exactly one 128-element K block of the down GEMM's input, so the
// epilogue quantises them itself from the fp32 values (tile [rows][128]
// floats): per row 8 threads, thread u the 16 values of record (stage u/4,
// part u%4) of the block's two 64-deep stages; block amax over the 8 threads,
// e as row_exponent, codes E4M3(v * 2^e), scale byte 127 - e.  The threads of
// a row are 8 aligned lanes of one wave and every wave runs the same number
// of rounds, so the DPP max always sees a whole group.
__device__ inline void store_act8_tile(const GemmArgs& a, const Chunk& ch, int grp, const char* smem,
                                       const RowInfo* rows) {
    constexpr int TW = kPrefillF8Cols / 2;
    const float* tile = reinterpret_cast<const float*>(smem + TILE_OFF);
    const int I = a.N / 2;
    __syncthreads();
    const int n8 = ch.nrows * 8;
    for (int i0 = 0; i0 < n8; i0 += blockDim.x) {
        const int idx = i0 + threadIdx.x;
        const bool ok = idx < n8;
        const int r = ok ? idx >> 3 : 0, u = idx & 7;
        const int k0 = 64 * (u >> 2) + 8 * (u & 3);
        float v[16];
        float amax = 0.f;
        if (ok) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x4 p0 = *reinterpret_cast<const f32x4*>(tile + r * TW + k0 + 32 * h);
                const f32x4 p1 = *reinterpret_cast<const f32x4*>(tile + r * TW + k0 + 32 * h + 4);
                v[8 * h + 0] = p0.x; v[8 * h + 1] = p0.y; v[8 * h + 2] = p0.z; v[8 * h + 3] = p0.w;
                v[8 * h + 4] = p1.x; v[8 * h + 5] = p1.y; v[8 * h + 6] = p1.z; v[8 * h + 7] = p1.w;
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) amax = fmaxf(amax, fabsf(v[q]));
        }
        amax = fmaxf(amax, dpp_f<kDppQuadXor1>(amax));
        amax = fmaxf(amax, dpp_f<kDppQuadXor2>(amax));
        amax = fmaxf(amax, dpp_f<kDppRowHalfMirror>(amax));
        if (!ok || rows[r].pid >= a.P_tot) continue;
        const int e = row_exponent(amax);
        const float up = ldexpf(1.f, e);
        uint32_t c[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            int h = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * d] * up, v[4 * d + 1] * up, 0, false);
            h = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * d + 2] * up, v[4 * d + 3] * up, h, true);
            c[d] = (uint32_t)h;
        }
        const size_t row = (size_t)(ch.row_start + r);
        *reinterpret_cast<u32x4*>(a.out_codes + row * I + (size_t)(2 * grp + (u >> 2)) * 64 + (u & 3) * 16) =
            u32x4{c[0], c[1], c[2], c[3]};
        if (u == 0) a.out_exps[row * a.out_exp_stride + grp] = (uint8_t)(127 - e);
    }
}

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
// barriers.  A8: FP8-activation variant (64-byte code records, the per
// (row, K block) scale bytes from the LDS exponent table as the MFMA's A
// scale, one MFMA per product and column block).
template <int GEMM, int NRW, int H, bool A8>
__device__ __attribute__((always_inline)) inline void f8_wave(const GemmArgs& a, char* smem, const Chunk& ch,
                                                               int grp, int s, int lane, const uint8_t* W,
                                                               const float* ws, RowInfo pre) {
    const int w = H * 4 + s;
    const int g2 = lane >> 5, r32 = lane & 31, hb = r32 >> 4, c16 = lane & 15;
    const int nkt = a.K / 64, nkb = a.K / 128;
    const int ntiles = a.N / 16;
    using L = F8Lds<A8>;
    constexpr int A_SLOT = L::A_SLOT, A_OFF = L::A_OFF, B_OFF = L::B_OFF, kRec = L::REC;
    constexpr int RPB = A8 ? 2 : 4;  // LDS reads of A fragments per row block per stage

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
    int srcv[NRW > 0 ? NRW : 1];  // source row of row (lane >> 3) of this wave's 8-row group
#pragma unroll
    for (int i = 0; i < NRW; ++i) {
        const int row0 = (H + 2 * i) * 32 + s * 8;  // rows row0 .. row0+7
        int row = row0 + (lane >> 3), src;
        if constexpr (GEMM == 1) {
            const int pid = row < ch.nrows && pidv[i] < a.P_tot ? pidv[i] : pid0;
            src = pid < a.P ? pid / a.topk : pid - a.P;
        } else {
            src = ch.row_start + (row < ch.nrows ? row : 0);
        }
        srcv[i] = src;
        int q = lane & 7;
        if constexpr (A8) {  // 4 lanes of 16 B per 64-byte record: lanes 0..31 cover the 8 rows
            row = row0 + ((lane >> 2) & 7);
            q = lane & 3;
            src = __shfl(src, ((lane >> 2) & 7) * 8, 64);
        }
        const int part = A8 ? (q ^ (row & 3)) : (q ^ ((row >> 1) & 7));  // logical part of this lane's slot
        a_src[i] = (const char*)a.A + (size_t)src * a.K * (kRec / 64) + part * 16;
        a_lds[i] = row0 * kRec;
    }
    auto issue_a1 = [&](int st, int i) {  // instruction i (8 rows) of stage st
        const int sc = min(st, nkt - 1);
        if constexpr (A8) {
            if (lane < 32) lds_dma16(a_src[i] + (size_t)sc * kRec, smem + A_OFF + (st % A_SLOTS) * A_SLOT + a_lds[i]);
        } else {
            lds_dma16(a_src[i] + (size_t)sc * kRec, smem + A_OFF + (st % A_SLOTS) * A_SLOT + a_lds[i]);
        }
    };
    // FP8 activations: this wave's rows of the chunk's scale-byte table, one
    // request per row block before stage 0's (so the stage-0 wait covers it):
    // exp_stride / 16 lanes per row, 8 rows
    auto issue_exps = [&]() {
        if constexpr (A8) {
            const int lpr = a.exp_stride >> 4;  // lanes per row (1 .. 8)
            const int r8 = lane / lpr;
#pragma unroll
            for (int i = 0; i < NRW; ++i) {
                const int row0 = (H + 2 * i) * 32 + s * 8;
                const int src = __shfl(srcv[i], min(r8, 7) * 8, 64);
                if (r8 < 8)
                    lds_dma16(a.a_exp + (size_t)src * a.exp_stride + (lane % lpr) * 16,
                              smem + L::EXP_OFF + row0 * a.exp_stride);
            }
        }
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
        const RowInfo* rows = publish_rows<GEMM, A8>(a, ch, smem, pre);
        if constexpr (GEMM == 1 && A8)
            store_act8_tile(a, ch, grp, smem, rows);
        else
            store_tile<GEMM>(a, ch, grp, smem, rows);
        return;
    } else {
        // ---- fragment addresses ----
        const int frow = H * 32 + r32;  // row block i adds 64 rows
        const uint32_t abase = lds_addr(smem + A_OFF);
        const uint32_t ah0 = abase + rec_off<A8>(frow, 2 * g2), ah1 = abase + rec_off<A8>(frow, 2 * g2 + 1);
        const uint32_t al0 = abase + rec_off<A8>(frow, 4 + 2 * g2), al1 = abase + rec_off<A8>(frow, 5 + 2 * g2);
        // FP8 activations: this lane's row in the scale-byte table (+ 64 rows per block)
        const uint32_t ebase = lds_addr(smem + L::EXP_OFF) + frow * a.exp_stride;
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
        u32x4 af[NRW][RPB], bA[2][2], bB[2][2];
        auto ldA = [&](uint32_t so, auto I) {
            constexpr int i = decltype(I)::value;
            constexpr int off = i * 64 * kRec;
            af[i][0] = ds_read16<off>(ah0 + so);
            af[i][1] = ds_read16<off>(ah1 + so);
            if constexpr (!A8) {
                af[i][2] = ds_read16<off>(al0 + so);
                af[i][3] = ds_read16<off>(al1 + so);
            }
        };
        // FP8 activations: the A scale byte of each row block.  Reads for K
        // block kb land in saN (issued during block kb-1's second stage, so
        // that stage's later row blocks keep using sa); each K block's first
        // stage copies them to sa after the wait that covers them.
        uint32_t sa[NRW > 0 ? NRW : 1], saN[NRW > 0 ? NRW : 1];
        auto ldE = [&](int kb) {
            if constexpr (A8) {
#pragma unroll
                for (int i = 0; i < NRW; ++i) saN[i] = ds_read_byte(ebase + (uint32_t)(i * 64 * a.exp_stride + kb));
            }
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
        // issue order so far: B of stages 0..B_AHEAD-1, (A8: the scale bytes,)
        // then A of stages 0..2
        issue_exps();
        for (int st = 0; st < A_AHEAD; ++st) issue_a(st);
        wait_vm<(A_AHEAD - 1) * NRW>();  // stage 0 landed (and the older requests)
        stage_barrier();                 // publishes stage 0
        ldE(0);
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
        // row blocks), before row block i > 0 at most 4 * NRW.  (A8: RPB = 2
        // reads per row block; the scale bytes of the next K block are read
        // after the B fragments in the K block's second stage, so before row
        // block 0 they are done, and before row block i > 0 the count leaves
        // room for the stage's B reads only: stricter when they are there.)
        auto stage = [&](int j, auto PARc, u32x4 (&b)[2][2], u32x4 (&nb)[2][2]) {
            constexpr int PAR = decltype(PARc)::value;  // 0: first stage of a K block
            float r[2] = {1.f, 1.f};
            if constexpr (PAR == 0) enter_block(j >> 1, r);
            const uint32_t so = ((j + 1) % A_SLOTS) * A_SLOT;
            i32x8 b0, b1;
            static_for<NRW>([&](auto I) {
                constexpr int i = decltype(I)::value;
                if constexpr (i == 0) {
                    lgkm_wait<RPB * (NRW - 1)>();
                    if constexpr (A8 && PAR == 0) {
#pragma unroll
                        for (int q = 0; q < NRW; ++q) {
                            tie_u(saN[q]);
                            sa[q] = saN[q];
                        }
                    }
                    tie(b[0][0]);
                    tie(b[0][1]);
                    tie(b[1][0]);
                    tie(b[1][1]);
                    b0 = cat8(b[0][0], b[0][1]);
                    b1 = cat8(b[1][0], b[1][1]);
                } else {
                    lgkm_wait<RPB * (NRW - 1) + 4>();
                }
#pragma unroll
                for (int q = 0; q < RPB; ++q) tie(af[i][q]);
                if constexpr (PAR == 0) {
                    acc[i][0] *= r[0];
                    acc[i][1] *= r[1];
                }
                const i32x8 hi = cat8(af[i][0], af[i][1]);
                if constexpr (A8) {
                    acc[i][0] = mfma_f8(hi, b0, acc[i][0], (int)sa[i], sb[0]);
                    acc[i][1] = mfma_f8(hi, b1, acc[i][1], (int)sa[i], sb[1]);
                } else {
                    const i32x8 lo = cat8(af[i][2], af[i][3]);
                    acc[i][0] = mfma_f8(hi, b0, acc[i][0], 127, sb[0]);
                    acc[i][1] = mfma_f8(hi, b1, acc[i][1], 127, sb[1]);
                    acc[i][0] = mfma_f8(lo, b0, acc[i][0], 127, sb[0]);
                    acc[i][1] = mfma_f8(lo, b1, acc[i][1], 127, sb[1]);
                }
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (i == 0) {
                    wait_vm<NRW + 2>();  // this wave's loads of stage j+1 landed
                    stage_barrier();     // stage j+1 published; stage j-1's slots are free
                    ldB(((j + 1) % B_SLOTS) * B_SLOT, nb);
                    // the next K block's scale bytes (its first stage is j+1);
                    // the last block reads past the table's used bytes: unused
                    if constexpr (PAR == 1) ldE((j >> 1) + 1);
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
            for (int q = 0; q < RPB; ++q) tie(af[decltype(I)::value][q]);
            if constexpr (A8) tie_u(saN[decltype(I)::value]);  // the last (unused) read
        });
        tie(bA[0][0]);
        tie(bA[0][1]);
        tie(bA[1][0]);
        tie(bA[1][1]);
        wait_vm<0>();  // every load has landed before the rings are reused
        const float mc[2] = {mlast[0], mlast[1]};
        const RowInfo* rows = publish_rows<GEMM, A8>(a, ch, smem, pre);

        // ---- epilogue: lane holds column r32 of both column blocks, rows
        // 8*(q/4) + 4*g2 + q%4 of each row block; bf16 results go to the
        // tile, whole rows go out in store_tile ----
        constexpr int TW = GEMM == 1 ? kPrefillF8Cols / 2 : kPrefillF8Cols;
        uint16_t* tile = reinterpret_cast<uint16_t*>(smem + TILE_OFF);
        float* tile_f = reinterpret_cast<float*>(smem + TILE_OFF);  // A8 GEMM1: fp32 values
#pragma unroll
        for (int i = 0; i < NRW; ++i) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = (H + 2 * i) * 32 + 8 * (q >> 2) + 4 * g2 + (q & 3);
                const float rs = rows[row].rs;  // 0 for padding rows (never stored)
                if constexpr (GEMM == 1) {
                    const float gv = acc[i][0][q] * mc[0] * rs, uv = acc[i][1][q] * mc[1] * rs;
                    if constexpr (A8)
                        tile_f[row * TW + 32 * s + r32] = silu(gv) * uv;
                    else
                        tile[row * TW + 32 * s + r32] = f32_to_bf16_bits(silu(gv) * uv);
                } else {
                    tile[row * TW + 64 * s + r32] = f32_to_bf16_bits(acc[i][0][q] * mc[0] * rs);
                    tile[row * TW + 64 * s + 32 + r32] = f32_to_bf16_bits(acc[i][1][q] * mc[1] * rs);
                }
            }
        }
        if constexpr (GEMM == 1 && A8)
            store_act8_tile(a, ch, grp, smem, rows);
        else
            store_tile<GEMM>(a, ch, grp, smem, rows);
    }
}

template <int GEMM, int H, bool A8>
__device__ __attribute__((always_inline)) inline void f8_dispatch(int nrw, const GemmArgs& a, char* smem,
                                                                  const Chunk& ch, int grp, int s, int lane,
                                                                  const uint8_t* W, const float* ws,
                                                                  RowInfo pre) {
    switch (nrw) {
        case 0: f8_wave<GEMM, 0, H, A8>(a, smem, ch, grp, s, lane, W, ws, pre); break;
        case 1: f8_wave<GEMM, 1, H, A8>(a, smem, ch, grp, s, lane, W, ws, pre); break;
        case 2: f8_wave<GEMM, 2, H, A8>(a, smem, ch, grp, s, lane, W, ws, pre); break;
        default: f8_wave<GEMM, 3, H, A8>(a, smem, ch, grp, s, lane, W, ws, pre); break;
    }
}

}  // namespace

template <int GEMM, bool A8>
__global__ __launch_bounds__(512, 1) void prefill_f8_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[F8Lds<A8>::SMEM];
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
    const RowInfo pre = prefetch_row<GEMM, A8>(a, ch);  // consumed by the epilogue
    const int nrb32 = (ch.nrows + 31) >> 5;  // row blocks of 32 (at most 6)
    const int s = wv & 3, h = wv >> 2;
    const int nrw = (nrb32 - h + 1) >> 1;    // blocks h, h+2, h+4 below nrb32
    if (h == 0)
        f8_dispatch<GEMM, 0, A8>(nrw, a, smem, ch, grp, s, lane, W, ws, pre);
    else
        f8_dispatch<GEMM, 1, A8>(nrw, a, smem, ch, grp, s, lane, W, ws, pre);
}

hipError_t launch_split_rows(const SplitArgs& a, hipStream_t st) {
    if (a.rows == 0) return hipSuccess;
    if (a.K % 64 != 0) return hipErrorInvalidValue;
    dim3 grid((unsigned)((a.rows + 3) / 4)), block(256);
    if (a.act8) {
        if (a.K % 128 != 0 || !a.exps || a.exp_stride < a.K / 128) return hipErrorInvalidValue;
        fp8_act_rows_kernel<<<grid, block, 0, st>>>(a);
    } else {
        const int units = a.K / 16;
        if (units <= 128)
            split_rows_wg_kernel<2, 1><<<dim3((unsigned)((a.rows + 1) / 2)), block, 0, st>>>(a);
        else if (units > 256 && units <= 512)
            split_rows_wg_kernel<4, 2><<<dim3((unsigned)a.rows), block, 0, st>>>(a);
        else
            split_rows_kernel<<<grid, block, 0, st>>>(a);
    }
    return hipGetLastError();
}

template <int GEMM>
static hipError_t launch_prefill_f8(const GemmArgs& a, int max_chunks, hipStream_t st) {
    // two stages per loop trip; block scales of at most 128 K blocks per lane pair
    if (a.K % 128 != 0 || a.K > kPrefillFp8MaxK || a.N % 128 != 0) return hipErrorInvalidValue;
    if (a.n_groups * kPrefillF8Cols < a.N) return hipErrorInvalidValue;
    const int slots_per_xcd = (max_chunks + 7) / 8;
    dim3 grid((unsigned)(8 * (size_t)slots_per_xcd * a.n_groups));
    if (a.act8) {
        // scale-byte rows of 16 .. 128 bytes (whole 16-byte requests)
        if (!a.a_exp || a.exp_stride % 16 || a.exp_stride < a.K / 128 || a.exp_stride > kMaxExpStride)
            return hipErrorInvalidValue;
        // GEMM1 writes the down GEMM's input records: 128 intermediate columns per group
        if (GEMM == 1 && (!a.out_codes || !a.out_exps || a.out_exp_stride < a.N / 256 || a.N % 256))
            return hipErrorInvalidValue;
        prefill_f8_kernel<GEMM, true><<<grid, 512, 0, st>>>(a);
    } else {
        prefill_f8_kernel<GEMM, false><<<grid, 512, 0, st>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_prefill_f8_gemm1(const GemmArgs& a, int max_chunks, hipStream_t st) {
    return launch_prefill_f8<1>(a, max_chunks, st);
}
hipError_t launch_prefill_f8_gemm2(const GemmArgs& a, int max_chunks, hipStream_t st) {
    return launch_prefill_f8<2>(a, max_chunks, st);
}

}  // namespace moe
