// moe_prefill.hip -- MFMA tile grouped GEMMs for many rows per expert.
//
// One workgroup (4 waves) owns one chunk of up to 128 sorted rows of one
// expert and 256 weight columns (GEMM1: 8 gate tiles + the 8 matching up
// tiles; GEMM2: 16 output tiles), over the full K range, so each weight byte
// of an expert column block is fetched once per chunk and the SiLU epilogue
// needs no cross-workgroup reduction.  Per 64-row K tile:
//   - the chunk's activation rows (gathered through sorted_ids for GEMM1) are
//     staged in LDS, double-buffered, one barrier per K tile;
//   - each wave streams its 4 weight tiles straight from HBM into registers
//     (prefetched one K tile ahead) and widens FP8 to bf16 with the 128x128
//     block scale folded in (dequantise-then-GEMM), bf16 and int8 as is;
//   - bf16 MFMA 16x16x32 (or i8 MFMA 16x16x64) over the chunk's 16-row blocks.
// Workgroup ids are dealt round-robin to the 8 XCDs; consecutive ids of one
// XCD take the column groups of one chunk, so the chunk's activation rows are
// shared through that XCD's L2.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

namespace {

template <int WT>
struct PF {
    static constexpr int EB = WT == W_BF16 ? 2 : 1;
    static constexpr int BV = WT == W_BF16 ? 2 : 1;
    static constexpr int AEB = WT == W_INT8 ? 1 : 2;
    static constexpr int A_ROW = 64 * AEB;         // bytes of one row per K tile
    static constexpr int A_STRIDE = A_ROW + 16;    // padded LDS row stride (bank spread)
    static constexpr int A_VEC_PER_ROW = A_ROW / 16;
    static constexpr int ROWS = kPrefillMB * 16;
    static constexpr int A_VEC_PER_THREAD = ROWS * A_VEC_PER_ROW / 256;
    typedef typename std::conditional<WT == W_INT8, i32x4, f32x4>::type Acc;
};

}  // namespace

template <int WT, int GEMM>
__global__ __launch_bounds__(256, 2) void prefill_kernel(GemmArgs a) {
    using T = PF<WT>;
    using Acc = typename T::Acc;
    constexpr int MB = kPrefillMB;
    constexpr int NT = kPrefillTilesPerWave;
    __shared__ __attribute__((aligned(16))) char lds[2][T::ROWS * T::A_STRIDE];
    __shared__ int row_src[T::ROWS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6, g = lane >> 4, c16 = lane & 15;
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
    const int ntiles = a.N / 16;

    // this wave's packed tiles and their logical first columns
    int tile[NT], col0[NT];
    bool tile_ok[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        if (GEMM == 1) {
            const int pt = (grp * kPrefillWaves + wv) * 2 + (n >> 1);  // pair tile
            const int h = n & 1;                                       // 0 gate, 1 up
            tile[n] = 2 * pt + h;
            col0[n] = h * (a.N / 2) + pt * 16;
        } else {
            tile[n] = (grp * kPrefillWaves + wv) * NT + n;
            col0[n] = tile[n] * 16;
        }
        tile_ok[n] = tile[n] < ntiles;
        if (!tile_ok[n]) {
            tile[n] = ntiles - 1;  // stream a valid tile; results discarded
            col0[n] = 0;
        }
    }
    const uint8_t* bptr[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n)
        bptr[n] = W + packed_tile_offset(T::EB, a.K, tile[n], 0) + lane * 16 * T::EB;
    constexpr size_t kt_bytes = 64 * 16 * T::EB;

    // source row of each chunk row (-1 = padding)
    if (tid < T::ROWS) {
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

    // per-thread share of the activation tile loads
    const char* a_src[T::A_VEC_PER_THREAD];
    int a_dst[T::A_VEC_PER_THREAD];
#pragma unroll
    for (int v = 0; v < T::A_VEC_PER_THREAD; ++v) {
        const int idx = tid + 256 * v;  // vector index in the tile
        const int row = idx / T::A_VEC_PER_ROW, part = idx % T::A_VEC_PER_ROW;
        const int src = row_src[row];
        a_src[v] = src >= 0 ? (const char*)a.A + (size_t)src * a.K * T::AEB + part * 16 : nullptr;
        a_dst[v] = row * T::A_STRIDE + part * 16;
    }
    u32x4 areg[T::A_VEC_PER_THREAD];
    auto load_a = [&](int kt) {
#pragma unroll
        for (int v = 0; v < T::A_VEC_PER_THREAD; ++v)
            areg[v] = a_src[v] ? ldg16(a_src[v] + (size_t)kt * T::A_ROW) : u32x4{0, 0, 0, 0};
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int v = 0; v < T::A_VEC_PER_THREAD; ++v)
            *reinterpret_cast<u32x4*>(&lds[buf][a_dst[v]]) = areg[v];
    };
    u32x4 bq[2][NT][T::BV];
    auto load_b = [&](int kt, int buf) {
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int v = 0; v < T::BV; ++v)
                bq[buf][n][v] = ldg16_nt(bptr[n] + (size_t)kt * kt_bytes + v * 16);
    };

    Acc acc[MB][NT];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[rb][n] = Acc{0, 0, 0, 0};

    const int nkt = a.K / 64;
    const int nbw = a.N / 128;
    auto compute = [&](int kt, int abuf, int bbuf) {
        bf16x8 b0[NT], b1[NT];
        if constexpr (WT == W_FP8) {
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const float s = ws[(kt >> 1) * nbw + col0[n] / 128];
                fp8x16_to_frags_scaled(bq[bbuf][n][0], s, b0[n], b1[n]);
            }
        } else if constexpr (WT == W_BF16) {
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                b0[n] = __builtin_bit_cast(bf16x8, bq[bbuf][n][0]);
                b1[n] = __builtin_bit_cast(bf16x8, bq[bbuf][n][1]);
            }
        }
        const char* base = &lds[abuf][0];
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) {
            if (rb < nrb) {
                const char* rp = base + (rb * 16 + c16) * T::A_STRIDE + g * 16;
                if constexpr (WT == W_INT8) {
                    const u32x4 av = *reinterpret_cast<const u32x4*>(rp);
#pragma unroll
                    for (int n = 0; n < NT; ++n) acc[rb][n] = mfma_i8(av, bq[bbuf][n][0], acc[rb][n]);
                } else {
                    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(rp);
                    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(rp + 64);
#pragma unroll
                    for (int n = 0; n < NT; ++n) {
                        acc[rb][n] = mfma_bf16(a0, b0[n], acc[rb][n]);
                        acc[rb][n] = mfma_bf16(a1, b1[n], acc[rb][n]);
                    }
                }
            }
        }
    };

    load_a(0);
    load_b(0, 0);
    store_a(0);
    __syncthreads();
    for (int kt = 0; kt < nkt; kt += 2) {
        // even step: compute from LDS buffer 0 / B buffer 0, prefetch into 1
        if (kt + 1 < nkt) {
            load_a(kt + 1);
            load_b(kt + 1, 1);
        }
        compute(kt, 0, 0);
        if (kt + 1 < nkt) store_a(1);
        __syncthreads();
        if (kt + 1 >= nkt) break;
        // odd step
        if (kt + 2 < nkt) {
            load_a(kt + 2);
            load_b(kt + 2, 0);
        }
        compute(kt + 1, 1, 1);
        if (kt + 2 < nkt) store_a(0);
        __syncthreads();
    }

    // epilogue
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
        if (rb >= nrb) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int lrow = rb * 16 + 4 * g + i;
            const int grow = ch.row_start + lrow;
            const int pid = a.sorted_ids[grow];
            if (pid >= a.P_tot) continue;
            if constexpr (GEMM == 1) {
                const int I = a.N / 2;
                float sx = 1.f;
                if constexpr (WT == W_INT8) sx = a.a_scale[pid < a.P ? pid / a.topk : pid - a.P];
#pragma unroll
                for (int p = 0; p < NT / 2; ++p) {
                    if (!tile_ok[2 * p]) continue;
                    float gv, uv;
                    if constexpr (WT == W_INT8) {
                        gv = (float)acc[rb][2 * p][i] * sx * ws[col0[2 * p] + c16];
                        uv = (float)acc[rb][2 * p + 1][i] * sx * ws[col0[2 * p + 1] + c16];
                    } else {
                        gv = acc[rb][2 * p][i];
                        uv = acc[rb][2 * p + 1][i];
                    }
                    ((uint16_t*)a.out)[(size_t)grow * I + col0[2 * p] + c16] =
                        f32_to_bf16_bits(silu(gv) * uv);
                }
            } else {
                float sa = 1.f;
                if constexpr (WT == W_INT8) sa = a.a_scale[grow];
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    if (!tile_ok[n]) continue;
                    float v;
                    if constexpr (WT == W_INT8)
                        v = (float)acc[rb][n][i] * sa * ws[col0[n] + c16];
                    else
                        v = acc[rb][n][i];
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
        prefill_kernel<W_FP8, GEMM><<<grid, 256, 0, st>>>(a);
    else if (wtype == W_INT8)
        prefill_kernel<W_INT8, GEMM><<<grid, 256, 0, st>>>(a);
    else
        prefill_kernel<W_BF16, GEMM><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_prefill_gemm1(int wtype, const GemmArgs& a, int max_chunks, hipStream_t st) {
    return launch_prefill<1>(wtype, a, max_chunks, st);
}
hipError_t launch_prefill_gemm2(int wtype, const GemmArgs& a, int max_chunks, hipStream_t st) {
    return launch_prefill<2>(wtype, a, max_chunks, st);
}

}  // namespace moe
