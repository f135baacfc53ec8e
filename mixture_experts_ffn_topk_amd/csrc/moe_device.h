// moe_device.h -- device-side building blocks shared by the libmoe kernels
// (gfx950 / CDNA4, wave64).  Internal header: not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum WType { W_BF16 = 0, W_FP8 = 1, W_INT8 = 2, W_INT4 = 3 };

// ---------------------------------------------------------------------------
// Packed weight layout (written by the prepack kernels, streamed by the GEMMs)
//
// A [K, N] expert matrix is stored as N/16 column tiles, each a run of K/64
// "k-tiles"; a k-tile holds 64 lanes x 16 elements (1 KiB for 8-bit weights,
// 2 KiB for bf16) so one wave-wide 16-byte-per-lane load fetches exactly one
// MFMA B-operand fragment pair, fully coalesced.  Lane l holds column
// (l % 16) of the tile; its element s maps to row
//   bf16 / fp8 (for the bf16 MFMA 16x16x32):  k = (s/8)*32 + (l/16)*8 + s%8
//   int8      (for the i8 MFMA 16x16x64):     k = (l/16)*16 + s
// so elements [0,8) and [8,16) of a bf16/fp8 fragment feed two consecutive
// K=32 MFMAs.  The activations use the same k-slot assignment, which is all
// the MFMA contraction needs.  In w13 the gate tile j and the up tile j (the
// columns SiLU(C1) and C2 of one intermediate column block) are adjacent:
// packed tile index 2j is gate j, 2j+1 is up j.
// ---------------------------------------------------------------------------
__host__ __device__ inline int packed_kslot(int wtype, int lane_group, int s) {
    return wtype == W_INT8 ? lane_group * 16 + s : (s >> 3) * 32 + lane_group * 8 + (s & 7);
}

// Byte offset of packed tile (nt, kt) of one expert.
__host__ __device__ inline size_t packed_tile_offset(int elem_bytes, int K, int nt, int kt) {
    return ((size_t)nt * (size_t)(K / 64) + (size_t)kt) * 64u * 16u * (size_t)elem_bytes;
}

// INT4 weights (decode kernels only): per 16-column tile, one 1 KiB block per
// 128 K rows, 64 lanes x 16 bytes, so one 16-byte load per lane covers both
// 64-row k-tiles of the block.  Lane l (column l % 16, lane group g = l / 16)
// holds four dwords: (k-tile kt, half d) at dword 2 kt + d, the 8 elements
// s = 8d .. 8d+7 of the bf16 fragment order (k = kt*64 + (s/8)*32 + g*8 + s%8)
// with element 2i in nibble i and element 2i+1 in nibble i+4, so one AND
// of the dword shifted by 4i with 0x000F000F yields the pair (2i, 2i+1) as
// two 16-bit halves.  Nibbles hold the code biased by 8 (u = q + 8, 0..15).
__host__ __device__ inline size_t packed_i4_offset(int K, int nt, int kb) {
    return ((size_t)nt * (size_t)(K / 128) + (size_t)kb) * 1024u;
}

// ---------------------------------------------------------------------------
// Number conversions
// ---------------------------------------------------------------------------
__device__ inline float bf16_bits_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ inline uint16_t f32_to_bf16_bits(float f) {  // round to nearest even (v_cvt_pk_bf16_f32)
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v;
    v.x = (__bf16)lo;
    v.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// Four E4M3FN codes (one dword) -> four bf16 (two dwords), exact: every
// E4M3FN value, subnormals included, is representable in bf16.  Uses the
// gfx950 scaled converter with a unit scale.
__device__ inline void fp8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);
    lo = __builtin_bit_cast(uint32_t, a);
    hi = __builtin_bit_cast(uint32_t, b);
}

// Four E4M3FN codes -> four bf16 of (code value * s), each rounded once to
// nearest even.  (Dequantise-then-GEMM form used by the MFMA tile kernels.)
__device__ inline void fp8x4_to_bf16x4_scaled(uint32_t w, float s, uint32_t& lo, uint32_t& hi) {
    f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    lo = pack_bf16x2(a.x * s, a.y * s);
    hi = pack_bf16x2(b.x * s, b.y * s);
}

// 16 fp8 codes (u32x4) -> two bf16x8 MFMA fragments (elements 0..7, 8..15).
__device__ inline void fp8x16_to_frags(u32x4 w, bf16x8& f0, bf16x8& f1) {
    uint32_t a[4], b[4];
    fp8x4_to_bf16x4(w.x, a[0], a[1]);
    fp8x4_to_bf16x4(w.y, a[2], a[3]);
    fp8x4_to_bf16x4(w.z, b[0], b[1]);
    fp8x4_to_bf16x4(w.w, b[2], b[3]);
    f0 = __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], a[2], a[3]});
    f1 = __builtin_bit_cast(bf16x8, u32x4{b[0], b[1], b[2], b[3]});
}
__device__ inline void fp8x16_to_frags_scaled(u32x4 w, float s, bf16x8& f0, bf16x8& f1) {
    uint32_t a[4], b[4];
    fp8x4_to_bf16x4_scaled(w.x, s, a[0], a[1]);
    fp8x4_to_bf16x4_scaled(w.y, s, a[2], a[3]);
    fp8x4_to_bf16x4_scaled(w.z, s, b[0], b[1]);
    fp8x4_to_bf16x4_scaled(w.w, s, b[2], b[3]);
    f0 = __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], a[2], a[3]});
    f1 = __builtin_bit_cast(bf16x8, u32x4{b[0], b[1], b[2], b[3]});
}

// One dword of INT4 codes (8 biased nibbles, see packed_i4_offset) -> an
// MFMA B fragment of 8 bf16 values 136 + q, exactly: (u | 0x4300) read as
// bf16 is 128 + u for u < 16.  The 136 is removed by a second product
// against a constant fragment of -136 (exact in bf16), so no per-element
// subtraction is needed.
__device__ inline bf16x8 int4x8_to_frag_biased(uint32_t w) {
    u32x4 r;
    r.x = (w & 0x000F000Fu) | 0x43004300u;
    r.y = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
    r.z = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
    r.w = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
    return __builtin_bit_cast(bf16x8, r);
}
constexpr uint32_t kBf16Minus136x2 = 0xC308C308u;  // two bf16 -136.0

// SiLU(v) = v / (1 + e^-v) with the hardware reciprocal (1 ulp): the result
// is rounded to bf16 (2^-9) right after, so an exact division buys nothing.
// v -> -inf gives -0, v -> +inf gives +inf, NaN stays NaN.
__device__ inline float silu(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

// ---------------------------------------------------------------------------
// MFMA wrappers (16x16 output tile; lane l holds column l%16, rows
// 4*(l/16) .. 4*(l/16)+3 of the accumulator).
// ---------------------------------------------------------------------------
__device__ inline f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                                 __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Global memory helpers
// ---------------------------------------------------------------------------
__device__ inline u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline u32x4 ldg16_nt(const void* p) {
    // weights are streamed once: non-temporal hint keeps them from evicting
    // the activations that are re-read from L2
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Direct global -> LDS load of 16 bytes per lane (gfx950
// global_load_lds_dwordx4): lane l's bytes land at lds + 16*l.  lds must be
// wave-uniform.  The builtin only exists for the device; the host pass sees
// an empty body (it never runs device code).
__device__ inline void lds_dma16(const void* gptr, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
#else
    (void)gptr;
    (void)lds;
#endif
}
// Same, with the non-temporal cache policy: for data read exactly once (the
// weight stream), so it does not evict the activation rows other workgroups
// re-read from L2.
__device__ inline void lds_dma16_stream(const void* gptr, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void*)lds, 16, 0, 2);
#else
    (void)gptr;
    (void)lds;
#endif
}

// ---------------------------------------------------------------------------
// Wave-level reductions.  Inside each row of 16 lanes the values meet through
// DPP lane permutations (quad swaps, then the half-row and row mirrors: a few
// cycles each, no LDS crossbar); the four row results are then read as
// scalars.  Each step combines a value with its partner's in a symmetric way,
// so every lane of a row holds bit-identical partial results and the outcome
// is one fixed order (deterministic).  Every lane of the wave must be active.
// ---------------------------------------------------------------------------
enum : int {
    kDppQuadXor1 = 0xB1,      // quad_perm [1,0,3,2]
    kDppQuadXor2 = 0x4E,      // quad_perm [2,3,0,1]
    kDppRowHalfMirror = 0x141,
    kDppRowMirror = 0x140,
};
template <int CTRL>
__device__ inline int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline float dpp_f(float v) {
    return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
__device__ inline float lane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ inline float wave_sum(float v) {
    v += dpp_f<kDppQuadXor1>(v);
    v += dpp_f<kDppQuadXor2>(v);
    v += dpp_f<kDppRowHalfMirror>(v);
    v += dpp_f<kDppRowMirror>(v);
    return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ inline float wave_max(float v) {
    v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
    v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
    v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppRowMirror>(v));
    return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// wave-wide maximum of an unsigned word, returned as a scalar
__device__ inline uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)dpp_i<kDppQuadXor1>((int)v));
    v = max(v, (uint32_t)dpp_i<kDppQuadXor2>((int)v));
    v = max(v, (uint32_t)dpp_i<kDppRowHalfMirror>((int)v));
    v = max(v, (uint32_t)dpp_i<kDppRowMirror>((int)v));
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// ---------------------------------------------------------------------------
// Router top-k: one wave per token, expert e lives in lane e%64, slot e/64.
// Each logit is mapped to an unsigned word of the same order (-0 and +0
// share one word, they compare equal; NaN orders below -inf, chosen last).
// k rounds: the largest word among the experts still in play (four DPP
// steps inside each row of 16 lanes, the four rows' maxima read as
// scalars), then the experts holding it by one ballot per slot, and the
// lowest expert id among them wins -- so among equal logits the lower id
// comes first.  This is an exact total order on (logit, -id): the winners
// and their order are those of a stable sort.
// Scores are computed in fp32 from the winning logits: softmax over all E,
// or the logistic sigmoid; optional renormalisation over the k chosen
// scores.  Outputs: w_out / id_out [T, k] (skipped when w_out is null) and
// ids_lds[t*k + j] (when not null).
// ---------------------------------------------------------------------------
__device__ inline uint32_t logit_order(float v) {
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    u = (u << 1) == 0u ? 0u : u;  // -0 -> +0
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return v != v ? 0u : o;
}
__device__ inline float logit_of_order(uint32_t o) {
    const uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
    return o == 0u ? __builtin_nanf("") : __builtin_bit_cast(float, u);
}

template <int VPL>
__device__ inline void topk_token(const float* __restrict__ logits, int t, int E, int k, int score,
                                  int renorm, float* __restrict__ w_out,
                                  int32_t* __restrict__ id_out, int32_t* ids_lds, int lane) {
    const float* l = logits + (size_t)t * E;
    float v[VPL];
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
        int e = lane + 64 * q;
        v[q] = e < E ? l[e] : -__builtin_inff();
    }
    uint32_t key[VPL];
    bool live[VPL];  // in range and not yet chosen
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
        live[q] = lane + 64 * q < E;
        key[q] = logit_order(v[q]);
    }
    uint32_t my_o = 0u;  // lane j: the word and the id chosen in round j
    int my_id = 0;
    for (int j = 0; j < k; ++j) {
        uint32_t b = 0u;
#pragma unroll
        for (int q = 0; q < VPL; ++q) b = live[q] && key[q] > b ? key[q] : b;
        b = wave_max_u32(b);
        int win = -1;  // the lowest id holding b (uniform)
#pragma unroll
        for (int q = 0; q < VPL; ++q) {
            const uint64_t m = __ballot(live[q] && key[q] == b);
            if (win < 0 && m != 0ull) win = 64 * q + (int)__builtin_ctzll(m);
        }
#pragma unroll
        for (int q = 0; q < VPL; ++q) live[q] = live[q] && lane + 64 * q != win;
        if (lane == j) {
            my_o = b;
            my_id = win;
        }
    }
    const float my_logit = logit_of_order(my_o);
    float s;
    if (score == 0) {  // softmax over all E logits
        float m = -__builtin_inff();
#pragma unroll
        for (int q = 0; q < VPL; ++q)
            if (lane + 64 * q < E) m = fmaxf(m, v[q]);
        m = wave_max(m);
        float z = 0.f;
#pragma unroll
        for (int q = 0; q < VPL; ++q)
            if (lane + 64 * q < E) z += expf(v[q] - m);
        z = wave_sum(z);
        s = expf(my_logit - m) / z;
    } else {
        s = 1.0f / (1.0f + expf(-my_logit));
    }
    if (lane >= k) s = 0.f;
    if (renorm) {
        float tot = wave_sum(s);
        s = s / tot;
    }
    if (lane < k) {
        if (w_out) {
            w_out[(size_t)t * k + lane] = s;
            id_out[(size_t)t * k + lane] = my_id;
        }
        if (ids_lds) ids_lds[t * k + lane] = my_id;
    }
}

// Dynamic symmetric INT8 quantisation, binary32: s = amax/127 (correctly
// rounded), q = clamp(rint(x/s), +-127), x/s the correctly rounded quotient.
//
// The quotients are taken as t = x * r, r = 1/s correctly rounded: for
// 2^-125 <= s <= 2^125 and |x| <= amax, |t - x/s| <= 2^-23 |x/s| (two
// roundings of at most 2^-24 each) and the rounded quotient lies within
// 2^-24 |x/s| of x/s, |x/s| <= 127.0001, so the two differ by less than
// 2.3e-5.  rint(t) is then rint of the rounded quotient unless t lies within
// that distance of a half-integer; a group of values in which any active
// lane has a t within 6e-5 of one (about one value in 8000, and every exact
// tie) is recomputed with the division.  Outside that range of s (and for
// s = 0, inf or NaN) quant_recip returns 0 and the division runs.
__device__ inline float quant_recip(float s) {
    return s >= 0x1p-125f && s <= 0x1p125f ? __fdiv_rn(1.0f, s) : 0.f;
}
template <int N>
__device__ inline void quant_codes(const float (&x)[N], float s, float r, int (&q)[N]) {
    float t[N];
    bool slow = r == 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        t[i] = x[i] * r;
        slow = slow || fabsf(t[i] - floorf(t[i]) - 0.5f) < 6e-5f;
    }
    if (__ballot(slow) != 0ull) {  // uniform over the active lanes
#pragma unroll
        for (int i = 0; i < N; ++i) t[i] = s != 0.f ? __fdiv_rn(x[i], s) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float tq = fminf(fmaxf(rintf(t[i]), -127.f), 127.f);
        q[i] = s != 0.f ? (int)tq : 0;
    }
}
// 4 codes packed into a word, the first in the low byte
__device__ inline uint32_t pack_codes4(const int (&q)[4]) {
    return (uint32_t)(q[0] & 0xff) | ((uint32_t)(q[1] & 0xff) << 8) | ((uint32_t)(q[2] & 0xff) << 16) |
           ((uint32_t)(q[3] & 0xff) << 24);
}

// Quantise 8 bf16 values (one 16-byte piece) with scale s, r = quant_recip(s):
// 8 INT8 codes.
__device__ inline uint2 quant8(u32x4 v, float s, float r) {
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = bf16_bits_to_f32((uint16_t)((w4[i >> 1] >> ((i & 1) * 16)) & 0xffff));
    int q[8];
    quant_codes<8>(x, s, r, q);
    const int lo[4] = {q[0], q[1], q[2], q[3]}, hi[4] = {q[4], q[5], q[6], q[7]};
    return make_uint2(pack_codes4(lo), pack_codes4(hi));
}

// Lanes holding the same value e as this lane (valid lanes only; e < 2^nbits):
// one ballot per bit.
__device__ inline uint64_t match_any(int e, bool valid, int nbits) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        bool bit = (e >> b) & 1;
        uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return m;
}

// ---------------------------------------------------------------------------
// Explicit LDS pipeline helpers for the MFMA tile kernels.  Waves that also
// issue direct global->LDS loads read LDS only through these, so the compiler
// (which does not track them) adds no vmcnt drains before the reads.
// ---------------------------------------------------------------------------
// LDS byte address of a __shared__ object
__device__ inline uint32_t lds_addr(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
#else
    return (uint32_t)(uintptr_t)p;
#endif
}

// Explicit LDS accesses: the compiler does not track these, so every use is
// preceded by an explicit lgkmcnt wait that names the destination registers.
template <int OFF>
__device__ inline u32x4 ds_read16(uint32_t addr) {
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
template <int OFF>
__device__ inline void ds_write16(uint32_t addr, u32x4 v) {
    asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(addr), "v"(v), "i"(OFF) : "memory");
}
__device__ inline void lgkm_wait0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// at most N of this wave's LDS reads outstanding (they complete in order)
template <int N>
__device__ inline void lgkm_wait() {
    static_assert(N >= 0 && N < 16, "lgkmcnt is a 4-bit counter");
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}
__device__ inline void tie(u32x4& v) { asm volatile("" : "+v"(v)); }

// At most N of this wave's vector-memory operations (its direct-to-LDS
// loads) may still be outstanding; they complete in issue order.
template <int N>
__device__ inline void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ inline void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int N, typename F>
__device__ inline void static_for(F&& f) {
    if constexpr (N > 0) {
        static_for<N - 1>(f);
        f(std::integral_constant<int, N - 1>{});
    }
}

// Row tables written by the alignment kernel for the fused layer.
struct Chunk {
    int expert;     // expert index; == E means the shared expert
    int row_start;  // first row in sorted_ids (a multiple of 16)
    int nrows;      // rows in this chunk including padding (multiple of 16)
    int pad;
};

}  // namespace moe
