// moe_route.hip -- router top-k, expert alignment, dynamic INT8 row
// quantisation and weight prepack kernels (gfx950).
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router top-k: one wave per token, expert e lives in lane e%64, slot e/64.
// k rounds of a wave-wide argmax over (logit, -expert id): ties go to the
// lower expert id, selection is on the fp32 logits themselves.  Scores are
// computed in fp32: softmax over all E, or the logistic sigmoid; optional
// renormalisation over the k chosen scores.
// ---------------------------------------------------------------------------
template <int VPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int score, int renorm,
                                                   float* __restrict__ w_out,
                                                   int32_t* __restrict__ id_out) {
    const int lane = threadIdx.x & 63;
    const int t = (int)((blockIdx.x * (size_t)blockDim.x + threadIdx.x) >> 6);
    if (t >= T) return;  // whole wave exits together
    const float* l = logits + (size_t)t * E;
    float v[VPL];
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
        int e = lane + 64 * q;
        v[q] = e < E ? l[e] : -__builtin_inff();
    }
    uint32_t taken = 0;
    float my_logit = 0.f;
    int my_id = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -__builtin_inff();
        int bi = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < VPL; ++q) {
            int e = lane + 64 * q;
            bool ok = e < E && !((taken >> q) & 1u);
            if (ok && (v[q] > bv || (v[q] == bv && e < bi))) {
                bv = v[q];
                bi = e;
            }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            float ov = __shfl_xor(bv, o, 64);
            int oi = __shfl_xor(bi, o, 64);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if (lane == (bi & 63)) taken |= 1u << (bi >> 6);
        if (lane == j) {
            my_logit = bv;
            my_id = bi;
        }
    }
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
        w_out[(size_t)t * k + lane] = s;
        id_out[(size_t)t * k + lane] = my_id;
    }
}

// ---------------------------------------------------------------------------
// Alignment (one workgroup, NW waves).
//
// The virtual id list is topk_ids.flat[0..P) followed, when n_shared > 0, by
// n_shared entries of id E (the shared expert, one per token).  Pass 1: every
// wave walks its own contiguous segment 64 ids at a time and counts ids per
// expert into its private LDS row; lanes holding the same id are found with a
// ballot per id bit (match-any), so no atomics are involved.  Pass 2: per
// expert totals, padding to the block size, an exclusive prefix sum over
// experts, and per-(wave, expert) bases in (expert, wave) order -- which keeps
// the canonical ascending-index order inside each expert.  Pass 3 re-walks
// the segments and scatters each index to base + rank-among-equal-lanes.
// The result is deterministic and bit-identical to the brute-force order.
// ---------------------------------------------------------------------------
__device__ inline uint64_t match_any(int e, bool valid, int nbits) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        bool bit = (e >> b) & 1;
        uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return m;
}

// Block-wide exclusive scan of `val` (one value per thread); returns the
// thread's exclusive prefix, and the total in *total.  scratch: >= NW ints.
__device__ inline int block_exclusive_scan(int val, int* scratch, int* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int inc = val;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int n = __shfl_up(inc, o, 64);
        if (lane >= o) inc += n;
    }
    if (lane == 63) scratch[w] = inc;
    __syncthreads();
    int wbase = 0, tot = 0;
    for (int i = 0; i < nw; ++i) {
        int s = scratch[i];
        if (i < w) wbase += s;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return wbase + inc - val;
}

__global__ void align_kernel(AlignArgs a) {
    extern __shared__ int smem[];
    const int nw = blockDim.x >> 6, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nthr = blockDim.x;
    const int E_tot = a.E + (a.n_shared > 0 ? 1 : 0);
    const int P_tot = a.P + a.n_shared;
    const int sentinel = P_tot;
    int* cnt = smem;                 // [nw][E_tot]
    int* scratch = cnt + nw * E_tot; // [64]
    for (int i = threadIdx.x; i < nw * E_tot; i += nthr) cnt[i] = 0;
    __syncthreads();

    const int seg = ((P_tot + nw - 1) / nw + 63) / 64 * 64;
    const int beg = w * seg;
    const int end = min(P_tot, beg + seg);
    const int nbits = 32 - __clz(E_tot > 1 ? E_tot - 1 : 1);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    // the expert of pair i (E for the shared-expert pairs), -1 past the
    // segment; loads go out U rows of 64 at a time so their latency is paid
    // once per U iterations
    constexpr int U = 8;
    auto load_rows = [&](int base, int (&ev)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * 64 + lane;
            ev[u] = i < end ? (i < a.P ? a.ids[i] : a.E) : -1;
        }
    };
    auto is_valid = [&](int i, int e) { return i < end && (i < a.P ? (e >= 0 && e < a.E) : true); };

    // pass 1: per-wave counts
    for (int base = beg; base < end; base += 64 * U) {
        int ev[U];
        load_rows(base, ev);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * 64 + lane, e = ev[u];
            const bool valid = is_valid(i, e);
            const uint64_t peers = match_any(e, valid, nbits);
            if (valid && (peers & lt) == 0) cnt[w * E_tot + e] += __popcll(peers);
        }
    }
    __syncthreads();

    // pass 2: totals, padding, prefix sums, per-(wave, expert) bases
    const int per = (E_tot + nthr - 1) / nthr;  // experts per thread (contiguous)
    const int e0 = threadIdx.x * per;
    int my_pad = 0, my_chunks = 0;
    for (int e = e0; e < min(E_tot, e0 + per); ++e) {
        int c = 0;
        for (int ww = 0; ww < nw; ++ww) c += cnt[ww * E_tot + e];
        const int p = (c + a.B - 1) / a.B * a.B;
        my_pad += p;
        if (a.chunks) my_chunks += (p + a.chunk_rows - 1) / a.chunk_rows;
    }
    int npp = 0, nchunks = 0;
    int off = block_exclusive_scan(my_pad, scratch, &npp);
    int coff = block_exclusive_scan(my_chunks, scratch, &nchunks);
    for (int e = e0; e < min(E_tot, e0 + per); ++e) {
        int run = off;
        for (int ww = 0; ww < nw; ++ww) {
            const int c = cnt[ww * E_tot + e];
            cnt[ww * E_tot + e] = run;
            run += c;
        }
        const int c = run - off;
        const int p = (c + a.B - 1) / a.B * a.B;
        for (int s = off + c; s < off + p; ++s) a.sorted_ids[s] = sentinel;
        if (a.expert_ids)
            for (int b = off / a.B; b < (off + p) / a.B; ++b) a.expert_ids[b] = e;
        if (a.chunks) {
            for (int r = 0; r < p; r += a.chunk_rows) {
                Chunk ch;
                ch.expert = e;
                ch.row_start = off + r;
                ch.nrows = min(a.chunk_rows, p - r);
                ch.pad = 0;
                a.chunks[coff++] = ch;
            }
        }
        off += p;
    }
    if (threadIdx.x == 0) {
        a.npp[0] = npp;
        if (a.meta) {
            a.meta[0] = npp;
            a.meta[1] = nchunks;
        }
    }
    for (int64_t s = npp + threadIdx.x; s < a.cap; s += nthr) a.sorted_ids[s] = sentinel;
    if (a.expert_ids) {
        const int64_t nblk = (a.cap + a.B - 1) / a.B;
        for (int64_t b = npp / a.B + threadIdx.x; b < nblk; b += nthr) a.expert_ids[b] = -1;
    }
    __syncthreads();

    // pass 3: stable scatter (rows of 64 in ascending pair order)
    for (int base = beg; base < end; base += 64 * U) {
        int ev[U];
        load_rows(base, ev);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * 64 + lane, e = ev[u];
            const bool valid = is_valid(i, e);
            const uint64_t peers = match_any(e, valid, nbits);
            if (valid) {
                const int b0 = cnt[w * E_tot + e];
                a.sorted_ids[b0 + __popcll(peers & lt)] = i;
                if ((peers & lt) == 0) cnt[w * E_tot + e] = b0 + __popcll(peers);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Dynamic symmetric INT8 row quantisation, one wave per row, binary32:
// s = amax/127 (correctly rounded), q = clamp(rint(x/s), +-127).
// Rows of a sorted-row table may be filtered: when row_ids != nullptr, row r
// is processed only if r < meta[0] and row_ids[r] < sentinel.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_rows_kernel(QuantArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)((blockIdx.x * (size_t)blockDim.x + threadIdx.x) >> 6);
    if (r >= a.rows) return;
    if (a.row_ids) {
        if (r >= a.meta[0] || a.row_ids[r] >= a.sentinel) return;
    }
    const uint16_t* x = a.x + r * (int64_t)a.cols;
    float amax = 0.f;
    for (int c = lane * 8; c < a.cols; c += 64 * 8) {
        u32x4 v = ldg16(x + c);
        uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            amax = fmaxf(amax, fabsf(bf16_bits_to_f32((uint16_t)(w4[i] & 0xffff))));
            amax = fmaxf(amax, fabsf(bf16_bits_to_f32((uint16_t)(w4[i] >> 16))));
        }
    }
    amax = wave_max(amax);
    const float s = __fdiv_rn(amax, 127.0f);
    if (lane == 0) a.scale[r] = s;
    int8_t* q = a.q + r * (int64_t)a.cols;
    for (int c = lane * 8; c < a.cols; c += 64 * 8) {
        u32x4 v = ldg16(x + c);
        uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint16_t bits = (uint16_t)((w4[i >> 1] >> ((i & 1) * 16)) & 0xffff);
            int qi = 0;
            if (s != 0.f) {
                float t = rintf(__fdiv_rn(bf16_bits_to_f32(bits), s));
                t = fminf(fmaxf(t, -127.f), 127.f);
                qi = (int)t;
            }
            packed[i >> 2] |= ((uint32_t)(qi & 0xff)) << ((i & 3) * 8);
        }
        *reinterpret_cast<uint2*>(q + c) = make_uint2(packed[0], packed[1]);
    }
}

// ---------------------------------------------------------------------------
// Prepack: logical [E, K, N] -> packed tiles (see moe_device.h).  One thread
// writes one lane's 16 elements of one k-tile.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void prepack_kernel(const T* __restrict__ w, int E, int K, int N,
                                                      int is_w13, int wtype, T* __restrict__ out) {
    const int ntiles = N / 16, ktiles = K / 64;
    const int64_t total = (int64_t)E * ntiles * ktiles * 64;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const int lane = (int)(gid & 63);
    int64_t rest = gid >> 6;
    const int kt = (int)(rest % ktiles);
    rest /= ktiles;
    const int nt = (int)(rest % ntiles);
    const int e = (int)(rest / ntiles);
    int col;
    if (is_w13) {
        const int j = nt >> 1, h = nt & 1;
        col = h * (N / 2) + j * 16;
    } else {
        col = nt * 16;
    }
    const int n = col + (lane & 15);
    const int g = lane >> 4;
    const T* src = w + (size_t)e * K * N;
    T* dst = out + (size_t)e * K * N + ((size_t)nt * ktiles + kt) * 64 * 16 + (size_t)lane * 16;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        const int k = kt * 64 + packed_kslot(wtype, g, s);
        dst[s] = src[(size_t)k * N + n];
    }
}

// ---------------------------------------------------------------------------
// FP8 block dequantisation (utility; uses the same converters as the GEMMs).
// codes [K, N] with scales [K/128, N/128] -> fp32 [K, N].
//   mode 0: value(code) * scale in fp32 via the exact bf16 converter
//   mode 1: bf16(value(code) * scale) via the scaled converter
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dequant_fp8_kernel(const uint8_t* __restrict__ codes,
                                                          const float* __restrict__ scale, int K,
                                                          int N, int mode, float* __restrict__ out) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nq = (int64_t)K * N / 4;
    if (gid >= nq) return;
    const int64_t idx = gid * 4;
    const int k = (int)(idx / N), n = (int)(idx % N);
    const float s = scale ? scale[(k / 128) * (N / 128) + n / 128] : 1.0f;
    const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + idx);
    uint32_t lo, hi;
    if (mode == 0)
        fp8x4_to_bf16x4(w, lo, hi);
    else
        fp8x4_to_bf16x4_scaled(w, s, lo, hi);
    const float m = mode == 0 ? s : 1.0f;
    out[idx + 0] = bf16_bits_to_f32((uint16_t)(lo & 0xffff)) * m;
    out[idx + 1] = bf16_bits_to_f32((uint16_t)(lo >> 16)) * m;
    out[idx + 2] = bf16_bits_to_f32((uint16_t)(hi & 0xffff)) * m;
    out[idx + 3] = bf16_bits_to_f32((uint16_t)(hi >> 16)) * m;
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
hipError_t launch_topk(const float* logits, int T, int E, int k, int score, int renorm,
                       float* w, int32_t* ids, hipStream_t st) {
    if (T == 0) return hipSuccess;
    const int waves_per_block = 4;
    dim3 grid((T + waves_per_block - 1) / waves_per_block), block(64 * waves_per_block);
    const int vpl = (E + 63) / 64;
    if (vpl <= 1)
        topk_kernel<1><<<grid, block, 0, st>>>(logits, T, E, k, score, renorm, w, ids);
    else if (vpl <= 2)
        topk_kernel<2><<<grid, block, 0, st>>>(logits, T, E, k, score, renorm, w, ids);
    else if (vpl <= 4)
        topk_kernel<4><<<grid, block, 0, st>>>(logits, T, E, k, score, renorm, w, ids);
    else if (vpl <= 8)
        topk_kernel<8><<<grid, block, 0, st>>>(logits, T, E, k, score, renorm, w, ids);
    else
        topk_kernel<16><<<grid, block, 0, st>>>(logits, T, E, k, score, renorm, w, ids);
    return hipGetLastError();
}

int align_waves(int E_tot) { return E_tot <= 512 ? 16 : 8; }

size_t align_lds_bytes(int E_tot) {
    return ((size_t)align_waves(E_tot) * E_tot + 64) * sizeof(int);
}

hipError_t launch_align(const AlignArgs& a, hipStream_t st) {
    const int E_tot = a.E + (a.n_shared > 0 ? 1 : 0);
    const int nw = align_waves(E_tot);
    align_kernel<<<1, nw * 64, align_lds_bytes(E_tot), st>>>(a);
    return hipGetLastError();
}

hipError_t launch_quant_rows(const QuantArgs& a, hipStream_t st) {
    if (a.rows == 0) return hipSuccess;
    const int64_t waves = a.rows;
    dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    quant_rows_kernel<<<grid, block, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_prepack(int elem_bytes, int wtype, const void* w, int E, int K, int N,
                          int is_w13, void* out, hipStream_t st) {
    const int64_t total = (int64_t)E * (N / 16) * (K / 64) * 64;
    dim3 grid((unsigned)((total + 255) / 256)), block(256);
    if (elem_bytes == 2)
        prepack_kernel<uint16_t><<<grid, block, 0, st>>>((const uint16_t*)w, E, K, N, is_w13,
                                                         wtype, (uint16_t*)out);
    else
        prepack_kernel<uint8_t><<<grid, block, 0, st>>>((const uint8_t*)w, E, K, N, is_w13, wtype,
                                                        (uint8_t*)out);
    return hipGetLastError();
}

hipError_t launch_dequant_fp8(const uint8_t* codes, const float* scale, int K, int N, int mode,
                              float* out, hipStream_t st) {
    const int64_t nq = (int64_t)K * N / 4;
    if (nq == 0) return hipSuccess;
    dim3 grid((unsigned)((nq + 255) / 256)), block(256);
    dequant_fp8_kernel<<<grid, block, 0, st>>>(codes, scale, K, N, mode, out);
    return hipGetLastError();
}

}  // namespace moe
