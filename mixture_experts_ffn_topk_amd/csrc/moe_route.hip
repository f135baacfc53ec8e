// moe_route.hip -- router top-k, expert alignment, dynamic INT8 row
// quantisation and weight prepack kernels (gfx950).
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

template <int VPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int score, int renorm,
                                                   float* __restrict__ w_out,
                                                   int32_t* __restrict__ id_out) {
    const int lane = threadIdx.x & 63;
    const int t = (int)((blockIdx.x * (size_t)blockDim.x + threadIdx.x) >> 6);
    if (t >= T) return;  // whole wave exits together
    topk_token<VPL>(logits, t, E, k, score, renorm, w_out, id_out, nullptr, lane);
}

// ---------------------------------------------------------------------------
// Dynamic symmetric INT8 quantisation of one row by one wave, binary32:
// s = amax/127 (correctly rounded), q = clamp(rint(x/s), +-127).  The whole
// wave must be active.
// ---------------------------------------------------------------------------
// rows up to 64 * 8 * PIECES values stay in registers (6 where the caller's
// own registers are many: 8 spilled inside the one-workgroup alignment)
constexpr int kQuantRegPieces = 6;

template <int PIECES = kQuantRegPieces, int LP = 1>
__device__ inline void quant_row(const uint16_t* __restrict__ x, int cols, int8_t* __restrict__ q,
                                 float* __restrict__ scale, int lane) {
    if (cols <= 64 * 8 * PIECES) {
        // the whole row in registers: every load in flight at once, one read
        u32x4 v[PIECES];
#pragma unroll
        for (int i = 0; i < PIECES; ++i) {
            const int c = lane * 8 + 512 * i;
            v[i] = c < cols ? ldg16(x + c) : u32x4{0, 0, 0, 0};
        }
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < PIECES; ++i) {
            const uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                amax = fmaxf(amax, fabsf(bf16_bits_to_f32((uint16_t)(w4[j] & 0xffff))));
                amax = fmaxf(amax, fabsf(bf16_bits_to_f32((uint16_t)(w4[j] >> 16))));
            }
        }
        amax = wave_max(amax);
        const float s = __fdiv_rn(amax, 127.0f), r = quant_recip(s);
        if (lane == 0) *scale = s;
#pragma unroll
        for (int i = 0; i < PIECES; ++i) {
            const int c = lane * 8 + 512 * i;
            if (c < cols) *reinterpret_cast<uint2*>(q + c) = quant8(v[i], s, r);
            // one piece's divisions at a time (interleaving all of them spills)
            __builtin_amdgcn_sched_barrier(0);
        }
        return;
    }
    // wider rows: two passes (amax, then codes), each in batches of LP loads
    // issued together, so a pass costs one round trip per batch (LP > 1
    // raises the kernel's register count: callers whose occupancy matters
    // keep LP = 1)
    float amax = 0.f;
    for (int c0 = lane * 8; c0 < cols; c0 += 512 * LP) {
        u32x4 v[LP];
#pragma unroll
        for (int i = 0; i < LP; ++i) {
            const int c = c0 + 512 * i;
            v[i] = c < cols ? ldg16(x + c) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < LP; ++i) {
            const uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                amax = fmaxf(amax, fabsf(bf16_bits_to_f32((uint16_t)(w4[j] & 0xffff))));
                amax = fmaxf(amax, fabsf(bf16_bits_to_f32((uint16_t)(w4[j] >> 16))));
            }
        }
    }
    amax = wave_max(amax);
    const float s = __fdiv_rn(amax, 127.0f), r = quant_recip(s);
    if (lane == 0) *scale = s;
    for (int c0 = lane * 8; c0 < cols; c0 += 512 * LP) {
        u32x4 v[LP];
#pragma unroll
        for (int i = 0; i < LP; ++i) {
            const int c = c0 + 512 * i;
            v[i] = c < cols ? ldg16(x + c) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < LP; ++i) {
            const int c = c0 + 512 * i;
            if (c < cols) *reinterpret_cast<uint2*>(q + c) = quant8(v[i], s, r);
            __builtin_amdgcn_sched_barrier(0);
        }
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
// the canonical ascending-index order inside each expert.  Pass 3 walks the
// segments again (from registers when a wave's segment is one batch of rows)
// and scatters each index to base + rank-among-equal-lanes.  The result is
// deterministic and bit-identical to the brute-force order.
//
// Blocks after the first quantise token rows to INT8 (one wave per row) when
// the arguments ask for it: independent work that shares the launch.
// ---------------------------------------------------------------------------

// Block-wide exclusive scans of two values per thread in the same steps;
// returns the prefixes in (*pa, *pb) and the totals in (*ta, *tb).
// scratch: >= 2 * NW ints.
__device__ inline void block_exclusive_scan2(int va, int vb, int* scratch, int* pa, int* pb,
                                             int* ta, int* tb) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int ia = va, ib = vb;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int na = __shfl_up(ia, o, 64);
        const int nb = __shfl_up(ib, o, 64);
        if (lane >= o) {
            ia += na;
            ib += nb;
        }
    }
    if (lane == 63) {
        scratch[2 * w] = ia;
        scratch[2 * w + 1] = ib;
    }
    __syncthreads();
    int wa = 0, wb = 0, sa = 0, sb = 0;
    for (int i = 0; i < nw; ++i) {
        const int xa = scratch[2 * i], xb = scratch[2 * i + 1];
        if (i < w) {
            wa += xa;
            wb += xb;
        }
        sa += xa;
        sb += xb;
    }
    *pa = wa + ia - va;
    *pb = wb + ib - vb;
    *ta = sa;
    *tb = sb;
}

constexpr int kAlignMaxWaves = 16;
constexpr int kAlignMaxPer = 2;  // experts per thread: E_tot <= 1024 and >= 512 threads

// ROUTE: the workgroup first runs the router top-k of all a.P / r.k tokens
// (wave w takes tokens w, w + NW, ...), writing the weights and ids out and
// the ids into LDS, from which the alignment then reads them: one dispatch,
// and no round trip of the ids through memory between two kernels.
// The tile kernels' schedule: the chunk list copied in order of decreasing
// rows (chunks of one size in any order).  Those kernels deal chunks to
// workgroups in list order and the hardware gives the next workgroup to the
// first CU that frees up, so the largest chunks start first and the smallest
// fill the last round: the launch ends when its slowest CU does, and a
// chunk's time grows with its rows.  Sizes are multiples of 16, at most
// chunk_rows: one class per size.  Called by the whole workgroup once the
// chunk list is written and a barrier has made it visible.
constexpr int kSchedClasses = 16;
__device__ inline int sched_class(int nrows, int chunk_rows) {
    return min(max((chunk_rows - nrows) >> 4, 0), kSchedClasses - 1);
}
__device__ void write_sched(const AlignArgs& a, int nchunks) {
    __shared__ int cls[kSchedClasses];
    if (!a.sched) return;  // kernel argument: uniform
    const int tid = threadIdx.x, nthr = blockDim.x;
    if (tid < kSchedClasses) cls[tid] = 0;
    __syncthreads();
    for (int c = tid; c < nchunks; c += nthr) atomicAdd(&cls[sched_class(a.chunks[c].nrows, a.chunk_rows)], 1);
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int k = 0; k < kSchedClasses; ++k) {
            const int v = cls[k];
            cls[k] = run;
            run += v;
        }
    }
    __syncthreads();
    for (int c = tid; c < nchunks; c += nthr) {
        const Chunk ch = a.chunks[c];
        a.sched[atomicAdd(&cls[sched_class(ch.nrows, a.chunk_rows)], 1)] = ch;
    }
}

template <bool ROUTE, int VPL>
__global__ __launch_bounds__(1024) void align_kernel(AlignArgs a, RouteArgs ra) {
    extern __shared__ int smem[];
    const int nw = blockDim.x >> 6, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (blockIdx.x > 0) {  // INT8 token rows (whole waves exit together)
        const int64_t r = (int64_t)(blockIdx.x - 1) * nw + w;
        if (r < a.q_rows)
            quant_row<kQuantRegPieces, 4>(a.qx + r * a.q_cols, a.q_cols, a.qq + r * a.q_cols, a.qs + r, lane);
        return;
    }
    const int nthr = blockDim.x;
    const int E_tot = a.E + (a.n_shared > 0 ? 1 : 0);
    const int P_tot = a.P + a.n_shared;
    const int sentinel = P_tot;
    int* cnt = smem;                 // [nw][E_tot]
    int* scratch = cnt + nw * E_tot; // [2 * nw]
    const int32_t* ids = a.ids;
    if constexpr (ROUTE) {
        int32_t* ids_lds = scratch + 2 * kAlignMaxWaves;  // [P]
        const int T = a.P / ra.k;
        for (int t = w; t < T; t += nw)
            topk_token<VPL>(ra.logits, t, a.E, ra.k, ra.score, ra.renorm, ra.w_out, ra.id_out, ids_lds,
                            lane);
        ids = ids_lds;
        __syncthreads();
    }
    for (int i = threadIdx.x; i < nw * E_tot; i += nthr) cnt[i] = 0;

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
            ev[u] = i < end ? (i < a.P ? ids[i] : a.E) : -1;
        }
    };
    auto is_valid = [&](int i, int e) { return i < end && (i < a.P ? (e >= 0 && e < a.E) : true); };
    const bool one_batch = end - beg <= 64 * U;
    int ev0[U];
    uint64_t pm0[U];
    if (one_batch) load_rows(beg, ev0);  // issued before the barrier that ends the zeroing
    __syncthreads();

    // pass 1: per-wave counts
    if (one_batch) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            pm0[u] = 0;
            if (beg + u * 64 < end) {  // rows past the segment hold no pair (uniform test)
                const int i = beg + u * 64 + lane, e = ev0[u];
                const bool valid = is_valid(i, e);
                pm0[u] = match_any(e, valid, nbits);
                if (valid && (pm0[u] & lt) == 0) cnt[w * E_tot + e] += __popcll(pm0[u]);
            }
        }
    } else {
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
    }
    __syncthreads();

    // pass 2: totals, padding, prefix sums, per-(wave, expert) bases.  A
    // thread owns at most kAlignMaxPer contiguous experts; their per-wave
    // counts are read once, all loads in flight together (the wave index is
    // clamped instead of tested, so no load waits behind a branch).
    const int per = (E_tot + nthr - 1) / nthr;
    const int e0 = threadIdx.x * per;
    int cw[kAlignMaxPer][kAlignMaxWaves];
    int my_pad = 0, my_chunks = 0;
#pragma unroll
    for (int q = 0; q < kAlignMaxPer; ++q) {
        const int e = e0 + q;
        const bool own = q < per && e < E_tot;
        int c = 0;
#pragma unroll
        for (int ww = 0; ww < kAlignMaxWaves; ++ww) {
            cw[q][ww] = own ? cnt[min(ww, nw - 1) * E_tot + min(e, E_tot - 1)] : 0;
            if (ww >= nw) cw[q][ww] = 0;
            c += cw[q][ww];
        }
        const int p = (c + a.B - 1) / a.B * a.B;
        my_pad += p;
        if (a.chunks) my_chunks += (p + a.chunk_rows - 1) / a.chunk_rows;
    }
    int off, coff, npp, nchunks;
    block_exclusive_scan2(my_pad, my_chunks, scratch, &off, &coff, &npp, &nchunks);
#pragma unroll
    for (int q = 0; q < kAlignMaxPer; ++q) {
        const int e = e0 + q;
        if (q >= per || e >= E_tot) break;
        int run = off;
#pragma unroll
        for (int ww = 0; ww < kAlignMaxWaves; ++ww) {
            if (ww < nw) cnt[ww * E_tot + e] = run;
            run += cw[q][ww];
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
    if (!a.skip_tail) {
        for (int64_t s = npp + threadIdx.x; s < a.cap; s += nthr) a.sorted_ids[s] = sentinel;
        if (a.expert_ids) {
            const int64_t nblk = (a.cap + a.B - 1) / a.B;
            for (int64_t b = npp / a.B + threadIdx.x; b < nblk; b += nthr) a.expert_ids[b] = -1;
        }
    }
    __syncthreads();
    write_sched(a, nchunks);  // (the barrier above made the chunk list visible)

    // pass 3: stable scatter (rows of 64 in ascending pair order)
    auto scatter = [&](int i, int e, uint64_t peers) {
        if (is_valid(i, e)) {
            const int b0 = cnt[w * E_tot + e];
            a.sorted_ids[b0 + __popcll(peers & lt)] = i;
            if ((peers & lt) == 0) cnt[w * E_tot + e] = b0 + __popcll(peers);
        }
    };
    if (one_batch) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (beg + u * 64 < end) scatter(beg + u * 64 + lane, ev0[u], pm0[u]);
    } else {
        for (int base = beg; base < end; base += 64 * U) {
            int ev[U];
            load_rows(base, ev);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = base + u * 64 + lane;
                scatter(i, ev[u], match_any(ev[u], is_valid(i, ev[u]), nbits));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Alignment over many workgroups, for large pair counts (one workgroup runs
// the per-pair passes of align_kernel on a single CU: 36864 pairs took about
// 70 us that way).  The pairs are cut into nblk blocks of bp consecutive
// pairs (bp a multiple of 64 * kAlignBlkWaves):
//   align_count_kernel   per block, the valid pairs of each expert (wave
//                        match-any groups, one LDS atomic per group) ->
//                        blk_cnt[b][e]; extra workgroups quantise INT8
//                        token rows, as in align_kernel;
//   align_scan_kernel    one workgroup: expert totals, padded sizes and
//                        offsets (block scan), padding sentinels,
//                        expert_ids, chunks, npp / meta; blk_cnt[b][e]
//                        becomes the first slot of block b's pairs of e
//                        (the expert's offset plus the earlier blocks'
//                        counts);
//   align_scatter_kernel per block, per-wave counts again, each wave's
//                        bases from blk_cnt, and the stable scatter.
// sorted_ids, expert_ids and the chunk list come out identical to
// align_kernel's: the pairs of an expert in ascending pair order.
// ---------------------------------------------------------------------------
constexpr int kAlignBlkWaves = 8;

__global__ __launch_bounds__(kAlignBlkWaves * 64) void align_count_kernel(AlignArgs a, int bp, int nblk) {
    extern __shared__ int h[];  // [E_tot]
    const int nw = blockDim.x >> 6, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if ((int)blockIdx.x >= nblk) {  // INT8 token rows (whole waves exit together)
        const int64_t r = (int64_t)(blockIdx.x - nblk) * nw + w;
        if (r < a.q_rows)  // rows up to 4096 values in registers
            quant_row<8, 4>(a.qx + r * a.q_cols, a.q_cols, a.qq + r * a.q_cols, a.qs + r, lane);
        return;
    }
    const int E_tot = a.E + (a.n_shared > 0 ? 1 : 0);
    const int P_tot = a.P + a.n_shared;
    const int nbits = 32 - __clz(E_tot > 1 ? E_tot - 1 : 1);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int i = threadIdx.x; i < E_tot; i += blockDim.x) h[i] = 0;
    const int beg = blockIdx.x * bp, end = min(P_tot, beg + bp);
    __syncthreads();
    // rows of 64 pairs, U per wave at a time (their loads in flight together)
    constexpr int U = 4;
    for (int base = beg + w * 64 * U; base < end; base += nw * 64 * U) {
        int ev[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * 64 + lane;
            ev[u] = i < end ? (i < a.P ? a.ids[i] : a.E) : -1;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * 64 + lane, e = ev[u];
            const bool valid = i < end && (i < a.P ? (e >= 0 && e < a.E) : true);
            const uint64_t peers = match_any(e, valid, nbits);
            if (valid && (peers & lt) == 0) atomicAdd(&h[e], __popcll(peers));
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E_tot; e += blockDim.x) a.blk_cnt[(size_t)blockIdx.x * E_tot + e] = h[e];
}

// one workgroup of 1024 threads: thread e owns expert e (E_tot <= 1024)
__global__ __launch_bounds__(1024) void align_scan_kernel(AlignArgs a, int nblk) {
    __shared__ int scratch[2 * 16];
    const int nthr = blockDim.x;
    const int E_tot = a.E + (a.n_shared > 0 ? 1 : 0);
    const int P_tot = a.P + a.n_shared;
    const int sentinel = P_tot;
    const int e = threadIdx.x;
    const bool own = e < E_tot;
    int c = 0;
    if (own) {
#pragma unroll 8
        for (int b = 0; b < nblk; ++b) c += a.blk_cnt[(size_t)b * E_tot + e];
    }
    const int p = (c + a.B - 1) / a.B * a.B;
    const int nch = a.chunks ? (p + a.chunk_rows - 1) / a.chunk_rows : 0;
    int off, coff, npp, nchunks;
    block_exclusive_scan2(own ? p : 0, own ? nch : 0, scratch, &off, &coff, &npp, &nchunks);
    if (own) {
        int run = off;
#pragma unroll 8
        for (int b = 0; b < nblk; ++b) {
            const size_t idx = (size_t)b * E_tot + e;
            const int v = a.blk_cnt[idx];
            a.blk_cnt[idx] = run;
            run += v;
        }
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
    }
    if (threadIdx.x == 0) {
        a.npp[0] = npp;
        if (a.meta) {
            a.meta[0] = npp;
            a.meta[1] = nchunks;
        }
    }
    if (!a.skip_tail) {
        for (int64_t s = npp + threadIdx.x; s < a.cap; s += nthr) a.sorted_ids[s] = sentinel;
        if (a.expert_ids) {
            const int64_t nblk_out = (a.cap + a.B - 1) / a.B;
            for (int64_t b = npp / a.B + threadIdx.x; b < nblk_out; b += nthr) a.expert_ids[b] = -1;
        }
    }
    if (a.sched) {
        __syncthreads();  // the chunk list is written
        write_sched(a, nchunks);
    }
}

__global__ __launch_bounds__(kAlignBlkWaves * 64) void align_scatter_kernel(AlignArgs a, int bp) {
    extern __shared__ int cnt[];  // [nw][E_tot]
    const int nw = blockDim.x >> 6, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int E_tot = a.E + (a.n_shared > 0 ? 1 : 0);
    const int P_tot = a.P + a.n_shared;
    const int nbits = 32 - __clz(E_tot > 1 ? E_tot - 1 : 1);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int i = threadIdx.x; i < nw * E_tot; i += blockDim.x) cnt[i] = 0;
    // wave w takes the contiguous pairs [beg, end) of the block, in order
    const int seg = bp / nw;
    const int beg = blockIdx.x * bp + w * seg, end = min(P_tot, beg + seg);
    auto is_valid = [&](int i, int e) { return i < end && (i < a.P ? (e >= 0 && e < a.E) : true); };
    constexpr int U = 4;
    auto load_rows = [&](int base, int (&ev)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * 64 + lane;
            ev[u] = i < end ? (i < a.P ? a.ids[i] : a.E) : -1;
        }
    };
    __syncthreads();
    // per-wave counts
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
    // per-wave bases: the block's first slot of each expert, then the
    // earlier waves' counts
    for (int e = threadIdx.x; e < E_tot; e += blockDim.x) {
        int run = a.blk_cnt[(size_t)blockIdx.x * E_tot + e];
        for (int ww = 0; ww < nw; ++ww) {
            const int t = cnt[ww * E_tot + e];
            cnt[ww * E_tot + e] = run;
            run += t;
        }
    }
    __syncthreads();
    // stable scatter (rows of 64 in ascending pair order)
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

__global__ __launch_bounds__(256) void quant_rows_kernel(QuantArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)((blockIdx.x * (size_t)blockDim.x + threadIdx.x) >> 6);
    if (r >= a.rows) return;
    if (a.row_ids) {
        // both loads in one round trip: row_ids has a slot for every row
        // (past npp it holds stale values, which the first test discards)
        const int npp = a.meta[0];
        const int rid = a.row_ids[r];
        if (r >= npp || rid >= a.sentinel) return;
    }
    quant_row(a.x + r * (int64_t)a.cols, a.cols, a.q + r * (int64_t)a.cols, a.scale + r, lane);
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

// Waves of the alignment workgroup: 8 (measured fastest for a few hundred
// pairs; 512 threads cover up to 1024 experts at two per thread), 16 for many
// pairs when the per-wave count table still fits in 32 KiB of LDS.
int align_waves(int E_tot, int P_tot) { return (P_tot > 4096 && E_tot <= 512) ? 16 : 8; }

size_t align_lds_bytes(int E_tot, int P_tot) {
    return ((size_t)align_waves(E_tot, P_tot) * E_tot + 2 * kAlignMaxWaves) * sizeof(int);
}

hipError_t launch_align(const AlignArgs& a, hipStream_t st) {
    const int E_tot = a.E + (a.n_shared > 0 ? 1 : 0);
    const int P_tot = a.P + a.n_shared;
    if (a.blk_cnt && P_tot >= kAlignMultiMin && E_tot <= 1024) {
        const int bp = align_blk_pairs(P_tot), nblk = align_blocks(P_tot);
        const int64_t qblocks = a.qx ? (a.q_rows + kAlignBlkWaves - 1) / kAlignBlkWaves : 0;
        align_count_kernel<<<(unsigned)(nblk + qblocks), kAlignBlkWaves * 64, E_tot * sizeof(int), st>>>(
            a, bp, nblk);
        align_scan_kernel<<<1, 1024, 0, st>>>(a, nblk);
        align_scatter_kernel<<<(unsigned)nblk, kAlignBlkWaves * 64, kAlignBlkWaves * E_tot * sizeof(int), st>>>(
            a, bp);
        return hipGetLastError();
    }
    const int nw = align_waves(E_tot, P_tot);
    if ((E_tot + nw * 64 - 1) / (nw * 64) > kAlignMaxPer) return hipErrorInvalidValue;
    const int64_t qblocks = a.qx ? (a.q_rows + nw - 1) / nw : 0;
    align_kernel<false, 1><<<(unsigned)(1 + qblocks), nw * 64, align_lds_bytes(E_tot, P_tot), st>>>(
        a, RouteArgs{});
    return hipGetLastError();
}

bool route_align_fits(int T, int E, int k) { return T <= kRouteAlignMaxTokens && E <= 1024 && k <= 32; }

hipError_t launch_route_align(const AlignArgs& a, const RouteArgs& r, hipStream_t st) {
    const int E_tot = a.E + (a.n_shared > 0 ? 1 : 0);
    const int P_tot = a.P + a.n_shared;
    const int T = a.P / r.k;
    if (!route_align_fits(T, a.E, r.k)) return hipErrorInvalidValue;
    const int nw = align_waves(E_tot, P_tot);
    if ((E_tot + nw * 64 - 1) / (nw * 64) > kAlignMaxPer) return hipErrorInvalidValue;
    const int64_t qblocks = a.qx ? (a.q_rows + nw - 1) / nw : 0;
    const size_t lds = ((size_t)nw * E_tot + 2 * kAlignMaxWaves + (size_t)a.P) * sizeof(int);
    const dim3 grid((unsigned)(1 + qblocks)), block(nw * 64);
    const int vpl = (a.E + 63) / 64;
    if (vpl <= 1)
        align_kernel<true, 1><<<grid, block, lds, st>>>(a, r);
    else if (vpl <= 2)
        align_kernel<true, 2><<<grid, block, lds, st>>>(a, r);
    else if (vpl <= 4)
        align_kernel<true, 4><<<grid, block, lds, st>>>(a, r);
    else if (vpl <= 8)
        align_kernel<true, 8><<<grid, block, lds, st>>>(a, r);
    else
        align_kernel<true, 16><<<grid, block, lds, st>>>(a, r);
    return hipGetLastError();
}

hipError_t launch_quant_rows(const QuantArgs& a, hipStream_t st) {
    if (a.rows == 0) return hipSuccess;
    const int64_t waves = a.rows;
    dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    quant_rows_kernel<<<grid, block, 0, st>>>(a);
    return hipGetLastError();
}

// INT4: logical [E, K, N/2] nibble pairs (column 2j low, 2j+1 high, two's
// complement) -> the packed blocks of packed_i4_offset.  One thread writes one
// lane's 16 bytes of one (tile, 128-row K block).
__global__ __launch_bounds__(256) void prepack_int4_kernel(const uint8_t* __restrict__ w, int E, int K, int N,
                                                           int is_w13, uint8_t* __restrict__ out) {
    const int ntiles = N / 16, kblocks = K / 128;
    const int64_t total = (int64_t)E * ntiles * kblocks * 64;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const int lane = (int)(gid & 63);
    int64_t rest = gid >> 6;
    const int kb = (int)(rest % kblocks);
    rest /= kblocks;
    const int nt = (int)(rest % ntiles);
    const int e = (int)(rest / ntiles);
    const int col = is_w13 ? (nt & 1) * (N / 2) + (nt >> 1) * 16 : nt * 16;
    const int n = col + (lane & 15), g = lane >> 4;
    const uint8_t* src = w + (size_t)e * K * (N / 2);
    uint32_t dw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // dword q = (k-tile q/2, half q%2)
        uint32_t v = 0;
#pragma unroll
        for (int el = 0; el < 8; ++el) {
            const int k = kb * 128 + (q >> 1) * 64 + (q & 1) * 32 + g * 8 + el;
            const uint8_t b = src[(size_t)k * (N / 2) + n / 2];
            const uint32_t u = (((n & 1) ? (b >> 4) : b) + 8u) & 15u;  // two's complement + 8
            v |= u << ((el & 1) ? 16 + 4 * (el >> 1) : 4 * (el >> 1));
        }
        dw[q] = v;
    }
    *reinterpret_cast<u32x4*>(out + (size_t)e * K * (N / 2) + packed_i4_offset(K, nt, kb) + (size_t)lane * 16) =
        u32x4{dw[0], dw[1], dw[2], dw[3]};
}

hipError_t launch_prepack(int elem_bytes, int wtype, const void* w, int E, int K, int N,
                          int is_w13, void* out, hipStream_t st) {
    if (wtype == W_INT4) {
        if (K % 128 || N % 16) return hipErrorInvalidValue;
        const int64_t total = (int64_t)E * (N / 16) * (K / 128) * 64;
        prepack_int4_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>((const uint8_t*)w, E, K, N,
                                                                            is_w13, (uint8_t*)out);
        return hipGetLastError();
    }
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
