/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU definition of the fused
 * Mixture-of-Experts FFN layer (router top-k -> expert-blocked alignment ->
 * gate/up GEMM with SiLU(C1)*C2 -> down GEMM -> top-k-weighted combine).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * generator with the HIP library.
 *
 * Arithmetic: every floating-point accumulation is fp64.  The one place where
 * floating point decides an integer -- the dynamic INT8 quantiser -- runs in
 * fp32, the precision the GPU kernels take the same decision in.
 *
 * Sources (the pages, by title and section):
 *  - Intel PyTorch team blog on SGLang's Xeon 6 CPU backend, section "MoE":
 *    the naive MoE loops experts and gathers their activations; the fast
 *    version argsorts topk_ids into sorted_ids blocked by expert id; the
 *    gate/up GEMM is A x [B1, B2] = [C1, C2] with SiLU(C1) * C2; INT8 uses
 *    dynamic activation quantisation and the identity
 *    A x B = (A + 128) x B - 128 x B.  Section "FP8 inference": FP8 is
 *    weight-only, converted to BF16 and computed against BF16 activations.
 *  - The author's own write-up of the same backend, section 03 (3) FusedMoE:
 *    GEMM-SiLU-GEMM per expert, W13 split with SiLU on the left half and MUL
 *    on the right, moe_align_index regrouping, and the remark that only the
 *    per-expert *set* of indices matters, not their order; section 02: INT8
 *    is per-channel, FP8 is block quantised.
 *  - The OSDI'26 local-MoE paper summary, section "CPU decode backend": FP8
 *    E4M3FN weights, 128-element scale blocks whose scale is applied after the
 *    block's partial dot product (mathematically the same sum as dequantising
 *    first, which is what this file does).
 *  - The OSDI'26 summary, section "CPU decode backend", and the author's
 *    write-up, section 06 (later work): INT4 weights for decode (ORC_INT4),
 *    the format a reading (see w_at).
 *  - The news rewrite of the LMSYS large-scale expert-parallel blog, section
 *    "DeepGEMM集成": FP8 grouped GEMMs for the MoE layer (contiguous layout
 *    for prefill).  The opt-in FP8-activation variant (ORC_FP8_ACT8) follows
 *    it: both GEMM inputs quantised to E4M3FN; the block size and scale form
 *    are a reading (see oracle_fp8_block_exponent).
 * Readings where the pages are silent (tie-break, sentinel, tails, layouts,
 * shared expert, quantiser rounding) are stated at each function.
 *
 * Parity pins: every function here is pinned by CPU tests against closed
 * forms, library routines, brute force or hand-worked fixtures (routing vs a
 * stable argsort and scipy softmax/expit; alignment vs a stable argsort on
 * exhaustive tiny inputs; E4M3FN table vs its closed form and torch's float8
 * cast; k=1 routing vs a dense float64 NumPy SiLU-gated FFN; INT8 GEMMs vs the
 * U8S8 identity in int64; quantiser round-trip and tie cases; token
 * permutation; zero input; linearity in the routing weights).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_NOMEM 2

/* ORC_FP8_ACT8: FP8 weights as ORC_FP8, and both GEMM inputs (the token row,
 * the intermediate row) quantised to E4M3FN per 128-element block. */
/* ORC_INT4: weight-only 4-bit weights (see w_at) against bf16 activations. */
enum { ORC_BF16 = 0, ORC_FP8 = 1, ORC_INT8 = 2, ORC_INT4 = 3, ORC_FP8_ACT8 = 4 };
enum { ORC_SOFTMAX = 0, ORC_SIGMOID = 1 };

/* ------------------------------------------------------------------------ */
/* Number formats                                                           */
/* ------------------------------------------------------------------------ */

/* bf16 is the top half of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP E4M3FN: sign, 4-bit exponent with bias 7, 3-bit mantissa.  Exponent
 * field 0 encodes subnormals m * 2^-9; S.1111.111 is NaN; there are no
 * infinities, so S.1111.110 = 448 is the largest finite magnitude. */
double oracle_e4m3fn_to_double(uint8_t code) {
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Round a double straight to the nearest bf16 (ties to even), without an
 * intermediate binary32 rounding.  bf16 keeps 8 significant bits; its
 * subnormal quantum is 2^-133. */
uint16_t oracle_double_to_bf16(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int e;
    frexp(a, &e); /* a in [2^(e-1), 2^e) */
    int q_exp = (e - 1) - 7;
    if (q_exp < -133) q_exp = -133;
    double r = nearbyint(ldexp(a, -q_exp)); /* default mode: nearest, ties even */
    double rv = ldexp(r, q_exp);
    if (rv >= ldexp(1.0, 128)) return sign | 0x7F80;
    float f = (float)rv; /* exact: rv is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

/* The 256-entry decode table is filled once when the library is loaded, so
 * calls running on several host threads (token shards) only read it. */
static double g_e4m3[256];
__attribute__((constructor)) static void e4m3_table_fill(void) {
    for (int c = 0; c < 256; ++c) g_e4m3[c] = oracle_e4m3fn_to_double((uint8_t)c);
}

/* Dynamic symmetric INT8 quantisation of one row, in binary32 (the precision
 * the kernels decide the codes in): s = amax / 127, q = clamp(rint(x / s),
 * -127, 127) with ties to even; an all-zero row gives s = 0 and q = 0.
 * (Blog "MoE" section: dynamic quantisation of the activations; the pages do
 * not fix the rounding, so round-to-nearest-even on the correctly rounded
 * quotient is the reading.) */
void oracle_quant_int8_row(const float* x, int n, int8_t* q, float* s) {
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    float sc = amax / 127.0f;
    *s = sc;
    for (int i = 0; i < n; ++i) {
        if (sc == 0.0f) {
            q[i] = 0;
            continue;
        }
        float v = rintf(x[i] / sc);
        if (v > 127.0f) v = 127.0f;
        if (v < -127.0f) v = -127.0f;
        q[i] = (int8_t)v;
    }
}

/* OCP E4M3FN encoding of a double: the E4M3FN value nearest to v, a tie
 * going to the even code (last mantissa bit 0), found by brute force over
 * the 127 non-negative finite codes (their values increase with the code).
 * Magnitudes of 448 and more give 448 (the activation quantiser below scales
 * every block so that none exceeds it); NaN gives 0x7F; the sign is kept,
 * -0 included. */
uint8_t oracle_double_to_e4m3fn(double v) {
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (a >= 448.0) return sign | 0x7E;
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double d = fabs(g_e4m3[c] - a);
        if (d < bd || (d == bd && (c & 1) == 0)) {
            best = c;
            bd = d;
        }
    }
    return sign | (uint8_t)best;
}

/* Power-of-two scale of one FP8 activation block (the FP8 fine-grained
 * quantisation of the grouped-GEMM inputs; the pages fix neither the block
 * nor the scale form, the reading is: one scale per row and per 128
 * consecutive K elements, the weights' block length, and a power of two so
 * that scaling is exact): the largest integer e in [-126, 126] with
 * amax * 2^e <= 448.  The block is stored as E4M3FN(x * 2^e) and read back
 * as code value * 2^-e.  An all-zero block takes e = 0. */
int oracle_fp8_block_exponent(double amax) {
    if (!(amax > 0.0)) return 0;
    int e = 0;
    while (e > -126 && ldexp(amax, e) > 448.0) --e;
    while (e < 126 && ldexp(amax, e + 1) <= 448.0) ++e;
    return e;
}

/* FP8 activation quantisation of a row of n values (n a multiple of 128),
 * block by block: codes[i] = E4M3FN(x[i] * 2^e_b), exps[b] = e_b, and the
 * values the GEMM then sees, xq[i] = value(codes[i]) * 2^-e_b. */
void oracle_quant_fp8_act_row(const double* x, int n, uint8_t* codes, int* exps, double* xq) {
    for (int b = 0; b < n / 128; ++b) {
        double amax = 0.0;
        for (int i = b * 128; i < (b + 1) * 128; ++i)
            if (fabs(x[i]) > amax) amax = fabs(x[i]);
        int e = oracle_fp8_block_exponent(amax);
        if (exps) exps[b] = e;
        for (int i = b * 128; i < (b + 1) * 128; ++i) {
            uint8_t c = oracle_double_to_e4m3fn(ldexp(x[i], e));
            if (codes) codes[i] = c;
            if (xq) xq[i] = ldexp(g_e4m3[c], -e);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Router top-k                                                              */
/* ------------------------------------------------------------------------ */

/* For each token: the k experts with the largest logits, in descending order,
 * ties to the lower expert id (softmax and sigmoid are both strictly
 * increasing, so selecting on logits selects the same set as selecting on
 * scores, without depending on exp() rounding).  Weight of slot j is the score
 * of its expert -- softmax over all E logits or the logistic sigmoid -- and,
 * with renorm, divided by the sum of the k selected scores.  Logits must be
 * finite. */
int oracle_topk(const float* logits, int T, int E, int k, int score, int renorm,
                double* topk_w, int32_t* topk_ids) {
    if (T < 0 || E < 1 || k < 1 || k > E || !logits || !topk_w || !topk_ids) return ORC_ERR_ARG;
    if (score != ORC_SOFTMAX && score != ORC_SIGMOID) return ORC_ERR_ARG;
    unsigned char* chosen = (unsigned char*)malloc((size_t)E);
    double* s = (double*)malloc(sizeof(double) * (size_t)E);
    if (!chosen || !s) {
        free(chosen);
        free(s);
        return ORC_ERR_NOMEM;
    }
    for (int t = 0; t < T; ++t) {
        const float* l = logits + (size_t)t * E;
        memset(chosen, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!chosen[e] && (best < 0 || l[e] > l[best])) best = e;
            chosen[best] = 1;
            topk_ids[(size_t)t * k + j] = best;
        }
        if (score == ORC_SOFTMAX) {
            double m = l[0];
            for (int e = 1; e < E; ++e)
                if (l[e] > m) m = l[e];
            double z = 0.0;
            for (int e = 0; e < E; ++e) z += exp((double)l[e] - m);
            for (int e = 0; e < E; ++e) s[e] = exp((double)l[e] - m) / z;
        } else {
            for (int e = 0; e < E; ++e) s[e] = 1.0 / (1.0 + exp(-(double)l[e]));
        }
        double sum = 0.0;
        for (int j = 0; j < k; ++j) sum += s[topk_ids[(size_t)t * k + j]];
        for (int j = 0; j < k; ++j) {
            double w = s[topk_ids[(size_t)t * k + j]];
            topk_w[(size_t)t * k + j] = renorm ? w / sum : w;
        }
    }
    free(chosen);
    free(s);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Alignment of topk_ids into expert-blocked sorted_ids                      */
/* ------------------------------------------------------------------------ */

/* Capacity of sorted_ids: every pair plus at most B-1 padding slots per
 * expert. */
int64_t oracle_align_capacity(int64_t P, int E, int B) { return P + (int64_t)E * (B - 1); }

/* Brute force, expert by expert: the flat pair indices i = t*k + j routed to
 * expert e, in ascending i (the canonical order; the pages say any order
 * inside an expert group is acceptable), then padding with the sentinel P up
 * to a multiple of B.  Experts with no pairs get no blocks.  expert_ids[b] is
 * the expert owning block b; num_tokens_post_pad is the padded total.  Slots
 * past it hold P, blocks past it hold -1. */
int oracle_align(const int32_t* ids, int64_t P, int E, int B, int32_t* sorted_ids,
                 int32_t* expert_ids, int32_t* num_tokens_post_pad) {
    if (P < 0 || E < 1 || B < 1 || !sorted_ids || !expert_ids || !num_tokens_post_pad)
        return ORC_ERR_ARG;
    if (P > 0 && !ids) return ORC_ERR_ARG;
    for (int64_t i = 0; i < P; ++i)
        if (ids[i] < 0 || ids[i] >= E) return ORC_ERR_ARG;
    int64_t cap = oracle_align_capacity(P, E, B);
    int64_t nblk = (cap + B - 1) / B;
    int64_t pos = 0;
    for (int e = 0; e < E; ++e) {
        int64_t start = pos, c = 0;
        for (int64_t i = 0; i < P; ++i)
            if (ids[i] == e) {
                sorted_ids[pos++] = (int32_t)i;
                ++c;
            }
        int64_t padded = (c + B - 1) / B * B;
        for (; c < padded; ++c) sorted_ids[pos++] = (int32_t)P;
        for (int64_t b = start / B; b < pos / B; ++b) expert_ids[b] = e;
    }
    *num_tokens_post_pad = (int32_t)pos;
    for (int64_t b = pos / B; b < nblk; ++b) expert_ids[b] = -1;
    for (; pos < cap; ++pos) sorted_ids[pos] = (int32_t)P;
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* One expert's FFN on one token                                             */
/* ------------------------------------------------------------------------ */

/* Signed value of the 4-bit code of element (kk, n) of an INT4 matrix
 * stored as [K, N/2] bytes: column n sits in byte n/2 of its row, the low
 * nibble for even n, the high nibble for odd n, in two's complement
 * (0..7 -> 0..7, 8..15 -> -8..-1). */
int oracle_int4_code(const uint8_t* w, int N, int64_t kk, int64_t n) {
    uint8_t b = w[kk * (N / 2) + n / 2];
    int v = (n & 1) ? (b >> 4) : (b & 15);
    return v >= 8 ? v - 16 : v;
}

/* Dequantised weight element W[kk][n] of a [K, N] row-major matrix.
 * BF16: the bf16 value.  FP8: E4M3FN value times the fp32 scale of the
 * 128x128 block (kk/128, n/128) -- block quantisation, multiplicative scale.
 * INT4 (weight-only 4-bit; the pages name INT4 weights for decode but fix no
 * layout -- reading: symmetric signed codes, one fp32 scale per output
 * column and 128-element K group, the FP8 block length): code times
 * scale[kk/128][n] of the [K/128, N] scale grid. */
static double w_at(int wdtype, const void* w, const float* scale, int N, int64_t kk, int64_t n) {
    if (wdtype == ORC_BF16) return oracle_bf16_to_double(((const uint16_t*)w)[kk * N + n]);
    if (wdtype == ORC_INT4)
        return (double)oracle_int4_code((const uint8_t*)w, N, kk, n) * (double)scale[(kk / 128) * N + n];
    double q = g_e4m3[((const uint8_t*)w)[kk * N + n]];
    return q * (double)scale[(kk / 128) * (N / 128) + n / 128];
}

static double silu(double v) { return v / (1.0 + exp(-v)); }

/* BF16 / FP8 expert: h = x W13 (length 2I), a = SiLU(h[0:I]) * h[I:2I],
 * y = a W2 (length H).  h and y may be NULL-free scratch supplied by caller. */
void oracle_float_ffn(int wdtype, const double* xt, int H, int I, const void* w13,
                      const float* w13_scale, const void* w2, const float* w2_scale, double* h,
                      double* y) {
    int N1 = 2 * I;
    for (int n = 0; n < N1; ++n) h[n] = 0.0;
    for (int64_t kk = 0; kk < H; ++kk) {
        double xv = xt[kk];
        for (int64_t n = 0; n < N1; ++n) h[n] += xv * w_at(wdtype, w13, w13_scale, N1, kk, n);
    }
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    for (int i = 0; i < I; ++i) a[i] = silu(h[i]) * h[I + i];
    for (int n = 0; n < H; ++n) y[n] = 0.0;
    for (int64_t i = 0; i < I; ++i) {
        double av = a[i];
        for (int64_t n = 0; n < H; ++n) y[n] += av * w_at(wdtype, w2, w2_scale, H, i, n);
    }
    free(a);
}

/* FP8 expert with FP8 activations (W8A8-FP8): the token row is quantised to
 * E4M3FN per 128-element block, h = xq W13 (fp64), a = SiLU(h[0:I]) * h[I:2I],
 * a is quantised the same way, y = aq W2 -- the FP8 path above with both
 * GEMM inputs passed through oracle_quant_fp8_act_row. */
void oracle_float_ffn_act8(const double* xt, int H, int I, const uint8_t* w13,
                           const float* w13_scale, const uint8_t* w2, const float* w2_scale,
                           double* h, double* y) {
    int N1 = 2 * I;
    double* xq = (double*)malloc(sizeof(double) * (size_t)H);
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    double* aq = (double*)malloc(sizeof(double) * (size_t)I);
    oracle_quant_fp8_act_row(xt, H, NULL, NULL, xq);
    for (int n = 0; n < N1; ++n) h[n] = 0.0;
    for (int64_t kk = 0; kk < H; ++kk) {
        double xv = xq[kk];
        for (int64_t n = 0; n < N1; ++n) h[n] += xv * w_at(ORC_FP8, w13, w13_scale, N1, kk, n);
    }
    for (int i = 0; i < I; ++i) a[i] = silu(h[i]) * h[I + i];
    oracle_quant_fp8_act_row(a, I, NULL, NULL, aq);
    for (int n = 0; n < H; ++n) y[n] = 0.0;
    for (int64_t i = 0; i < I; ++i) {
        double av = aq[i];
        for (int64_t n = 0; n < H; ++n) y[n] += av * w_at(ORC_FP8, w2, w2_scale, H, i, n);
    }
    free(xq);
    free(a);
    free(aq);
}

/* INT8 expert (W8A8 with dynamic activations).  xq/sx: the token's quantised
 * row.  h = (sum xq * w13, exact integer) * sx * s13[n];  a = SiLU(h_gate) *
 * h_up;  (qa, sa) = quant(a) per (token, slot) row, in binary32;
 * y = (sum qa * w2, exact integer) * sa * s2[n].  The optional trace outputs
 * expose every intermediate for the pins. */
void oracle_int8_ffn(const int8_t* xq, float sx, int H, int I, const int8_t* w13,
                     const float* w13_scale, const int8_t* w2, const float* w2_scale, double* y,
                     int64_t* h_int_out, double* a_out, int8_t* qa_out, float* sa_out,
                     int64_t* y_int_out) {
    int N1 = 2 * I;
    int64_t* hi = (int64_t*)calloc((size_t)N1, sizeof(int64_t));
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    float* af = (float*)malloc(sizeof(float) * (size_t)I);
    int8_t* qa = (int8_t*)malloc((size_t)I);
    int64_t* yi = (int64_t*)calloc((size_t)H, sizeof(int64_t));
    for (int64_t kk = 0; kk < H; ++kk) {
        int64_t xv = xq[kk];
        for (int64_t n = 0; n < N1; ++n) hi[n] += xv * (int64_t)w13[kk * N1 + n];
    }
    for (int i = 0; i < I; ++i) {
        double g = (double)hi[i] * (double)sx * (double)w13_scale[i];
        double u = (double)hi[I + i] * (double)sx * (double)w13_scale[I + i];
        a[i] = silu(g) * u;
        af[i] = (float)a[i];
    }
    float sa;
    oracle_quant_int8_row(af, I, qa, &sa);
    for (int64_t i = 0; i < I; ++i) {
        int64_t av = qa[i];
        for (int64_t n = 0; n < H; ++n) yi[n] += av * (int64_t)w2[i * H + n];
    }
    for (int n = 0; n < H; ++n) y[n] = (double)yi[n] * (double)sa * (double)w2_scale[n];
    if (h_int_out) memcpy(h_int_out, hi, sizeof(int64_t) * (size_t)N1);
    if (a_out) memcpy(a_out, a, sizeof(double) * (size_t)I);
    if (qa_out) memcpy(qa_out, qa, (size_t)I);
    if (sa_out) *sa_out = sa;
    if (y_int_out) memcpy(y_int_out, yi, sizeof(int64_t) * (size_t)H);
    free(hi);
    free(a);
    free(af);
    free(qa);
    free(yi);
}

/* ------------------------------------------------------------------------ */
/* The layer                                                                 */
/* ------------------------------------------------------------------------ */

/* out[t] = bf16( sum_j topk_w[t,j] * FFN_{topk_ids[t,j]}(x[t])  +  FFN_shared(x[t]) )
 *
 * A plain loop over tokens and their k slots, no sorting -- the naive per-token
 * definition that the expert-blocked method regroups.  Slots are summed in
 * ascending j, the shared expert (weight 1, same format and shape as a routed
 * expert with intermediate size shared_I; pass NULL to omit it) is added last,
 * and the fp64 sum is rounded once to bf16.
 *
 * tokens: optional list of n_tokens token indices to evaluate (NULL = all T);
 * outputs are [n_tokens, H] in that order.  out_acc (fp64, pre-rounding) may
 * be NULL.
 * Weights are in logical layout: w13 [E, H, 2I], w2 [E, I, H]; FP8 scales
 * [E, H/128, 2I/128] and [E, I/128, H/128]; INT8 scales [E, 2I] and [E, H]. */
int oracle_moe(int wdtype, const uint16_t* x, int T, int H, int I, int E, int k,
               const void* w13, const float* w13_scale, const void* w2, const float* w2_scale,
               const float* topk_w, const int32_t* topk_ids, const void* sh13,
               const float* sh13_scale, const void* sh2, const float* sh2_scale, int shared_I,
               const int32_t* tokens, int n_tokens, double* out_acc, uint16_t* out_bf16) {
    if (wdtype < ORC_BF16 || wdtype > ORC_FP8_ACT8) return ORC_ERR_ARG;
    if (T < 0 || H < 1 || I < 1 || E < 1 || k < 1 || k > E) return ORC_ERR_ARG;
    if (!x || !w13 || !w2 || !topk_w || !topk_ids || !out_bf16) return ORC_ERR_ARG;
    if (wdtype != ORC_BF16 && (!w13_scale || !w2_scale)) return ORC_ERR_ARG;
    const int fp8w = wdtype == ORC_FP8 || wdtype == ORC_FP8_ACT8;
    if ((fp8w || wdtype == ORC_INT4) && (H % 128 || I % 128)) return ORC_ERR_ARG;
    if (sh13 && (!sh2 || shared_I < 1)) return ORC_ERR_ARG;
    if (sh13 && (fp8w || wdtype == ORC_INT4) && shared_I % 128) return ORC_ERR_ARG;
    if (sh13 && wdtype != ORC_BF16 && (!sh13_scale || !sh2_scale)) return ORC_ERR_ARG;
    int nt = tokens ? n_tokens : T;
    int Imax = (sh13 && shared_I > I) ? shared_I : I;
    double* xt = (double*)malloc(sizeof(double) * (size_t)H);
    float* xf = (float*)malloc(sizeof(float) * (size_t)H);
    int8_t* xq = (int8_t*)malloc((size_t)H);
    double* h = (double*)malloc(sizeof(double) * 2 * (size_t)Imax);
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    double* acc = (double*)malloc(sizeof(double) * (size_t)H);
    if (!xt || !xf || !xq || !h || !y || !acc) return ORC_ERR_NOMEM;
    /* bytes per expert matrix (INT4: two codes per byte) and scales per expert */
    size_t n13 = (size_t)H * 2 * I, n2 = (size_t)I * H;
    if (wdtype == ORC_BF16) {
        n13 *= 2;
        n2 *= 2;
    } else if (wdtype == ORC_INT4) {
        n13 /= 2;
        n2 /= 2;
    }
    size_t s13 = fp8w ? (size_t)(H / 128) * (2 * I / 128) : (size_t)2 * I;
    size_t s2 = fp8w ? (size_t)(I / 128) * (H / 128) : (size_t)H;
    if (wdtype == ORC_INT4) {
        s13 = (size_t)(H / 128) * 2 * I;
        s2 = (size_t)(I / 128) * H;
    }
    int rc = ORC_OK;
    for (int r = 0; r < nt; ++r) {
        int t = tokens ? tokens[r] : r;
        if (t < 0 || t >= T) {
            rc = ORC_ERR_ARG;
            break;
        }
        for (int n = 0; n < H; ++n) {
            xt[n] = oracle_bf16_to_double(x[(size_t)t * H + n]);
            xf[n] = (float)xt[n];
            acc[n] = 0.0;
        }
        float sx = 0.0f;
        if (wdtype == ORC_INT8) oracle_quant_int8_row(xf, H, xq, &sx);
        for (int j = 0; j < k; ++j) {
            int e = topk_ids[(size_t)t * k + j];
            if (e < 0 || e >= E) {
                rc = ORC_ERR_ARG;
                break;
            }
            const char* a13 = (const char*)w13 + (size_t)e * n13;
            const char* a2 = (const char*)w2 + (size_t)e * n2;
            const float* c13 = w13_scale ? w13_scale + (size_t)e * s13 : NULL;
            const float* c2 = w2_scale ? w2_scale + (size_t)e * s2 : NULL;
            if (wdtype == ORC_INT8)
                oracle_int8_ffn(xq, sx, H, I, (const int8_t*)a13, c13, (const int8_t*)a2, c2, y,
                                NULL, NULL, NULL, NULL, NULL);
            else if (wdtype == ORC_FP8_ACT8)
                oracle_float_ffn_act8(xt, H, I, (const uint8_t*)a13, c13, (const uint8_t*)a2, c2, h, y);
            else
                oracle_float_ffn(wdtype, xt, H, I, a13, c13, a2, c2, h, y);
            double w = (double)topk_w[(size_t)t * k + j];
            for (int n = 0; n < H; ++n) acc[n] += w * y[n];
        }
        if (rc != ORC_OK) break;
        if (sh13) {
            if (wdtype == ORC_INT8)
                oracle_int8_ffn(xq, sx, H, shared_I, (const int8_t*)sh13, sh13_scale,
                                (const int8_t*)sh2, sh2_scale, y, NULL, NULL, NULL, NULL, NULL);
            else if (wdtype == ORC_FP8_ACT8)
                oracle_float_ffn_act8(xt, H, shared_I, (const uint8_t*)sh13, sh13_scale,
                                      (const uint8_t*)sh2, sh2_scale, h, y);
            else
                oracle_float_ffn(wdtype, xt, H, shared_I, sh13, sh13_scale, sh2, sh2_scale, h, y);
            for (int n = 0; n < H; ++n) acc[n] += y[n];
        }
        for (int n = 0; n < H; ++n) {
            if (out_acc) out_acc[(size_t)r * H + n] = acc[n];
            out_bf16[(size_t)r * H + n] = oracle_double_to_bf16(acc[n]);
        }
    }
    free(xt);
    free(xf);
    free(xq);
    free(h);
    free(y);
    free(acc);
    return rc;
}
