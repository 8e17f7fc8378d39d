/*
 * q4_oracle.c -- plain, slow CPU oracle for the 4-bit block-quantised matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, table or helper with the HIP library; the two are built by
 * different compilers from different files.
 *
 * What it computes (the plain definition; nothing is blocked, fused or
 * reordered):
 *
 *   w[n,k] = (c[n,k] - 8) * s[n, k/32]
 *   y[m,n] = sum_{k=0}^{K-1} x[m,k] * w[n,k]        (double, k ascending)
 *   t[m,n] = sum_k |x[m,k] * w[n,k]|                 (the tolerance scale)
 *
 *   MoE:  y[t,n] = sum_j g[t,j] * (sum_k x[t,k] * w_{id[t,j]}[n,k])
 *         t[t,n] = sum_j |g[t,j]| * (sum_k |x[t,k] * w_{id[t,j]}[n,k]|)
 *
 *   Routed expert FFN (gate/up, SwiGLU, down, weighted sum), per selected
 *   expert e = id[t,j]:
 *         gate_f = sum_k x[t,k] * w13_e[2f,k],  up_f = sum_k x[t,k] * w13_e[2f+1,k]
 *         a_f    = silu(gate_f) * up_f,  silu(z) = z / (1 + exp(-z))
 *         y[t,h] = sum_j g[t,j] * sum_f a_f * w2_e[h,f]
 *
 * Sources.  The specialised-runtime spec ("spec: specialized model runtimes")
 * names quant/dequant and GEMM as T0 kernel-tier ops (section
 * "Architecture"), a quantised GEMM as the first measured kernel (section
 * "Feasibility gate"), groupwise-int weights as the first weight profile
 * (section "Target package and artifact"), and asks for a clear, slow,
 * independent reference for every tuned kernel (section "Kernel and
 * portability contract", rule 1).  The layer-package spec ("Layer Package
 * Repository Spec", the MoE fixture paragraph under "Policy Resolution")
 * describes routed top-k expert matmuls followed by a weighted sum over the
 * selected experts, and a routed FFN layer as gate/up expert matmuls, a
 * fused SwiGLU split (silu(gate) * up), the down expert matmul and that
 * weighted sum.  The pages fix no bit layout; the readings used here are:
 *   - a code is 4 bits, value = code - 8 (symmetric, no zero point);
 *   - one IEEE binary16 scale per 32 consecutive k of a row;
 *   - codes of row n are packed two per byte, k = 2j in the LOW nibble of
 *     byte j and k = 2j+1 in the HIGH nibble; rows are K/2 bytes apart;
 *   - scales of row n are K/32 consecutive fp16 values;
 *   - activations are bf16, row-major [M][K];
 *   - oracle option bf16_weights rounds each dequantised weight to bf16,
 *     nearest-even, before the product (a pinned variant of the oracle; the
 *     product paths use the weights exactly);
 *   - FFN: gate and up weights of an expert are one [2F][H] matrix whose row
 *     2f is the gate row and row 2f+1 the up row of hidden unit f; the
 *     SwiGLU output a_f feeds the down product unrounded.
 *
 * RMSNorm prologue.  The specialised-runtime spec's first measured kernel is
 * "one quantized GEMM plus fused RMSNorm" (section "Feasibility gate"; also
 * Phase 1 of "Development sequence").  The pages do not define RMSNorm; the
 * reading taken is the usual one, per activation row m:
 *         r_m      = 1 / sqrt( (1/K) * sum_k x[m,k]^2 + eps )
 *         x'[m,k]  = x[m,k] * r_m * gamma[k]          (gamma: bf16 [K])
 *         y[m,n]   = sum_k x'[m,k] * w[n,k],  t[m,n] = sum_k |x'[m,k] * w[n,k]|
 *         u[m,n]   = sum_k hulp(x'[m,k]) * |w[n,k]|
 * where hulp(v) is half a bf16 unit in the last place of v: the normalised
 * activations are the matmul's activation operand, whose type is bf16, and u
 * is what their rounding to bf16 can move y by.  Everything in double.
 *
 * Quantiser (bf16 weights -> this format).  The spec's build flow converts
 * model weights into the runtime's profile before qualifying it (section
 * "Target package and artifact": Convert, then Qualify) but fixes no method.
 * The reading taken, per 32-element block of a row (symmetric absmax, the
 * block's largest-magnitude element landing exactly on code 0):
 *         m    = the element of largest |w| (the first one in k on ties)
 *         s    = fp16(m / -8), nearest-even, |s| clamped to 65504
 *         c_k  = clamp(rint(w_k / s) + 8, 0, 15)      (s != 0; else c_k = 8)
 * The quotient and its rounding decide an integer, so they are taken in the
 * kernel's precision: an IEEE fp32 division and round-half-even in fp32.
 *
 * Super-block (two-level) scales.  The layer-package spec names K-quant
 * profiles (Q4_K-class, q2_K / q3_K; sections "Repository Identity" and
 * "Policy Resolution") without defining them.  The reading taken keeps this
 * format's codes and builds the structure the K-quants share: 256-element
 * super-blocks of eight 32-element blocks, one fp16 scale d per super-block
 * and an unsigned 8-bit multiplier sc per block:
 *         w[n,k] = (c[n,k] - 8) * d[n, k/256] * sc[n, k/32]
 * (d * sc has at most 19 significant bits, exact in float and double).
 *
 * 4-bit float blocks.  The specialised-runtime spec names a 4-bit float block
 * format as the performance path after groupwise-int weights (section "Target
 * package and artifact") but fixes no bits.  The reading taken is the public
 * microscaling definition with 32-element blocks:
 *   - an element is e2m1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0
 *     mantissa; exponent 0 is subnormal (m * 2^-1), otherwise
 *     (1 + m/2) * 2^(e-1); no infinity or NaN;
 *   - one E8M0 byte per 32 consecutive k scales the block by 2^(E-127);
 *     E = 255 is NaN;
 *   - elements are packed like the int4 codes (k = 2j in the low nibble),
 *     scales are K/32 bytes per row:
 *         w[n,k] = e2m1(c[n,k]) * 2^(E[n, k/32] - 127)
 *
 * Floating point: every fp16 / bf16 value is decoded from its IEEE fields
 * into a double (exact); (c-8)*s is exact in double and in float; products
 * x*w are exact in double; only the k-ordered sum rounds.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define Q4O_BLOCK 32

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double fp16_value(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* 0.f * 2^-14 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* 1.f * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
static double bf16_value(uint16_t b) {
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xFF;
    int f = b & 0x7F;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);                /* 0.f * 2^-126 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);     /* 1.f * 2^(e-127) */
    return sign ? -v : v;
}

/* Round a double to the nearest bf16 value, ties to even, and return the
 * rounded value as a double.  Written from the definition: keep 8
 * significant bits in the normal range, a fixed 2^-133 quantum in the
 * subnormal range, and overflow to infinity past the largest finite value. */
static double bf16_round(double v) {
    if (isnan(v) || isinf(v) || v == 0.0)
        return v;
    double a = fabs(v);
    int e;
    frexp(a, &e);                       /* a = m * 2^e, m in [0.5, 1) */
    double r;
    if (e - 1 < -126)                   /* below the smallest normal */
        r = ldexp(rint(ldexp(a, 133)), -133);
    else
        r = ldexp(rint(ldexp(a, 8 - e)), e - 8);
    if (r >= ldexp(1.0, 128))           /* 2^128 is past the largest finite */
        r = INFINITY;
    return v < 0 ? -r : r;
}

static uint16_t bf16_bits_of(double v) {
    /* v is a bf16 value (or inf/nan): it converts to float exactly. */
    float f = (float)v;
    uint32_t u;
    if (isnan(v))
        return (uint16_t)(signbit(v) ? 0xFFC0u : 0x7FC0u);
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static int code_at(const uint8_t *row, int64_t k) {
    uint8_t byte = row[k / 2];
    return (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
}

static double weight_at(const uint8_t *wq_row, const uint16_t *ws_row, int64_t k,
                        int bf16_weights) {
    double w = (double)(code_at(wq_row, k) - 8) * fp16_value(ws_row[k / Q4O_BLOCK]);
    return bf16_weights ? bf16_round(w) : w;
}

/* e2m1 element from its fields. */
static double e2m1_value(int c) {
    int sign = (c >> 3) & 1;
    int e = (c >> 1) & 3;
    int m = c & 1;
    double v = (e == 0) ? ldexp((double)m, -1) : ldexp(2.0 + m, e - 2);   /* (1 + m/2) 2^(e-1) */
    return sign ? -v : v;
}

/* E8M0 scale byte: 2^(E-127), E = 255 is NaN. */
static double e8m0_value(uint8_t e) {
    return e == 255 ? NAN : ldexp(1.0, (int)e - 127);
}

static double mx_weight_at(const uint8_t *wq_row, const uint8_t *we_row, int64_t k) {
    return e2m1_value(code_at(wq_row, k)) * e8m0_value(we_row[k / Q4O_BLOCK]);
}

/* ---- exported ---------------------------------------------------------- */

double oracle_e2m1_value(int c) { return e2m1_value(c & 15); }
double oracle_e8m0_value(uint8_t e) { return e8m0_value(e); }

/* 4-bit float blocks dequantised to double [N][K] (exact). */
void oracle_mx_dequant(const uint8_t *wq, const uint8_t *we, int64_t N, int64_t K,
                       double *out) {
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            out[n * K + k] = mx_weight_at(wq + n * (K / 2), we + n * (K / Q4O_BLOCK), k);
}

/* y = x . w^T with 4-bit float block weights; y, t: double [M][N]. */
void oracle_mx_matmul(const uint16_t *x, const uint8_t *wq, const uint8_t *we,
                      int64_t M, int64_t N, int64_t K, double *y, double *t) {
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m) {
            const uint16_t *xr = x + m * K;
            const uint8_t *wr = wq + n * (K / 2), *er = we + n * (K / Q4O_BLOCK);
            double sum = 0.0, abs_sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double prod = bf16_value(xr[k]) * mx_weight_at(wr, er, k);
                sum += prod;
                abs_sum += fabs(prod);
            }
            y[m * N + n] = sum;
            t[m * N + n] = abs_sum;
        }
}

int oracle_block(void) { return Q4O_BLOCK; }

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

double oracle_fp16_value(uint16_t h) { return fp16_value(h); }
double oracle_bf16_value(uint16_t b) { return bf16_value(b); }
uint16_t oracle_bf16_round_bits(double v) { return bf16_bits_of(bf16_round(v)); }

/* Dequantise to float32 [N][K]; (c-8)*s is exact in float. */
void oracle_dequant_f32(const uint8_t *wq, const uint16_t *ws, int64_t N, int64_t K,
                        float *out) {
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            out[n * K + k] = (float)weight_at(wq + n * (K / 2), ws + n * (K / Q4O_BLOCK), k, 0);
}

/* Dequantise and round to bf16 (nearest-even); bf16 bit patterns [N][K]. */
void oracle_dequant_bf16(const uint8_t *wq, const uint16_t *ws, int64_t N, int64_t K,
                         uint16_t *out) {
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            out[n * K + k] = bf16_bits_of(
                weight_at(wq + n * (K / 2), ws + n * (K / Q4O_BLOCK), k, 1));
}

/* One output: sequential double dot product over k and its |.| companion. */
static void dot_one(const uint16_t *x_row, const uint8_t *wq_row, const uint16_t *ws_row,
                    int64_t K, int bf16_weights, double *y, double *t) {
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = bf16_value(x_row[k]) * weight_at(wq_row, ws_row, k, bf16_weights);
        acc += p;
        mag += fabs(p);
    }
    *y = acc;
    *t = mag;
}

/* y, t: double [M][N]. */
void oracle_matmul(const uint16_t *x, const uint8_t *wq, const uint16_t *ws,
                   int64_t M, int64_t N, int64_t K, int bf16_weights,
                   double *y, double *t) {
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m)
            dot_one(x + m * K, wq + n * (K / 2), ws + n * (K / Q4O_BLOCK), K, bf16_weights,
                    &y[m * N + n], &t[m * N + n]);
}

/* Only the listed outputs (ms[i], ns[i]); y, t: double [count]. */
void oracle_matmul_sampled(const uint16_t *x, const uint8_t *wq, const uint16_t *ws,
                           int64_t M, int64_t N, int64_t K, int bf16_weights,
                           const int64_t *ms, const int64_t *ns, int64_t count,
                           double *y, double *t) {
    (void)M; (void)N;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i)
        dot_one(x + ms[i] * K, wq + ns[i] * (K / 2), ws + ns[i] * (K / Q4O_BLOCK), K,
                bf16_weights, &y[i], &t[i]);
}

/* Expert-routed rows.  x: bf16 [T][K]; wq: [E][N][K/2]; ws: [E][N][K/32];
 * ids: int32 [T][topk]; gates: float [T][topk]; y, t: double [T][N].
 * An id outside [0, E) selects no expert and contributes nothing. */
void oracle_moe(const uint16_t *x, const uint8_t *wq, const uint16_t *ws,
                const int32_t *ids, const float *gates,
                int64_t T, int64_t topk, int64_t E, int64_t N, int64_t K,
                double *y, double *t) {
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t tok = 0; tok < T; ++tok) {
            double acc = 0.0, mag = 0.0;
            for (int64_t j = 0; j < topk; ++j) {
                int64_t e = ids[tok * topk + j];
                if (e < 0 || e >= E) continue;
                double d, dm;
                dot_one(x + tok * K, wq + (e * N + n) * (K / 2),
                        ws + (e * N + n) * (K / Q4O_BLOCK), K, 0, &d, &dm);
                double g = (double)gates[tok * topk + j];
                acc += g * d;
                mag += fabs(g) * dm;
            }
            y[tok * N + n] = acc;
            t[tok * N + n] = mag;
        }
    }
}

/* Routed expert FFN.  x: bf16 [T][H]; w13q: [E][2F][H/2]; w13s: [E][2F][H/32]
 * (row 2f = gate row, row 2f+1 = up row of unit f); w2q: [E][H][F/2];
 * w2s: [E][H][F/32]; ids: int32 [T][topk]; gates: float [T][topk];
 * y, b: double [T][H].  An id outside [0, E) adds nothing.
 *
 * b is the tolerance scale: each first-stage sum may be off by a fraction of
 * its own |.|-sum (tg, tu), carried to first order through the SwiGLU
 * (|silu'| <= 1.1), plus the down product's own |.|-sum:
 *   b[t,h] = sum_j |g[t,j]| * sum_f |w2_e[h,f]| * (|a_f| + 1.1*|up_f|*tg_f + |silu(gate_f)|*tu_f)
 */
static double silu(double z) { return z / (1.0 + exp(-z)); }

void oracle_moe_ffn(const uint16_t *x, const uint8_t *w13q, const uint16_t *w13s,
                    const uint8_t *w2q, const uint16_t *w2s, const int32_t *ids,
                    const float *gates, int64_t T, int64_t topk, int64_t E, int64_t H,
                    int64_t F, double *y, double *b) {
    double *a = (double *)malloc(sizeof(double) * (size_t)(F > 0 ? F : 1));
    double *da = (double *)malloc(sizeof(double) * (size_t)(F > 0 ? F : 1));
    for (int64_t i = 0; i < T * H; ++i) { y[i] = 0.0; b[i] = 0.0; }
    for (int64_t tok = 0; tok < T; ++tok) {
        for (int64_t j = 0; j < topk; ++j) {
            int64_t e = ids[tok * topk + j];
            if (e < 0 || e >= E) continue;
            double g = (double)gates[tok * topk + j];
            #pragma omp parallel for schedule(static)
            for (int64_t f = 0; f < F; ++f) {
                int64_t rg = e * 2 * F + 2 * f, ru = rg + 1;
                double gv, tg, uv, tu;
                dot_one(x + tok * H, w13q + rg * (H / 2), w13s + rg * (H / Q4O_BLOCK), H, 0, &gv, &tg);
                dot_one(x + tok * H, w13q + ru * (H / 2), w13s + ru * (H / Q4O_BLOCK), H, 0, &uv, &tu);
                double sg = silu(gv);
                a[f] = sg * uv;
                da[f] = fabs(a[f]) + 1.1 * fabs(uv) * tg + fabs(sg) * tu;
            }
            #pragma omp parallel for schedule(static)
            for (int64_t h = 0; h < H; ++h) {
                const uint8_t *wr = w2q + (e * H + h) * (F / 2);
                const uint16_t *sr = w2s + (e * H + h) * (F / Q4O_BLOCK);
                double o = 0.0, m = 0.0;
                for (int64_t f = 0; f < F; ++f) {
                    double w = weight_at(wr, sr, f, 0);
                    o += a[f] * w;
                    m += fabs(w) * da[f];
                }
                y[tok * H + h] += g * o;
                b[tok * H + h] += fabs(g) * m;
            }
        }
    }
    free(a);
    free(da);
}

/* ---- RMSNorm prologue + matmul ------------------------------------------ */

/* Half a bf16 unit in the last place of |v|: 8 significant bits in the
 * normal range (|v| >= 2^-126), a fixed quantum of 2^-133 below it. */
static double bf16_half_ulp(double v) {
    double a = fabs(v);
    if (a == 0.0 || isnan(a) || isinf(a))
        return a == 0.0 ? ldexp(1.0, -134) : a;
    int e;
    frexp(a, &e);                       /* a = m * 2^e, m in [0.5, 1) */
    if (e - 1 < -126)
        return ldexp(1.0, -134);
    return ldexp(1.0, (e - 1) - 8);     /* ulp 2^(e-1-7), half of it */
}

/* x' = RMSNorm(x) * gamma as double [M][K]. */
void oracle_rmsnorm(const uint16_t *x, const uint16_t *gamma, double eps, int64_t M,
                    int64_t K, double *xn) {
    for (int64_t m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = bf16_value(x[m * K + k]);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / (double)K + eps);
        for (int64_t k = 0; k < K; ++k)
            xn[m * K + k] = bf16_value(x[m * K + k]) * r * bf16_value(gamma[k]);
    }
}

double oracle_bf16_half_ulp(double v) { return bf16_half_ulp(v); }

/* One output of the normalised product: xn_row is a row of oracle_rmsnorm. */
static void rms_dot_one(const double *xn_row, const uint8_t *wq_row, const uint16_t *ws_row,
                        int64_t K, double *y, double *t, double *u) {
    double acc = 0.0, mag = 0.0, rnd = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double w = weight_at(wq_row, ws_row, k, 0);
        double p = xn_row[k] * w;
        acc += p;
        mag += fabs(p);
        rnd += bf16_half_ulp(xn_row[k]) * fabs(w);
    }
    *y = acc;
    *t = mag;
    *u = rnd;
}

/* y, t, u: double [M][N] (see the header). */
void oracle_rmsnorm_matmul(const uint16_t *x, const uint16_t *gamma, double eps,
                           const uint8_t *wq, const uint16_t *ws, int64_t M, int64_t N,
                           int64_t K, double *y, double *t, double *u) {
    double *xn = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    oracle_rmsnorm(x, gamma, eps, M, K, xn);
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m)
            rms_dot_one(xn + m * K, wq + n * (K / 2), ws + n * (K / Q4O_BLOCK), K,
                        &y[m * N + n], &t[m * N + n], &u[m * N + n]);
    free(xn);
}

/* Only the listed outputs (ms[i], ns[i]); y, t, u: double [count]. */
void oracle_rmsnorm_matmul_sampled(const uint16_t *x, const uint16_t *gamma, double eps,
                                   const uint8_t *wq, const uint16_t *ws, int64_t M,
                                   int64_t N, int64_t K, const int64_t *ms, const int64_t *ns,
                                   int64_t count, double *y, double *t, double *u) {
    (void)N;
    double *xn = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    oracle_rmsnorm(x, gamma, eps, M, K, xn);
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i)
        rms_dot_one(xn + ms[i] * K, wq + ns[i] * (K / 2), ws + ns[i] * (K / Q4O_BLOCK), K,
                    &y[i], &t[i], &u[i]);
    free(xn);
}

/* ---- quantiser ------------------------------------------------------------- */

/* Round a double to the nearest fp16 value, ties to even, written from the
 * format: 11 significant bits in the normal range (>= 2^-14), a fixed
 * quantum of 2^-24 below it; values past 65504 are clamped to +-65504. */
static double fp16_round_clamped(double v) {
    if (v == 0.0 || isnan(v))
        return v;
    double a = fabs(v);
    int e;
    frexp(a, &e);                       /* a = m * 2^e, m in [0.5, 1) */
    double r;
    if (e - 1 < -14)
        r = ldexp(rint(ldexp(a, 24)), -24);
    else
        r = ldexp(rint(ldexp(a, 11 - e)), e - 11);
    if (r > 65504.0)
        r = 65504.0;
    return v < 0 ? -r : r;
}

static uint16_t fp16_bits_of(double v) {
    /* v is an fp16 value (finite): encode its fields */
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);
    if (e - 1 < -14)                    /* subnormal: f * 2^-24 */
        return (uint16_t)(sign | (uint16_t)ldexp(a, 24));
    int f = (int)(ldexp(a, 11 - e)) - 1024;   /* 1.f * 2^(e-1) */
    return (uint16_t)(sign | ((e - 1 + 15) << 10) | f);
}

/* bf16 weights [N][K] -> codes [N][K/2] and fp16 scales [N][K/32]. */
void oracle_quantize(const uint16_t *w, int64_t N, int64_t K, uint8_t *wq, uint16_t *ws) {
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < K / Q4O_BLOCK; ++b) {
            const uint16_t *blk = w + n * K + b * Q4O_BLOCK;
            double m = 0.0;
            for (int i = 0; i < Q4O_BLOCK; ++i) {
                double v = bf16_value(blk[i]);
                if (fabs(v) > fabs(m))
                    m = v;
            }
            double s = fp16_round_clamped(m / -8.0);
            ws[n * (K / Q4O_BLOCK) + b] = fp16_bits_of(s);
            for (int i = 0; i < Q4O_BLOCK; ++i) {
                int c = 8;
                if (s != 0.0) {
                    float q = rintf((float)bf16_value(blk[i]) / (float)s);
                    c = (int)fmaxf(0.0f, fminf(15.0f, q + 8.0f));
                }
                int64_t k = b * Q4O_BLOCK + i;
                uint8_t *byte = &wq[n * (K / 2) + k / 2];
                if (k % 2 == 0)
                    *byte = (uint8_t)((*byte & 0xF0) | c);
                else
                    *byte = (uint8_t)((*byte & 0x0F) | (c << 4));
            }
        }
    }
}

/* ---- super-block (two-level) scales ------------------------------------------ */

static double sb_weight_at(const uint8_t *wq_row, const uint16_t *wd_row, const uint8_t *wsc_row,
                           int64_t k) {
    return (double)(code_at(wq_row, k) - 8) * fp16_value(wd_row[k / 256]) *
           (double)wsc_row[k / Q4O_BLOCK];
}

/* Dequantised to double [N][K] (exact). */
void oracle_sb_dequant(const uint8_t *wq, const uint16_t *wd, const uint8_t *wsc, int64_t N,
                       int64_t K, double *out) {
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            out[n * K + k] = sb_weight_at(wq + n * (K / 2), wd + n * (K / 256),
                                          wsc + n * (K / Q4O_BLOCK), k);
}

/* y, t: double [M][N]. */
void oracle_sb_matmul(const uint16_t *x, const uint8_t *wq, const uint16_t *wd,
                      const uint8_t *wsc, int64_t M, int64_t N, int64_t K, double *y,
                      double *t) {
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m) {
            const uint8_t *qr = wq + n * (K / 2), *sr = wsc + n * (K / Q4O_BLOCK);
            const uint16_t *dr = wd + n * (K / 256);
            double sum = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = bf16_value(x[m * K + k]) * sb_weight_at(qr, dr, sr, k);
                sum += p;
                mag += fabs(p);
            }
            y[m * N + n] = sum;
            t[m * N + n] = mag;
        }
}
