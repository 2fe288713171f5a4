/*
 * moe_oracle.c -- plain, slow CPU oracle for the fused MoE expert-FFN forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  The GPU library
 * never links, includes or calls it, and it shares no source with it.
 *
 * What it computes (the "MegaMoE" forward of the DeepGEMM/sglang pages):
 *   route tokens by their top-k expert ids (expert count, stable index
 *   write: DeepGEMM SM90 MegaMoE dev log, Phase-2 entry), the L1 grouped GEMM
 *   hidden -> 2 x intermediate (sglang PR #36657 digest, "key code": the
 *   mega_l1_weights argument), the SwiGLU activation with activation_clamp
 *   (same snippet: activation="swiglu", activation_clamp=swiglu_limit),
 *   re-quantisation of the activation into l2_acts / l2_acts_sf (dev log,
 *   Phase-1 entry: the eight buffer views), the L2 grouped GEMM
 *   (mega_l2_weights) and the top-k weighted combine into y (PR #36657
 *   digest: y sliced to num_tokens; DeepGEMM PR #451: the combine step).
 *   Block-scale recipe (1, 1, 32): one e8m0 scale per 1 x 32 block along
 *   the contraction dimension for both operands (PR #36657 digest, recipe
 *   argument).  Recipe (1, 128, 128) with float scale factors (SM90 MegaMoE
 *   dev log, Phase-1 entry): e4m3 operands, one fp32 scale per 1 x 128
 *   activation block and per 128 x 128 weight block.
 *
 * All reductions run in double in ascending index order; every intermediate
 * that the method stores in a narrow type is rounded exactly once to it.
 * Readings of points the pages leave open (scale rule, clamp form, nibble
 * order, where the top-k weight is applied, output precision) are listed in
 * the header comment of each function below.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_RECIPE_BF16 0
#define OR_RECIPE_FP8_FP8 1
#define OR_RECIPE_FP8_FP4 2
#define OR_RECIPE_FP8_B128 3   /* e4m3 x e4m3 with fp32 scales: 1 x 128 (activations), 128 x 128 (weights) */

#define OR_OK 0
#define OR_BAD_ARG -1
#define OR_NO_MEMORY -2
#define OR_BAD_EXPERT_INDEX 1  /* returned (positive) when an index outside [-1, E) was seen */

typedef struct {
    int64_t num_tokens;   /* T */
    int64_t hidden;       /* H */
    int64_t intermediate; /* I */
    int64_t num_experts;  /* E */
    int64_t top_k;        /* k */
    int32_t recipe;       /* OR_RECIPE_* */
    int32_t y_fp32;       /* 1: y is float32, 0: y is bfloat16 */
    float activation_clamp; /* finite and > 0: clamp; otherwise no clamp */
    int32_t pad_;
} oracle_problem;

/* ------------------------------------------------------------------------ */
/* O1: element codecs.  OCP 8-bit (E4M3FN), 4-bit (E2M1) and scale (E8M0)    */
/* formats of the 1x32 block-scale recipe.                                   */
/* ------------------------------------------------------------------------ */

/* E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
   S.1111.111 is NaN; largest finite 448; subnormals m * 2^-9. */
double oracle_dec_e4m3(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp((double)(8 + m), e - 10);   /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit: magnitudes
   0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double oracle_dec_e2m1(uint8_t nibble) {
    int s = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
    double v;
    if (e == 0) v = 0.5 * m;
    else v = ldexp((double)(2 + m), e - 2);    /* (1 + m/2) * 2^(e-1) */
    return s ? -v : v;
}

/* E8M0: 2^(b - 127); 0xFF is NaN. */
double oracle_dec_e8m0(uint8_t b) {
    if (b == 255) return NAN;
    return ldexp(1.0, (int)b - 127);
}

double oracle_dec_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round v to the nearest number with `mbits` fraction bits whose exponent is
   at least `emin` (below 2^emin the spacing stays 2^(emin - mbits)), ties to
   the even neighbour.  No range limit is applied here. */
static double round_to_grid(double v, int mbits, int emin) {
    int e;
    double q;
    if (v == 0.0 || !isfinite(v)) return v;
    frexp(fabs(v), &e);             /* |v| in [2^(e-1), 2^e) */
    e -= 1;
    if (e < emin) e = emin;
    q = ldexp(1.0, e - mbits);      /* grid spacing around v */
    return nearbyint(v / q) * q;    /* exact scaling; nearbyint is round-half-even */
}

/* Nearest E4M3FN value, ties to even, saturating at +-448 (never NaN). */
double oracle_round_e4m3_sat(double v) {
    double r;
    if (isnan(v)) return v;
    r = round_to_grid(v, 3, -6);
    if (r > 448.0) r = 448.0;
    if (r < -448.0) r = -448.0;
    return r;
}

/* Bit pattern of an E4M3FN-representable value (|r| <= 448). */
uint8_t oracle_enc_e4m3(double r) {
    uint8_t s = signbit(r) ? 0x80 : 0x00;
    double a = fabs(r);
    int e;
    if (a == 0.0) return s;
    frexp(a, &e);
    e -= 1;                          /* a in [2^e, 2^(e+1)) */
    if (e < -6) return (uint8_t)(s | (int)ldexp(a, 9));          /* subnormal m * 2^-9 */
    return (uint8_t)(s | ((e + 7) << 3) | ((int)ldexp(a, 3 - e) - 8));
}

/* Nearest bfloat16 value, ties to even; beyond the largest finite bf16 the
   result is +-inf (round-to-nearest overflow). */
double oracle_round_bf16(double v) {
    const double maxbf = 3.3895313892515355e38;  /* (2 - 2^-7) * 2^127 */
    double r;
    if (isnan(v)) return v;
    r = round_to_grid(v, 7, -126);
    if (r > maxbf) r = INFINITY;
    if (r < -maxbf) r = -INFINITY;
    return r;
}

uint16_t oracle_enc_bf16(double r) {
    float f = (float)r;   /* exact: r is bf16-representable */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* O5 scale rule (a reading: the pages do not state it): the e8m0 exponent of
   a 1x32 block is the smallest integer E with amax <= 448 * 2^E, i.e. the
   finest power-of-two scale that clips nothing; clamped to [-127, 127];
   an all-zero block takes E = 0. */
int oracle_scale_exp(double amax) {
    int E;
    if (!(amax > 0.0)) return 0;
    frexp(amax / 448.0, &E);
    while (ldexp(448.0, E - 1) >= amax) E--;
    while (ldexp(448.0, E) < amax) E++;
    if (E < -127) E = -127;
    if (E > 127) E = 127;
    return E;
}

/* O4 activation, fp32 result: clamp BOTH gate and up to [-c, c] when c is
   finite and positive (reading of activation_clamp), then silu(g) * u with
   silu(g) = g * sigmoid(g), evaluated in double and rounded once to fp32. */
float oracle_swiglu(float gate, float up, float clamp) {
    double g = gate, u = up, c = clamp;
    if (isfinite(c) && c > 0.0) {
        g = fmin(fmax(g, -c), c);
        u = fmin(fmax(u, -c), c);
    }
    return (float)(g / (1.0 + exp(-g)) * u);
}

/* ------------------------------------------------------------------------ */
/* O1 applied to whole rows: dequantised operand values in double.           */
/* ------------------------------------------------------------------------ */

/* Activation row (x or the re-quantised h): K values.  The (1, 128, 128)
   recipe scales each 1 x 128 block of a row by one fp32 factor, sf[row][k/128]. */
static void dequant_act_row(int recipe, const void* base, const uint8_t* sf, int64_t row, int64_t K, double* out) {
    int64_t k;
    if (recipe == OR_RECIPE_BF16) {
        const uint16_t* p = (const uint16_t*)base + row * K;
        for (k = 0; k < K; k++) out[k] = oracle_dec_bf16(p[k]);
    } else if (recipe == OR_RECIPE_FP8_B128) {
        const uint8_t* p = (const uint8_t*)base + row * K;
        const float* s = (const float*)(const void*)sf + row * (K / 128);
        for (k = 0; k < K; k++) out[k] = oracle_dec_e4m3(p[k]) * (double)s[k / 128];
    } else {
        const uint8_t* p = (const uint8_t*)base + row * K;
        const uint8_t* s = sf + row * (K / 32);
        for (k = 0; k < K; k++) out[k] = oracle_dec_e4m3(p[k]) * oracle_dec_e8m0(s[k / 32]);
    }
}

/* Weight row `row` of a [rows, K] matrix (rows of all experts stacked).  The
   (1, 128, 128) recipe scales each 128 x 128 block by one fp32 factor,
   sf[row / 128][k / 128] (every expert's row count is a multiple of 128). */
static void dequant_weight_row(int recipe, const void* base, const uint8_t* sf, int64_t row, int64_t K, double* out) {
    int64_t k;
    if (recipe == OR_RECIPE_BF16) {
        const uint16_t* p = (const uint16_t*)base + row * K;
        for (k = 0; k < K; k++) out[k] = oracle_dec_bf16(p[k]);
    } else if (recipe == OR_RECIPE_FP8_B128) {
        const uint8_t* p = (const uint8_t*)base + row * K;
        const float* s = (const float*)(const void*)sf + (row / 128) * (K / 128);
        for (k = 0; k < K; k++) out[k] = oracle_dec_e4m3(p[k]) * (double)s[k / 128];
    } else if (recipe == OR_RECIPE_FP8_FP8) {
        const uint8_t* p = (const uint8_t*)base + row * K;
        const uint8_t* s = sf + row * (K / 32);
        for (k = 0; k < K; k++) out[k] = oracle_dec_e4m3(p[k]) * oracle_dec_e8m0(s[k / 32]);
    } else {
        /* E2M1, two per byte along K: element k sits in byte k/2, even k in
           the low nibble (a reading: the pages do not fix the packing). */
        const uint8_t* p = (const uint8_t*)base + row * (K / 2);
        const uint8_t* s = sf + row * (K / 32);
        for (k = 0; k < K; k++) {
            uint8_t byte = p[k / 2];
            uint8_t nib = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
            out[k] = oracle_dec_e2m1(nib) * oracle_dec_e8m0(s[k / 32]);
        }
    }
}

static double dot(const double* a, const double* b, int64_t n) {
    double acc = 0.0;
    int64_t i;
    for (i = 0; i < n; i++) acc += a[i] * b[i];
    return acc;
}

/* ------------------------------------------------------------------------ */
/* O3-O6: one routed row (token t through expert e).                         */
/*   c_out  [2I] fp32 L1 output (optional)                                   */
/*   h_out  [I]  fp32 activation (optional)                                  */
/*   hq_out [I]  re-quantised activation value (optional)                    */
/*   hq_codes [I] (e4m3 byte, or bf16 bits as uint16 when recipe is BF16),   */
/*   hq_sf [I/32] e8m0 bytes (optional; FP8 recipes only)                    */
/*   o_out  [H]  L2 output as fp32: bf16 values for the e4m3 recipes        */
/*               (required)                                                  */
/*   o_exact, o_eps [H]  exact L2 sums before that rounding and their      */
/*               contraction-error bound (optional)                        */
/* ------------------------------------------------------------------------ */
/* Spacing of the E4M3 grid around |v| (v finite, |v| <= 448). */
static double e4m3_spacing(double v) {
    int e;
    double a = fabs(v);
    if (a < ldexp(1.0, -6)) return ldexp(1.0, -9);
    frexp(a, &e);
    e -= 1;
    if (e > 8) e = 8;
    return ldexp(1.0, e - 3);
}

/* Rounding-decision band (parity infrastructure, not part of the method).
   The re-quantisation turns the fp32 activation into a code.  An
   implementation whose L1 outputs differ from the exact ones sees each
   activation move, and may pick another code for an element whose exact
   value lies close to a rounding midpoint (or another block exponent when the
   block amax lies close to a boundary 448 * 2^E).  The error model is the
   one of a blocked contraction: the K dimension is summed in steps of 128
   elements, each step with an error of at most rho times the step's largest
   |product|, and the step results are added in fp32 (at most 2^-24 times the
   sum of |products| per addition).  So L1 output n is off by at most
     eps[n] = rho * S[n] + steps * 2^-24 * A[n],
     S[n] = sum over steps of max |x_k w_nk|,  A[n] = sum_k |x_k w_nk|,
   and, the clamp being 1-Lipschitz and |silu'| <= 1.1, activation i by at most
     band_i = 1.1 * eps_g * (|u| + eps_u) + |silu(g)| * eps_u
   (g, u the clamped gate and up values, eps_g = eps[i], eps_u = eps[I+i]).
   delta[i] receives the largest change of the dequantised value such a
   deviation can cause: 0 when no rounding midpoint lies within band_i of the
   exact activation and the block exponent is unambiguous, else band_i plus one
   grid spacing at |h_i| + band_i, taken at the coarsest block exponent the
   block amax (within its largest band) can select. */
static double e4m3_spacing_at(double v, int E) {   /* grid spacing at |v| for block exponent E, in v's units */
    double q = ldexp(fabs(v), -E);
    return ldexp(e4m3_spacing(q > 448.0 ? 448.0 : q), E);
}

/* O5 of the (1, 128, 128) recipe (a reading: the pages name the recipe and its
   float scale factors, not the quantiser): per 1 x 128 block of h,
   s = max(fp32(amax / 448), 2^-126), code = E4M3FN code of the IEEE fp32
   quotient fp32(h / s), rounded to nearest even and saturating; the value is
   code * s.  (Rounding the double quotient to fp32 gives the correctly
   rounded fp32 quotient: double has more than twice fp32's precision.) */
static float b128_scale(double amax) {
    float sc = (float)(amax / 448.0);
    return sc < FLT_MIN ? FLT_MIN : sc;
}

static double b128_quotient(float h, float sc) { return (double)(float)((double)h / (double)sc); }

/* The band of the (1, 128, 128) recipe (same activation band as requant_band):
   the block's scale follows its amax continuously, so within the band it can
   move from s_lo = scale(amax - bmax) to s_hi = scale(amax + bmax), changing
   every value of the block by up to (|q| + spacing) * (s_hi - s_lo); an
   element whose quotient lies within band / s_lo + |q| (s_hi - s_lo) / s_lo
   of a rounding midpoint may also take the other code, adding band + one
   spacing at s_hi. */
static void requant_band_b128(const float* h, const double* band, int64_t I, double* delta) {
    int64_t b, i;
    for (b = 0; b < I / 128; b++) {
        double amax = 0.0, bmax = 0.0;
        for (i = 128 * b; i < 128 * b + 128; i++) {
            if (band[i] > bmax) bmax = band[i];
            if (fabs((double)h[i]) > amax) amax = fabs((double)h[i]);
        }
        const double sc = b128_scale(amax), s_lo = b128_scale(amax - bmax > 0.0 ? amax - bmax : 0.0);
        const double s_hi = b128_scale(amax + bmax);
        for (i = 128 * b; i < 128 * b + 128; i++) {
            double q = (double)h[i] / sc;
            double sp = e4m3_spacing(fabs(q) > 448.0 ? 448.0 : q);
            double lo = floor(q / sp) * sp, mid = lo + 0.5 * sp;
            double eq = band[i] / s_lo + fabs(q) * (s_hi - s_lo) / s_lo;
            double sp_hi = e4m3_spacing(fmin(448.0, fabs(q) + eq));
            delta[i] = (fabs(q) + sp) * (s_hi - s_lo);
            if (fabs(q - mid) <= eq || fabs(q) + eq > 448.0) delta[i] += band[i] + sp_hi * s_hi;
        }
    }
}

/* Activation band of every element (see above), into band[I]. */
static void activation_band(const float* c, const double* eps, int64_t I, float clamp, double* band) {
    int64_t i;
    double cc = clamp;
    int clamp_on = isfinite(cc) && cc > 0.0;
    for (i = 0; i < I; i++) {
        double g = c[i], u = c[I + i], eg = eps[i], eu = eps[I + i];
        if (clamp_on) { g = fmin(fmax(g, -cc), cc); u = fmin(fmax(u, -cc), cc); }
        band[i] = 1.1 * eg * (fabs(u) + eu) + fabs(g / (1.0 + exp(-g))) * eu;
    }
}

static void requant_band(const float* h, const float* c, const double* eps, int64_t I, float clamp, double* delta) {
    int64_t b, i;
    double cc = clamp;
    int clamp_on = isfinite(cc) && cc > 0.0;
    for (b = 0; b < I / 32; b++) {
        double amax = 0.0, bmax = 0.0, band[32];
        int E, Ehi, scale_amb;
        for (i = 32 * b; i < 32 * b + 32; i++) {
            double g = c[i], u = c[I + i], eg = eps[i], eu = eps[I + i];
            if (clamp_on) { g = fmin(fmax(g, -cc), cc); u = fmin(fmax(u, -cc), cc); }
            band[i - 32 * b] = 1.1 * eg * (fabs(u) + eu) + fabs(g / (1.0 + exp(-g))) * eu;
            if (band[i - 32 * b] > bmax) bmax = band[i - 32 * b];
            if (fabs((double)h[i]) > amax) amax = fabs((double)h[i]);
        }
        E = oracle_scale_exp(amax);
        Ehi = oracle_scale_exp(amax + bmax);
        if (amax > 0.0)
            scale_amb = Ehi != E || oracle_scale_exp(amax - bmax > 0.0 ? amax - bmax : 0.0) != E;
        else
            scale_amb = bmax > 0.0;
        for (i = 32 * b; i < 32 * b + 32; i++) {
            double q = ldexp((double)h[i], -E);
            double sp = e4m3_spacing(q);
            double lo = floor(q / sp) * sp;       /* grid neighbours of q (exact: sp is a power of two) */
            double mid = lo + 0.5 * sp;
            double bd = band[i - 32 * b];
            if (scale_amb) delta[i] = bd + e4m3_spacing_at(fabs((double)h[i]) + bd, Ehi);
            else if (ldexp(fabs(q - mid), E) <= bd) delta[i] = bd + e4m3_spacing_at(fabs((double)h[i]) + bd, E);
            else delta[i] = 0.0;
        }
    }
}

static int ffn_row(const oracle_problem* p, const void* x, const uint8_t* x_sf, int64_t t, int64_t e,
                   const void* w1, const uint8_t* w1_sf, const void* w2, const uint8_t* w2_sf,
                   float* c_out, float* h_out, double* hq_out, void* hq_codes, uint8_t* hq_sf, float* o_out,
                   double rho, double* o_allow, double* delta_out, double* o_exact, double* o_eps) {
    const int64_t H = p->hidden, I = p->intermediate;
    double* xd = (double*)malloc(sizeof(double) * (size_t)H);
    double* wd = (double*)malloc(sizeof(double) * (size_t)(H > I ? H : I));
    float* c = (float*)malloc(sizeof(float) * (size_t)(2 * I));
    float* h = (float*)malloc(sizeof(float) * (size_t)I);
    double* hq = (double*)malloc(sizeof(double) * (size_t)I);
    int64_t n, i, b;
    if (!xd || !wd || !c || !h || !hq) {
        free(xd); free(wd); free(c); free(h); free(hq);
        return OR_NO_MEMORY;
    }
    /* O3: L1 = x_t . W1[e]^T over the hidden dimension, exact in double,
       rounded once to fp32 (fp32 accumulator of the grouped GEMM).  With a
       band requested, also the error bound eps[n] of requant_band. */
    const int want_band = (o_allow || delta_out) && p->recipe != OR_RECIPE_BF16;
    double* eps = want_band ? (double*)calloc((size_t)(2 * I), sizeof(double)) : NULL;
    if (want_band && !eps) { free(xd); free(wd); free(c); free(h); free(hq); return OR_NO_MEMORY; }
    dequant_act_row(p->recipe, x, x_sf, t, H, xd);
    for (n = 0; n < 2 * I; n++) {
        dequant_weight_row(p->recipe, w1, w1_sf, e * 2 * I + n, H, wd);
        c[n] = (float)dot(xd, wd, H);
        if (eps) {
            double S = 0.0, A = 0.0, m = 0.0;
            int64_t k, steps = (H + 127) / 128;
            for (k = 0; k < H; k++) {
                double a = fabs(xd[k] * wd[k]);
                A += a;
                if (a > m) m = a;
                if (k % 128 == 127 || k == H - 1) { S += m; m = 0.0; }
            }
            /* fp32 step sums; the (1, 128, 128) recipe rounds once more (its fp32 scale product) */
            eps[n] = rho * S + (double)steps * (p->recipe == OR_RECIPE_FP8_B128 ? 2.0 : 1.0) * ldexp(A, -24);
        }
    }
    /* O4: rows [0, I) of W1 are the gate, rows [I, 2I) the up projection. */
    for (i = 0; i < I; i++) h[i] = oracle_swiglu(c[i], c[I + i], p->activation_clamp);
    /* O5: re-quantise h for the L2 GEMM. */
    if (p->recipe == OR_RECIPE_BF16) {
        for (i = 0; i < I; i++) {
            hq[i] = oracle_round_bf16((double)h[i]);
            if (hq_codes) ((uint16_t*)hq_codes)[i] = oracle_enc_bf16(hq[i]);
        }
    } else if (p->recipe == OR_RECIPE_FP8_B128) {
        for (b = 0; b < I / 128; b++) {
            double amax = 0.0;
            float sc;
            for (i = 128 * b; i < 128 * b + 128; i++)
                if (fabs((double)h[i]) > amax) amax = fabs((double)h[i]);
            sc = b128_scale(amax);
            if (hq_sf) ((float*)(void*)hq_sf)[b] = sc;
            for (i = 128 * b; i < 128 * b + 128; i++) {
                double q = oracle_round_e4m3_sat(b128_quotient(h[i], sc));
                if (hq_codes) ((uint8_t*)hq_codes)[i] = oracle_enc_e4m3(q);
                hq[i] = q * (double)sc;
            }
        }
    } else {
        for (b = 0; b < I / 32; b++) {
            double amax = 0.0;
            int E;
            for (i = 32 * b; i < 32 * b + 32; i++)
                if (fabs((double)h[i]) > amax) amax = fabs((double)h[i]);
            E = oracle_scale_exp(amax);
            if (hq_sf) hq_sf[b] = (uint8_t)(E + 127);
            for (i = 32 * b; i < 32 * b + 32; i++) {
                double q = oracle_round_e4m3_sat(ldexp((double)h[i], -E));
                if (hq_codes) ((uint8_t*)hq_codes)[i] = oracle_enc_e4m3(q);
                hq[i] = ldexp(q, E);
            }
        }
    }
    /* O6: L2 = hq . W2[e]^T over the intermediate dimension, exact in double,
       rounded once to the per-slot output type: fp32 for the BF16 recipe, bf16
       (round to nearest even) for the e4m3 recipes, whose y is bf16 (a
       reading: the pages name y's type, not that of the per-expert results the
       combine adds).  o_exact receives the exact sums; o_eps (e4m3 recipes)
       the bound of the blocked contraction's error on each, the model of
       requant_band applied to hq and W2: rho * (sum over 128-element steps of
       the step's largest |hq_i w_ni|) + steps * 2^-24 * sum_i |hq_i w_ni|
       (twice that for the (1, 128, 128) recipe). */
    {
        double* delta = NULL;
        if (want_band) {
            delta = (double*)calloc((size_t)(2 * I), sizeof(double));
            if (!delta) { free(xd); free(wd); free(c); free(h); free(hq); free(eps); return OR_NO_MEMORY; }
            if (p->recipe == OR_RECIPE_FP8_B128) {
                activation_band(c, eps, I, p->activation_clamp, delta + I);
                requant_band_b128(h, delta + I, I, delta);
            } else {
                requant_band(h, c, eps, I, p->activation_clamp, delta);
            }
        }
        for (n = 0; n < H; n++) {
            dequant_weight_row(p->recipe, w2, w2_sf, e * H + n, I, wd);
            {
                double v = dot(hq, wd, I);
                o_out[n] = p->recipe == OR_RECIPE_BF16 ? (float)v : (float)oracle_round_bf16(v);
                if (o_exact) o_exact[n] = v;
            }
            if (o_eps) {
                double S = 0.0, A = 0.0, m = 0.0;
                int64_t steps = (I + 127) / 128;
                for (i = 0; i < I; i++) {
                    double a = fabs(hq[i] * wd[i]);
                    A += a;
                    if (a > m) m = a;
                    if (i % 128 == 127 || i == I - 1) { S += m; m = 0.0; }
                }
                o_eps[n] = p->recipe == OR_RECIPE_BF16
                               ? 0.0
                               : rho * S + (double)steps * (p->recipe == OR_RECIPE_FP8_B128 ? 2.0 : 1.0) * ldexp(A, -24);
            }
            if (o_allow) {
                double a = 0.0;
                if (delta)
                    for (i = 0; i < I; i++)
                        if (delta[i] != 0.0) a += delta[i] * fabs(wd[i]);
                o_allow[n] = a;
            }
        }
        if (delta_out) {
            for (i = 0; i < I; i++) delta_out[i] = delta ? delta[i] : 0.0;
        }
        free(delta);
    }
    free(eps);
    if (c_out) memcpy(c_out, c, sizeof(float) * (size_t)(2 * I));
    if (h_out) memcpy(h_out, h, sizeof(float) * (size_t)I);
    if (hq_out) memcpy(hq_out, hq, sizeof(double) * (size_t)I);
    free(xd); free(wd); free(c); free(h); free(hq);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* O2: routing.  A slot s = t*k + j is valid iff 0 <= idx[s] < E; index -1   */
/* masks a slot, any other out-of-range index also masks it and is reported. */
/* counts[e] = valid slots with expert e; offsets = exclusive prefix sum     */
/* (E+1 entries); rows of expert e are its valid slots in ascending slot     */
/* order: row_to_slot[offsets[e] + r] = the r-th such slot; slot_to_row is   */
/* the inverse, -1 for masked slots.  (Expert count and source token/top-k   */
/* index write of the dispatch stage: DeepGEMM SM90 MegaMoE dev log, Phase   */
/* 2; the in-expert order is a reading: ascending slot.)                     */
/* ------------------------------------------------------------------------ */
int oracle_route(const int32_t* idx, int64_t T, int64_t k, int64_t E,
                 int32_t* counts, int32_t* offsets, int32_t* row_to_slot, int32_t* slot_to_row) {
    int64_t s, e;
    int bad = 0;
    int32_t* cursor;
    if (T < 0 || k <= 0 || E <= 0) return OR_BAD_ARG;
    for (e = 0; e < E; e++) counts[e] = 0;
    for (s = 0; s < T * k; s++) {
        int32_t v = idx[s];
        if (v >= 0 && v < E) counts[v]++;
        else if (v != -1) bad = 1;
    }
    offsets[0] = 0;
    for (e = 0; e < E; e++) offsets[e + 1] = offsets[e] + counts[e];
    cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    if (!cursor) return OR_NO_MEMORY;
    for (e = 0; e < E; e++) cursor[e] = offsets[e];
    for (s = 0; s < T * k; s++) {
        int32_t v = idx[s];
        if (v >= 0 && v < E) {
            int32_t r = cursor[v]++;
            row_to_slot[r] = (int32_t)s;
            slot_to_row[s] = r;
        } else {
            slot_to_row[s] = -1;
        }
    }
    free(cursor);
    return bad ? OR_BAD_EXPERT_INDEX : OR_OK;
}

/* O7: combine.  y[t, n] = sum over valid j (ascending) of w[t, j] * o[row, n]
   in double, rounded once to y's type; a token with no valid slot gets 0. */
static void store_y(const oracle_problem* p, void* y, int64_t yrow, int64_t n, double acc) {
    if (p->y_fp32) ((float*)y)[yrow * p->hidden + n] = (float)acc;
    else ((uint16_t*)y)[yrow * p->hidden + n] = oracle_enc_bf16(oracle_round_bf16(acc));
}

/* Inputs the forward reads must be present when there are tokens to process. */
static int check_inputs(const oracle_problem* p, const void* x, const uint8_t* x_sf, const int32_t* topk_idx,
                        const float* topk_w, const void* w1, const uint8_t* w1_sf, const void* w2,
                        const uint8_t* w2_sf) {
    int fp8 = p->recipe != OR_RECIPE_BF16;
    if (p->num_tokens == 0) return OR_OK;
    if (!x || !topk_idx || !topk_w || !w1 || !w2) return OR_BAD_ARG;
    if (fp8 && (!x_sf || !w1_sf || !w2_sf)) return OR_BAD_ARG;
    return OR_OK;
}

static int check_problem(const oracle_problem* p) {
    if (!p) return OR_BAD_ARG;
    if (p->num_tokens < 0 || p->hidden <= 0 || p->intermediate <= 0 || p->num_experts <= 0 || p->top_k <= 0) return OR_BAD_ARG;
    if (p->recipe < 0 || p->recipe > 3) return OR_BAD_ARG;
    if (p->recipe == OR_RECIPE_FP8_B128 && (p->hidden % 128 || p->intermediate % 128)) return OR_BAD_ARG;
    if (p->hidden % 32 || p->intermediate % 32) return OR_BAD_ARG;
    return OR_OK;
}

/*
 * Full routed forward.  y rows [0, T) are written; optional outputs:
 *   counts[E], offsets[E+1], row_to_slot[T*k] (first R entries used),
 *   slot_to_row[T*k], o_rows[T*k, H]: each routed row's L2 result (O6) as fp32
 *   (bf16 values for the e4m3 recipes).
 * Returns OR_OK, OR_BAD_EXPERT_INDEX (y still computed with those slots
 * masked) or a negative error.
 */
int oracle_forward(const oracle_problem* p, const void* x, const uint8_t* x_sf,
                   const int32_t* topk_idx, const float* topk_w,
                   const void* w1, const uint8_t* w1_sf, const void* w2, const uint8_t* w2_sf,
                   void* y, int32_t* counts_out, int32_t* offsets_out,
                   int32_t* row_to_slot_out, int32_t* slot_to_row_out, float* o_rows_out) {
    int64_t T, H, E, k, R, r, t;
    int32_t *counts, *offsets, *r2s, *s2r;
    float* o;
    int rc, err = 0;
    if (check_problem(p) != OR_OK) return OR_BAD_ARG;
    if (check_inputs(p, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf) != OR_OK) return OR_BAD_ARG;
    T = p->num_tokens; H = p->hidden; E = p->num_experts; k = p->top_k;
    counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
    r2s = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k + 1));
    s2r = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k + 1));
    if (!counts || !offsets || !r2s || !s2r) { free(counts); free(offsets); free(r2s); free(s2r); return OR_NO_MEMORY; }
    rc = oracle_route(topk_idx, T, k, E, counts, offsets, r2s, s2r);
    if (rc < 0) { free(counts); free(offsets); free(r2s); free(s2r); return rc; }
    R = offsets[E];
    o = (float*)malloc(sizeof(float) * (size_t)((R > 0 ? R : 1) * H));
    if (!o) { free(counts); free(offsets); free(r2s); free(s2r); return OR_NO_MEMORY; }
    /* Rows are independent: row r of expert e is token row_to_slot[r] / k. */
#pragma omp parallel for schedule(dynamic, 1) reduction(|:err)
    for (r = 0; r < R; r++) {
        int64_t e = 0;
        while (offsets[e + 1] <= r) e++;
        if (ffn_row(p, x, x_sf, r2s[r] / k, e, w1, w1_sf, w2, w2_sf, NULL, NULL, NULL, NULL, NULL, o + r * H,
                    0.0, NULL, NULL, NULL, NULL) != OR_OK)
            err |= 1;
    }
    if (err) { free(counts); free(offsets); free(r2s); free(s2r); free(o); return OR_NO_MEMORY; }
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; t++) {
        int64_t n, j;
        for (n = 0; n < H; n++) {
            double acc = 0.0;
            for (j = 0; j < k; j++) {
                int32_t row = s2r[t * k + j];
                if (row >= 0) acc += (double)topk_w[t * k + j] * (double)o[(int64_t)row * H + n];
            }
            store_y(p, y, t, n, acc);
        }
    }
    if (counts_out) memcpy(counts_out, counts, sizeof(int32_t) * (size_t)E);
    if (offsets_out) memcpy(offsets_out, offsets, sizeof(int32_t) * (size_t)(E + 1));
    if (row_to_slot_out) memcpy(row_to_slot_out, r2s, sizeof(int32_t) * (size_t)R);
    if (slot_to_row_out) memcpy(slot_to_row_out, s2r, sizeof(int32_t) * (size_t)(T * k));
    if (o_rows_out) memcpy(o_rows_out, o, sizeof(float) * (size_t)(R * H));
    free(counts); free(offsets); free(r2s); free(s2r); free(o);
    return rc;
}

/*
 * Per-token forward (no routing tables): for each listed token, run the FFN
 * of expert topk_idx[t, j] directly for every valid j and combine.  Rows of
 * y_rows follow the order of `tokens`.  Used for sampled checks at sizes the
 * routed forward cannot reach in seconds, and as an independent path to the
 * routed one.  When allow_rows is not NULL it receives, per output element,
 * sum_j |w_j| * sum_i delta_i |W2(e_j, n, i)|: the largest change of y that
 * re-quantisation decisions inside the band `rho` can cause (requant_band),
 * before the rounding of each slot's L2 result to its type (O6; that
 * rounding's own decisions are bounded from ox_rows / oeps_rows).
 */
static int forward_tokens_impl(const oracle_problem* p, const void* x, const uint8_t* x_sf,
                               const int32_t* topk_idx, const float* topk_w,
                               const void* w1, const uint8_t* w1_sf, const void* w2, const uint8_t* w2_sf,
                               const int64_t* tokens, int64_t ntok, void* y_rows,
                               double rho, double* allow_rows, double* hq_rows, double* delta_rows,
                               double* ox_rows, double* oeps_rows) {
    int64_t H, I, E, k, q;
    int err = 0, bad = 0;
    if (check_problem(p) != OR_OK) return OR_BAD_ARG;
    if (check_inputs(p, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf) != OR_OK) return OR_BAD_ARG;
    H = p->hidden; I = p->intermediate; E = p->num_experts; k = p->top_k;
    for (q = 0; q < ntok; q++)
        if (tokens[q] < 0 || tokens[q] >= p->num_tokens) return OR_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1) reduction(|:err) reduction(|:bad)
    for (q = 0; q < ntok; q++) {
        int64_t t = tokens[q], j, n;
        float* o = (float*)malloc(sizeof(float) * (size_t)(k * H));
        double* oa = allow_rows ? (double*)calloc((size_t)(k * H), sizeof(double)) : NULL;
        if (!o || (allow_rows && !oa)) { free(o); free(oa); err |= 1; continue; }
        for (j = 0; j < k; j++) {
            int32_t e = topk_idx[t * k + j];
            if (e >= 0 && e < E) {
                if (ffn_row(p, x, x_sf, t, e, w1, w1_sf, w2, w2_sf, NULL, NULL,
                            hq_rows ? hq_rows + (q * k + j) * I : NULL, NULL, NULL, o + j * H,
                            rho, oa ? oa + j * H : NULL, delta_rows ? delta_rows + (q * k + j) * I : NULL,
                            ox_rows ? ox_rows + (q * k + j) * H : NULL,
                            oeps_rows ? oeps_rows + (q * k + j) * H : NULL) != OR_OK)
                    err |= 1;
            } else if (e != -1) {
                bad |= 1;
            }
        }
        for (n = 0; n < H; n++) {
            double acc = 0.0, al = 0.0;
            for (j = 0; j < k; j++) {
                int32_t e = topk_idx[t * k + j];
                if (e >= 0 && e < E) {
                    acc += (double)topk_w[t * k + j] * (double)o[j * H + n];
                    if (oa) al += fabs((double)topk_w[t * k + j]) * oa[j * H + n];
                }
            }
            store_y(p, y_rows, q, n, acc);
            if (allow_rows) allow_rows[q * H + n] = al;
        }
        free(o);
        free(oa);
    }
    if (err) return OR_NO_MEMORY;
    return bad ? OR_BAD_EXPERT_INDEX : OR_OK;
}

int oracle_forward_tokens_band(const oracle_problem* p, const void* x, const uint8_t* x_sf,
                               const int32_t* topk_idx, const float* topk_w,
                               const void* w1, const uint8_t* w1_sf, const void* w2, const uint8_t* w2_sf,
                               const int64_t* tokens, int64_t ntok, void* y_rows,
                               double rho, double* allow_rows) {
    return forward_tokens_impl(p, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, tokens, ntok, y_rows, rho,
                               allow_rows, NULL, NULL, NULL, NULL);
}

/* Per-token forward that also hands back, for slot j of listed token q (row
   q*k + j of hq_rows / delta_rows, each [ntok*k, I]), the re-quantised
   activation values of that routed row and the rounding-decision band of each
   of them for `rho` (requant_band; zero for the BF16 recipe), and (rows
   q*k + j of ox_rows / oeps_rows, each [ntok*k, H]; either may be NULL) the
   exact L2 sums of the row before their rounding to the per-slot type and the
   contraction-error bound of each (O6).  Rows of masked slots are left
   untouched.  For unit checks of an implementation's h and o. */
int oracle_forward_tokens_rows(const oracle_problem* p, const void* x, const uint8_t* x_sf,
                               const int32_t* topk_idx, const float* topk_w,
                               const void* w1, const uint8_t* w1_sf, const void* w2, const uint8_t* w2_sf,
                               const int64_t* tokens, int64_t ntok, void* y_rows,
                               double rho, double* hq_rows, double* delta_rows, double* ox_rows,
                               double* oeps_rows) {
    return forward_tokens_impl(p, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, tokens, ntok, y_rows, rho,
                               NULL, hq_rows, delta_rows, ox_rows, oeps_rows);
}

int oracle_forward_tokens(const oracle_problem* p, const void* x, const uint8_t* x_sf,
                          const int32_t* topk_idx, const float* topk_w,
                          const void* w1, const uint8_t* w1_sf, const void* w2, const uint8_t* w2_sf,
                          const int64_t* tokens, int64_t ntok, void* y_rows) {
    return oracle_forward_tokens_band(p, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, tokens, ntok, y_rows,
                                      0.0, NULL);
}

/* One row's intermediates (token t through expert e), for unit checks;
   delta_out (optional, [I]) receives the rounding-decision band of each
   re-quantised element for the given rho (see requant_band). */
int oracle_ffn_row(const oracle_problem* p, const void* x, const uint8_t* x_sf, int64_t t, int64_t e,
                   const void* w1, const uint8_t* w1_sf, const void* w2, const uint8_t* w2_sf,
                   float* c_out, float* h_out, double* hq_out, void* hq_codes, uint8_t* hq_sf, float* o_out,
                   double rho, double* delta_out, double* o_exact, double* o_eps) {
    if (check_problem(p) != OR_OK) return OR_BAD_ARG;
    if (t < 0 || t >= p->num_tokens || e < 0 || e >= p->num_experts || !o_out) return OR_BAD_ARG;
    return ffn_row(p, x, x_sf, t, e, w1, w1_sf, w2, w2_sf, c_out, h_out, hq_out, hq_codes, hq_sf, o_out,
                   rho, NULL, delta_out, o_exact, o_eps);
}

/* ------------------------------------------------------------------------ */
/* Pre-dispatch activation quantisation: bf16 activations -> e4m3 codes and */
/* one e8m0 scale per 1x32 block along the hidden dimension, the x / x_sf   */
/* the forward consumes.  The pages place the step before the kernel call   */
/* ("[Blackwell] Reserve SMs for DeepGEMM MegaMoE grid barriers", Fix       */
/* section; its digest, key-code section) without its arithmetic; the       */
/* reading is the forward's own O5 rule on the exact bf16 values: for each  */
/* block, E = oracle_scale_exp(max |x|), sf = E + 127, and each code is the */
/* E4M3FN pattern of round_e4m3_sat(x * 2^-E) (the scaling by 2^-E is exact */
/* in double).  Rows are independent; parity status: pinned (tests).        */
/* ------------------------------------------------------------------------ */
int oracle_quantize_act(const uint16_t* x, int64_t T, int64_t H, uint8_t* codes, uint8_t* sf) {
    int64_t t, b;
    int i;
    if (T < 0 || H <= 0 || H % 32 != 0 || (T > 0 && (!x || !codes || !sf))) return OR_BAD_ARG;
    for (t = 0; t < T; t++) {
        for (b = 0; b < H / 32; b++) {
            const uint16_t* xb = x + t * H + b * 32;
            double amax = 0.0;
            int E;
            for (i = 0; i < 32; i++) {
                const double a = fabs(oracle_dec_bf16(xb[i]));
                if (a > amax) amax = a;
            }
            E = oracle_scale_exp(amax);
            sf[t * (H / 32) + b] = (uint8_t)(E + 127);
            for (i = 0; i < 32; i++)
                codes[t * H + b * 32 + i] = oracle_enc_e4m3(oracle_round_e4m3_sat(ldexp(oracle_dec_bf16(xb[i]), -E)));
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Gate and top-k (the step that produces topk_idx / topk_weights before    */
/* dispatch; the sglang page's Fix section: gate computation and top-k      */
/* selection run before the MegaMoE call).  The pages give no formula; the  */
/* reading is a softmax router:                                             */
/*   logits[t, e] = sum_h x[t, h] * Wg[e, h]   (bf16 inputs, double sum in  */
/*                                              ascending h; stored fp64)   */
/*   the k slots of token t are its k largest logits in descending order,   */
/*   equal logits ordered by the lower expert id (softmax is monotonic, so  */
/*   this is the top-k of the probabilities);                               */
/*   weight of slot j = softmax over the selected logits only, i.e. the     */
/*   top-k probabilities renormalised to sum 1, rounded once to fp32.       */
/* ------------------------------------------------------------------------ */
int oracle_route_topk(const uint16_t* x, const uint16_t* wg, int64_t T, int64_t H, int64_t E, int64_t k,
                      double* logits, int32_t* topk_idx, float* topk_w) {
    int64_t t;
    if (T < 0 || H <= 0 || E <= 0 || k <= 0 || k > E || (T > 0 && (!x || !wg || !logits || !topk_idx || !topk_w)))
        return OR_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 4)
    for (t = 0; t < T; t++) {
        double* l = logits + t * E;
        unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
        double lmax = 0.0, den = 0.0;
        int64_t e, h, j;
        for (e = 0; e < E; e++) {
            double acc = 0.0;
            for (h = 0; h < H; h++) acc += oracle_dec_bf16(x[t * H + h]) * oracle_dec_bf16(wg[e * H + h]);
            l[e] = acc;
        }
        for (j = 0; j < k; j++) {
            int64_t best = -1;
            for (e = 0; e < E; e++)
                if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;   /* strict: ties keep the lower id */
            taken[best] = 1;
            topk_idx[t * k + j] = (int32_t)best;
        }
        lmax = l[topk_idx[t * k]];
        for (j = 0; j < k; j++) den += exp(l[topk_idx[t * k + j]] - lmax);
        for (j = 0; j < k; j++) topk_w[t * k + j] = (float)(exp(l[topk_idx[t * k + j]] - lmax) / den);
        free(taken);
    }
    return OR_OK;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
