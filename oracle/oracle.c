/*
 * CPU oracle for the scaled low-precision GEMM of LLM prefill linears.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The HIP product path
 * never links, imports or calls it, and it shares no code, header or table
 * with that path.
 *
 * Plain, slow, obviously correct: table decode of every code, a bisection
 * search for the nearest representable value, IEEE binary32 arithmetic where
 * the method rounds to fp32, fp64 accumulation, and a single direct rounding
 * from fp64 to bf16.  OpenMP only splits independent rows; no blocking,
 * fusion or reordering of the arithmetic.
 *
 * Sources (web pages; section names as they appear there):
 *  [P1] ninfer PR #167, "The fp8 A8 GEMM stages its operands through TMA"
 *       - opening summary: FP8 row-scaled "A8" GEMM, fp32 accumulator, scales
 *         applied to the accumulator, then the linear / linear_add /
 *         linear_swiglu epilogue and output policies;
 *       - "Measured": weights stored as FP8_E4M3FN with row scales;
 *       - maintainer review item 3 and the reply: the contract is the Op
 *         against an independent mathematical oracle.
 *  [P2] AstrAI commit log for csrc/kernels/fp8/gemm.cuh
 *       - its E4M3 benchmark entry: per-tensor scaled NT GEMM on
 *         pre-quantized operands;
 *       - an API of two primitives (quantize, then the FP8 GEMM), with
 *         amax references computed in fp32; 3D operands through batch
 *         strides.
 *  [P3] ninfer PR #160, "The NVFP4 TMA route reads activation scales as one
 *       tile": NVFP4 = E2M1 codes, one E4M3 scale per 16-element K group
 *       (scale tiles of a block of tokens by 16 groups), linear_add and
 *       linear_swiglu at T=4096.
 * The pages print no formulas for the scales.  Where they are silent this
 * file takes the plainest reading:
 *  - FP8 scale s = fl32(amax / 448); code = RNE-to-E4M3, saturating at 448;
 *  - NVFP4: tensor scale t = fl32(amax / 2688) (448 * 6, both format maxima),
 *    block scale code = RNE-to-E4M3(fl32(amax_g / fl32(6 t))), element code =
 *    RNE-to-E2M1(fl32(x / fl32(S_g t))), saturating at 6;
 *  - signed zeros are kept in codes; a zero scale gives signed-zero codes;
 *  - SwiGLU pairs weight rows j (gate) and j + N/2 (up).
 *
 * Every function here is pinned by tests marked "not gpu": exhaustive decode
 * tables against torch's float8_e4m3fn, a brute-force nearest search, exact
 * integer dot products, power-of-two cases and naive triple loops.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

/* Threads an OpenMP region of this library uses. */
EXPORT int spo_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------- */
/* bf16 and fp32 bit helpers                                                 */
/* ------------------------------------------------------------------------- */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* A bf16 value is the upper half of a binary32. */
EXPORT float spo_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* Round an fp64 value to the nearest bf16 (ties to even) in one step, with no
 * intermediate fp32 rounding.  bf16 keeps 8 significant bits; below 2^-126 the
 * quantum is fixed at 2^-133 (subnormals). */
EXPORT uint16_t spo_bf16_from_f64(double y)
{
    if (isnan(y)) return 0x7FC0;
    uint16_t sign = signbit(y) ? 0x8000 : 0;
    double a = fabs(y);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int e;
    frexp(a, &e);                       /* a = m * 2^e, 0.5 <= m < 1 */
    int qexp = e - 8;                   /* quantum of an 8-bit significand */
    if (qexp < -133) qexp = -133;
    double n = nearbyint(ldexp(a, -qexp));  /* default mode: nearest, ties even */
    double r = ldexp(n, qexp);
    float f = (float)r;                 /* exact, or +inf past the bf16 range */
    return sign | (uint16_t)(bits_from_f32(f) >> 16);
}

/* ------------------------------------------------------------------------- */
/* Number formats: decode by definition, encode by nearest-value search      */
/* ------------------------------------------------------------------------- */

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
 * S.1111.111 is NaN; largest finite magnitude 448 (0x7E). */
EXPORT double spo_e4m3_value(uint32_t code)
{
    code &= 0xFF;
    double sgn = (code & 0x80) ? -1.0 : 1.0;
    uint32_t e = (code >> 3) & 0xF, m = code & 0x7;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0) return sgn * ldexp((double)m, -9);           /* m/8 * 2^-6 */
    return sgn * ldexp(1.0 + m / 8.0, (int)e - 7);
}

/* E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7; bit 3 is the sign. */
EXPORT double spo_e2m1_value(uint32_t code)
{
    code &= 0xF;
    double sgn = (code & 0x8) ? -1.0 : 1.0;
    uint32_t e = (code >> 1) & 0x3, m = code & 0x1;
    if (e == 0) return sgn * 0.5 * m;
    return sgn * ldexp(1.0 + m / 2.0, (int)e - 1);
}

/* Index of the representable magnitude nearest to a (>= 0) in a strictly
 * increasing table mag[0..n-1] (mag[i] is the value of code i); ties go to
 * the even code; anything at or above mag[n-1] saturates to n-1. */
static uint32_t nearest_code(double a, const double *mag, int n)
{
    if (a >= mag[n - 1]) return (uint32_t)(n - 1);
    int lo = 0, hi = n - 1;              /* mag[lo] <= a < mag[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (mag[mid] <= a) lo = mid; else hi = mid;
    }
    double midpoint = 0.5 * (mag[lo] + mag[hi]);   /* exact: few-bit values */
    if (a < midpoint) return (uint32_t)lo;
    if (a > midpoint) return (uint32_t)hi;
    return (lo & 1) ? (uint32_t)hi : (uint32_t)lo;
}

static double e4m3_mag[127];   /* codes 0x00..0x7E */
static double e2m1_mag[8];     /* codes 0x0..0x7 */

__attribute__((constructor)) static void build_tables(void)
{
    for (int c = 0; c < 127; ++c) e4m3_mag[c] = spo_e4m3_value((uint32_t)c);
    for (int c = 0; c < 8; ++c) e2m1_mag[c] = spo_e2m1_value((uint32_t)c);
}

/* Round a finite binary32 to E4M3FN: nearest, ties to even, saturating at
 * +-448, sign kept (so -0 and small negatives give 0x80).  Never NaN. */
EXPORT uint32_t spo_e4m3_encode(float v)
{
    uint32_t sign = signbit(v) ? 0x80u : 0u;
    return sign | nearest_code(fabs((double)v), e4m3_mag, 127);
}

/* Round a finite binary32 to E2M1: nearest, ties to even, saturating at
 * +-6, sign kept (bit 3). */
EXPORT uint32_t spo_e2m1_encode(float v)
{
    uint32_t sign = signbit(v) ? 0x8u : 0u;
    return sign | nearest_code(fabs((double)v), e2m1_mag, 8);
}

/* ------------------------------------------------------------------------- */
/* FP8 quantization: per row and per tensor                                  */
/* ------------------------------------------------------------------------- */

/* One element: fl32(x / s) rounded to E4M3; a zero scale gives a signed
 * zero code. */
static uint8_t e4m3_quant_one(float x, float s)
{
    if (s > 0.0f) {
        float r = x / s;                 /* IEEE binary32 division */
        return (uint8_t)spo_e4m3_encode(r);
    }
    return signbit(x) ? 0x80 : 0x00;
}

/* Per-row ("row-scaled", [P1] opening summary and "Measured") quantization.
 * x: bf16 bits [rows, K] with row stride ldx; q: codes [rows, K] with row
 * stride ldq; scale: fp32 [rows].  s_r = fl32(max_k |x_rk| / 448). */
EXPORT void spo_quantize_rowwise(const uint16_t *x, int64_t rows, int64_t K, int64_t ldx,
                                 uint8_t *q, int64_t ldq, float *scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * ldx;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) amax = fmaxf(amax, fabsf(spo_bf16_to_f32(xr[k])));
        float s = amax / 448.0f;
        scale[r] = s;
        for (int64_t k = 0; k < K; ++k) q[r * ldq + k] = e4m3_quant_one(spo_bf16_to_f32(xr[k]), s);
    }
}

/* Largest magnitude over a [rows, K] bf16 matrix (exact in fp32). */
EXPORT float spo_amax_bf16(const uint16_t *x, int64_t rows, int64_t K, int64_t ldx)
{
    float amax = 0.0f;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k) amax = fmaxf(amax, fabsf(spo_bf16_to_f32(x[r * ldx + k])));
    return amax;
}

/* Per-tensor quantization ([P2], the per-tensor E4M3 benchmark; one scale per
 * matrix, per batch element for a batched operand).  x: batch matrices
 * [rows, K], matrix b at x + b*bstride, row stride K; q likewise with stride
 * rows*K per matrix; scale: fp32 [batch]. */
EXPORT void spo_quantize_tensor(const uint16_t *x, int64_t batch, int64_t rows, int64_t K,
                                int64_t bstride, uint8_t *q, float *scale)
{
    for (int64_t b = 0; b < batch; ++b) {
        const uint16_t *xb = x + b * bstride;
        float s = spo_amax_bf16(xb, rows, K, K) / 448.0f;
        scale[b] = s;
        uint8_t *qb = q + b * rows * K;
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t k = 0; k < K; ++k)
                qb[r * K + k] = e4m3_quant_one(spo_bf16_to_f32(xb[r * K + k]), s);
    }
}

/* Quantize rows with a given per-row or shared scale (used to quantize only
 * the rows a sampled check needs).  scale_stride 1: scale[r]; 0: scale[0]. */
EXPORT void spo_quantize_rows_with_scale(const uint16_t *x, int64_t rows, int64_t K, int64_t ldx,
                                         const float *scale, int64_t scale_stride,
                                         uint8_t *q, int64_t ldq)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float s = scale[r * scale_stride];
        for (int64_t k = 0; k < K; ++k)
            q[r * ldq + k] = e4m3_quant_one(spo_bf16_to_f32(x[r * ldx + k]), s);
    }
}

/* ------------------------------------------------------------------------- */
/* NVFP4 block quantization ([P3]: E2M1 codes, E4M3 scale per 16 K-elements,  */
/* fp32 tensor scale)                                                         */
/* ------------------------------------------------------------------------- */

/* t = fl32(amax / (448 * 6)). */
EXPORT float spo_nvfp4_tensor_scale(const uint16_t *x, int64_t rows, int64_t K, int64_t ldx)
{
    return spo_amax_bf16(x, rows, K, ldx) / 2688.0f;
}

/* Quantize rows [rows, K] (K % 16 == 0) given the tensor scale t.
 * q: [rows, K/2] bytes, element k in the low nibble when k is even;
 * bscale: [rows, K/16] E4M3 codes, row-major. */
EXPORT void spo_quantize_block16_rows(const uint16_t *x, int64_t rows, int64_t K, int64_t ldx,
                                      float t, uint8_t *q, uint8_t *bscale)
{
    const int64_t G = K / 16;
    const float six_t = 6.0f * t;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * ldx;
        for (int64_t g = 0; g < G; ++g) {
            float amax_g = 0.0f;
            for (int k = 0; k < 16; ++k) amax_g = fmaxf(amax_g, fabsf(spo_bf16_to_f32(xr[16 * g + k])));
            uint32_t b = 0;
            if (t > 0.0f) b = spo_e4m3_encode(amax_g / six_t);
            bscale[r * G + g] = (uint8_t)b;
            float S = (float)spo_e4m3_value(b);      /* exact */
            float e = S * t;                         /* fl32(S_g * t) */
            for (int k = 0; k < 16; k += 2) {
                uint32_t c[2];
                for (int h = 0; h < 2; ++h) {
                    float xv = spo_bf16_to_f32(xr[16 * g + k + h]);
                    if (e > 0.0f) c[h] = spo_e2m1_encode(xv / e);
                    else c[h] = signbit(xv) ? 0x8u : 0x0u;
                }
                q[r * (K / 2) + (16 * g + k) / 2] = (uint8_t)(c[0] | (c[1] << 4));
            }
        }
    }
}

/* Whole-tensor NVFP4 quantization: tensor scale, then every row. */
EXPORT void spo_quantize_block16(const uint16_t *x, int64_t rows, int64_t K, int64_t ldx,
                                 uint8_t *q, uint8_t *bscale, float *tscale)
{
    float t = spo_nvfp4_tensor_scale(x, rows, K, ldx);
    *tscale = t;
    spo_quantize_block16_rows(x, rows, K, ldx, t, q, bscale);
}

/* ------------------------------------------------------------------------- */
/* GEMM: exact sums of decoded code products, fp64                           */
/* ------------------------------------------------------------------------- */

/* D[i,j] = sum_k dec(A[i,k]) dec(W[j,k]) for E4M3 codes, NT layout (both
 * operands K-contiguous).  Every product is a multiple of 2^-18 below 2^18,
 * so the fp64 sum is exact for K < 2^17.  Dabs[i,j] = sum_k |products|.
 * Rows of the result have stride N. */
EXPORT void spo_gemm_e4m3(const uint8_t *A, int64_t lda, const uint8_t *W, int64_t ldw,
                          int64_t M, int64_t N, int64_t K, double *D, double *Dabs)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        double a[K > 0 ? K : 1];
        for (int64_t k = 0; k < K; ++k) a[k] = spo_e4m3_value(A[i * lda + k]);
        for (int64_t j = 0; j < N; ++j) {
            const uint8_t *w = W + j * ldw;
            double s = 0.0, sa = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = a[k] * spo_e4m3_value(w[k]);
                s += p;
                sa += fabs(p);
            }
            D[i * N + j] = s;
            Dabs[i * N + j] = sa;
        }
    }
}

/* NVFP4: D[i,j] = sum_g S^A_ig S^W_jg sum_{k in g} dec(a_ik) dec(w_jk), with
 * the group sums of E2M1 products exact and the scaled terms summed in fp64.
 * Aq/Wq: packed codes [rows, K/2]; As/Ws: E4M3 block scales [rows, K/16]. */
EXPORT void spo_gemm_nvfp4(const uint8_t *Aq, const uint8_t *As, const uint8_t *Wq,
                           const uint8_t *Ws, int64_t M, int64_t N, int64_t K,
                           double *D, double *Dabs)
{
    const int64_t G = K / 16;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        double a[K > 0 ? K : 1];
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = Aq[i * (K / 2) + k / 2];
            a[k] = spo_e2m1_value((k & 1) ? (byte >> 4) : (byte & 0xF));
        }
        for (int64_t j = 0; j < N; ++j) {
            double s = 0.0, sa = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                double gs = 0.0, gsa = 0.0;
                for (int64_t k = 16 * g; k < 16 * g + 16; ++k) {
                    uint8_t byte = Wq[j * (K / 2) + k / 2];
                    double w = spo_e2m1_value((k & 1) ? (byte >> 4) : (byte & 0xF));
                    gs += a[k] * w;
                    gsa += fabs(a[k] * w);
                }
                double sc = spo_e4m3_value(As[i * G + g]) * spo_e4m3_value(Ws[j * G + g]);
                s += sc * gs;
                sa += fabs(sc) * gsa;
            }
            D[i * N + j] = s;
            Dabs[i * N + j] = sa;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Epilogue ([P1] opening summary: linear, linear_add, linear_swiglu)        */
/* ------------------------------------------------------------------------- */

enum { SPO_STORE = 0, SPO_ADD = 1, SPO_SWIGLU = 2 };

static double silu(double z) { return z / (1.0 + exp(-z)); }
static double silu_prime(double z)
{
    double sg = 1.0 / (1.0 + exp(-z));
    return sg * (1.0 + z * (1.0 - sg));
}

/* silu'' vanishes only at +-T0, the root of t tanh(t/2) = 2, so silu' is
 * monotone on (-inf, -T0], [-T0, T0] and [T0, inf): its largest magnitude on
 * [lo, hi] is taken at an end or at +-T0 when they lie inside. */
#define SILU_T0 2.3993572805154675
static double silu_slope_max(double lo, double hi)
{
    double m = fmax(fabs(silu_prime(lo)), fabs(silu_prime(hi)));
    if (lo <= SILU_T0 && SILU_T0 <= hi) m = fmax(m, fabs(silu_prime(SILU_T0)));
    if (lo <= -SILU_T0 && -SILU_T0 <= hi) m = fmax(m, fabs(silu_prime(-SILU_T0)));
    return m;
}

/* Scale the exact sums and apply the epilogue, all in fp64.
 * D, Dabs: [M, Nw] (row stride Nw); ascale[M], wscale[Nw] are the fp32 scales
 * as doubles (per-tensor and NVFP4 tensor scales are passed replicated).
 * STORE:  y = sa_i sw_j D_ij                        (Nout = Nw)
 * ADD:    y = sa_i sw_j D_ij + r_ij + b_j           (Nout = Nw)
 * SWIGLU: y = silu(v_ij) v_i,j+Nw/2, v = sa sw D    (Nout = Nw/2)
 * r (bf16 bits, row stride ldr) and b (fp64 [Nout], a bias already
 * dequantized) may each be NULL (taken as zero).  The bias enters after the
 * operand scales and before the one rounding to bf16 (AstrAI commit log, the
 * commit fusing the bias into the GEMM epilogue).
 * y, tol_S: [M, Nout]; out: bf16 bits of y, rounded once from fp64.
 * tol_S is the error scale S of the acceptance bound |gpu - y| <=
 * 2^-8 |y| + 2^-12 S: S = |sa sw| Dabs for STORE and ADD.  For SWIGLU the
 * gate g and up u may each be off by 2^-12 of their own scales Sg, Su; then
 * |silu(g') u' - silu(g) u| <= L Sg' (|u| + 2^-12 Su) + |silu(g)| Su' with
 * Sg' = 2^-12 Sg, Su' = 2^-12 Su and L the largest |silu'| within Sg' of g,
 * so S = L Sg (|u| + 2^-12 Su) + |silu(g)| Su.  Where the gate sum cancels
 * (|g| far below Sg) the slope at g alone would understate the error. */
EXPORT void spo_epilogue(int epi, const double *D, const double *Dabs, int64_t M, int64_t Nw,
                         const double *ascale, const double *wscale,
                         const uint16_t *residual, int64_t ldr, const double *bias,
                         double *y, double *tol_S, uint16_t *out)
{
    const int64_t Nout = (epi == SPO_SWIGLU) ? Nw / 2 : Nw;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < Nout; ++j) {
            double yv, S;
            if (epi == SPO_SWIGLU) {
                int64_t ju = j + Nout;
                double vg = ascale[i] * wscale[j] * D[i * Nw + j];
                double vu = ascale[i] * wscale[ju] * D[i * Nw + ju];
                double Sg = fabs(ascale[i] * wscale[j]) * Dabs[i * Nw + j];
                double Su = fabs(ascale[i] * wscale[ju]) * Dabs[i * Nw + ju];
                yv = silu(vg) * vu;
                double dg = 0x1p-12 * Sg;
                S = silu_slope_max(vg - dg, vg + dg) * Sg * (fabs(vu) + 0x1p-12 * Su) + fabs(silu(vg)) * Su;
            } else {
                double v = ascale[i] * wscale[j] * D[i * Nw + j];
                S = fabs(ascale[i] * wscale[j]) * Dabs[i * Nw + j];
                yv = v;
                if (epi == SPO_ADD && residual) yv += (double)spo_bf16_to_f32(residual[i * ldr + j]);
                if (epi == SPO_ADD && bias) yv += bias[j];
            }
            y[i * Nout + j] = yv;
            tol_S[i * Nout + j] = S;
            out[i * Nout + j] = spo_bf16_from_f64(yv);
        }
    }
}
