/*
 * NVFP4 W4A4 reference oracle -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.
 *
 * A plain, slow CPU statement of what the quantized linear layer computes, used only to check the
 * HIP library: only the test suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the GPU library and includes nothing from it.
 *
 * Sources (paper: "Why Gated DeltaNet Survives 4-Bit Quantization: NVFP4 W4A4 for the Recurrent Half
 * of a Hybrid 27B LLM", arXiv:2609.04098, as presented by the pages):
 *  - NVFP4 format: 4-bit E2M1 values, one E4M3 scale per 16 consecutive elements, the block maximum
 *    setting the scale -- Japanese article, "Mechanism 1: block scaling localizes outliers" and the
 *    FAQ "What is NVFP4?"; English abstract, point (i) "16-element block scaling".
 *  - One FP32 global scale per linear module, and several separately calibrated modules fused into
 *    one GEMM, each needing its own global scale -- Japanese article, "Trap 1: per-module calibration
 *    vs. fused GEMM scale mismatch"; English abstract ("global-scale mismatch ... fuse those modules
 *    into one GEMM"); aimodeling.com English translation, "What engineers should actually take away".
 *  - Gates g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b) -- Japanese article,
 *    "Mechanism 2: the protected gate projections were the most robust".
 *  - The E2M1 and E4M3 encodings themselves follow the OCP Microscaling / FP8 definitions, which the
 *    article's reference list cites ("Microscaling Data Formats", arXiv:2310.10537).
 *  - Companions on the same serving path (section "Serving-path companions" below): the FP8 KV cache
 *    with calibrated static per-tensor scales -- Japanese article, "Is FP8 enough for the KV cache?
 *    The 'ship KV scales' recipe"; the fold-in repair of the fused-module scale mismatch (common global
 *    scale, ratio folded into the block scales, re-rounding error at most 6.2%) -- Japanese article,
 *    "Trap 1"; the BF16 normalization layers ahead of the quantized projections -- Japanese article,
 *    "Minima, quantized 'all 4-bit': the experiment design"; the Gated DeltaNet delta-rule recurrence
 *    that consumes the gates -- Japanese article, "How Gated DeltaNet works".
 *
 * Readings where the pages are silent:
 *  - every FP32 step is one IEEE binary32 operation rounded to nearest-even, in the order
 *    t = 6*g, s_raw = amax/t, S = s*g, v = |x|/S (this file is compiled with -ffp-contract=off);
 *  - the E4M3 block scale is rounded to nearest-even and saturates at 448 (OCP E4M3FN);
 *  - a block whose scale rounds to zero encodes all its elements as zero magnitude;
 *  - a code keeps the sign bit of its input, so -0.0 and small negatives encode as 0x8;
 *  - codes pack two per byte, the even element in the low nibble; scales are one byte per block;
 *  - GEMM products are accumulated exactly (integers in units of 2^-20), then scaled in double.
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if defined(__FAST_MATH__)
#error "the oracle must be compiled without fast-math"
#endif

/* ------------------------------------------------------------------------------------------------
 * Format definitions
 * ---------------------------------------------------------------------------------------------- */

/* E2M1 (OCP MX FP4): bit 3 sign, bits 2:1 exponent (bias 1), bit 0 mantissa.
 * Exponent 0 is subnormal: value = m * 0.5. Otherwise value = 2^(e-1) * (1 + m/2). */
double oracle_e2m1_value(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? m * 0.5 : ldexp(1.0 + m / 2.0, e - 1);
    return s ? -mag : mag;
}

/* E4M3FN (OCP FP8): bit 7 sign, bits 6:3 exponent (bias 7), bits 2:0 mantissa. Exponent 0 is
 * subnormal: m * 2^-9. Bytes 0x7F and 0xFF are NaN; there is no infinity. */
double oracle_e4m3_value(int byte) {
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Round a non-negative finite value to the nearest of the given ascending grid of candidates,
 * ties going to the candidate with the even index (even index == even mantissa LSB for both grids
 * below). Values above the largest candidate saturate to it. Distances are compared exactly by
 * testing 2*v against lo+hi, which is exact in double for these grids. */
static int nearest_even(double v, const double* grid, int n) {
    if (!(v >= 0.0)) return 0; /* caller guarantees v >= 0 and not NaN */
    if (v >= grid[n - 1]) return n - 1;
    int lo = 0;
    while (lo + 1 < n && grid[lo + 1] <= v) ++lo;
    int hi = lo + 1;
    double twice = 2.0 * v, mid2 = grid[lo] + grid[hi];
    if (twice < mid2) return lo;
    if (twice > mid2) return hi;
    return (lo % 2 == 0) ? lo : hi;
}

/* The two rounding grids, ascending: the 127 finite non-negative E4M3FN values (bytes 0x00..0x7E)
 * and the 8 E2M1 magnitudes (codes 0..7). */
static void e4m3_grid(double* grid) {
    for (int b = 0; b < 127; ++b) grid[b] = oracle_e4m3_value(b);
}
static void e2m1_grid(double* grid) {
    for (int c = 0; c < 8; ++c) grid[c] = oracle_e2m1_value(c);
}

/* E4M3FN round-to-nearest-even with saturation to the largest finite value 448 (byte 0x7E).
 * Input: non-negative, not NaN. Returns the byte. */
int oracle_e4m3_from_float(float v) {
    double grid[127];
    e4m3_grid(grid);
    return nearest_even((double)v, grid, 127);
}

/* E2M1 round-to-nearest-even with saturation to 6 (magnitude code 7). Input non-negative, not NaN.
 * Returns the 3-bit magnitude code. */
int oracle_e2m1_from_float(float v) {
    double grid[8];
    e2m1_grid(grid);
    return nearest_even((double)v, grid, 8);
}

static float bf16_to_float(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ------------------------------------------------------------------------------------------------
 * Global scale: g = amax_T / (6 * 448), the decode-direction FP32 scale that maps the tensor's
 * largest magnitude to the top of the E2M1 range (6) times the top of the E4M3 range (448).
 * ---------------------------------------------------------------------------------------------- */
float oracle_tensor_amax(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx) {
    float amax = 0.0f;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(bf16_to_float(x[r * ldx + k]));
            if (a > amax) amax = a;
        }
    return amax;
}

float oracle_global_scale(float amax) {
    float denom = 6.0f * 448.0f; /* 2688, exact */
    return amax / denom;
}

/* ------------------------------------------------------------------------------------------------
 * Quantizer: bf16 [rows, K] -> packed E2M1 codes [rows, K/2] + E4M3 block scales [rows, K/16].
 * Steps per 16-element block along K:
 *   amax_b = max |x|;  t = RN32(6 g);  s_raw = RN32(amax_b / t);  s = E4M3_RNE_SAT(s_raw);
 *   if s == 0: magnitudes 0; else S = RN32(s g), v = RN32(|x| / S), mag = E2M1_RNE_SAT(v);
 *   code = sign(x) * 8 + mag.
 * Returns 0, or -1 if K is not a multiple of 16.
 * ---------------------------------------------------------------------------------------------- */
int oracle_quantize(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, float g,
                    uint8_t* codes, int64_t ldc, uint8_t* scales, int64_t lds) {
    if (K % 16 != 0) return -1;
    double g4[127], g2[8];
    e4m3_grid(g4);
    e2m1_grid(g2);
    float t = 6.0f * g;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < K / 16; ++b) {
            float xs[16];
            float amax = 0.0f;
            for (int i = 0; i < 16; ++i) {
                xs[i] = bf16_to_float(x[r * ldx + 16 * b + i]);
                if (fabsf(xs[i]) > amax) amax = fabsf(xs[i]);
            }
            float s_raw = amax / t;
            int sbyte = nearest_even((double)s_raw, g4, 127);
            float s = (float)oracle_e4m3_value(sbyte); /* exact in binary32 */
            int code[16];
            for (int i = 0; i < 16; ++i) {
                int mag = 0;
                if (s != 0.0f) {
                    float S = s * g;
                    float v = fabsf(xs[i]) / S;
                    mag = nearest_even((double)v, g2, 8);
                }
                code[i] = (signbit(xs[i]) ? 8 : 0) | mag;
            }
            for (int j = 0; j < 8; ++j)
                codes[r * ldc + 8 * b + j] = (uint8_t)(code[2 * j] | (code[2 * j + 1] << 4));
            scales[r * lds + b] = (uint8_t)sbyte;
        }
    }
    return 0;
}

/* Dequantized element as an exact integer in units of 2^-10: (2 * e2m1) * (2^9 * e4m3).
 * 2*e2m1 is an integer in [-12, 12]; 2^9 * e4m3 is an integer in [0, 229376]. */
static int64_t deq_units(const uint8_t* codes, const uint8_t* scales, int64_t row, int64_t k,
                         int64_t ldc, int64_t lds) {
    int byte = codes[row * ldc + k / 2];
    int code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
    double v2 = 2.0 * oracle_e2m1_value(code);                       /* exact integer */
    double s512 = ldexp(oracle_e4m3_value(scales[row * lds + k / 16]), 9); /* exact integer */
    return (int64_t)v2 * (int64_t)s512;
}

void oracle_dequantize(const uint8_t* codes, int64_t ldc, const uint8_t* scales, int64_t lds,
                       int64_t rows, int64_t K, float g, double* out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k)
            out[r * K + k] = ldexp((double)deq_units(codes, scales, r, k, ldc, lds), -10) * (double)g;
}

/* ------------------------------------------------------------------------------------------------
 * GEMM: y[m, n] = g_a * g_w[seg(n)] * sum_k a[m,k] w[n,k], with a, w the block-decoded operands
 * (decoded without their global scales). The sum is exact: int64 in units of 2^-20 (each term is
 * below 2^44 in magnitude and K stays far below 2^19). Also returns T[m, n] = g_a * g_w[seg(n)] *
 * sum_k |a w|, the scale of the accumulation-error bound.
 * rows: the list of A rows to evaluate (n_rows of them); outputs are [n_rows, N] row-major.
 * seg_begin: n_segs+1 ascending column boundaries, seg_begin[0] = 0, seg_begin[n_segs] = N.
 * ---------------------------------------------------------------------------------------------- */
int oracle_gemm_rows(const uint8_t* a_codes, const uint8_t* a_scales, int64_t lda_c, int64_t lda_s,
                     float g_a, const uint8_t* w_codes, const uint8_t* w_scales, int64_t ldw_c,
                     int64_t ldw_s, int64_t N, int64_t K, const int64_t* seg_begin,
                     const float* g_w, int n_segs, const int64_t* rows, int64_t n_rows, double* y,
                     double* T) {
    if (K % 16 != 0) return -1;
    int32_t* wq = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N * K));
    if (!wq) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            wq[n * K + k] = (int32_t)deq_units(w_codes, w_scales, n, k, ldw_c, ldw_s);
    int64_t* seg_of = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
    if (!seg_of) { free(wq); return -2; }
    for (int s = 0; s < n_segs; ++s)
        for (int64_t n = seg_begin[s]; n < seg_begin[s + 1]; ++n) seg_of[n] = s;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t m = rows[i];
        int32_t* aq = (int32_t*)malloc(sizeof(int32_t) * (size_t)(K > 0 ? K : 1));
        if (!aq) { err = -2; continue; }
        for (int64_t k = 0; k < K; ++k)
            aq[k] = (int32_t)deq_units(a_codes, a_scales, m, k, lda_c, lda_s);
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0, aacc = 0;
            const int32_t* wr = wq + n * K;
            for (int64_t k = 0; k < K; ++k) {
                int64_t p = (int64_t)aq[k] * (int64_t)wr[k];
                acc += p;
                aacc += p < 0 ? -p : p;
            }
            double scale = (double)g_a * (double)g_w[seg_of[n]];
            y[i * N + n] = ldexp((double)acc, -20) * scale;
            T[i * N + n] = ldexp((double)aacc, -20) * scale;
        }
        free(aq);
    }
    free(seg_of);
    free(wq);
    return err;
}

/* ------------------------------------------------------------------------------------------------
 * Gate epilogues, in double on the GEMM output y (per column j of the gate segment):
 *   beta  = sigmoid(y)                                   (write strength)
 *   alpha = exp(-exp(A_log[j]) * softplus(y + dt_bias[j]))  (decay; the exponent is the gate g_t)
 * softplus(z) = max(z, 0) + log1p(exp(-|z|)).
 * ---------------------------------------------------------------------------------------------- */
double oracle_sigmoid(double y) { return 1.0 / (1.0 + exp(-y)); }

double oracle_softplus(double z) { return (z > 0.0 ? z : 0.0) + log1p(exp(-fabs(z))); }

double oracle_gdn_decay(double y, double a_log, double dt_bias) {
    return exp(-exp(a_log) * oracle_softplus(y + dt_bias));
}

void oracle_sigmoid_array(const double* y, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_sigmoid(y[i]);
}

/* y is [rows, ncols]; A_log and dt_bias are per column. */
void oracle_gdn_decay_array(const double* y, int64_t rows, int64_t ncols, const float* a_log,
                            const float* dt_bias, double* out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < ncols; ++j)
            out[r * ncols + j] = oracle_gdn_decay(y[r * ncols + j], a_log[j], dt_bias[j]);
}

/* Element-wise helpers exposed for the format pins. */
void oracle_e4m3_from_float_array(const float* v, int64_t n, uint8_t* out) {
    double grid[127];
    e4m3_grid(grid);
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)nearest_even((double)v[i], grid, 127);
}

void oracle_e2m1_from_float_array(const float* v, int64_t n, uint8_t* out) {
    double grid[8];
    e2m1_grid(grid);
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)nearest_even((double)v[i], grid, 8);
}

/* ------------------------------------------------------------------------------------------------
 * Serving-path companions
 * ---------------------------------------------------------------------------------------------- */

/* bf16 round-to-nearest-even of a binary32 value (NaN -> canonical quiet NaN 0x7FC0). */
static uint16_t bf16_from_float(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* E4M3FN byte of a finite binary32 value: sign bit kept, magnitude rounded to nearest-even with
 * saturation at 448. NaN -> 0x7F. */
static int e4m3_signed(float v, const double* grid) {
    if (isnan(v)) return 0x7F;
    int mag = nearest_even(fabs((double)v), grid, 127);
    return (signbit(v) ? 0x80 : 0) | mag;
}

/* FP8 KV-cache scale, static per tensor, from a calibration amax: s = RN32(amax / 448), so that the
 * largest calibrated magnitude maps to the top of the E4M3 range. */
float oracle_kv_scale(float amax) { return amax / 448.0f; }

/* FP8 KV-cache quantize: q = E4M3_RNE_SAT(RN32(x / s)) per element, x bf16 [rows, cols] with row
 * stride ldx, q bytes with row stride ldq. Infinite inputs saturate to +-448, NaN gives 0x7F. */
void oracle_kv_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, float s, uint8_t* q,
                        int64_t ldq) {
    double grid[127];
    e4m3_grid(grid);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float t = bf16_to_float(x[r * ldx + c]) / s;
            q[r * ldq + c] = (uint8_t)e4m3_signed(t, grid);
        }
}

/* FP8 KV-cache dequantize: y = bf16_RNE(RN32(e4m3(q) * s)); NaN codes give NaN. */
void oracle_kv_dequantize(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, float s, uint16_t* y,
                          int64_t ldy) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float v = (float)oracle_e4m3_value(q[r * ldq + c]); /* exact in binary32 (or NaN) */
            y[r * ldy + c] = bf16_from_float(v * s);
        }
}

/* Fold-in repair of a fused group (pages' own repair of the global-scale mismatch): the group is
 * rewritten to one common global scale G and each module's ratio r = g / G is folded into its block
 * scales: s' = E4M3_RNE_SAT(RN32(s * r)), codes unchanged. With G the group maximum (a reading: the
 * pages do not say which common scale), r <= 1 and no folded scale can overflow 448. */
float oracle_fold_common_scale(const float* g, int n) {
    float G = 0.0f;
    for (int i = 0; i < n; ++i)
        if (g[i] > G) G = g[i];
    return G;
}

float oracle_fold_ratio(float g, float G) { return g / G; }

/* In place over a [rows, nblocks] scale array with row stride lds. The sign bit of a byte is kept
 * and NaN bytes stay 0x7F. */
void oracle_fold_scales(uint8_t* scales, int64_t rows, int64_t nblocks, int64_t lds, float ratio) {
    double grid[127];
    e4m3_grid(grid);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nblocks; ++b) {
            int byte = scales[r * lds + b];
            double v = oracle_e4m3_value(byte);
            if (isnan(v)) {
                scales[r * lds + b] = 0x7F;
                continue;
            }
            float t = (float)fabs(v) * ratio; /* RN32 */
            scales[r * lds + b] = (uint8_t)((byte & 0x80) | nearest_even((double)t, grid, 127));
        }
}

/* RMSNorm ahead of the quantizer, norm in BF16 (the pages keep normalization layers in BF16):
 *   ms = (sum_k x_k^2) / K in double;  r = RN32(1 / sqrt(ms + eps)) (double, then one rounding);
 *   y1_k = bf16_RNE(RN32(x_k * r));   y_k = bf16_RNE(y1_k * w_k)   (the product is exact in binary32).
 * The two BF16 roundings follow the usual BF16 RMSNorm (normalize in FP32, round, scale by the
 * weight); the pages do not spell the formula out. Also returns r per row. */
void oracle_rmsnorm(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, const uint16_t* w, float eps,
                    uint16_t* y, int64_t ldy, float* r_out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = (double)bf16_to_float(x[i * ldx + k]);
            ss += v * v;
        }
        double ms = ss / (double)K;
        float r = (float)(1.0 / sqrt(ms + (double)eps));
        if (r_out) r_out[i] = r;
        for (int64_t k = 0; k < K; ++k) {
            float y1 = bf16_to_float(bf16_from_float(bf16_to_float(x[i * ldx + k]) * r));
            y[i * ldy + k] = bf16_from_float(y1 * bf16_to_float(w[k]));
        }
    }
}

/* Gated DeltaNet recurrence fed by the gates (Japanese article, "How Gated DeltaNet works"): per
 * sequence b and value head h, with key head hk = h / (Hv / Hk) and state S [D (key), D (value)],
 *   S_t = alpha_t S_{t-1} + beta_t k_t (v_t - S_{t-1}^T k_t)^T,     o_t = S_t^T q_t,
 * exactly the pages' update (its erase term carries no alpha); the readout o_t = S_t^T q_t is the
 * usual linear-attention readout (the pages do not write it). Rows are tokens, row r = b * T + t;
 * q, k: bf16 [B*T, Hk*D] (strides ldq, ldk); v: bf16 [B*T, Hv*D] (ldv); alpha, beta: float
 * [B*T, Hv] (lda, ldb); S0: double [B, Hv, D, D] (NULL = zeros); outputs o: double [B*T, Hv*D]
 * (dense) and S_T: double [B, Hv, D, D]. Everything in double. */
void oracle_gdn_recurrence(const uint16_t* q, int64_t ldq, const uint16_t* k, int64_t ldk, const uint16_t* v,
                           int64_t ldv, const float* alpha, int64_t lda, const float* beta, int64_t ldb,
                           const double* S0, int64_t B, int64_t T, int64_t Hv, int64_t Hk, int64_t D, double* o,
                           double* S_out) {
    const int64_t group = Hv / Hk;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hv; ++h) {
            const int64_t hk = h / group;
            double* S = S_out + (b * Hv + h) * D * D;
            for (int64_t i = 0; i < D * D; ++i) S[i] = S0 ? S0[(b * Hv + h) * D * D + i] : 0.0;
            double* kt = (double*)malloc(sizeof(double) * (size_t)D);
            double* qt = (double*)malloc(sizeof(double) * (size_t)D);
            double* u = (double*)malloc(sizeof(double) * (size_t)D);
            for (int64_t t = 0; t < T; ++t) {
                const int64_t r = b * T + t;
                for (int64_t i = 0; i < D; ++i) {
                    kt[i] = bf16_to_float(k[r * ldk + hk * D + i]);
                    qt[i] = bf16_to_float(q[r * ldq + hk * D + i]);
                }
                const double a = alpha[r * lda + h], be = beta[r * ldb + h];
                for (int64_t j = 0; j < D; ++j) { /* u = v - S^T k, with the old S */
                    double sk = 0.0;
                    for (int64_t i = 0; i < D; ++i) sk += S[i * D + j] * kt[i];
                    u[j] = (double)bf16_to_float(v[r * ldv + h * D + j]) - sk;
                }
                for (int64_t i = 0; i < D; ++i)
                    for (int64_t j = 0; j < D; ++j) S[i * D + j] = a * S[i * D + j] + be * kt[i] * u[j];
                for (int64_t j = 0; j < D; ++j) {
                    double oq = 0.0;
                    for (int64_t i = 0; i < D; ++i) oq += S[i * D + j] * qt[i];
                    o[r * Hv * D + h * D + j] = oq;
                }
            }
            free(kt);
            free(qt);
            free(u);
        }
}

/* The same recurrence in binary32 with the natural order (sequential sums), used only to size the
 * rounding error of an FP32 implementation on a given input. */
void oracle_gdn_recurrence_f32(const uint16_t* q, int64_t ldq, const uint16_t* k, int64_t ldk, const uint16_t* v,
                               int64_t ldv, const float* alpha, int64_t lda, const float* beta, int64_t ldb,
                               const float* S0, int64_t B, int64_t T, int64_t Hv, int64_t Hk, int64_t D, float* o,
                               float* S_out) {
    const int64_t group = Hv / Hk;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hv; ++h) {
            const int64_t hk = h / group;
            float* S = S_out + (b * Hv + h) * D * D;
            for (int64_t i = 0; i < D * D; ++i) S[i] = S0 ? S0[(b * Hv + h) * D * D + i] : 0.0f;
            float* u = (float*)malloc(sizeof(float) * (size_t)D);
            for (int64_t t = 0; t < T; ++t) {
                const int64_t r = b * T + t;
                const float a = alpha[r * lda + h], be = beta[r * ldb + h];
                for (int64_t j = 0; j < D; ++j) {
                    float sk = 0.0f;
                    for (int64_t i = 0; i < D; ++i) sk += S[i * D + j] * bf16_to_float(k[r * ldk + hk * D + i]);
                    u[j] = bf16_to_float(v[r * ldv + h * D + j]) - sk;
                }
                for (int64_t i = 0; i < D; ++i) {
                    const float ki = bf16_to_float(k[r * ldk + hk * D + i]);
                    for (int64_t j = 0; j < D; ++j) S[i * D + j] = a * S[i * D + j] + be * ki * u[j];
                }
                for (int64_t j = 0; j < D; ++j) {
                    float oq = 0.0f;
                    for (int64_t i = 0; i < D; ++i) oq += S[i * D + j] * bf16_to_float(q[r * ldq + hk * D + i]);
                    o[r * Hv * D + h * D + j] = oq;
                }
            }
            free(u);
        }
}

/* Number of threads the OpenMP row loops use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the number of threads later OpenMP row loops use (n >= 1; ignored without OpenMP). Only the
 * CPU-baseline timing uses it, to time the oracle single-threaded as well. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
