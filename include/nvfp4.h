/*
 * nvfp4.h -- C interface of the MI355X (gfx950) NVFP4 W4A4 quantized-linear library (libnvfp4.so).
 *
 * The library implements the data-parallel hot path of an all-linear-layers NVFP4 W4A4 recipe
 * (paper arXiv:2609.04098, "Why Gated DeltaNet Survives 4-Bit Quantization"):
 *
 *   1. online activation quantization to NVFP4: E2M1 4-bit elements, one E4M3 scale per 16
 *      consecutive elements along K chosen from the block maximum, and one FP32 global scale per
 *      linear module (Japanese article, "Mechanism 1" and FAQ "What is NVFP4?"; English abstract,
 *      point (i));
 *   2. the block-scaled W4A4 GEMM Y = X W^T with FP32 accumulation, where one GEMM may serve several
 *      separately calibrated modules fused along N, each output-column segment applying its own
 *      global scale after accumulation -- the repair of the fused-module global-scale mismatch
 *      (Japanese article, "Trap 1"; English abstract; aimodeling.com English translation, "What
 *      engineers should actually take away"), with an optional Gated DeltaNet gate epilogue
 *      (Japanese article, "Mechanism 2").
 *
 * It also carries the companions of that layer on the same serving path: the FP8 E4M3 KV-cache
 * codec with static scales, the pages' own fold-in repair of the scale mismatch, BF16 RMSNorm
 * fused with the quantizer, and the Gated DeltaNet recurrence fed by the gates (declared at the end
 * of this file).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers; `stream` is a hipStream_t passed as void* (NULL means
 *    the null stream). Work is enqueued on `stream` and the call returns without synchronizing.
 *  - The caller owns every buffer. The library never allocates, frees or synchronizes device
 *    memory. Device buffers must stay valid until the stream has executed the work.
 *  - Host arrays (segment tables, scale vectors) are read only during the call.
 *  - Argument errors are returned synchronously before anything is enqueued; a failed launch
 *    returns NVFP4_ERR_HIP. nvfp4_last_error() then gives a thread-local description.
 *  - Results are bitwise deterministic for identical inputs and shapes (no floating-point atomics).
 *  - No exceptions cross this interface. Calls from several host threads are safe.
 *
 * Data layouts (row-major; all strides are in ELEMENTS of the buffer's own type, i.e. bytes for the
 * uint8 code/scale buffers)
 *  - bf16 activations X [rows, K], row stride ldx >= K.
 *  - NVFP4 tensor = codes [rows, K/2] uint8 + scales [rows, K/16] uint8:
 *      codes byte j of a row holds element 2j in bits 0-3 and element 2j+1 in bits 4-7;
 *      a 4-bit code is sign (bit 3) | E2M1 magnitude (bits 2-0) with magnitudes
 *      {0, 0.5, 1, 1.5, 2, 3, 4, 6};
 *      scales byte b of a row is the OCP E4M3FN scale of elements [16b, 16b+16), never negative;
 *      decoded value x ~= e2m1(code) * e4m3(scale) * g, with g the tensor's FP32 global scale.
 *    Weights use the same layout with rows = N (as nn.Linear: W [N, K], Y = X W^T).
 *  - Alignment: every base pointer is 16-byte aligned and every row stride is a multiple of 16
 *    bytes (ldx a multiple of 8 elements; ldc and lds multiples of 16). A buffer of R rows holds
 *    at least R * stride bytes. Violations return NVFP4_ERR_ALIGN; there is no slow fallback.
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL = 1,      /* a required pointer is NULL */
    NVFP4_ERR_SHAPE = 2,     /* negative size, K not a multiple of 16, stride smaller than a row */
    NVFP4_ERR_ALIGN = 3,     /* pointer or stride misaligned (see "Alignment" above) */
    NVFP4_ERR_SEGMENTS = 4,  /* segment table empty, too long, unsorted, overlapping or not covering N */
    NVFP4_ERR_SCALE = 5,     /* a global scale is not finite and > 0 */
    NVFP4_ERR_EPILOGUE = 6,  /* unknown epilogue/out dtype, or a gate without FP32 output/parameters */
    NVFP4_ERR_WORKSPACE = 7, /* workspace smaller than the call's *_workspace_bytes() */
    NVFP4_ERR_HIP = 8        /* the HIP runtime reported an error (launch failure, bad stream) */
} nvfp4_status;

enum { NVFP4_OUT_F32 = 0, NVFP4_OUT_BF16 = 1 };
enum { NVFP4_EPI_NONE = 0, NVFP4_EPI_SIGMOID = 1, NVFP4_EPI_GDN_DECAY = 2 };
enum { NVFP4_MAX_SEGMENTS = 16 };
enum { NVFP4_NOALLOC_SCRATCH_BYTES = 16 << 20 }; /* scratch of nvfp4_gemm_noalloc, per GPU */

/*
 * nvfp4_global_scale -- calibration of a module's FP32 global scale from a bf16 tensor:
 *   g = RN32(amax / 2688), amax = max |x| over the tensor, 2688 = 6 * 448 (largest E2M1 magnitude
 *   times largest E4M3 scale), so that the tensor maximum lands on the top of both grids.
 * The pages fix one global scale per linear module by calibration ("Trap 1", "Experiment design");
 * the synthetic workloads take it from the tensor itself. Writes one float to the device pointer
 * g_out (which the call also uses as its reduction accumulator). rows == 0 or K == 0 gives g = 0.
 * x: device bf16 [rows, K], stride ldx (elements). Errors: NULL, SHAPE, ALIGN, HIP.
 */
nvfp4_status nvfp4_global_scale(const void* x_bf16, int64_t rows, int64_t K, int64_t ldx,
                                float* g_out, void* stream);

/*
 * nvfp4_quantize -- NVFP4 quantization of bf16 rows (activations online; weights offline).
 * For every 16-element block along K, with RN32 = one IEEE binary32 operation rounded to nearest
 * even:
 *   amax_b = max |x|;  s = E4M3_RNE_SAT(RN32(amax_b / RN32(6 g)))  (saturating at 448);
 *   if s == 0 every magnitude is 0, else  code = signbit(x) * 8 + E2M1_RNE_SAT(RN32(|x| / RN32(s g)))
 *   (E2M1 saturating at 6; ties to the even code; -0.0 and values rounding to zero keep their sign).
 * Block scaling per the Japanese article, "Mechanism 1"; one FP32 global scale g per module per
 * "Trap 1" and the English abstract.
 *   x_bf16: device bf16 [rows, K], stride ldx elements;  g: host float, finite and > 0;
 *   codes: device uint8 [rows, K/2], stride ldc bytes;  scales: device uint8 [rows, K/16], stride lds.
 * K must be a multiple of 16. rows == 0 or K == 0 is a no-op.
 * Errors: NULL, SHAPE, ALIGN, SCALE, HIP.
 */
nvfp4_status nvfp4_quantize(const void* x_bf16, int64_t rows, int64_t K, int64_t ldx, float g,
                            uint8_t* codes, int64_t ldc, uint8_t* scales, int64_t lds,
                            void* stream);

/*
 * One output-column segment of a (possibly fused) GEMM: columns [n_begin, n_begin + n_len) of W,
 * i.e. one separately calibrated linear module ("Trap 1": the fused in_proj_qkv+z and in_proj_b+a
 * GEMMs). The segment writes its own output matrix out [M, n_len] with row stride ldo (elements):
 *   y[m, j] = g_a * g_w[s] * sum_k a[m, k] w[n_begin + j, k]    (accumulated in FP32)
 *   epilogue NONE:      out = y                     (out_dtype F32, or BF16 rounded to nearest even)
 *   epilogue SIGMOID:   out = 1 / (1 + exp(-y))     (write strength beta; out_dtype must be F32)
 *   epilogue GDN_DECAY: out = exp(-exp(A_log[j]) * softplus(y + dt_bias[j]))
 *                       (decay alpha; out_dtype must be F32; A_log, dt_bias: device float [n_len])
 * Gates follow the Gated DeltaNet parameterization of the Japanese article, "Mechanism 2"; their
 * outputs are FP32 because a decay close to 1 is not representable in bf16.
 * Several segments may share one output buffer by pointing `out` at column n_begin of it.
 */
typedef struct {
    int64_t n_begin;
    int64_t n_len;
    int32_t epilogue;   /* NVFP4_EPI_* */
    int32_t out_dtype;  /* NVFP4_OUT_* */
    void* out;          /* device, [M, n_len], stride ldo elements; 16-byte aligned, ldo*size%16==0 */
    int64_t ldo;
    const float* A_log;   /* GDN_DECAY only, else ignored */
    const float* dt_bias; /* GDN_DECAY only, else ignored */
} nvfp4_segment;

/*
 * nvfp4_gemm -- block-scaled W4A4 GEMM with a per-segment global-scale epilogue.
 *   a_codes/a_scales: device NVFP4 activations [M, K] (strides lda_c, lda_s bytes), global scale g_a;
 *   w_codes/w_scales: device NVFP4 weights [N, K] (strides ldw_c, ldw_s bytes);
 *   every row stride is below 2^23 bytes (so K < 2^24 for dense codes), else SHAPE;
 *   M and N at most 2^31, and for M > 64 at most 2^30 output tiles of 256 x 256, else SHAPE;
 *   segs[n_segs]: host array, sorted by n_begin, contiguous, non-overlapping, covering [0, N),
 *                 every n_len > 0, 1 <= n_segs <= NVFP4_MAX_SEGMENTS;
 *   g_w[n_segs]: host array, the weight global scale of each segment (finite, > 0); each
 *                product RN32(g_a * g_w[s]) must be a normal positive float, else SCALE.
 * The product of the decoded operands is accumulated in FP32 from exact FP16 products (an E2M1
 * value times an E4M3 scale is exact in FP16), then scaled once by RN32(g_a * g_w[s]).
 * M == 0 or N == 0 is a no-op; K == 0 writes the epilogue of y = 0.
 * workspace: device scratch of at least nvfp4_gemm_workspace_bytes(M, N, K) bytes, 16-byte aligned
 * (may be NULL when that is 0; it is not when 32 < M <= 64 and K is long enough to be split over
 * workgroups, where the decode kernel's partial sums live there). Owned by the caller; its contents
 * on entry do not matter, and calls that share one workspace must be ordered on one stream.
 * Errors: NULL, SHAPE, ALIGN, SEGMENTS, SCALE, EPILOGUE, WORKSPACE, HIP.
 */
nvfp4_status nvfp4_gemm(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales,
                        int64_t lda_s, float g_a, const uint8_t* w_codes, int64_t ldw_c,
                        const uint8_t* w_scales, int64_t ldw_s, int64_t M, int64_t N, int64_t K,
                        const nvfp4_segment* segs, const float* g_w, int32_t n_segs,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace nvfp4_gemm needs for this shape (0 when none). For 32 < M <= 64 with
 * n = ceil(K / 256) chunks: s0 = min(8, max(1, n / 11)), p = ceil(n / s0) rounded up to even,
 * splits = ceil(n / p); the size is splits * N * 64 * 4 when splits > 1, else 0. */
size_t nvfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * nvfp4_gemm_noalloc -- nvfp4_gemm for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments (without the
 * workspace), same kernels and bitwise the same results as nvfp4_gemm. The call allocates nothing:
 * where nvfp4_gemm would use the caller's workspace (the decode kernel's split-K partial sums,
 * 32 < M <= 64 with K split), it uses a static device array of NVFP4_NOALLOC_SCRATCH_BYTES (16 MiB)
 * that the library holds on every GPU it runs on until the process ends. A shape whose
 * nvfp4_gemm_workspace_bytes() exceeds that returns NVFP4_ERR_WORKSPACE before anything is enqueued.
 * Every call on one GPU shares that GPU's array (its contents carry over between calls and need no
 * clearing: each call writes every partial sum it reads), so calls that may overlap on one GPU --
 * different streams, or host threads not ordered on one stream -- race and must be serialized by
 * the caller. Errors: as nvfp4_gemm.
 */
nvfp4_status nvfp4_gemm_noalloc(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales,
                                int64_t lda_s, float g_a, const uint8_t* w_codes, int64_t ldw_c,
                                const uint8_t* w_scales, int64_t ldw_s, int64_t M, int64_t N, int64_t K,
                                const nvfp4_segment* segs, const float* g_w, int32_t n_segs, void* stream);

/*
 * Decode weight layout -- NVFP4 weights repacked once, offline, for the decode GEMMs (M <= 64), where
 * the weights are nearly all of the traffic (Japanese article, "Running 27B at home": decode is
 * weight streaming). With T = ceil(N / 16) tiles of 16 rows and C = ceil(K / 256) chunks of 256
 * elements, tile t and chunk c hold:
 *   codes  at (t C + c) * 2048: piece h = 0, 1 of 1024 bytes; within a piece, 16 bytes per lane
 *          l = r + 16 g (r < 16, g < 4): code bytes 64 h + 16 g .. + 15 of chunk c of row 16 t + r;
 *   scales at T C 2048 + (t C + c) * 256: 4 bytes per lane l: the E4M3 scale bytes of blocks
 *          2g, 2g + 1, 8 + 2g, 9 + 2g of chunk c of row 16 t + r.
 * Codes and scales are those of the row-major weights, moved; rows past N and bytes past K are zero.
 * In this order each load of the decode kernels is one contiguous run and needs no lane exchange.
 */

/* Bytes of the decode layout of N x K weights: T * C * 2304 (0 when N <= 0, K <= 0 or K % 16 != 0). */
size_t nvfp4_packed_weight_bytes(int64_t N, int64_t K);

/*
 * nvfp4_pack_weights -- write the decode layout of row-major NVFP4 weights (codes [N, K/2] stride
 * ldw_c, scales [N, K/16] stride ldw_s, as for nvfp4_gemm) into packed: a device buffer of
 * nvfp4_packed_weight_bytes(N, K) bytes, 16-byte aligned, owned by the caller. N == 0 or K == 0 is a
 * no-op. Errors: NULL, SHAPE, ALIGN, HIP.
 */
nvfp4_status nvfp4_pack_weights(const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s,
                                int64_t N, int64_t K, uint8_t* packed, void* stream);

/*
 * nvfp4_gemm_packed -- nvfp4_gemm for 1 <= M <= 64 activation rows with weights in the decode layout
 * (w_packed from nvfp4_pack_weights for the same N and K). Same activations, segments, global scales,
 * epilogues and workspace (nvfp4_gemm_workspace_bytes) as nvfp4_gemm; for 2 <= M <= 64 the results
 * are bitwise those of nvfp4_gemm with the row-major weights (same kernels, same order of every sum).
 * At M = 1 nvfp4_gemm streams whole row-major rows and is the faster of the two.
 * M > 64: NVFP4_ERR_SHAPE (the prefill kernel reads row-major weights). Errors: as nvfp4_gemm.
 */
nvfp4_status nvfp4_gemm_packed(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s,
                               float g_a, const uint8_t* w_packed, int64_t M, int64_t N, int64_t K,
                               const nvfp4_segment* segs, const float* g_w, int32_t n_segs, void* workspace,
                               size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Companions on the same serving path
 * --------------------------------------------------------------------------------------------- */

/*
 * nvfp4_kv_scale -- static per-tensor FP8 KV-cache scale from a calibration tensor:
 *   s = RN32(amax / 448), amax = max |x|, so that the calibrated maximum lands on the largest E4M3
 *   value. The pages calibrate such scales offline and ship them with the checkpoint, one per K and
 *   V tensor of each attention layer (Japanese article, "Is FP8 enough for the KV cache? The 'ship
 *   KV scales' recipe"). Writes one float to the device pointer s_out (also used as the reduction
 *   accumulator). x: device bf16 [rows, cols], stride ldx elements. Errors: NULL, SHAPE, ALIGN, HIP.
 */
nvfp4_status nvfp4_kv_scale(const void* x_bf16, int64_t rows, int64_t cols, int64_t ldx, float* s_out,
                            void* stream);

/*
 * nvfp4_kv_quantize -- FP8 E4M3FN KV-cache quantization with a static scale (same passage):
 *   q = E4M3_RNE_SAT(RN32(x / s)) per element: round to nearest even, saturating at +-448 (also
 *   for infinities), sign kept (-0.0 and values rounding to zero give 0x80), NaN -> 0x7F.
 *   x_bf16: device bf16 [rows, cols], stride ldx elements, 16-byte aligned, ldx % 8 == 0;
 *   q: device uint8 [rows, cols], stride ldq bytes, 16-byte aligned, ldq % 16 == 0;
 *   s: host float, finite and > 0. cols must be a multiple of 16. rows == 0 or cols == 0: no-op.
 * Errors: NULL, SHAPE, ALIGN, SCALE, HIP.
 */
nvfp4_status nvfp4_kv_quantize(const void* x_bf16, int64_t rows, int64_t cols, int64_t ldx, float s,
                               uint8_t* q, int64_t ldq, void* stream);

/*
 * nvfp4_kv_dequantize -- FP8 E4M3FN KV-cache dequantization with the same static scale:
 *   y = bf16_RNE(RN32(e4m3(q) * s)); NaN codes (0x7F, 0xFF) give the bf16 NaN 0x7FC0.
 *   q: device uint8 [rows, cols], stride ldq bytes (16-byte aligned, ldq % 16 == 0);
 *   y_bf16: device bf16 [rows, cols], stride ldy elements (16-byte aligned, ldy % 8 == 0).
 * cols must be a multiple of 16. Errors: NULL, SHAPE, ALIGN, SCALE, HIP.
 */
nvfp4_status nvfp4_kv_dequantize(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, float s,
                                 void* y_bf16, int64_t ldy, void* stream);

/*
 * nvfp4_fold_scales -- the fold-in step of the pages' own repair of the fused-module scale mismatch
 * (Japanese article, "Trap 1": the fused group is rewritten to one common global scale and each
 * module's ratio is folded into its block scales, with a re-rounding error of at most 6.2%). In
 * place over E4M3 scale bytes [rows, nblocks] (stride lds bytes):
 *   s' = sign(s) | E4M3_RNE_SAT(RN32(|e4m3(s)| * ratio)); NaN bytes become 0x7F.
 * For 0 < ratio <= 1 the relative re-rounding error is at most 2^-4 in the E4M3 normal range.
 * ratio: host float, finite and > 0. Errors: NULL, SHAPE, SCALE, HIP.
 */
nvfp4_status nvfp4_fold_scales(uint8_t* scales, int64_t rows, int64_t nblocks, int64_t lds, float ratio,
                               void* stream);

/*
 * nvfp4_fold_group -- the whole fold-in repair of one fused weight tensor W [N, K] made of n_segs
 * modules stacked along N (seg_rows[s] rows each, host array), with per-module global scales g_w
 * (host array, finite, > 0): G = max_s g_w[s] (a reading: the pages do not name the common scale;
 * the maximum keeps every ratio <= 1, so no folded scale overflows), r_s = RN32(g_w[s] / G), and
 * nvfp4_fold_scales of module s's rows with r_s. Writes G to the host pointer g_common. Afterwards
 * the group runs as one GEMM segment with global scale G (codes are unchanged).
 *   w_scales: device uint8 [N, K/16], stride ldw_s bytes; K a multiple of 16.
 * Every argument (including each ratio, which must not underflow to 0) is validated before
 * anything is written or enqueued, so an error leaves the scales and *g_common untouched.
 * Errors: NULL, SHAPE, SEGMENTS, SCALE, HIP.
 */
nvfp4_status nvfp4_fold_group(uint8_t* w_scales, int64_t ldw_s, int64_t K, const int64_t* seg_rows,
                              const float* g_w, int32_t n_segs, float* g_common, void* stream);

/*
 * nvfp4_rmsnorm_quantize -- BF16 RMSNorm fused with the NVFP4 quantizer of its output, so the
 * normalized activations never go through HBM. The pages keep normalization layers in BF16
 * (Japanese article, "Minima, quantized 'all 4-bit': the experiment design"); the formula below is
 * the usual BF16 RMSNorm, which the pages do not spell out. Per row:
 *   ms = (sum_k x_k^2) / K in double;  r = RN32(1 / sqrt(ms + eps)) (double, then one rounding);
 *   y_k = bf16_RNE(bf16_RNE(RN32(x_k * r)) * w_k);   then y is quantized as by nvfp4_quantize.
 *   x_bf16: device bf16 [rows, K], stride ldx;  w_bf16: device bf16 [K] (16-byte aligned);
 *   eps: host float >= 0;  g: host float global scale of the consuming module (finite, > 0);
 *   codes/scales: as nvfp4_quantize;  y_bf16: optional device bf16 [rows, K] (stride ldy) that also
 *   receives y, or NULL.
 * K must be a multiple of 16. Errors: NULL, SHAPE, ALIGN, SCALE, HIP.
 */
nvfp4_status nvfp4_rmsnorm_quantize(const void* x_bf16, int64_t rows, int64_t K, int64_t ldx,
                                    const void* w_bf16, float eps, float g, uint8_t* codes, int64_t ldc,
                                    uint8_t* scales, int64_t lds, void* y_bf16, int64_t ldy,
                                    void* stream);

/* Static English name of a status code (any int: values that are no nvfp4_status give
 * "unknown status"). */
const char* nvfp4_status_string(int status);

/* Thread-local description of the last non-OK status returned on this thread ("" if none). */
const char* nvfp4_last_error(void);

/*
 * nvfp4_gdn_recurrence -- the Gated DeltaNet delta-rule recurrence that consumes the gates of the
 * fused in_proj GEMM (Japanese article, "How Gated DeltaNet works"; gates per "Mechanism 2"), in
 * FP32 as in the pages' "FP32 lockstep" experiment ("Mechanism 3"). For each sequence b, value head
 * h (key head h / (Hv / Hk)) and token t, with S the [D, D] state (key rows, value columns):
 *   S_t = alpha_t S_{t-1} + beta_t k_t (v_t - S_{t-1}^T k_t)^T,     o_t = S_t^T q_t
 * (the update exactly as the pages write it; the readout is the usual linear-attention readout).
 *   q_bf16, k_bf16: device bf16 [B*T, Hk*D], row r = b*T + t, strides ldq, ldk (elements), bases
 *                   16-byte aligned, strides multiples of 8 elements (the GEMM's q and k segments);
 *   v_bf16: device bf16 [B*T, Hv*D], stride ldv (the v segment); ldq, ldk, ldv, ldo below 2^23;
 *   alpha, beta: device float [B*T, Hv], strides lda, ldb (the decay and write-strength gates, as the
 *                GEMM's GDN_DECAY and SIGMOID epilogues write them);
 *   state: device float [B, Hv, D, D] holding each head's S value-major, i.e. S^T:
 *          state[b][h][j][i] = S[i][j] (i key, j value), 16-byte aligned; read as S_0 and
 *          overwritten with S_T;
 *   o: device float [B*T, Hv*D], stride ldo;
 *   workspace: device scratch of at least nvfp4_gdn_workspace_bytes(B, T, Hv, Hk, D) bytes, 16-byte
 *              aligned (may be NULL when that is 0); its contents on entry do not matter.
 * D must be 128; Hv must be a multiple of Hk. B == 0 or T == 0 is a no-op (state unchanged).
 * Calls of 32 tokens or more take the chunked form of the same recurrence (the update unrolled
 * exactly over 64-token chunks: within a chunk the deltas v_t - S_{t-1}^T k_t solve a unit
 * lower-triangular system and the state advances once per chunk); shorter calls go token by token.
 * Both compute in FP32 and differ only in rounding order; a call split at multiples of 64 tokens
 * gives the same bits as the whole call.
 * Tokens are processed in order; sequences and heads in parallel. Deterministic.
 * Errors: NULL, SHAPE, ALIGN, WORKSPACE, HIP.
 */
nvfp4_status nvfp4_gdn_recurrence(const void* q_bf16, int64_t ldq, const void* k_bf16, int64_t ldk,
                                  const void* v_bf16, int64_t ldv, const float* alpha, int64_t lda,
                                  const float* beta, int64_t ldb, float* state, int64_t B, int64_t T,
                                  int32_t Hv, int32_t Hk, int32_t D, float* o, int64_t ldo, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Bytes of device workspace nvfp4_gdn_recurrence needs for this call (0 when none: token-by-token
 * calls, or an invalid shape). */
size_t nvfp4_gdn_workspace_bytes(int64_t B, int64_t T, int32_t Hv, int32_t Hk, int32_t D);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H_ */
