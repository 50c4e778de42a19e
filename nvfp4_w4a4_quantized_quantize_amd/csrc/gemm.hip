// Block-scaled W4A4 GEMM with a per-segment global-scale epilogue, for gfx950 (CDNA4).
//
//   y[m, n] = g_a * g_w[seg(n)] * sum_k e2m1(qa[m,k]) sa[m,k/16] * e2m1(qw[n,k]) sw[n,k/16]
//
// The fused-module case (several separately calibrated projections in one GEMM, each output-column
// segment with its own global scale) is the repair of the global-scale mismatch of the paper
// arXiv:2609.04098 (Japanese article, "Trap 1"; English abstract); the optional gate epilogues are
// the Gated DeltaNet parameterization of "Mechanism 2".
//
// Design (a dense contraction, so it runs on the matrix cores):
//  * An E2M1 value times an E4M3 scale has at most 6 significant bits and lies in [2^-10, 2688], so
//    it is exact in FP16; FP16 x FP16 products are exact in FP32. The kernel dequantizes both
//    operands to FP16 in registers and issues v_mfma_f32_32x32x16_f16 with FP32 accumulation.
//    (The FP4 matrix instructions take power-of-two E8M0 scales per 32 elements, which cannot
//    express an E4M3 scale per 16 elements exactly.)
//  * The dequantization is two VALU instructions per pair of elements: the gfx950 FP4->FP16
//    conversion (its scale operand only contributes a power of two, so it runs with 1.0) and a
//    packed FP16 multiply by the block scale.
//  * Workgroup tile 256 x 256, K chunk 128, 4 waves as 2 x 2, each wave 128 x 128 = 4 x 4 MFMA tiles
//    of 32 x 32 accumulated in 256 registers. Codes (4 bits) and FP16 block scales are staged in LDS
//    (double buffered, 100 KB), so LDS traffic stays at 4.5 bits per element; each wave dequantizes
//    its own operand fragments.
//  * K order inside a 64-element half chunk is permuted identically for A and W (lane half h of the
//    MFMA takes elements [32h + 8j, 32h + 8j + 8) at step j), so each lane reads its 32 codes with one
//    16-byte LDS read; a sum does not depend on the order of its terms.
#include "internal.h"

namespace nvfp4 {
namespace {

typedef _Float16 half_t;
typedef half_t half2_t __attribute__((ext_vector_type(2)));
typedef half_t half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int NTHREADS = 256;
constexpr int CODE_STRIDE = 80;   // LDS bytes per tile row of codes: 64 used, padded against bank conflicts
constexpr int SCALE_STRIDE = 20;  // LDS bytes per tile row of FP16 scales: 16 used
constexpr int A_CODES = 0;
constexpr int A_SCALES = A_CODES + BM * CODE_STRIDE;
constexpr int B_CODES = A_SCALES + BM * SCALE_STRIDE;
constexpr int B_SCALES = B_CODES + BN * CODE_STRIDE;
constexpr int STAGE_BYTES = B_SCALES + BN * SCALE_STRIDE;

// Global -> register staging of one K chunk for one operand (rows = 256).
struct Staged {
    uint4 codes[4];   // pieces p = tid + 256 i: row p / 4, 16-byte piece p % 4 of the row's 64 bytes
    uint2 scales;     // row tid: the 8 scale bytes of the chunk
};

__device__ __forceinline__ void load_chunk(Staged& st, const uint8_t* __restrict__ codes, int64_t ldc,
                                           const uint8_t* __restrict__ scales, int64_t lds,
                                           int64_t row0, int64_t nrows, int64_t k0, int64_t K, int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = tid + NTHREADS * i;
        const int r = p >> 2, q = p & 3;
        const int64_t gr = row0 + r;
        const int64_t e0 = k0 + 32 * q;  // first element of this piece
        uint4 v = make_uint4(0, 0, 0, 0);
        if (gr < nrows) {
            const uint8_t* src = codes + gr * ldc + (e0 >> 1);
            if (e0 + 32 <= K) {
                v = *reinterpret_cast<const uint4*>(src);
            } else if (e0 + 16 <= K) {
                const uint2 h = *reinterpret_cast<const uint2*>(src);
                v = make_uint4(h.x, h.y, 0, 0);
            }
        }
        st.codes[i] = v;
    }
    {
        const int64_t gr = row0 + tid;
        uint2 s = make_uint2(0, 0);
        if (gr < nrows) {
            const uint8_t* src = scales + gr * lds + (k0 >> 4);
            const int64_t nvalid = (K - k0) >> 4;  // blocks of this chunk inside K
            if (nvalid >= 8) {
                s = *reinterpret_cast<const uint2*>(src);
            } else {
                uint32_t b[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                for (int j = 0; j < 8; ++j)
                    if (j < nvalid) b[j] = src[j];
                s = make_uint2(b[0] | b[1] << 8 | b[2] << 16 | b[3] << 24, b[4] | b[5] << 8 | b[6] << 16 | b[7] << 24);
            }
        }
        st.scales = s;
    }
}

__device__ __forceinline__ uint32_t e4m3_pair_to_f16x2(uint32_t lo_byte, uint32_t hi_byte) {
    const half_t lo = (half_t)__builtin_amdgcn_cvt_f32_fp8((int)lo_byte, 0);
    const half_t hi = (half_t)__builtin_amdgcn_cvt_f32_fp8((int)hi_byte, 0);
    half2_t h = {lo, hi};
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ void store_chunk(uint8_t* stage, int codes_off, int scales_off, const Staged& st,
                                            int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = tid + NTHREADS * i;
        const int r = p >> 2, q = p & 3;
        *reinterpret_cast<uint4*>(stage + codes_off + r * CODE_STRIDE + q * 16) = st.codes[i];
    }
    // E4M3 -> FP16 (exact: every E4M3 value is an FP16 normal number)
    const uint32_t s0 = st.scales.x, s1 = st.scales.y;
    uint32_t* dst = reinterpret_cast<uint32_t*>(stage + scales_off + tid * SCALE_STRIDE);
    dst[0] = e4m3_pair_to_f16x2(s0 & 0xff, (s0 >> 8) & 0xff);
    dst[1] = e4m3_pair_to_f16x2((s0 >> 16) & 0xff, s0 >> 24);
    dst[2] = e4m3_pair_to_f16x2(s1 & 0xff, (s1 >> 8) & 0xff);
    dst[3] = e4m3_pair_to_f16x2((s1 >> 16) & 0xff, s1 >> 24);
}

// 8 codes (one dword) times one FP16 block scale -> 8 exact FP16 values.
__device__ __forceinline__ half8_t dequant8(uint32_t w, half_t s) {
    const half2_t ss = {s, s};
    const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
    const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
    const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
    const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
    return half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int j) {
    return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

__device__ __forceinline__ float sigmoid_f32(float y) { return 1.0f / (1.0f + expf(-y)); }

__device__ __forceinline__ float softplus_f32(float z) { return fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z))); }

__global__ __launch_bounds__(NTHREADS, 1) void gemm_kernel(
    const uint8_t* __restrict__ a_codes, int64_t lda_c, const uint8_t* __restrict__ a_scales, int64_t lda_s,
    const uint8_t* __restrict__ w_codes, int64_t ldw_c, const uint8_t* __restrict__ w_scales, int64_t ldw_s,
    int64_t M, int64_t N, int64_t K, int32_t tiles_n, const SegParams sp) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31;  // row of the MFMA fragment this lane feeds
    const int lh = lane >> 5;  // lane half: which 8-element K group of an MFMA step

    const int64_t tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int64_t m0 = tm * BM, n0 = tn * BN;

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t nk = (K + BK - 1) / BK;
    Staged sa, sb;
    if (nk > 0) {
        load_chunk(sa, a_codes, lda_c, a_scales, lda_s, m0, M, 0, K, tid);
        load_chunk(sb, w_codes, ldw_c, w_scales, ldw_s, n0, N, 0, K, tid);
        store_chunk(smem, A_CODES, A_SCALES, sa, tid);
        store_chunk(smem, B_CODES, B_SCALES, sb, tid);
    }
    __syncthreads();

    for (int64_t kc = 0; kc < nk; ++kc) {
        uint8_t* cur = smem + (kc & 1) * STAGE_BYTES;
        const bool more = kc + 1 < nk;
        if (more) {
            load_chunk(sa, a_codes, lda_c, a_scales, lda_s, m0, M, (kc + 1) * BK, K, tid);
            load_chunk(sb, w_codes, ldw_c, w_scales, ldw_s, n0, N, (kc + 1) * BK, K, tid);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {  // two 64-element halves of the chunk
            uint4 araw[4], braw[4];
            half2_t ascl[4], bscl[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ra = wm * 128 + 32 * i + lr;
                const int rb = wn * 128 + 32 * i + lr;
                araw[i] = *reinterpret_cast<const uint4*>(cur + A_CODES + ra * CODE_STRIDE + c * 32 + lh * 16);
                braw[i] = *reinterpret_cast<const uint4*>(cur + B_CODES + rb * CODE_STRIDE + c * 32 + lh * 16);
                ascl[i] = *reinterpret_cast<const half2_t*>(cur + A_SCALES + ra * SCALE_STRIDE + (4 * c + 2 * lh) * 2);
                bscl[i] = *reinterpret_cast<const half2_t*>(cur + B_SCALES + rb * SCALE_STRIDE + (4 * c + 2 * lh) * 2);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {  // MFMA K steps of 16
                half8_t aop[4], bop[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    aop[i] = dequant8(word_of(araw[i], j), ascl[i][j >> 1]);
                    bop[i] = dequant8(word_of(braw[i], j), bscl[i][j >> 1]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int jn = 0; jn < 4; ++jn)
                        acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[i], bop[jn], acc[i][jn], 0, 0, 0);
            }
        }
        if (more) {
            uint8_t* nxt = smem + ((kc + 1) & 1) * STAGE_BYTES;
            store_chunk(nxt, A_CODES, A_SCALES, sa, tid);
            store_chunk(nxt, B_CODES, B_SCALES, sb, tid);
        }
        __syncthreads();
    }

    // ---- epilogue ---------------------------------------------------------------------------------
    // Each wave stages one 128 x 32 column group of its FP32 accumulators in LDS (wave-private
    // region, 33-float row pitch), then lane l handles column l % 32 of the group for every other
    // row: 32 consecutive columns per store instruction, per-column segment lookup, global scale,
    // optional gate, FP32 or bf16 store. The LDS is free here: the K loop ended with a barrier.
    float* ep = reinterpret_cast<float*>(smem) + wave * (128 * 33);
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                ep[(32 * i + (r >> 2) * 8 + lh * 4 + (r & 3)) * 33 + lr] = acc[i][jn][r];
        __syncthreads();
        const int64_t col = n0 + wn * 128 + 32 * jn + lr;
        if (col < N) {
            int s = 0;
            for (int t = 1; t < sp.n_segs; ++t)
                if (col >= sp.n_begin[t]) s = t;
            const float scale = sp.scale[s];
            const int epi = sp.epilogue[s];
            const int dtype = sp.out_dtype[s];
            const int64_t ldo = sp.ldo[s];
            const int64_t j = col - sp.n_begin[s];
            float a_coef = 0.0f, dtb = 0.0f;
            if (epi == NVFP4_EPI_GDN_DECAY) {
                a_coef = expf(sp.A_log[s][j]);
                dtb = sp.dt_bias[s][j];
            }
            const int64_t row_base = m0 + wm * 128;
            const int nrows = (int)(M - row_base < 128 ? M - row_base : 128);
            for (int rr = lh; rr < nrows; rr += 2) {
                float y = ep[rr * 33 + lr] * scale;
                if (epi == NVFP4_EPI_SIGMOID) {
                    y = sigmoid_f32(y);
                } else if (epi == NVFP4_EPI_GDN_DECAY) {
                    y = expf(-(a_coef * softplus_f32(y + dtb)));
                }
                const int64_t off = (row_base + rr) * ldo + j;
                if (dtype == NVFP4_OUT_F32) {
                    reinterpret_cast<float*>(sp.out[s])[off] = y;
                } else {
                    uint32_t u = __float_as_uint(y);
                    u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest even
                    reinterpret_cast<uint16_t*>(sp.out[s])[off] = (uint16_t)(u >> 16);
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s,
                       const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s,
                       int64_t M, int64_t N, int64_t K, const SegParams& sp, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    hipLaunchKernelGGL(gemm_kernel, dim3((uint32_t)(tiles_m * tiles_n)), dim3(NTHREADS), 0, stream, a_codes,
                       lda_c, a_scales, lda_s, w_codes, ldw_c, w_scales, ldw_s, M, N, K, (int32_t)tiles_n, sp);
    return hipGetLastError();
}

}  // namespace nvfp4
