// Block-scaled W4A4 GEMM for one activation row (decode), for gfx950 (CDNA4).
//
//   y[0, n] = g_a * g_w[seg(n)] * sum_k e2m1(qa[0,k]) sa[0,k/16] * e2m1(qw[n,k]) sw[n,k/16]
//
// (The kernel is written for MA activation rows; it is instantiated for MA = 1: at two rows its VALU
// dot products cost more than the matrix cores of the skinny kernel, 16.1 against about 14.7 us.)
// At M = 1 the GEMM is a weight stream: every weight byte is read once and used for one product, so
// the kernel is bound by HBM bandwidth and is built for memory-level parallelism and an even split of
// the weight bytes over the compute units (the fused-module epilogue is that of the
// paper arXiv:2609.04098: Japanese article, "Trap 1"; gates per "Mechanism 2"):
//  * One wave computes one weight row over all of K; a workgroup is four waves (four rows), so the
//    decode projections (N = 17408 or 5120) give every CU exactly 17 or 5 workgroups.
//  * Each lane owns the 16-element blocks lane, lane + 64, lane + 128, ... of its row. A wave issues
//    all of its row's loads at once (8 code bytes and 1 scale byte per block, unconditional buffer
//    loads whose out-of-range part returns zeros), so a CU keeps tens of KB in flight.
//  * The activation rows are decoded once per workgroup into LDS as FP16 (an E2M1 value times an
//    E4M3 scale is exact in FP16), while the weight loads are in flight.
//  * Per block, the 16 weight codes are converted to FP16 (exact E2M1 values) and multiplied with the
//    FP16 activations by eight v_dot2_f32_f16 (the products are exact in FP32), and the block sum is
//    scaled once by the weight block scale: 18 VALU instructions per 16 weights for one row.
//  * The 64 lane sums of a row are added in a fixed butterfly order; the result is scaled by
//    RN32(g_a * g_w[s]) and passes through the segment's epilogue. No sum depends on N or on the
//    grid, so a fused call and its modules called alone give the same bits.
// (A persistent variant, one 16-wave workgroup per CU streaming contiguous 64-block units with 8 or
// 16 units in flight per wave, was measured 1.45-1.7x slower on both decode shapes and not kept.)
#include "device_common.h"

namespace nvfp4 {
namespace {

constexpr int GV_WAVES = 4;
constexpr int GV_THREADS = 64 * GV_WAVES;
constexpr int BUF_RAW = 0x00020000;  // raw buffer resource, 32-bit data format (gfx9 family)

__device__ __forceinline__ float e4m3_to_f32_dev(uint32_t byte) { return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint8_t* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)bytes, BUF_RAW);
}

// Lane sum over the wave in a fixed butterfly order.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Weight row n (one per wave) against the MA = M activation rows. BPL >= ceil(K / 16 / 64)
// blocks per lane (the lane's blocks beyond K load zeros and are skipped); the activation occupies
// MA * ceil(BPL / 4) * 256 * 32 bytes of dynamic LDS.
template <int MA, int BPL>
__global__ __launch_bounds__(GV_THREADS) void gemm_gemv_kernel(
    const uint8_t* __restrict__ a_codes, int64_t lda_c, const uint8_t* __restrict__ a_scales, int64_t lda_s,
    const uint8_t* __restrict__ w_codes, int64_t ldw_c, const uint8_t* __restrict__ w_scales, int64_t ldw_s,
    int64_t M, int64_t N, int64_t K, const SegParams sp) {
    // [MA][ABPT * 256 blocks][16] e2m1(qa) * sa, exact in FP16
    extern __shared__ __attribute__((aligned(16))) half_t act[];
    constexpr int ABPT = (BPL + GV_WAVES - 1) / GV_WAVES;  // activation blocks per thread
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t n = (int64_t)blockIdx.x * GV_WAVES + wave;
    const int nb = (int)(K >> 4);    // blocks per row
    const int nbl = (nb + 63) >> 6;  // blocks per lane that exist somewhere in the row (<= BPL)

    // 1. activation loads (L2), then this wave's whole weight row (HBM), all unconditional
    uint32_t a_cw[MA][ABPT][2], a_sb[MA][ABPT];
#pragma unroll
    for (int m = 0; m < MA; ++m) {
        const __amdgpu_buffer_rsrc_t rc = rsrc(a_codes + m * lda_c, (uint32_t)nb * 8u);
        const __amdgpu_buffer_rsrc_t rs = rsrc(a_scales + m * lda_s, (uint32_t)nb);
#pragma unroll
        for (int i = 0; i < ABPT; ++i) {
            const uint32_t blk = (uint32_t)(tid + GV_THREADS * i);
            const u32x2 c = __builtin_amdgcn_raw_buffer_load_b64(rc, (int)(blk * 8u), 0, 0);
            a_cw[m][i][0] = c[0];
            a_cw[m][i][1] = c[1];
            a_sb[m][i] = __builtin_amdgcn_raw_buffer_load_b8(rs, (int)blk, 0, 0);
        }
    }
    const int64_t nrow = n < N ? n : N - 1;  // a wave past N streams the last row again, stores nothing
    const __amdgpu_buffer_rsrc_t wr_c = rsrc(w_codes + nrow * ldw_c, (uint32_t)nb * 8u);
    const __amdgpu_buffer_rsrc_t wr_s = rsrc(w_scales + nrow * ldw_s, (uint32_t)nb);
    u32x2 wc[BPL];
    uint32_t wsb[BPL];
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
        const uint32_t blk = (uint32_t)(lane + 64 * j);
        wc[j] = __builtin_amdgcn_raw_buffer_load_b64(wr_c, (int)(blk * 8u), 0, 0);
        wsb[j] = __builtin_amdgcn_raw_buffer_load_b8(wr_s, (int)blk, 0, 0);
    }

    // 2. decode the activation rows into LDS: every thread stores all of its blocks (those past K hold
    // zeros), so no load hides behind a branch and the wait covers only the activation loads
#pragma unroll
    for (int m = 0; m < MA; ++m) {
#pragma unroll
        for (int i = 0; i < ABPT; ++i) {
            const int blk = tid + GV_THREADS * i;
            const half_t s = (half_t)e4m3_to_f32_dev(a_sb[m][i]);
            const half8_t lo = dequant8(a_cw[m][i][0], s), hi = dequant8(a_cw[m][i][1], s);
            half8_t* dst = reinterpret_cast<half8_t*>(act + ((m * ABPT * GV_THREADS) + blk) * 16);
            dst[0] = lo;
            dst[1] = hi;
        }
    }
    __syncthreads();

    // 3. per block: 8 dot2 over exact FP16 products, then one multiply-add by the weight block scale
    float acc[MA];
#pragma unroll
    for (int m = 0; m < MA; ++m) acc[m] = 0.0f;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
        if (j < nbl) {  // uniform
            const int blk = lane + 64 * j;
            const int blk_c = blk < nb ? blk : nb - 1;  // past K: weights are zero, read any block
            const float sw = e4m3_to_f32_dev(wsb[j]);
            const half2_t w[8] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wc[j][0], 1.0f, 0),
                                  __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wc[j][0], 1.0f, 1),
                                  __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wc[j][0], 1.0f, 2),
                                  __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wc[j][0], 1.0f, 3),
                                  __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wc[j][1], 1.0f, 0),
                                  __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wc[j][1], 1.0f, 1),
                                  __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wc[j][1], 1.0f, 2),
                                  __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wc[j][1], 1.0f, 3)};
#pragma unroll
            for (int m = 0; m < MA; ++m) {
                const half8_t* src = reinterpret_cast<const half8_t*>(act + ((m * ABPT * GV_THREADS) + blk_c) * 16);
                const half8_t a0 = src[0], a1 = src[1];
                float s = 0.0f;
#pragma unroll
                for (int b = 0; b < 4; ++b) s = __builtin_amdgcn_fdot2(w[b], half2_t{a0[2 * b], a0[2 * b + 1]}, s, false);
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    s = __builtin_amdgcn_fdot2(w[4 + b], half2_t{a1[2 * b], a1[2 * b + 1]}, s, false);
                acc[m] = __builtin_fmaf(s, sw, acc[m]);
            }
        }
    }

    // 4. row sums and the segment epilogue
    float y[MA];
#pragma unroll
    for (int m = 0; m < MA; ++m) y[m] = wave_sum(acc[m]);
    if (n < N && lane < MA) {
        const ColumnOut co = column_out(sp, n);
        column_store(co, lane, lane == 0 ? y[0] : y[MA - 1]);
    }
}

template <int MA>
hipError_t launch_ma(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s,
                     const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s, int64_t M,
                     int64_t N, int64_t K, const SegParams& sp, hipStream_t stream) {
    using fn_t = void (*)(const uint8_t*, int64_t, const uint8_t*, int64_t, const uint8_t*, int64_t, const uint8_t*,
                          int64_t, int64_t, int64_t, int64_t, const SegParams);
    const int nbl = (int)((K / 16 + 63) / 64);
    fn_t fn;
    int bpl;
    if (nbl <= 2) fn = gemm_gemv_kernel<MA, 2>, bpl = 2;
    else if (nbl <= 4) fn = gemm_gemv_kernel<MA, 4>, bpl = 4;
    else if (nbl <= 5) fn = gemm_gemv_kernel<MA, 5>, bpl = 5;
    else if (nbl <= 8) fn = gemm_gemv_kernel<MA, 8>, bpl = 8;
    else if (nbl <= 12) fn = gemm_gemv_kernel<MA, 12>, bpl = 12;
    else if (nbl <= 17) fn = gemm_gemv_kernel<MA, 17>, bpl = 17;
    else if (nbl <= 24) fn = gemm_gemv_kernel<MA, 24>, bpl = 24;
    else fn = gemm_gemv_kernel<MA, 32>, bpl = 32;
    const size_t lds = (size_t)MA * (size_t)((bpl + GV_WAVES - 1) / GV_WAVES) * GV_THREADS * 32;
    hipLaunchKernelGGL(fn, dim3((uint32_t)((N + GV_WAVES - 1) / GV_WAVES)), dim3(GV_THREADS), lds, stream, a_codes,
                       lda_c, a_scales, lda_s, w_codes, ldw_c, w_scales, ldw_s, M, N, K, sp);
    return hipGetLastError();
}

}  // namespace

bool gemv_supported(int64_t M, int64_t K) { return M >= 1 && M <= GEMV_MAX_M && K >= 16 && K <= GEMV_MAX_K; }

hipError_t launch_gemm_gemv(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s,
                            const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s,
                            int64_t M, int64_t N, int64_t K, const SegParams& sp, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    if (!gemv_supported(M, K)) return hipErrorInvalidValue;
    return launch_ma<1>(a_codes, lda_c, a_scales, lda_s, w_codes, ldw_c, w_scales, ldw_s, M, N, K, sp, stream);
}

}  // namespace nvfp4
