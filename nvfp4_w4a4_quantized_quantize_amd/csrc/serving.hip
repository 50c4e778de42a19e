// Companions of the NVFP4 linear layer on the same serving path, for gfx950 (CDNA4):
//  * FP8 E4M3 KV-cache codec with static per-tensor scales, calibrated offline and shipped with the
//    checkpoint (paper arXiv:2609.04098; Japanese article, "Is FP8 enough for the KV cache? The 'ship
//    KV scales' recipe"): q = E4M3_RNE_SAT(RN32(x / s)), x^ = bf16_RNE(RN32(e4m3(q) s)).
//  * The fold-in repair of the fused-module global-scale mismatch (Japanese article, "Trap 1"): the
//    fused group takes one common global scale G and each module's ratio r = g / G is folded into
//    its block scales, s' = E4M3_RNE_SAT(RN32(s r)); codes are unchanged.
//  * BF16 RMSNorm fused with the NVFP4 quantizer of its output (the pages keep normalization layers
//    in BF16; Japanese article, experiment design), so the normalized activations never go to HBM.
// All three are streaming kernels bound by HBM bandwidth.
#include <cmath>

#include "quant_common.h"

namespace nvfp4 {
namespace {

// RN32(a / S) for a = |x| of a bf16 value, S > 0: quotient_fast (the reciprocal with one
// exact-residual correction) inside its range, where it gives the same E4M3 byte as the correctly
// rounded quotient, else the IEEE division.
__device__ __forceinline__ float quotient_rn(float a, float S, float y, bool s_ok) {
    if (s_ok && a * 0x1p-100f <= S) return quotient_fast(a, S, y);
    return __fdiv_rn(a, S);
}

// One signed E4M3FN byte: saturating round to nearest even, sign kept, NaN -> 0x7F.
__device__ __forceinline__ uint32_t e4m3_signed(float q, float xsign) {
    if (q != q) return 0x7Fu;
    const uint32_t mag = e4m3_rne_sat(q);  // q >= 0 here
    return (__float_as_uint(xsign) >> 24 & 0x80u) | mag;
}

// ---- FP8 KV codec: one thread = 16 consecutive elements (32 bytes of bf16, 16 bytes of FP8) ----
__device__ __forceinline__ uint32_t kv_pair(uint32_t w, float s, float y, bool s_ok) {
    const float f0 = bf16_lo(w), f1 = bf16_hi(w);
    const uint32_t b0 = e4m3_signed(quotient_rn(fabsf(f0), s, y, s_ok), f0);
    const uint32_t b1 = e4m3_signed(quotient_rn(fabsf(f1), s, y, s_ok), f1);
    return b0 | (b1 << 8);
}

__global__ __launch_bounds__(256) void kv_quantize_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                          uint8_t* __restrict__ q, int64_t ldq, float s,
                                                          uint32_t units, uint32_t blocks_per_row) {
    const uint32_t row = blockIdx.x / blocks_per_row;
    const uint32_t u = (blockIdx.x - row * blocks_per_row) * 256u + threadIdx.x;
    if (u >= units) return;
    const qu32x4* src = reinterpret_cast<const qu32x4*>(x + (int64_t)row * ldx + 16u * u);
    const qu32x4 p0 = __builtin_nontemporal_load(src), p1 = __builtin_nontemporal_load(src + 1);
    const float y = __builtin_amdgcn_rcpf(s);
    const bool s_ok = divisor_fast_ok(s);
    qu32x4 o;
    o[0] = kv_pair(p0[0], s, y, s_ok) | (kv_pair(p0[1], s, y, s_ok) << 16);
    o[1] = kv_pair(p0[2], s, y, s_ok) | (kv_pair(p0[3], s, y, s_ok) << 16);
    o[2] = kv_pair(p1[0], s, y, s_ok) | (kv_pair(p1[1], s, y, s_ok) << 16);
    o[3] = kv_pair(p1[2], s, y, s_ok) | (kv_pair(p1[3], s, y, s_ok) << 16);
    __builtin_nontemporal_store(o, reinterpret_cast<qu32x4*>(q + (int64_t)row * ldq + 16u * u));
}

__device__ __forceinline__ uint32_t bf16_bits_rne(float v) {
    if (v != v) return 0x7FC0u;
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v);
}

__global__ __launch_bounds__(256) void kv_dequantize_kernel(const uint8_t* __restrict__ q, int64_t ldq,
                                                            uint16_t* __restrict__ y, int64_t ldy, float s,
                                                            uint32_t units, uint32_t blocks_per_row) {
    const uint32_t row = blockIdx.x / blocks_per_row;
    const uint32_t u = (blockIdx.x - row * blocks_per_row) * 256u + threadIdx.x;
    if (u >= units) return;
    const qu32x4 p = __builtin_nontemporal_load(reinterpret_cast<const qu32x4*>(q + (int64_t)row * ldq + 16u * u));
    qu32x4 o[2];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const int w = (int)p[h];
        const float v0 = __builtin_amdgcn_cvt_f32_fp8(w, 0) * s;
        const float v1 = __builtin_amdgcn_cvt_f32_fp8(w, 1) * s;
        const float v2 = __builtin_amdgcn_cvt_f32_fp8(w, 2) * s;
        const float v3 = __builtin_amdgcn_cvt_f32_fp8(w, 3) * s;
        o[h >> 1][2 * (h & 1)] = bf16_bits_rne(v0) | (bf16_bits_rne(v1) << 16);
        o[h >> 1][2 * (h & 1) + 1] = bf16_bits_rne(v2) | (bf16_bits_rne(v3) << 16);
    }
    qu32x4* dst = reinterpret_cast<qu32x4*>(y + (int64_t)row * ldy + 16u * u);
    __builtin_nontemporal_store(o[0], dst);
    __builtin_nontemporal_store(o[1], dst + 1);
}

// ---- fold-in repair: one thread = one scale byte, in place -------------------------------------
__global__ __launch_bounds__(256) void fold_scales_kernel(uint8_t* __restrict__ scales, int64_t lds, float ratio,
                                                          uint32_t nblocks, uint32_t blocks_per_row) {
    const uint32_t row = blockIdx.x / blocks_per_row;
    const uint32_t b = (blockIdx.x - row * blocks_per_row) * 256u + threadIdx.x;
    if (b >= nblocks) return;
    uint8_t* p = scales + (int64_t)row * lds + b;
    const uint32_t byte = *p;
    uint32_t out = 0x7Fu;
    if ((byte & 0x7Fu) != 0x7Fu) out = (byte & 0x80u) | e4m3_rne_sat(e4m3_to_f32(byte & 0x7Fu) * ratio);
    *p = (uint8_t)out;
}

// ---- RMSNorm + NVFP4 quantize: one wave = one row ----------------------------------------------
//   ms = sum(x^2) / K in double; r = RN32(1 / sqrt(ms + eps)) (double, then one rounding);
//   y1 = bf16_RNE(RN32(x r)); y = bf16_RNE(y1 w) (the product of two bf16 values is exact in FP32);
//   then y is encoded as NVFP4 with the static global scale g.
// Lane l owns the 16-element blocks l, l + 64, ... of its row. With NBL > 0 (rows of at most
// 64 * NBL blocks) the row stays in registers between the sum and the encoding, so it is read
// once; NBL == 0 handles any K with a second pass over the row, which finds it in L2.

// The block's 16 elements widened to FP32 (exact), in order.
__device__ __forceinline__ void widen16(const qu32x4& p0, const qu32x4& p1, float (&xf)[16]) {
    const uint32_t wv[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        xf[2 * i] = bf16_lo(wv[i]);
        xf[2 * i + 1] = bf16_hi(wv[i]);
    }
}

__device__ __forceinline__ double sum_squares_f(const float (&xf)[16]) {
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) ss += (double)xf[i] * (double)xf[i];
    return ss;
}

// xf: the block's 16 elements as FP32; wf: its 16 norm weights as FP32 (exact bf16 values).
__device__ __forceinline__ void norm_encode_block(const float (&xf)[16], const float* wf, int64_t b, float r, float g,
                                                  uint8_t* __restrict__ codes_row, uint8_t* __restrict__ scales_row,
                                                  uint16_t* __restrict__ y_row) {
    float f[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // two elements per bf16 rounding instruction
        const uint32_t y1 = bf16x2_rne(xf[2 * i] * r, xf[2 * i + 1] * r);
        const uint32_t y = bf16x2_rne(bf16_lo(y1) * wf[2 * i], bf16_hi(y1) * wf[2 * i + 1]);
        f[2 * i] = bf16_lo(y);
        f[2 * i + 1] = bf16_hi(y);
    }
    const Block16 q = encode_block16(f, g);
    __builtin_nontemporal_store(qu32x2{q.c0, q.c1}, reinterpret_cast<qu32x2*>(codes_row + 8 * b));
    scales_row[b] = (uint8_t)q.sb;
    if (y_row) {
        qu32x4 o0, o1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o0[i] = (__float_as_uint(f[2 * i]) >> 16) | (__float_as_uint(f[2 * i + 1]) & 0xffff0000u);
            o1[i] = (__float_as_uint(f[8 + 2 * i]) >> 16) | (__float_as_uint(f[8 + 2 * i + 1]) & 0xffff0000u);
        }
        qu32x4* dst = reinterpret_cast<qu32x4*>(y_row + 16 * b);
        dst[0] = o0;
        dst[1] = o1;
    }
}

__device__ __forceinline__ float row_rscale(double ss, int64_t K, float eps) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    const double ms = __ddiv_rn(ss, (double)K);
    return (float)__ddiv_rn(1.0, __dsqrt_rn(ms + (double)eps));
}

template <int NBL>
__global__ __launch_bounds__(256) void rmsnorm_quantize_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t K, int64_t ldx, const uint16_t* __restrict__ w, float eps,
    float g, uint8_t* __restrict__ codes, int64_t ldc, uint8_t* __restrict__ scales, int64_t lds,
    uint16_t* __restrict__ y_out, int64_t ldy) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (NBL == 0 && row >= rows) return;
    const int64_t nb = K / 16;
    const uint16_t* xr = x + row * ldx;
    uint8_t* codes_row = codes + row * ldc;
    uint8_t* scales_row = scales + row * lds;
    uint16_t* y_row = y_out ? y_out + row * ldy : nullptr;

    if constexpr (NBL > 0) {
        // the row is loaded first; the norm weights are staged once per workgroup in LDS meanwhile,
        // widened to FP32 (exact)
        __shared__ __attribute__((aligned(16))) float w_lds[NBL * 64 * 16];
        qu32x4 p[NBL][2];
#pragma unroll
        for (int j = 0; j < NBL; ++j) {
            const int64_t b = lane + 64 * j;
            if (b < nb && row < rows) {
                const qu32x4* src = reinterpret_cast<const qu32x4*>(xr + 16 * b);
                p[j][0] = __builtin_nontemporal_load(src);
                p[j][1] = __builtin_nontemporal_load(src + 1);
            }
        }
        for (int64_t i = threadIdx.x; i < nb * 2; i += 256) {
            const qu32x4 wq = reinterpret_cast<const qu32x4*>(w)[i];  // 8 weights
            qu32x4 lo, hi;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                lo[2 * e] = wq[e] << 16;
                lo[2 * e + 1] = wq[e] & 0xffff0000u;
                hi[2 * e] = wq[2 + e] << 16;
                hi[2 * e + 1] = wq[2 + e] & 0xffff0000u;
            }
            reinterpret_cast<qu32x4*>(w_lds)[2 * i] = lo;
            reinterpret_cast<qu32x4*>(w_lds)[2 * i + 1] = hi;
        }
        __syncthreads();
        if (row >= rows) return;
        // the elements are widened once, for the sum and for the norm
        float xf[NBL][16];
        double ss = 0.0;
#pragma unroll
        for (int j = 0; j < NBL; ++j)
            if (lane + 64 * j < nb) {
                widen16(p[j][0], p[j][1], xf[j]);
                ss += sum_squares_f(xf[j]);
            }
        const float r = row_rscale(ss, K, eps);
#pragma unroll
        for (int j = 0; j < NBL; ++j) {
            const int64_t b = lane + 64 * j;
            if (b < nb) norm_encode_block(xf[j], w_lds + 16 * b, b, r, g, codes_row, scales_row, y_row);
        }
    } else {
        double ss = 0.0;
        for (int64_t b = lane; b < nb; b += 64) {
            const qu32x4* src = reinterpret_cast<const qu32x4*>(xr + 16 * b);
            float xf[16];
            widen16(src[0], src[1], xf);
            ss += sum_squares_f(xf);
        }
        const float r = row_rscale(ss, K, eps);
        for (int64_t b = lane; b < nb; b += 64) {
            const qu32x4* src = reinterpret_cast<const qu32x4*>(xr + 16 * b);
            const qu32x4* wsrc = reinterpret_cast<const qu32x4*>(w + 16 * b);
            const qu32x4 w0 = wsrc[0], w1 = wsrc[1];
            float wf[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                wf[2 * i] = bf16_lo(w0[i]);
                wf[2 * i + 1] = bf16_hi(w0[i]);
                wf[8 + 2 * i] = bf16_lo(w1[i]);
                wf[8 + 2 * i + 1] = bf16_hi(w1[i]);
            }
            float xf[16];
            widen16(src[0], src[1], xf);
            norm_encode_block(xf, wf, b, r, g, codes_row, scales_row, y_row);
        }
    }
}

// Rows of `units` work items (256 per block): returns false when the grid would not fit one launch.
bool row_grid(int64_t rows, int64_t units, uint32_t* blocks_per_row, uint32_t* grid) {
    const int64_t bpr = (units + 255) / 256;
    if (units > 0xFFFFFFFFll || bpr == 0 || rows * bpr > 0x7FFFFFFFll) return false;
    *blocks_per_row = (uint32_t)bpr;
    *grid = (uint32_t)(rows * bpr);
    return true;
}

}  // namespace

hipError_t launch_kv_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, float s, uint8_t* q,
                              int64_t ldq, hipStream_t stream) {
    if (rows == 0 || cols == 0) return hipSuccess;
    if (ldx == cols && ldq == cols) {  // contiguous: one long row
        cols *= rows;
        rows = 1;
    }
    uint32_t bpr, grid;
    if (!row_grid(rows, cols / 16, &bpr, &grid)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kv_quantize_kernel, dim3(grid), dim3(256), 0, stream, x, ldx, q, ldq, s, (uint32_t)(cols / 16), bpr);
    return hipGetLastError();
}

hipError_t launch_kv_dequantize(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, float s, uint16_t* y,
                                int64_t ldy, hipStream_t stream) {
    if (rows == 0 || cols == 0) return hipSuccess;
    if (ldq == cols && ldy == cols) {
        cols *= rows;
        rows = 1;
    }
    uint32_t bpr, grid;
    if (!row_grid(rows, cols / 16, &bpr, &grid)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kv_dequantize_kernel, dim3(grid), dim3(256), 0, stream, q, ldq, y, ldy, s, (uint32_t)(cols / 16), bpr);
    return hipGetLastError();
}

hipError_t launch_fold_scales(uint8_t* scales, int64_t rows, int64_t nblocks, int64_t lds, float ratio,
                              hipStream_t stream) {
    if (rows == 0 || nblocks == 0) return hipSuccess;
    if (lds == nblocks) {
        nblocks *= rows;
        rows = 1;
    }
    uint32_t bpr, grid;
    if (!row_grid(rows, nblocks, &bpr, &grid)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fold_scales_kernel, dim3(grid), dim3(256), 0, stream, scales, lds, ratio, (uint32_t)nblocks, bpr);
    return hipGetLastError();
}

hipError_t launch_rmsnorm_quantize(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, const uint16_t* w,
                                   float eps, float g, uint8_t* codes, int64_t ldc, uint8_t* scales, int64_t lds,
                                   uint16_t* y, int64_t ldy, hipStream_t stream) {
    if (rows == 0 || K == 0) return hipSuccess;
    const int64_t grid = (rows + 3) / 4;
    if (grid > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
    typedef void (*fn_t)(const uint16_t*, int64_t, int64_t, int64_t, const uint16_t*, float, float, uint8_t*, int64_t,
                         uint8_t*, int64_t, uint16_t*, int64_t);
    static const fn_t by_nbl[9] = {rmsnorm_quantize_kernel<0>, rmsnorm_quantize_kernel<1>, rmsnorm_quantize_kernel<2>,
                                   rmsnorm_quantize_kernel<3>, rmsnorm_quantize_kernel<4>, rmsnorm_quantize_kernel<5>,
                                   rmsnorm_quantize_kernel<6>, rmsnorm_quantize_kernel<7>, rmsnorm_quantize_kernel<8>};
    const int64_t nbl = (K / 16 + 63) / 64;  // blocks per lane
    hipLaunchKernelGGL(by_nbl[nbl <= 8 ? nbl : 0], dim3((uint32_t)grid), dim3(256), 0, stream, x, rows, K, ldx, w, eps,
                       g, codes, ldc, scales, lds, y, ldy);
    return hipGetLastError();
}

}  // namespace nvfp4
