// NVFP4 activation/weight quantizer and global-scale calibration for gfx950.
//
// Format: E2M1 elements, one E4M3 scale per 16 elements along K chosen from the block maximum, one
// FP32 global scale per linear module (paper arXiv:2609.04098; Japanese article, "Mechanism 1" and
// FAQ "What is NVFP4?"; "Trap 1" for the per-module global scale).
//
// The quantizer is a streaming kernel bound by HBM bandwidth: it reads 2 bytes and writes 9/16 byte
// per element. One lane owns one 16-element block (two 16-byte loads, one 8-byte code store, one
// scale byte), so a wave reads 2 KB of contiguous bf16 and writes 512 contiguous code bytes.
// Every rounding decision is taken in IEEE binary32 exactly as specified:
//   t = RN32(6 g); s = E4M3_RNE_SAT(RN32(amax / t)); S = RN32(s g); v = RN32(|x| / S);
//   code = sign(x) | E2M1_RNE_SAT(v).
#include "quant_common.h"

namespace nvfp4 {
namespace {

typedef qu32x4 u32x4;
typedef qu32x2 u32x2;

__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                       uint8_t* __restrict__ codes, int64_t ldc,
                                                       uint8_t* __restrict__ scales, int64_t lds,
                                                       float g, uint32_t nb, uint32_t tiles_per_row,
                                                       uint64_t total_tiles) {
    // one wave = one tile of 64 consecutive blocks of one row
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63;
    const uint64_t tile = (uint64_t)blockIdx.x * 4 + wave;
    if (tile >= total_tiles) return;
    const uint64_t row = tile / tiles_per_row;
    const uint32_t b = (uint32_t)(tile - row * tiles_per_row) * 64u + lane;
    if (b >= nb) return;

    const u32x4* src = reinterpret_cast<const u32x4*>(x + row * ldx + (uint64_t)b * 16u);
    const u32x4 p0 = __builtin_nontemporal_load(src);
    const u32x4 p1 = __builtin_nontemporal_load(src + 1);
    const uint32_t w[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
    float f[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        f[2 * i] = bf16_lo(w[i]);
        f[2 * i + 1] = bf16_hi(w[i]);
    }
    const Block16 q = encode_block16(f, g);

    u32x2* dst = reinterpret_cast<u32x2*>(codes + row * ldc + (uint64_t)b * 8u);
    __builtin_nontemporal_store(u32x2{q.c0, q.c1}, dst);
    scales[row * lds + b] = (uint8_t)q.sb;
}

// ---- scale from a tensor amax: RN32(amax / divisor) (2688 = 6 * 448 for NVFP4, 448 for FP8 KV) ----
__global__ void clear_word_kernel(uint32_t* p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0u;
}

__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                   int64_t K, int64_t ldx, uint32_t* acc) {
    float m = 0.0f;
    const int64_t nvec = K / 8;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const uint4* row = reinterpret_cast<const uint4*>(x + r * ldx);
        for (int64_t c = threadIdx.x; c < nvec; c += blockDim.x) {
            const uint4 p = row[c];
            const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
        }
        for (int64_t k = nvec * 8 + threadIdx.x; k < K; k += blockDim.x)
            m = fmaxf(m, fabsf(__uint_as_float((uint32_t)x[r * ldx + k] << 16)));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    // one atomic per workgroup: same-address atomics serialize in L2
    __shared__ float wave_max[4];
    if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
        // non-negative floats order like their bit patterns, so an integer max is exact
        if (m > 0.0f) atomicMax(acc, __float_as_uint(m));
    }
}

__global__ void finish_scale_kernel(float* g_out, float divisor) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        const float amax = __uint_as_float(*reinterpret_cast<uint32_t*>(g_out));
        *g_out = __fdiv_rn(amax, divisor);
    }
}

}  // namespace

hipError_t launch_amax_scale(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, float divisor,
                             float* g_out, hipStream_t stream) {
    uint32_t* acc = reinterpret_cast<uint32_t*>(g_out);
    hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(64), 0, stream, acc);
    if (rows > 0 && K > 0) {
        const int64_t grid = rows < 1024 ? rows : 1024;
        hipLaunchKernelGGL(amax_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, x, rows, K, ldx, acc);
    }
    hipLaunchKernelGGL(finish_scale_kernel, dim3(1), dim3(64), 0, stream, g_out, divisor);
    return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, float g,
                           uint8_t* codes, int64_t ldc, uint8_t* scales, int64_t lds,
                           hipStream_t stream) {
    if (rows == 0 || K == 0) return hipSuccess;
    const uint32_t nb = (uint32_t)(K / 16);
    const uint32_t tiles_per_row = (nb + 63u) / 64u;
    const uint64_t total_tiles = (uint64_t)rows * tiles_per_row;
    const uint64_t grid = (total_tiles + 3) / 4;
    hipLaunchKernelGGL(quantize_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, x, ldx, codes, ldc,
                       scales, lds, g, nb, tiles_per_row, total_tiles);
    return hipGetLastError();
}

}  // namespace nvfp4
