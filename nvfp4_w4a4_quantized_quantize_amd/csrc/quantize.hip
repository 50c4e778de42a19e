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
#include "internal.h"

namespace nvfp4 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// E4M3FN round-to-nearest-even with saturation at 448. The gfx950 conversion rounds to nearest
// even in the OCP E4M3FN format but turns inputs of 464 and above into NaN, so clamp first.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
    v = fminf(v, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xffu;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
    return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// Two signed E2M1 codes (round to nearest even, saturating at 6, sign kept for zero) into byte
// `sel` of `word`: the first value goes to the low nibble.
template <int sel>
__device__ __forceinline__ uint32_t put_e2m1_pair(uint32_t word, float lo, float hi) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, lo, hi, 1.0f, sel);
}

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
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));

    const float t = 6.0f * g;
    const float s_raw = __fdiv_rn(amax, t);
    const uint32_t sb = e4m3_rne_sat(s_raw);
    const float s = e4m3_to_f32(sb);
    const float S = s * g;

    // v = RN32(|x| / S). Fast path: y = rcp(S) then one exact-residual correction
    //   q0 = |x| y;  r = fma(-q0, S, |x|) (exact);  q1 = fma(r, y, q0)
    // which equals the correctly rounded quotient for bf16 |x| whenever S, 1/S and the quotient
    // stay inside the normal range (checked against IEEE division for every bf16 significand and
    // every binary32 significand of S). A zero scale takes y = 0, giving q1 = 0. Blocks outside
    // that range (extreme global scales) use the IEEE division.
    const bool fast = (s == 0.0f) || (S >= 0x1p-100f && S <= 0x1p100f && amax * 0x1p-100f <= S);
    float v[16];
    if (fast) {
        const float y = (s == 0.0f) ? 0.0f : __builtin_amdgcn_rcpf(S);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float a = fabsf(f[i]);
            const float q0 = a * y;
            const float r = __builtin_fmaf(-q0, S, a);
            const float q1 = __builtin_fmaf(r, y, q0);
            v[i] = __builtin_copysignf(q1, f[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = __builtin_copysignf(__fdiv_rn(fabsf(f[i]), S), f[i]);
    }
    uint32_t c0 = 0, c1 = 0;
    c0 = put_e2m1_pair<0>(c0, v[0], v[1]);
    c0 = put_e2m1_pair<1>(c0, v[2], v[3]);
    c0 = put_e2m1_pair<2>(c0, v[4], v[5]);
    c0 = put_e2m1_pair<3>(c0, v[6], v[7]);
    c1 = put_e2m1_pair<0>(c1, v[8], v[9]);
    c1 = put_e2m1_pair<1>(c1, v[10], v[11]);
    c1 = put_e2m1_pair<2>(c1, v[12], v[13]);
    c1 = put_e2m1_pair<3>(c1, v[14], v[15]);

    u32x2* dst = reinterpret_cast<u32x2*>(codes + row * ldc + (uint64_t)b * 8u);
    __builtin_nontemporal_store(u32x2{c0, c1}, dst);
    scales[row * lds + b] = (uint8_t)sb;
}

// ---- global scale: g = RN32(amax / 2688) ------------------------------------------------------
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
    // non-negative floats order like their bit patterns, so an integer max is exact
    if ((threadIdx.x & 63) == 0 && m > 0.0f) atomicMax(acc, __float_as_uint(m));
}

__global__ void finish_scale_kernel(float* g_out) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        const float amax = __uint_as_float(*reinterpret_cast<uint32_t*>(g_out));
        *g_out = __fdiv_rn(amax, 6.0f * 448.0f);
    }
}

}  // namespace

hipError_t launch_global_scale(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, float* g_out,
                               hipStream_t stream) {
    uint32_t* acc = reinterpret_cast<uint32_t*>(g_out);
    hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(64), 0, stream, acc);
    if (rows > 0 && K > 0) {
        const int64_t grid = rows < 8192 ? rows : 8192;
        hipLaunchKernelGGL(amax_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, x, rows, K, ldx, acc);
    }
    hipLaunchKernelGGL(finish_scale_kernel, dim3(1), dim3(64), 0, stream, g_out);
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
