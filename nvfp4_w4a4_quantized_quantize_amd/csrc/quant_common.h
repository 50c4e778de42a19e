// Device helpers shared by the kernels that encode NVFP4 or FP8 E4M3: bf16 unpacking, the E4M3 and
// E2M1 conversions and the encoding of one 16-element NVFP4 block.
#pragma once

#include "internal.h"

namespace nvfp4 {

typedef uint32_t qu32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t qu32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// E4M3FN round-to-nearest-even with saturation at 448, for a non-negative input. The gfx950
// conversion rounds to nearest even in the OCP E4M3FN format but turns inputs of 464 and above into
// NaN, so clamp first.
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

struct Block16 {
    uint32_t c0, c1;  // 16 packed codes, element 2i in the low nibble of byte i
    uint32_t sb;      // E4M3 scale byte
};

// One NVFP4 block, every rounding taken in IEEE binary32 as specified:
//   t = RN32(6 g); s = E4M3_RNE_SAT(RN32(amax / t)); S = RN32(s g); v = RN32(|x| / S);
//   code = sign(x) | E2M1_RNE_SAT(v).
__device__ __forceinline__ Block16 encode_block16(const float (&f)[16], float g) {
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
    Block16 b;
    b.c0 = 0;
    b.c1 = 0;
    b.c0 = put_e2m1_pair<0>(b.c0, v[0], v[1]);
    b.c0 = put_e2m1_pair<1>(b.c0, v[2], v[3]);
    b.c0 = put_e2m1_pair<2>(b.c0, v[4], v[5]);
    b.c0 = put_e2m1_pair<3>(b.c0, v[6], v[7]);
    b.c1 = put_e2m1_pair<0>(b.c1, v[8], v[9]);
    b.c1 = put_e2m1_pair<1>(b.c1, v[10], v[11]);
    b.c1 = put_e2m1_pair<2>(b.c1, v[12], v[13]);
    b.c1 = put_e2m1_pair<3>(b.c1, v[14], v[15]);
    b.sb = sb;
    return b;
}

}  // namespace nvfp4
