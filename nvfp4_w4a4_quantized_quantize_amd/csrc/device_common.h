// Device helpers shared by the GEMM kernels: operand types, NVFP4 -> FP16 dequantization, the
// segment lookup and the gate epilogues.
#pragma once

#include "internal.h"

namespace nvfp4 {

typedef _Float16 half_t;
typedef half_t half2_t __attribute__((ext_vector_type(2)));
typedef half_t half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 8 codes (one dword, element 2i in the low nibble of byte i) times one FP16 block scale -> 8 exact
// FP16 values. An E2M1 value times an E4M3 scale has at most 6 significant bits and lies in
// [2^-10, 2688], so the product is exact in FP16. The conversion's own scale operand only
// contributes a power of two, so it runs with 1.0 and the block scale is a packed FP16 multiply.
__device__ __forceinline__ half8_t dequant8(uint32_t w, half_t s) {
    const half2_t ss = {s, s};
    const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
    const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
    const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
    const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
    return half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

__device__ __forceinline__ float sigmoid_f32(float y) { return 1.0f / (1.0f + expf(-y)); }

__device__ __forceinline__ float softplus_f32(float z) { return fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z))); }

// Index of the segment holding output column col.
__device__ __forceinline__ int segment_of(const SegParams& sp, int64_t col) {
    int s = 0;
    for (int t = 1; t < sp.n_segs; ++t)
        if (col >= sp.n_begin[t]) s = t;
    return s;
}

// Gate epilogues of the Gated DeltaNet input projection: beta = sigmoid(b) and
// alpha = exp(-exp(A_log) * softplus(a + dt_bias)); a_coef = exp(A_log) of the column.
__device__ __forceinline__ float apply_gate(float y, int epi, float a_coef, float dtb) {
    if (epi == NVFP4_EPI_SIGMOID) return sigmoid_f32(y);
    if (epi == NVFP4_EPI_GDN_DECAY) return expf(-(a_coef * softplus_f32(y + dtb)));
    return y;
}

// What the epilogue of one output column needs: its segment's tensor, stride, column in it, scale
// RN32(g_a * g_w) and gate (with the column's gate parameters).
struct ColumnOut {
    uint8_t* out;
    int64_t ldo, j;
    float scale, a_coef, dtb;
    int epi;
    bool f32;
};

// Resolves column col (< N). The segments are walked with a wave-uniform index, so their fields come
// from the kernel arguments by scalar loads; indexing them by a per-lane segment number instead
// becomes a chain of dependent vector loads per element.
__device__ __forceinline__ ColumnOut column_out(const SegParams& sp, int64_t col) {
    ColumnOut c = {};
    for (int t = 0; t < sp.n_segs; ++t) {
        if (col >= sp.n_begin[t] && col < sp.n_end[t]) {
            c.out = reinterpret_cast<uint8_t*>(sp.out[t]);
            c.ldo = sp.ldo[t];
            c.j = col - sp.n_begin[t];
            c.scale = sp.scale[t];
            c.epi = sp.epilogue[t];
            c.f32 = sp.out_dtype[t] == NVFP4_OUT_F32;
            if (c.epi == NVFP4_EPI_GDN_DECAY) {
                c.a_coef = expf(sp.A_log[t][c.j]);
                c.dtb = sp.dt_bias[t][c.j];
            }
        }
    }
    return c;
}

// Scales acc by the column's g_a * g_w, applies its segment's epilogue and stores output element
// (row, col) of the fused GEMM into the segment's tensor.
__device__ __forceinline__ void column_store(const ColumnOut& c, int64_t row, float acc) {
    const float y = apply_gate(acc * c.scale, c.epi, c.a_coef, c.dtb);
    const int64_t off = row * c.ldo + c.j;
    if (c.f32)
        reinterpret_cast<float*>(c.out)[off] = y;
    else
        reinterpret_cast<__bf16*>(c.out)[off] = (__bf16)y;
}

}  // namespace nvfp4
