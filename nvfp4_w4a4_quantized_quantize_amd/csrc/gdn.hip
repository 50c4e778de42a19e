// Gated DeltaNet recurrence consuming the gates of the fused in_proj GEMM, for gfx950 (CDNA4):
//
//   S_t = alpha_t S_{t-1} + beta_t k_t (v_t - S_{t-1}^T k_t)^T,      o_t = S_t^T q_t
//
// the delta-rule update of the paper arXiv:2609.04098 (Japanese article, "How Gated DeltaNet works"),
// with the erase term as the pages write it (no alpha on it), in FP32 like the pages' "FP32 lockstep"
// experiment ("Mechanism 3"). S is [D key, D value] per (sequence, value head), stored value-major
// (as S^T, one value column's key entries contiguous); value head h reads key head h / (Hv / Hk).
// The readout o_t = S_t^T q_t is the usual linear-attention readout.
//
// Design: the value columns of S evolve independently (the delta rule couples key rows only), so a
// wave owns 4 columns of one head's state, 8 key rows per lane: lane = 16 * column + row group. Both
// dot products over the key dimension are reduced inside a 16-lane row with DPP (quad swaps, then
// row rotations by 4 and 8), so a wave needs no LDS and no barrier, and a workgroup of 4 waves
// covers 16 columns. Token inputs (k, q: 16 bytes per lane; v; the gates) stream through an 8-token
// register ring: each load is issued 8 tokens ahead (prefill) and is unconditional (pointers that advance by
// one row per token, clamped to the last token near the end), so the compiler waits for exactly one
// token's loads at a time.
#include <algorithm>

#include "quant_common.h"

namespace nvfp4 {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int GDN_D = 128;    // head dimension (keys and values)

// Sum over the 16 lanes of a DPP row, returned in every lane of the row.
__device__ __forceinline__ float row16_sum(float x) {
    int v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false));  // row_ror 4
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));  // row_ror 8
    return x;
}

struct Token {
    qu32x4 k, q;  // 8 bf16 key / query elements of this lane's row group
    uint32_t v;   // bf16 value of this lane's column (low half)
    float a, b;   // the token's decay and write-strength gates
};

__device__ __forceinline__ void load_token(Token& tk, const uint16_t* kp, const uint16_t* qp, const uint16_t* vp,
                                           const float* ap, const float* bp, int64_t r, int64_t ldk, int64_t ldq,
                                           int64_t ldv, int64_t lda, int64_t ldb) {
    tk.k = *reinterpret_cast<const qu32x4*>(kp + r * ldk);
    tk.q = *reinterpret_cast<const qu32x4*>(qp + r * ldq);
    tk.v = vp[r * ldv];
    tk.a = ap[r * lda];
    tk.b = bp[r * ldb];
}

// One token for this lane's 8 key rows of one value column: u = v - S^T k, S = a S + b u k, o = S^T q.
__device__ __forceinline__ void gdn_step(const Token& cur, float (&S)[8], int kg, float* o_elem) {
    float kf[8], qf[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        kf[2 * j] = bf16_lo(cur.k[j]);
        kf[2 * j + 1] = bf16_hi(cur.k[j]);
        qf[2 * j] = bf16_lo(cur.q[j]);
        qf[2 * j + 1] = bf16_hi(cur.q[j]);
    }
    float sk = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) sk = __builtin_fmaf(S[j], kf[j], sk);
    sk = row16_sum(sk);
    const float bu = cur.b * (bf16_lo(cur.v) - sk);
#pragma unroll
    for (int j = 0; j < 8; ++j) S[j] = __builtin_fmaf(bu, kf[j], cur.a * S[j]);
    float oq = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) oq = __builtin_fmaf(S[j], qf[j], oq);
    oq = row16_sum(oq);
    if (kg == 0) *o_elem = oq;
}

// GDN_RING tokens in flight: 8 for prefill; 1 for decode-sized calls, where a deeper ring would only
// reload the same few tokens and cost registers (occupancy).
template <int GDN_RING>
__global__ __launch_bounds__(256) void gdn_recurrence_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const uint16_t* __restrict__ k, int64_t ldk,
    const uint16_t* __restrict__ v, int64_t ldv, const float* __restrict__ alpha, int64_t lda,
    const float* __restrict__ beta, int64_t ldb, float* __restrict__ state, int64_t T, int32_t Hv, int32_t group,
    float* __restrict__ o, int64_t ldo) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kg = lane & 15;                     // key rows 8 kg .. 8 kg + 7
    const int slices = GDN_D / 16;                // workgroups per head
    const int64_t bh = blockIdx.x / slices;       // b * Hv + h
    const int h = (int)(bh % Hv);
    const int64_t b = bh / Hv;
    const int c = (int)(blockIdx.x % slices) * 16 + wave * 4 + (lane >> 4);  // value column
    const int hk = h / group;

    // the state is stored value-major (S^T): this lane's 8 key rows of column c are contiguous
    float* Sp = state + bh * GDN_D * GDN_D + (int64_t)c * GDN_D + 8 * kg;
    float S[8];
    {
        const f32x4_t s0 = *reinterpret_cast<const f32x4_t*>(Sp), s1 = *reinterpret_cast<const f32x4_t*>(Sp + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            S[i] = s0[i];
            S[4 + i] = s1[i];
        }
    }

    const int64_t r0 = b * T;  // first row of this sequence
    const uint16_t* kp = k + r0 * ldk + hk * GDN_D + 8 * kg;
    const uint16_t* qp = q + r0 * ldq + hk * GDN_D + 8 * kg;
    const uint16_t* vp = v + r0 * ldv + h * GDN_D + c;
    // The gates' addresses are the same in every lane, which would make them scalar loads; those
    // complete out of order, so every token would wait for all of them. A zero the compiler cannot
    // see through (a register move) makes them vector loads, counted in order with the others.
    int vzero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
    const float* ap = alpha + r0 * lda + h + vzero;
    const float* bp = beta + r0 * ldb + h + vzero;
    float* op = o + r0 * ldo + h * GDN_D + c;

    Token ring[GDN_RING];
#pragma unroll
    for (int i = 0; i < GDN_RING; ++i)
        load_token(ring[i], kp, qp, vp, ap, bp, std::min<int64_t>(i, T - 1), ldk, ldq, ldv, lda, ldb);

    // Full blocks of GDN_RING tokens: each step issues the loads of the token GDN_RING ahead, then
    // computes; no condition in the body, so the waits stay exact. While the token ahead is inside
    // the sequence the load pointers just advance by one row per token (no index arithmetic); the
    // last blocks clamp it to the last token.
    int64_t t0 = 0;
    {
        const uint16_t* kn = kp + GDN_RING * ldk;
        const uint16_t* qn = qp + GDN_RING * ldq;
        const uint16_t* vn = vp + GDN_RING * ldv;
        const float* an = ap + GDN_RING * lda;
        const float* bn = bp + GDN_RING * ldb;
        float* ot = op;
        for (; t0 + 2 * GDN_RING <= T; t0 += GDN_RING) {
#pragma unroll
            for (int i = 0; i < GDN_RING; ++i) {
                const Token cur = ring[i];
                load_token(ring[i], kn, qn, vn, an, bn, 0, 0, 0, 0, 0, 0);
                kn += ldk;
                qn += ldq;
                vn += ldv;
                an += lda;
                bn += ldb;
                __builtin_amdgcn_sched_barrier(0);
                gdn_step(cur, S, kg, ot);
                ot += ldo;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    for (; t0 + GDN_RING <= T; t0 += GDN_RING) {
#pragma unroll
        for (int i = 0; i < GDN_RING; ++i) {
            const Token cur = ring[i];
            load_token(ring[i], kp, qp, vp, ap, bp, std::min<int64_t>(t0 + i + GDN_RING, T - 1), ldk, ldq, ldv, lda,
                       ldb);
            __builtin_amdgcn_sched_barrier(0);
            gdn_step(cur, S, kg, op + (t0 + i) * ldo);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // the last T % GDN_RING tokens are already in the ring
#pragma unroll
    for (int i = 0; i < GDN_RING - 1; ++i)
        if (t0 + i < T) gdn_step(ring[i], S, kg, op + (t0 + i) * ldo);
    *reinterpret_cast<f32x4_t*>(Sp) = f32x4_t{S[0], S[1], S[2], S[3]};
    *reinterpret_cast<f32x4_t*>(Sp + 4) = f32x4_t{S[4], S[5], S[6], S[7]};
}

}  // namespace

hipError_t launch_gdn_recurrence(const uint16_t* q, int64_t ldq, const uint16_t* k, int64_t ldk, const uint16_t* v,
                                 int64_t ldv, const float* alpha, int64_t lda, const float* beta, int64_t ldb,
                                 float* state, int64_t B, int64_t T, int32_t Hv, int32_t Hk, float* o, int64_t ldo,
                                 hipStream_t stream) {
    if (B == 0 || T == 0) return hipSuccess;
    const int64_t grid = B * Hv * (GDN_D / 16);
    if (grid > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(T >= 16 ? gdn_recurrence_kernel<8> : gdn_recurrence_kernel<1>, dim3((uint32_t)grid), dim3(256),
                       0, stream, q, ldq, k, ldk, v, ldv, alpha, lda, beta, ldb, state, T, Hv, Hv / Hk, o, ldo);
    return hipGetLastError();
}

}  // namespace nvfp4
