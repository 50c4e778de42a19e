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
constexpr int64_t GDN_CHUNK_MIN_T = 32;  // calls with at least this many tokens take the chunked form

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


// ---------------------------------------------------------------------------------------------------
// Chunked form, for prefill. Within a chunk of CH tokens starting from state S0, with
// P(t, j) = prod_{j < i <= t} alpha_i and P(t, start) the product over the chunk up to t, the deltas
// u_t = v_t - S_{t-1}^T k_t solve the unit lower-triangular system
//     u_t + sum_{j < t} P(t-1, j) beta_j (k_t . k_j) u_j = v_t - P(t-1, start) S0^T k_t,
// i.e. (I + L) U = R, and then
//     o_t   = P(t, start) S0^T q_t + sum_{j <= t} P(t, j) beta_j (q_t . k_j) u_j     (O = G Q S0 + Mq U)
//     S_end = P(end, start) S0 + sum_j P(end, j) beta_j k_j u_j^T.
// This is the recurrence unrolled over the chunk, exact up to rounding. Each workgroup owns 16 value
// columns of one head (the columns evolve independently) and walks the chunks in order, holding its
// 128 x 16 slice of S in registers (FP32). The matrix products run on the matrix cores:
//   * K K^T, K Q^T (bf16 inputs: the products are exact, FP32 sums): v_mfma_f32_16x16x32_bf16;
//   * K S0, Q S0, K^T (w U): the FP32 operand is split into three bf16 parts x = h + m + l (each part
//     the rounded remainder of the previous ones, so the sum carries 24 significant bits), which keeps
//     FP32 accuracy at bf16 matrix rate;
//   * T R, L U, Mq U (both operands FP32, 16 x 16 blocks): v_mfma_f32_16x16x4_f32.
// The triangular system is solved by blocks of 16: T_bb = (I + L_bb)^-1 for the two diagonal blocks
// by back substitution (VALU), then U_0 = T_00 R_0, U_1 = T_11 (R_1 - L_10 U_0).
// The decay products P(t, j) are running products (robust to underflow, no logarithms). Tokens past
// the end of the sequence are padded with k = q = v = 0, alpha = 1, beta = 0, which leave the state
// unchanged. A chunk's inputs are loaded into registers one chunk ahead and staged in LDS (two buffers).

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

constexpr int CH = 32;          // tokens per chunk
constexpr int NV = 16;          // value columns per workgroup
constexpr int KP = GDN_D + 8;   // LDS pitch (bf16) of a key / query row and of a state split row
constexpr int FP = 36;          // LDS pitch (floats) of the 32-wide tables
constexpr int WP = CH + 8;      // LDS pitch (bf16) of a w U split row

struct ChunkLds {
    __bf16 k[2][CH][KP];   // keys of the chunk (two buffers)
    __bf16 q[2][CH][KP];   // queries
    float v[2][NV][FP];    // the workgroup's value columns, value-major
    float beta[2][CH];
    float p[2][CH][FP];    // p[t][j] = P(t, j) for j <= t; p[t][32] = P(t, start)
    float l[CH][FP];       // L, row-major (blocks 00, 10, 11)
    float mq[CH][FP];      // Mq, row-major (blocks 00, 10, 11)
    float ti[CH][FP];      // T_00 and T_11, row-major
    float r[NV][FP];       // R, value-major
    float u[NV][FP];       // U, value-major
    __bf16 wu[3][NV][WP];  // P(end, j) beta_j U, split in three bf16 parts, value-major
    __bf16 s[3][NV][KP];   // S split in three bf16 parts, value-major
};

struct ChunkIn {
    qu32x4 k[2], q[2];  // 16-byte pieces tid and tid + 256 of the chunk: token piece / 16, keys 8 (piece % 16) ..
    uint32_t v[2];     // value elements tid and tid + 256: token e / 16, column e % 16
    float a, b;        // alpha, beta of token tid % 32
};

struct GdnIo {
    const uint16_t *k, *q, *v;  // this workgroup's key head, query head, first value column (row 0 of its sequence)
    const float *a, *b;         // its value head's gates
    int64_t ldk, ldq, ldv, lda, ldb;
};

__device__ __forceinline__ f32x4_t mma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A 16 x 16 x 16 FP32 product: lane (g, r) supplies A[r][4g .. 4g + 3] and B[4g .. 4g + 3][r]; the
// result lands as usual, lane (g, r) holding rows 4g .. 4g + 3 of column r (which is again the
// B-operand layout of a following product).
__device__ __forceinline__ f32x4_t mma16_f32(f32x4_t a, f32x4_t b, f32x4_t c) {
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ void split3(f32x4_t x, bf16x4_t& h, bf16x4_t& m, bf16x4_t& l) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = (__bf16)x[e];
        const float r1 = x[e] - (float)h[e];
        m[e] = (__bf16)r1;
        l[e] = (__bf16)(r1 - (float)m[e]);
    }
}

__device__ __forceinline__ void store_split(__bf16 (*dst)[NV][KP], int row, int col, f32x4_t x) {
    bf16x4_t h, m, l;
    split3(x, h, m, l);
    *reinterpret_cast<bf16x4_t*>(&dst[0][row][col]) = h;
    *reinterpret_cast<bf16x4_t*>(&dst[1][row][col]) = m;
    *reinterpret_cast<bf16x4_t*>(&dst[2][row][col]) = l;
}

__device__ __forceinline__ void load_chunk(ChunkIn& in, const GdnIo& io, int64_t c0, int64_t T, int tid) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int pc = tid + 256 * i;
        const int64_t row = std::min<int64_t>(c0 + (pc >> 4), T - 1);
        in.k[i] = *reinterpret_cast<const qu32x4*>(io.k + row * io.ldk + 8 * (pc & 15));
        in.q[i] = *reinterpret_cast<const qu32x4*>(io.q + row * io.ldq + 8 * (pc & 15));
        in.v[i] = io.v[row * io.ldv + (pc & 15)];
    }
    const int64_t row = std::min<int64_t>(c0 + (tid & 31), T - 1);
    in.a = io.a[row * io.lda];
    in.b = io.b[row * io.ldb];
}

// Writes a loaded chunk (n valid tokens) into LDS buffer bi; wave 1 builds its decay table.
__device__ __forceinline__ void stage_chunk(ChunkLds& sm, int bi, const ChunkIn& in, int n, int tid) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int pc = tid + 256 * i, t = pc >> 4, col = 8 * (pc & 15);
        const bool ok = t < n;
        const qu32x4 zero = {0u, 0u, 0u, 0u};
        *reinterpret_cast<qu32x4*>(&sm.k[bi][t][col]) = ok ? in.k[i] : zero;
        *reinterpret_cast<qu32x4*>(&sm.q[bi][t][col]) = ok ? in.q[i] : zero;
        sm.v[bi][pc & 15][t] = ok ? bf16_lo(in.v[i]) : 0.0f;
    }
    if ((tid >> 6) == 1) {
        const int lane = tid & 63, t = lane & 31;
        const float a = t < n ? in.a : 1.0f;
        if (lane < 32) sm.beta[bi][lane] = t < n ? in.b : 0.0f;
        // lane j < 32: P(t, j), the product of alpha_i for j < i <= t; lane 32: P(t, start)
        const int j = lane < 32 ? lane : -1;
        float pr = 1.0f;
#pragma unroll
        for (int tt = 0; tt < CH; ++tt) {
            const float at = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), tt));
            if (tt > j) pr *= at;
            if (lane <= 32) sm.p[bi][tt][lane] = pr;
        }
    }
}

// 16 x 16 tile of X K^T: lane (g, r) receives row t = 16 ti + r of X dotted with keys 16 tj + 4g + e.
__device__ __forceinline__ f32x4_t gram_tile(const __bf16 (*kk)[KP], const __bf16 (*xx)[KP], int ti, int tj, int g,
                                             int r) {
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < GDN_D / 32; ++ks)
        acc = mma_bf16(*reinterpret_cast<const bf16x8_t*>(&kk[16 * tj + r][32 * ks + 8 * g]),
                       *reinterpret_cast<const bf16x8_t*>(&xx[16 * ti + r][32 * ks + 8 * g]), acc);
    return acc;
}

// L (strict: j < t, weight P(t-1, j) beta_j) or Mq (j <= t, weight P(t, j) beta_j) from a gram tile.
template <bool STRICT>
__device__ __forceinline__ void decay_tile(ChunkLds& sm, int bi, float (*dst)[FP], int ti, int tj, int g, int r,
                                           f32x4_t x) {
    const int t = 16 * ti + r, j0 = 16 * tj + 4 * g;
    const int prow = STRICT ? (t > 0 ? t - 1 : 0) : t;
    const f32x4_t pv = *reinterpret_cast<const f32x4_t*>(&sm.p[bi][prow][j0]);
    const f32x4_t bv = *reinterpret_cast<const f32x4_t*>(&sm.beta[bi][j0]);
    f32x4_t out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = (STRICT ? j0 + e < t : j0 + e <= t) ? pv[e] * bv[e] * x[e] : 0.0f;
    *reinterpret_cast<f32x4_t*>(&dst[t][j0]) = out;
}

// T_bb = (I + L_bb)^-1 for diagonal block blk: lane (g, c) computes row c of T_bb by back substitution
// (row c of T solves y (I + L) = e_c) and writes its columns 4g .. 4g + 3.
__device__ __forceinline__ void invert_block(ChunkLds& sm, int blk, int g, int c) {
    float y[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) y[t] = t == c ? 1.0f : 0.0f;
#pragma unroll
    for (int j = 15; j >= 1; --j) {
        const float* lrow = &sm.l[16 * blk + j][16 * blk];
        float lv[16];
#pragma unroll
        for (int q4 = 0; q4 < (j + 3) / 4; ++q4) {
            const f32x4_t x = *reinterpret_cast<const f32x4_t*>(lrow + 4 * q4);
#pragma unroll
            for (int e = 0; e < 4; ++e) lv[4 * q4 + e] = x[e];
        }
#pragma unroll
        for (int t = 0; t < j; ++t) y[t] = __builtin_fmaf(-y[j], lv[t], y[t]);
    }
    f32x4_t out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = g == 0 ? y[e] : g == 1 ? y[4 + e] : g == 2 ? y[8 + e] : y[12 + e];
    *reinterpret_cast<f32x4_t*>(&sm.ti[16 * blk + c][16 * blk + 4 * g]) = out;
}

__global__ __launch_bounds__(256) void gdn_chunk_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const uint16_t* __restrict__ k, int64_t ldk,
    const uint16_t* __restrict__ v, int64_t ldv, const float* __restrict__ alpha, int64_t lda,
    const float* __restrict__ beta, int64_t ldb, float* __restrict__ state, int64_t T, int32_t Hv, int32_t group,
    float* __restrict__ o, int64_t ldo) {
    __shared__ __attribute__((aligned(16))) ChunkLds sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;
    constexpr int slices = GDN_D / NV;
    const int64_t bh = blockIdx.x / slices;  // b * Hv + h
    const int h = (int)(bh % Hv), slice = (int)(blockIdx.x % slices);
    const int64_t b = bh / Hv, r0 = b * T;
    const int hk = h / group;
    const GdnIo io{k + r0 * ldk + hk * GDN_D, q + r0 * ldq + hk * GDN_D, v + r0 * ldv + h * GDN_D + slice * NV,
                   alpha + r0 * lda + h, beta + r0 * ldb + h, ldk, ldq, ldv, lda, ldb};
    float* ob = o + r0 * ldo + h * GDN_D + slice * NV;

    // S rows (keys) 16 kt + 4g + e of column r, for this wave's key tiles kt = 2 wave, 2 wave + 1;
    // stored value-major, so the four rows are contiguous
    float* sg = state + bh * GDN_D * GDN_D + (int64_t)(slice * NV + r) * GDN_D + 32 * wave + 4 * g;
    f32x4_t S[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        S[kk] = *reinterpret_cast<const f32x4_t*>(sg + 16 * kk);
        store_split(sm.s, r, 32 * wave + 16 * kk + 4 * g, S[kk]);
    }

    const int64_t nch = (T + CH - 1) / CH;
    ChunkIn in;
    load_chunk(in, io, 0, T, tid);
    stage_chunk(sm, 0, in, (int)std::min<int64_t>(CH, T), tid);
    load_chunk(in, io, CH, T, tid);
    __syncthreads();

    for (int64_t ch = 0; ch < nch; ++ch) {
        const int bi = (int)(ch & 1);
        const int64_t c0 = ch * CH;
        const int n = (int)std::min<int64_t>(CH, T - c0);

        // ---- phase 1: K S0 (waves 0, 1) or Q S0 (waves 2, 3) for token tile wave % 2; the L and Mq
        // blocks; R = V - P(t-1, start) K S0
        const int tt = wave & 1;
        f32x4_t xs;
        {
            const __bf16 (*src)[KP] = wave < 2 ? sm.k[bi] : sm.q[bi];
            f32x4_t a0 = {0.0f, 0.0f, 0.0f, 0.0f}, a1 = a0, a2 = a0;
#pragma unroll
            for (int ks = 0; ks < GDN_D / 32; ++ks) {
                const bf16x8_t A = *reinterpret_cast<const bf16x8_t*>(&src[16 * tt + r][32 * ks + 8 * g]);
                a0 = mma_bf16(A, *reinterpret_cast<const bf16x8_t*>(&sm.s[0][r][32 * ks + 8 * g]), a0);
                a1 = mma_bf16(A, *reinterpret_cast<const bf16x8_t*>(&sm.s[1][r][32 * ks + 8 * g]), a1);
                a2 = mma_bf16(A, *reinterpret_cast<const bf16x8_t*>(&sm.s[2][r][32 * ks + 8 * g]), a2);
            }
            xs = (a2 + a1) + a0;
        }
        if (wave == 0) {
            decay_tile<true>(sm, bi, sm.l, 0, 0, g, r, gram_tile(sm.k[bi], sm.k[bi], 0, 0, g, r));
        } else if (wave == 1) {
            decay_tile<true>(sm, bi, sm.l, 1, 0, g, r, gram_tile(sm.k[bi], sm.k[bi], 1, 0, g, r));
        } else if (wave == 2) {
            decay_tile<true>(sm, bi, sm.l, 1, 1, g, r, gram_tile(sm.k[bi], sm.k[bi], 1, 1, g, r));
            decay_tile<false>(sm, bi, sm.mq, 0, 0, g, r, gram_tile(sm.k[bi], sm.q[bi], 0, 0, g, r));
        } else {
            decay_tile<false>(sm, bi, sm.mq, 1, 0, g, r, gram_tile(sm.k[bi], sm.q[bi], 1, 0, g, r));
            decay_tile<false>(sm, bi, sm.mq, 1, 1, g, r, gram_tile(sm.k[bi], sm.q[bi], 1, 1, g, r));
        }
        if (wave < 2) {
            const int t0 = 16 * tt + 4 * g;
            const f32x4_t vv = *reinterpret_cast<const f32x4_t*>(&sm.v[bi][r][t0]);
            f32x4_t rr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = t0 + e;
                const float gp = t > 0 ? sm.p[bi][t - 1][32] : 1.0f;
                rr[e] = vv[e] - gp * xs[e];
            }
            *reinterpret_cast<f32x4_t*>(&sm.r[r][t0]) = rr;
        }
        __syncthreads();

        // ---- phase 2: T_00, T_11
        if (wave < 2) invert_block(sm, wave, g, r);
        __syncthreads();

        // ---- phase 3: U_0 = T_00 R_0, U_1 = T_11 (R_1 - L_10 U_0); U and w U to LDS
        if (wave == 0) {
            const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
            const f32x4_t R0 = *reinterpret_cast<const f32x4_t*>(&sm.r[r][4 * g]);
            const f32x4_t R1 = *reinterpret_cast<const f32x4_t*>(&sm.r[r][16 + 4 * g]);
            const f32x4_t U0 = mma16_f32(*reinterpret_cast<const f32x4_t*>(&sm.ti[r][4 * g]), R0, zero);
            const f32x4_t Y = mma16_f32(*reinterpret_cast<const f32x4_t*>(&sm.l[16 + r][4 * g]), U0, zero);
            const f32x4_t U1 = mma16_f32(*reinterpret_cast<const f32x4_t*>(&sm.ti[16 + r][16 + 4 * g]), R1 - Y, zero);
            *reinterpret_cast<f32x4_t*>(&sm.u[r][4 * g]) = U0;
            *reinterpret_cast<f32x4_t*>(&sm.u[r][16 + 4 * g]) = U1;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int t0 = 16 * half + 4 * g;
                const f32x4_t pe = {sm.p[bi][CH - 1][t0], sm.p[bi][CH - 1][t0 + 1], sm.p[bi][CH - 1][t0 + 2],
                                    sm.p[bi][CH - 1][t0 + 3]};
                const f32x4_t be = *reinterpret_cast<const f32x4_t*>(&sm.beta[bi][t0]);
                const f32x4_t uu = half ? U1 : U0;
                const f32x4_t wu = (pe * be) * uu;
                bf16x4_t hh, mm, ll;
                split3(wu, hh, mm, ll);
                *reinterpret_cast<bf16x4_t*>(&sm.wu[0][r][t0]) = hh;
                *reinterpret_cast<bf16x4_t*>(&sm.wu[1][r][t0]) = mm;
                *reinterpret_cast<bf16x4_t*>(&sm.wu[2][r][t0]) = ll;
            }
        }
        __syncthreads();

        // ---- phase 4: outputs (waves 2, 3), S update (all), next chunk staged
        if (wave >= 2) {
            const int t0 = 16 * tt + 4 * g;
            f32x4_t acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = sm.p[bi][t0 + e][32] * xs[e];
            acc = mma16_f32(*reinterpret_cast<const f32x4_t*>(&sm.mq[16 * tt + r][4 * g]),
                            *reinterpret_cast<const f32x4_t*>(&sm.u[r][4 * g]), acc);
            if (tt == 1)
                acc = mma16_f32(*reinterpret_cast<const f32x4_t*>(&sm.mq[16 + r][16 + 4 * g]),
                                *reinterpret_cast<const f32x4_t*>(&sm.u[r][16 + 4 * g]), acc);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (t0 + e < n) ob[(c0 + t0 + e) * ldo + r] = acc[e];
        }
        {
            const bf16x8_t B0 = *reinterpret_cast<const bf16x8_t*>(&sm.wu[0][r][8 * g]);
            const bf16x8_t B1 = *reinterpret_cast<const bf16x8_t*>(&sm.wu[1][r][8 * g]);
            const bf16x8_t B2 = *reinterpret_cast<const bf16x8_t*>(&sm.wu[2][r][8 * g]);
            const float gend = sm.p[bi][CH - 1][32];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int key = 32 * wave + 16 * kk + r;
                bf16x8_t A;
#pragma unroll
                for (int e = 0; e < 8; ++e) A[e] = sm.k[bi][8 * g + e][key];
                f32x4_t acc = gend * S[kk];
                acc = mma_bf16(A, B2, acc);
                acc = mma_bf16(A, B1, acc);
                acc = mma_bf16(A, B0, acc);
                S[kk] = acc;
            }
        }
        // the state split was last read in phase 1, buffer bi ^ 1 in the previous chunk
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) store_split(sm.s, r, 32 * wave + 16 * kk + 4 * g, S[kk]);
        if (ch + 1 < nch) {
            stage_chunk(sm, bi ^ 1, in, (int)std::min<int64_t>(CH, T - c0 - CH), tid);
            load_chunk(in, io, c0 + 2 * CH, T, tid);
        }
        __syncthreads();
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) *reinterpret_cast<f32x4_t*>(sg + 16 * kk) = S[kk];
}

}  // namespace

hipError_t launch_gdn_recurrence(const uint16_t* q, int64_t ldq, const uint16_t* k, int64_t ldk, const uint16_t* v,
                                 int64_t ldv, const float* alpha, int64_t lda, const float* beta, int64_t ldb,
                                 float* state, int64_t B, int64_t T, int32_t Hv, int32_t Hk, float* o, int64_t ldo,
                                 hipStream_t stream) {
    if (B == 0 || T == 0) return hipSuccess;
    const int64_t grid = B * Hv * (GDN_D / 16);
    if (grid > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
    if (T >= GDN_CHUNK_MIN_T)
        hipLaunchKernelGGL(gdn_chunk_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, q, ldq, k, ldk, v, ldv, alpha,
                           lda, beta, ldb, state, T, Hv, Hv / Hk, o, ldo);
    else
        hipLaunchKernelGGL(T >= 16 ? gdn_recurrence_kernel<8> : gdn_recurrence_kernel<1>, dim3((uint32_t)grid),
                           dim3(256), 0, stream, q, ldq, k, ldk, v, ldv, alpha, lda, beta, ldb, state, T, Hv, Hv / Hk,
                           o, ldo);
    return hipGetLastError();
}

}  // namespace nvfp4
