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
// Two forms of the same recurrence: token by token (decode-sized calls, below) and chunked (prefill,
// further down): the recurrence unrolled exactly over 32-token chunks, so that most of its work
// becomes matrix products.
//
// Token by token: the value columns of S evolve independently (the delta rule couples key rows only),
// so a wave owns 4 columns of one head's state, 8 key rows per lane: lane = 16 * column + row group.
// Both dot products over the key dimension are reduced inside a 16-lane row with DPP (quad swaps, then
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
// This is the recurrence unrolled over the chunk, exact up to rounding. Everything built from k, q,
// alpha and beta alone (the decay products, T = (I + L)^-1, Mq and the gate vectors) does not depend
// on the state; a first kernel computes it for every (sequence, value head, chunk) at once into the
// caller's workspace. Only S0 -> R -> U -> S_end runs chunk after chunk, in a second kernel where each
// workgroup owns 16 value columns of one head (the columns evolve independently) and holds its
// 128 x 16 slice of S in registers (FP32), each of its four waves 32 key rows.
// The matrix products run on the matrix cores:
//   * K K^T, K Q^T (bf16 inputs: the products are exact, FP32 sums): v_mfma_f32_16x16x32_bf16;
//   * K S0, Q S0, K^T (w U): the FP32 operand is split into three bf16 parts x = h + m + l (each part
//     the rounded remainder of the previous ones, so the sum carries 24 significant bits), which keeps
//     FP32 accuracy at bf16 matrix rate;
//   * T R, Mq U and the off-diagonal blocks of T (both operands FP32): v_mfma_f32_16x16x4_f32.
// T is formed by 16-blocks: T_ii = (I + L_ii)^-1 by back substitution, then level by level
// T_ij = -T_ii sum_{j <= k < i} L_ik T_kj. The decay products P(t, j) are running products (robust to
// underflow, no logarithms). Tokens past the end of the sequence are padded with k = q = v = 0,
// alpha = 1, beta = 0, which leave the state unchanged.
// Per chunk the sequential kernel has three phases separated by two barriers: (1) every wave's key
// rows of K S0 and Q S0; (2) wave w builds R_0 .. R_w and U_w = sum_j T_wj R_j, and the next chunk is
// staged; (3) wave w writes the outputs of token tile 3 - w (so each wave does five 16-block products
// per chunk) and updates its key rows of S.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

constexpr int CH = 64;          // tokens per chunk
constexpr int NTT = CH / 16;    // token tiles of 16 per chunk
constexpr int NV = 16;          // value columns per workgroup of the sequential kernel
constexpr int KP = GDN_D + 8;   // LDS pitch (bf16) of a key / query row
constexpr int FP = CH + 4;      // LDS pitch (floats) of the chunk-wide tables (column CH: P(t, start))
constexpr int WP = CH + 8;      // LDS pitch (bf16) of a w U split row
constexpr int NBLK = NTT * (NTT + 1) / 2;  // 16 x 16 blocks on and below the diagonal

// Lower-triangular 16-block (i, j), j <= i, stored at i (i + 1) / 2 + j.
__host__ __device__ constexpr int blk(int i, int j) { return i * (i + 1) / 2 + j; }

// What the sequential kernel needs of one chunk of one (sequence, value head), state aside.
struct ChunkFactors {
    float t[NBLK][16][16];   // T = (I + L)^-1: its lower blocks, row-major
    float mq[NBLK][16][16];  // Mq[t][j] = P(t, j) beta_j (q_t . k_j), j <= t: lower blocks
    float gp[CH];            // P(t-1, start), the weight of S0^T k_t in R
    float ga[CH];            // P(t, start), the weight of S0^T q_t in O
    float w[CH];             // P(end, j) beta_j, the weight of k_j u_j^T in the state update
    float gend[CH];          // [0]: P(end, start); the rest unused
};
static_assert(sizeof(ChunkFactors) % 16 == 0, "chunk factors keep 16-byte alignment");

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

__device__ __forceinline__ f32x4_t ld4(const float* p) { return *reinterpret_cast<const f32x4_t*>(p); }

__device__ __forceinline__ void split3(f32x4_t x, bf16x4_t& h, bf16x4_t& m, bf16x4_t& l) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = (__bf16)x[e];
        const float r1 = x[e] - (float)h[e];
        m[e] = (__bf16)r1;
        l[e] = (__bf16)(r1 - (float)m[e]);
    }
}

constexpr int BUF_FLAGS = 0x00020000;  // raw buffer resource, 32-bit data format (gfx9 family)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, BUF_FLAGS);
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
__device__ __forceinline__ void decay_tile(const float (*p)[FP], const float* beta, float (*dst)[FP], bool strict,
                                           int ti, int tj, int g, int r, f32x4_t x) {
    const int t = 16 * ti + r, j0 = 16 * tj + 4 * g;
    const f32x4_t pv = ld4(&p[strict ? (t > 0 ? t - 1 : 0) : t][j0]);
    const f32x4_t bv = ld4(&beta[j0]);
    f32x4_t out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = (strict ? j0 + e < t : j0 + e <= t) ? pv[e] * bv[e] * x[e] : 0.0f;
    *reinterpret_cast<f32x4_t*>(&dst[t][j0]) = out;
}

// T_bb = (I + L_bb)^-1 for diagonal block bb: lane (g, c) computes row c of T_bb by back substitution
// (row c of T solves y (I + L) = e_c; y_t = 0 for t > c, y_c = 1); lanes of group 0 write it.
__device__ __forceinline__ void invert_block(const float (*l)[FP], float (*ti)[FP], int bb, int g, int c) {
    float y[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) y[t] = 0.0f;
#pragma unroll
    for (int j = 15; j >= 1; --j) {
        // y_j is final here: 1 at j = c, 0 above c, and below c complete after the updates from j + 1 ..
        const float yv = j > c ? 0.0f : (j == c ? 1.0f : y[j]);
        const float* lrow = &l[16 * bb + j][16 * bb];
#pragma unroll
        for (int q4 = 0; q4 < (j + 3) / 4; ++q4) {
            const f32x4_t x = ld4(lrow + 4 * q4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * q4 + e < j) y[4 * q4 + e] = __builtin_fmaf(-yv, x[e], y[4 * q4 + e]);
        }
    }
    if (g == 0) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            f32x4_t out;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * q4 + e;
                out[e] = t > c ? 0.0f : (t == c ? 1.0f : y[t]);
            }
            *reinterpret_cast<f32x4_t*>(&ti[16 * bb + c][16 * bb + 4 * q4]) = out;
        }
    }
}

// Off-diagonal block T_ij = -T_ii sum_{j <= k < i} L_ik T_kj (from (I + L) T = I, row block i).
__device__ __forceinline__ void offdiag_block(const float (*l)[FP], float (*ti)[FP], int i, int j, int g, int r) {
    f32x4_t X = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = j; k < i; ++k) {
        const f32x4_t tkj = {ti[16 * k + 4 * g][16 * j + r], ti[16 * k + 4 * g + 1][16 * j + r],
                             ti[16 * k + 4 * g + 2][16 * j + r], ti[16 * k + 4 * g + 3][16 * j + r]};
        X = mma16_f32(ld4(&l[16 * i + r][16 * k + 4 * g]), tkj, X);
    }
    const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4_t Y = mma16_f32(ld4(&ti[16 * i + r][16 * i + 4 * g]), X, zero);
#pragma unroll
    for (int e = 0; e < 4; ++e) ti[16 * i + 4 * g + e][16 * j + r] = -Y[e];
}

// Keys and queries are dead once the gram tiles are in registers, so L and T reuse their space
// (about 52 KB in all: three workgroups per CU).
struct PrepLds {
    union {
        struct {
            __bf16 k[CH][KP];
            __bf16 q[CH][KP];
        } in;
        struct {
            float l[CH][FP];   // L, row-major (lower blocks)
            float ti[CH][FP];  // T, row-major (lower blocks)
        } tri;
    };
    float p[CH][FP];  // p[t][j] = P(t, j) for j <= t; p[t][CH] = P(t, start)
    float beta[CH];
};

// One workgroup per (sequence, value head, chunk): blockIdx = (b Hv + h) nch + c.
__global__ __launch_bounds__(256) void gdn_chunk_prep_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const uint16_t* __restrict__ k, int64_t ldk,
    const float* __restrict__ alpha, int64_t lda, const float* __restrict__ beta, int64_t ldb, int64_t T, int32_t Hv,
    int32_t group, int64_t nch, ChunkFactors* __restrict__ fac) {
    __shared__ __attribute__((aligned(16))) PrepLds sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;
    const int64_t c = blockIdx.x % nch, bh = blockIdx.x / nch;
    const int h = (int)(bh % Hv);
    const int64_t b = bh / Hv, c0 = c * CH;
    const int hk = h / group;
    const int n = (int)std::min<int64_t>(CH, T - c0);
    ChunkFactors* F = fac + blockIdx.x;

    // keys and queries of the chunk; rows past the sequence read as zeros (bounds-checked loads)
    {
        const int64_t row0 = b * T + c0;
        const __amdgpu_buffer_rsrc_t rk = rsrc(k + row0 * ldk + hk * GDN_D, (int64_t)n * ldk * 2);
        const __amdgpu_buffer_rsrc_t rq = rsrc(q + row0 * ldq + hk * GDN_D, (int64_t)n * ldq * 2);
#pragma unroll
        for (int m = 0; m < CH * 16 / 256; ++m) {
            const int pc = tid + 256 * m, t = pc >> 4, col = 8 * (pc & 15);
            *reinterpret_cast<qu32x4*>(&sm.in.k[t][col]) =
                __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(t * (uint32_t)ldk * 2u + 2u * col), 0, 0);
            *reinterpret_cast<qu32x4*>(&sm.in.q[t][col]) =
                __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(t * (uint32_t)ldq * 2u + 2u * col), 0, 0);
        }
    }
    float a = 1.0f;
    if (wave == 0) {  // lane t: alpha_t, beta_t (padding: alpha 1, beta 0)
        const int64_t row = b * T + std::min<int64_t>(c0 + lane, T - 1);
        const float av = alpha[row * lda + h], bv = beta[row * ldb + h];
        a = lane < n ? av : 1.0f;
        sm.beta[lane] = lane < n ? bv : 0.0f;
    }
    __syncthreads();

    // wave 0: decay table; waves 1-3: the 20 gram tiles (10 of K K^T for L, 10 of K Q^T for Mq)
    constexpr int JOBS_PER_WAVE = 7;
    f32x4_t G[JOBS_PER_WAVE];
    if (wave == 0) {
        // lane j: P(t, j), the product of alpha_i for j < i <= t
        float pr = 1.0f;
#pragma unroll
        for (int tt = 0; tt < CH; ++tt) {
            const float at = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), tt));
            if (tt > lane) pr *= at;
            sm.p[tt][lane] = pr;
        }
        // P(t, start) = alpha_0 P(t, 0)
        const float a0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 0));
        sm.p[lane][CH] = a0 * sm.p[lane][0];
    } else {
#pragma unroll
        for (int s = 0; s < JOBS_PER_WAVE; ++s) {
            const int job = JOBS_PER_WAVE * (wave - 1) + s;
            if (job < 2 * NBLK) {
                const int tri = job % NBLK;
                const int ti = tri >= 6 ? 3 : tri >= 3 ? 2 : tri >= 1 ? 1 : 0, tj = tri - blk(ti, 0);
                G[s] = gram_tile(sm.in.k, job < NBLK ? sm.in.k : sm.in.q, ti, tj, g, r);
            }
        }
    }
    __syncthreads();  // every gram tile is in registers: the key and query space is free

    if (wave == 0) {
        F->gp[lane] = lane > 0 ? sm.p[lane - 1][CH] : 1.0f;
        F->ga[lane] = sm.p[lane][CH];
        F->w[lane] = sm.p[CH - 1][lane] * sm.beta[lane];
        F->gend[lane] = sm.p[CH - 1][CH];
    } else {
#pragma unroll
        for (int s = 0; s < JOBS_PER_WAVE; ++s) {
            const int job = JOBS_PER_WAVE * (wave - 1) + s;
            if (job < 2 * NBLK) {
                const int tri = job % NBLK;
                const int ti = tri >= 6 ? 3 : tri >= 3 ? 2 : tri >= 1 ? 1 : 0, tj = tri - blk(ti, 0);
                if (job < NBLK) {
                    decay_tile(sm.p, sm.beta, sm.tri.l, true, ti, tj, g, r, G[s]);
                } else {  // Mq goes straight to the chunk factors: lane (g, r) holds row r, columns 4g ..
                    const int t = 16 * ti + r, j0 = 16 * tj + 4 * g;
                    const f32x4_t pv = ld4(&sm.p[t][j0]), bv = ld4(&sm.beta[j0]);
                    f32x4_t out;
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = j0 + e <= t ? pv[e] * bv[e] * G[s][e] : 0.0f;
                    *reinterpret_cast<f32x4_t*>(&F->mq[tri][r][4 * g]) = out;
                }
            }
        }
    }
    __syncthreads();

    invert_block(sm.tri.l, sm.tri.ti, wave, g, r);  // T_ww
    __syncthreads();
    if (wave < 3) offdiag_block(sm.tri.l, sm.tri.ti, wave + 1, wave, g, r);  // T_10, T_21, T_32
    __syncthreads();
    if (wave < 2) offdiag_block(sm.tri.l, sm.tri.ti, wave + 2, wave, g, r);  // T_20, T_31
    __syncthreads();
    if (wave == 0) offdiag_block(sm.tri.l, sm.tri.ti, 3, 0, g, r);  // T_30
    __syncthreads();

    // the lower blocks of T, 16 bytes per thread and round: piece = block * 64 + row * 4 + quarter
#pragma unroll
    for (int m = 0; m < (NBLK * 64 + 255) / 256; ++m) {
        const int pc = tid + 256 * m;
        if (pc < NBLK * 64) {
            const int bk = pc >> 6, row = (pc >> 2) & 15, col = 4 * (pc & 3);
            const int bi = bk >= 6 ? 3 : bk >= 3 ? 2 : bk >= 1 ? 1 : 0, bj = bk - blk(bi, 0);
            *reinterpret_cast<f32x4_t*>(&F->t[bk][row][col]) = ld4(&sm.tri.ti[16 * bi + row][16 * bj + col]);
        }
    }
}

// The chunk factors wave w of the sequential kernel reads (loaded a chunk ahead; the same number of
// loads in every wave): rows r, columns 4g .. 4g + 3 of T_wj and Mq_oj (o = 3 - w, the output tile
// of wave w), j = 0 .. 3 (blocks past the diagonal repeat the diagonal one, unused); gp of every token
// tile; ga of tile o; w of tile w; P(end, start).
struct FactorRegs {
    f32x4_t t[NTT], mq[NTT], gp[NTT];
    f32x4_t ga, wt;
    float gend;
};

// A chunk's keys, queries and value columns, staged by thread i (0 .. 255): 16-byte pieces i + 256 m
// (token piece / 16, elements 8 (piece % 16) ..) and value elements i + 256 m (token e / 16, column
// e % 16), m = 0 .. 3.
constexpr int PIECES = CH * 16 / 256;
struct PieceRegs {
    qu32x4 k[PIECES], q[PIECES];
    uint32_t v[PIECES];
};

struct MainLds {
    __bf16 k[2][CH][KP];            // keys of chunks c and c + 1
    __bf16 q[2][CH][KP];            // queries
    float v[2][NV][FP];             // the workgroup's value columns, value-major
    f32x4_t red[4][2 * NTT][64];    // partial K S0 and Q S0 tiles of each wave's key rows
    float u[NV][FP];                // U, value-major
    __bf16 wu[3][NV][WP];           // w U split in three bf16 parts, value-major
};

__device__ __forceinline__ void load_factors(FactorRegs& fr, const ChunkFactors* F, int wave, int g, int r,
                                             int vzero) {
    const int o = 3 - wave, off = 16 * r + 4 * g;
#pragma unroll
    for (int j = 0; j < NTT; ++j) {
        fr.t[j] = ld4(&F->t[blk(wave, j <= wave ? j : wave)][0][0] + off);
        fr.mq[j] = ld4(&F->mq[blk(o, j <= o ? j : o)][0][0] + off);
        fr.gp[j] = ld4(F->gp + 16 * j + 4 * g);
    }
    fr.ga = ld4(F->ga + 16 * o + 4 * g);
    fr.wt = ld4(F->w + 16 * wave + 4 * g);
    fr.gend = F->gend[vzero];  // a vector load (see the note at the token-by-token kernel)
}

// Per-thread byte offsets of a thread's pieces inside a chunk (the same for every chunk).
struct PieceOffs {
    uint32_t k[PIECES], q[PIECES], v[PIECES];
};

__device__ __forceinline__ PieceOffs piece_offsets(int64_t ldk, int64_t ldq, int64_t ldv, int i) {
    PieceOffs po;
#pragma unroll
    for (int m = 0; m < PIECES; ++m) {
        const uint32_t t = (uint32_t)((i >> 4) + 16 * m);
        po.k[m] = t * (uint32_t)ldk * 2u + 16u * (uint32_t)(i & 15);
        po.q[m] = t * (uint32_t)ldq * 2u + 16u * (uint32_t)(i & 15);
        po.v[m] = t * (uint32_t)ldv * 2u + 2u * (uint32_t)(i & 15);
    }
    return po;
}

// Buffer loads of chunk cl: each descriptor spans exactly the chunk's rows inside the sequence, so
// the hardware returns zeros for the padding rows past the end (and for a chunk past the end).
__device__ __forceinline__ void load_pieces(PieceRegs& pr, const PieceOffs& po, const uint16_t* kb, int64_t ldk,
                                            const uint16_t* qb, int64_t ldq, const uint16_t* vb, int64_t ldv,
                                            int64_t cl, int64_t T) {
    const int64_t c0 = cl * CH;
    const int64_t nv = std::max<int64_t>(0, std::min<int64_t>(CH, T - c0));
    const __amdgpu_buffer_rsrc_t rk = rsrc(kb + c0 * ldk, nv * ldk * 2);
    const __amdgpu_buffer_rsrc_t rq = rsrc(qb + c0 * ldq, nv * ldq * 2);
    const __amdgpu_buffer_rsrc_t rv = rsrc(vb + c0 * ldv, nv * ldv * 2);
#pragma unroll
    for (int m = 0; m < PIECES; ++m) {
        pr.k[m] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)po.k[m], 0, 0);
        pr.q[m] = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)po.q[m], 0, 0);
        pr.v[m] = __builtin_amdgcn_raw_buffer_load_b16(rv, (int)po.v[m], 0, 0);
    }
}

__device__ __forceinline__ void stage_pieces(MainLds& sm, int bi, const PieceRegs& pr, int i) {
#pragma unroll
    for (int m = 0; m < PIECES; ++m) {
        const int pc = i + 256 * m, t = pc >> 4, col = 8 * (pc & 15);
        *reinterpret_cast<qu32x4*>(&sm.k[bi][t][col]) = pr.k[m];
        *reinterpret_cast<qu32x4*>(&sm.q[bi][t][col]) = pr.q[m];
        sm.v[bi][pc & 15][t] = bf16_lo(pr.v[m]);
    }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(qu32x2 lo, qu32x2 hi) {
    const qu32x4 x = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8_t, x);
}

__global__ __launch_bounds__(256) void gdn_chunk_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const uint16_t* __restrict__ k, int64_t ldk,
    const uint16_t* __restrict__ v, int64_t ldv, float* __restrict__ state, int64_t T, int32_t Hv, int32_t group,
    int64_t nch, int64_t nbh, const ChunkFactors* __restrict__ fac, float* __restrict__ o, int64_t ldo) {
    __shared__ __attribute__((aligned(16))) MainLds sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;
    const int ot = 3 - wave;  // the output tile of this wave (its U tile is wave)
    // Workgroups are dealt to the 8 XCDs round-robin; the 8 value slices of one (sequence, head) go to
    // one XCD (its L2 then serves their shared keys, queries and chunk factors, and whole value rows):
    // workgroup i -> head 8 (i / 64) + i % 8, slice (i / 8) % 8. The grid is rounded up to 64.
    const int64_t bh = 8 * (int64_t)(blockIdx.x / 64) + blockIdx.x % 8;  // b * Hv + h
    if (bh >= nbh) return;
    const int h = (int)(bh % Hv), slice = (int)((blockIdx.x / 8) % 8);
    const int64_t b = bh / Hv, r0 = b * T;
    const int hk = h / group;
    const uint16_t* kb = k + r0 * ldk + hk * GDN_D;
    const uint16_t* qb = q + r0 * ldq + hk * GDN_D;
    const uint16_t* vb = v + r0 * ldv + h * GDN_D + slice * NV;
    const ChunkFactors* Fh = fac + bh * nch;
    float* ob = o + r0 * ldo + h * GDN_D + slice * NV;
    int vzero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));

    // S rows (keys) 32 wave + 16 kk + 4g + e of column r; value-major in memory, so the four rows are
    // contiguous
    float* sg = state + bh * GDN_D * GDN_D + (int64_t)(slice * NV + r) * GDN_D + 32 * wave + 4 * g;
    f32x4_t S[2] = {ld4(sg), ld4(sg + 16)};

    // Every wave issues the same sequence of vector memory instructions, so that the compiler can
    // count what is in flight and waits for a load only where its data is used.
    PieceRegs pieces;
    const PieceOffs po = piece_offsets(ldk, ldq, ldv, tid);
    load_pieces(pieces, po, kb, ldk, qb, ldq, vb, ldv, 0, T);
    stage_pieces(sm, 0, pieces, tid);
    load_pieces(pieces, po, kb, ldk, qb, ldq, vb, ldv, 1, T);
    FactorRegs nxt;
    load_factors(nxt, Fh, wave, g, r, vzero);
    __syncthreads();

    for (int64_t c = 0; c < nch; ++c) {
        const int bi = (int)(c & 1);
        const FactorRegs cur = nxt;
        load_factors(nxt, Fh + (c + 1 < nch ? c + 1 : c), wave, g, r, vzero);

        // ---- phase 1: this wave's 32 key rows of K S0 and Q S0 for the 4 token tiles. The matrix
        // instruction's 8 k-slots of lane group g hold keys 32w + 4g + e and 32w + 16 + 4g + e, which are
        // exactly the state rows the lane holds.
        bf16x8_t B[3];
        {
            bf16x4_t h0, m0, l0, h1, m1, l1;
            split3(S[0], h0, m0, l0);
            split3(S[1], h1, m1, l1);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                B[0][e] = h0[e];
                B[0][4 + e] = h1[e];
                B[1][e] = m0[e];
                B[1][4 + e] = m1[e];
                B[2][e] = l0[e];
                B[2][4 + e] = l1[e];
            }
        }
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int t2 = 0; t2 < NTT; ++t2) {
                const __bf16* row = x == 0 ? &sm.k[bi][16 * t2 + r][32 * wave + 4 * g]
                                           : &sm.q[bi][16 * t2 + r][32 * wave + 4 * g];
                const bf16x8_t A = as_bf16x8(*reinterpret_cast<const qu32x2*>(row),
                                             *reinterpret_cast<const qu32x2*>(row + 16));
                f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
                acc = mma_bf16(A, B[2], acc);
                acc = mma_bf16(A, B[1], acc);
                acc = mma_bf16(A, B[0], acc);
                sm.red[wave][NTT * x + t2][lane] = acc;
            }
        __syncthreads();

        // ---- phase 2: U_w = sum_{j <= w} T_wj R_j with R_j = V_j - P(t-1, start) K_j S0 (each wave
        // rebuilds the R tiles it needs); P(t, start) Q S0 of the output tile; the next chunk staged
        // (its buffer was last read before the barrier above) and the one after it loaded; the state
        // update's K^T operands (independent of U) read before the barrier.
        {
            const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
            f32x4_t U = zero;
#pragma unroll
            for (int j = 0; j < NTT; ++j) {
                if (j > wave) break;
                const f32x4_t ks =
                    ((sm.red[0][j][lane] + sm.red[1][j][lane]) + sm.red[2][j][lane]) + sm.red[3][j][lane];
                const f32x4_t R = ld4(&sm.v[bi][r][16 * j + 4 * g]) - cur.gp[j] * ks;
                U = mma16_f32(cur.t[j], R, U);
            }
            const int t0 = 16 * wave + 4 * g;
            *reinterpret_cast<f32x4_t*>(&sm.u[r][t0]) = U;
            bf16x4_t hh, mm, ll;
            split3(cur.wt * U, hh, mm, ll);
            *reinterpret_cast<bf16x4_t*>(&sm.wu[0][r][t0]) = hh;
            *reinterpret_cast<bf16x4_t*>(&sm.wu[1][r][t0]) = mm;
            *reinterpret_cast<bf16x4_t*>(&sm.wu[2][r][t0]) = ll;
        }
        const f32x4_t qs = ((sm.red[0][NTT + ot][lane] + sm.red[1][NTT + ot][lane]) + sm.red[2][NTT + ot][lane]) +
                           sm.red[3][NTT + ot][lane];
        const f32x4_t xs = cur.ga * qs;
        // also past the end (zeros into the free buffer), so the loads in flight are the same every time
        stage_pieces(sm, bi ^ 1, pieces, tid);
        load_pieces(pieces, po, kb, ldk, qb, ldq, vb, ldv, c + 2, T);
        bf16x8_t KT[2][2];  // [key tile][token half]
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int e = 0; e < 8; ++e) KT[kk][hf][e] = sm.k[bi][32 * hf + 8 * g + e][32 * wave + 16 * kk + r];
        __syncthreads();

        // ---- phase 3: outputs of tile ot = 3 - w (so every wave does 5 block products per chunk) and
        // the state update of each wave's key rows
        {
            f32x4_t acc = xs;
#pragma unroll
            for (int j = 0; j < NTT; ++j) {
                if (j > ot) break;
                acc = mma16_f32(cur.mq[j], ld4(&sm.u[r][16 * j + 4 * g]), acc);
            }
            // bounds-checked stores: rows past the end of the sequence fall outside the descriptor
            const int rows = (int)std::min<int64_t>(CH, T - c * CH);
            const __amdgpu_buffer_rsrc_t ro = rsrc(ob + c * CH * ldo, ((int64_t)(rows - 1) * ldo + NV) * 4);
            const int t0 = 16 * ot + 4 * g;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[e]), ro,
                                                      (int)(((t0 + e) * (uint32_t)ldo + r) * 4u), 0, 0);
        }
        {
            bf16x8_t W[2][3];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int x = 0; x < 3; ++x)
                    W[hf][x] = *reinterpret_cast<const bf16x8_t*>(&sm.wu[x][r][32 * hf + 8 * g]);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                f32x4_t acc = cur.gend * S[kk];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    acc = mma_bf16(KT[kk][hf], W[hf][2], acc);
                    acc = mma_bf16(KT[kk][hf], W[hf][1], acc);
                    acc = mma_bf16(KT[kk][hf], W[hf][0], acc);
                }
                S[kk] = acc;
            }
        }
    }
    *reinterpret_cast<f32x4_t*>(sg) = S[0];
    *reinterpret_cast<f32x4_t*>(sg + 16) = S[1];
}

}  // namespace

size_t gdn_workspace_bytes(int64_t B, int64_t T, int32_t Hv) {
    if (B <= 0 || T < GDN_CHUNK_MIN_T || Hv <= 0) return 0;
    return (size_t)B * (size_t)Hv * (size_t)((T + CH - 1) / CH) * sizeof(ChunkFactors);
}

hipError_t launch_gdn_recurrence(const uint16_t* q, int64_t ldq, const uint16_t* k, int64_t ldk, const uint16_t* v,
                                 int64_t ldv, const float* alpha, int64_t lda, const float* beta, int64_t ldb,
                                 float* state, int64_t B, int64_t T, int32_t Hv, int32_t Hk, float* o, int64_t ldo,
                                 void* workspace, hipStream_t stream) {
    if (B == 0 || T == 0) return hipSuccess;
    const int64_t grid = B * Hv * (GDN_D / 16);
    if (grid > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
    if (T >= GDN_CHUNK_MIN_T) {
        const int64_t nch = (T + CH - 1) / CH;
        if (B * Hv * nch > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
        ChunkFactors* fac = static_cast<ChunkFactors*>(workspace);
        hipLaunchKernelGGL(gdn_chunk_prep_kernel, dim3((uint32_t)(B * Hv * nch)), dim3(256), 0, stream, q, ldq, k, ldk,
                           alpha, lda, beta, ldb, T, Hv, Hv / Hk, nch, fac);
        const int64_t nbh = B * Hv;
        hipLaunchKernelGGL(gdn_chunk_kernel, dim3((uint32_t)((nbh + 7) / 8 * 64)), dim3(256), 0, stream, q, ldq, k,
                           ldk, v, ldv, state, T, Hv, Hv / Hk, nch, nbh, fac, o, ldo);
    } else {
        hipLaunchKernelGGL(T >= 16 ? gdn_recurrence_kernel<8> : gdn_recurrence_kernel<1>, dim3((uint32_t)grid),
                           dim3(256), 0, stream, q, ldq, k, ldk, v, ldv, alpha, lda, beta, ldb, state, T, Hv, Hv / Hk,
                           o, ldo);
    }
    return hipGetLastError();
}

}  // namespace nvfp4
