// Skinny block-scaled W4A4 GEMM for decode (M <= 64 activation rows), for gfx950 (CDNA4).
//
//   y[m, n] = g_a * g_w[seg(n)] * sum_k e2m1(qa[m,k]) sa[m,k/16] * e2m1(qw[n,k]) sw[n,k/16]
//
// Same product, segment table and epilogues as the tiled kernel. With a handful of activation rows
// against an N x K weight matrix the weights are nearly all of the traffic, and the kernel is bound
// by HBM: every weight byte has to be read once, by enough waves to keep HBM busy, while the
// activation rows (a few hundred KB at most) are re-read from L2.
//
// Design:
//  * One workgroup per 16*NT weight rows (output columns). Its KW waves split K into contiguous
//    ranges of 256-element chunks; KW depends on K alone, so the order of the additions, and with it
//    every output bit, does not depend on N, the column tile or the segment table (a fused GEMM and
//    the same modules called one by one agree bitwise).
//  * Operands go straight from global memory into registers: each weight byte is used by exactly
//    one wave, so staging through LDS would buy nothing. Lane (r, g), r = lane % 16 and
//    g = lane / 16, loads the 32 code bytes (64 elements) at byte 32g of row r's 128-byte chunk and
//    the 4 scale bytes of those elements. Activation rows are loaded the same way, so lane group g
//    holds the same K elements of both operands, as the matrix instruction requires; within a chunk
//    the 256 elements are thus summed in a permuted order, which a sum does not depend on.
//  * v_mfma_f32_16x16x32_f16 with 16 weight rows as the rows of A and 16 activation rows as the
//    columns of B; at step j (0..7) each lane feeds its elements [8j, 8j + 8). Both operands are
//    dequantized to FP16 exactly (see dequant8), products are exact in FP32 and accumulate in FP32.
//    MT = ceil(M / 16) activation tiles and NT weight tiles per wave.
//  * The loads of the next DEPTH chunks are in flight while a chunk is dequantized and multiplied.
//  * The KW partial sums meet in LDS and are added in wave order (deterministic), then scaled by
//    g_a * g_w of the column's segment, gated and stored, consecutive threads on consecutive columns.
#include <algorithm>

#include "device_common.h"

namespace nvfp4 {
namespace {

constexpr int MAX_WAVES = 4;  // K-split of a workgroup
constexpr int CHUNK = 256;  // K elements per chunk: 128 code bytes and 16 scale bytes per row
constexpr int DEPTH = 2;    // chunks in flight ahead of the one being multiplied

// One lane's share of one row of a chunk: 64 codes (two 16-byte pieces) and their 4 scale bytes.
struct RowFrag {
    u32x4 c[2];
    uint32_t s;
};

// codes/scales point at the lane's first byte of the row (row base + 32g, row base + 4g).
__device__ __forceinline__ void load_full(const uint8_t* codes, const uint8_t* scales, int64_t c, RowFrag& f) {
    const uint8_t* p = codes + c * (CHUNK / 2);
    f.c[0] = *reinterpret_cast<const u32x4*>(p);
    f.c[1] = *reinterpret_cast<const u32x4*>(p + 16);
    f.s = *reinterpret_cast<const uint32_t*>(scales + c * (CHUNK / 16));
}

// The chunk that crosses K: only bytes of elements below K are read; the rest is zero, and a zero
// scale byte makes a block contribute 0. K is a multiple of 16, so a piece is full, half or empty.
__device__ __forceinline__ void load_tail(const uint8_t* codes, const uint8_t* scales, int64_t c, int g, int64_t K,
                                          RowFrag& f) {
    const int64_t cvalid = K / 2 - (c * (CHUNK / 2) + 32 * g);
    const int64_t svalid = K / 16 - (c * (CHUNK / 16) + 4 * g);
    const uint8_t* p = codes + c * (CHUNK / 2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t v = cvalid - 16 * h;
        if (v >= 16) {
            f.c[h] = *reinterpret_cast<const u32x4*>(p + 16 * h);
        } else if (v >= 8) {
            const u32x2 lo = *reinterpret_cast<const u32x2*>(p + 16 * h);
            f.c[h] = u32x4{lo[0], lo[1], 0u, 0u};
        } else {
            f.c[h] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    const uint8_t* q = scales + c * (CHUNK / 16);
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (i < svalid) s |= (uint32_t)q[i] << (8 * i);
    f.s = s;
}

template <int MT, int NT>
struct Frags {
    RowFrag w[NT];
    RowFrag a[MT];
};

template <int MT, int NT>
__device__ __forceinline__ void load_full_chunk(Frags<MT, NT>& f, const uint8_t* const (&wc)[NT],
                                                const uint8_t* const (&ws)[NT], const uint8_t* const (&ac)[MT],
                                                const uint8_t* const (&as)[MT], int64_t c) {
#pragma unroll
    for (int t = 0; t < NT; ++t) load_full(wc[t], ws[t], c, f.w[t]);
#pragma unroll
    for (int u = 0; u < MT; ++u) load_full(ac[u], as[u], c, f.a[u]);
}

template <int MT, int NT>
__device__ __forceinline__ void compute_chunk(const Frags<MT, NT>& f, f32x4 (&acc)[NT][MT]) {
    half2_t sw[NT][2], sa[MT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        sw[t][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.w[t].s, 1.0f, false);
        sw[t][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.w[t].s, 1.0f, true);
    }
#pragma unroll
    for (int u = 0; u < MT; ++u) {
        sa[u][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.a[u].s, 1.0f, false);
        sa[u][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.a[u].s, 1.0f, true);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        // elements [8j, 8j + 8): dword j & 3 of piece j >> 2, block j >> 1
        half8_t wv[NT], av[MT];
#pragma unroll
        for (int t = 0; t < NT; ++t) wv[t] = dequant8(f.w[t].c[j >> 2][j & 3], sw[t][j >> 2][(j >> 1) & 1]);
#pragma unroll
        for (int u = 0; u < MT; ++u) av[u] = dequant8(f.a[u].c[j >> 2][j & 3], sa[u][j >> 2][(j >> 1) & 1]);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int u = 0; u < MT; ++u)
                acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv[t], av[u], acc[t][u], 0, 0, 0);
    }
}

template <int MT, int NT>
__global__ __launch_bounds__(64 * MAX_WAVES) void gemm_skinny_kernel(
    const uint8_t* __restrict__ a_codes, int64_t lda_c, const uint8_t* __restrict__ a_scales, int64_t lda_s,
    const uint8_t* __restrict__ w_codes, int64_t ldw_c, const uint8_t* __restrict__ w_scales, int64_t ldw_s,
    int64_t M, int64_t N, int64_t K, const SegParams sp) {
    extern __shared__ float red[];  // [KW][NT][MT][4][64] partial sums
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, kw = blockDim.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * (16 * NT);

    // rows past N or M are clamped to the last row: their results are never stored
    const uint8_t* wc[NT];
    const uint8_t* ws[NT];
    const uint8_t* ac[MT];
    const uint8_t* as[MT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int64_t n = std::min<int64_t>(n0 + 16 * t + r, N - 1);
        wc[t] = w_codes + n * ldw_c + 32 * g;
        ws[t] = w_scales + n * ldw_s + 4 * g;
    }
#pragma unroll
    for (int u = 0; u < MT; ++u) {
        const int64_t m = std::min<int64_t>(16 * u + r, M - 1);
        ac[u] = a_codes + m * lda_c + 32 * g;
        as[u] = a_scales + m * lda_s + 4 * g;
    }

    const int64_t nch = (K + CHUNK - 1) / CHUNK, nfull = K / CHUNK;
    const int64_t c_lo = nch * wave / kw, c_hi = nch * (wave + 1) / kw;

    f32x4 acc[NT][MT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int u = 0; u < MT; ++u) acc[t][u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // Full chunks [c_lo, c_end) go through a ring of DEPTH + 1 register buffers: chunk c is multiplied
    // while chunks c + 1 .. c + DEPTH are in flight. The loop is unrolled over the ring, so no buffer
    // is ever copied, and its loads are unconditional (indices past the range are clamped to its last
    // chunk), so the compiler can wait for exactly one chunk's loads at a time; a copy or a load under
    // a branch would make it wait for all of them.
    const int64_t c_end = std::min(c_hi, nfull);
    if (c_lo < c_end) {
        constexpr int RING = DEPTH + 1;
        Frags<MT, NT> f[RING];
#pragma unroll
        for (int i = 0; i < DEPTH; ++i) load_full_chunk<MT, NT>(f[i], wc, ws, ac, as, std::min(c_lo + i, c_end - 1));
        int64_t c = c_lo;
        for (; c + RING <= c_end; c += RING) {
#pragma unroll
            for (int i = 0; i < RING; ++i) {
                load_full_chunk<MT, NT>(f[(i + DEPTH) % RING], wc, ws, ac, as, std::min(c + i + DEPTH, c_end - 1));
                // keep the loads ahead of this chunk's arithmetic: sunk below it they would be waited for
                __builtin_amdgcn_sched_barrier(0);
                compute_chunk<MT, NT>(f[i], acc);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // fewer than RING chunks left, already loaded into f[0 ..]
#pragma unroll
        for (int i = 0; i < DEPTH; ++i)
            if (c + i < c_end) compute_chunk<MT, NT>(f[i], acc);
    }
    // the chunk that crosses K, if any, is the last chunk of the last wave
    if (c_hi > nfull && c_lo <= nfull) {
        Frags<MT, NT> t;
#pragma unroll
        for (int i = 0; i < NT; ++i) load_tail(wc[i], ws[i], nfull, g, K, t.w[i]);
#pragma unroll
        for (int u = 0; u < MT; ++u) load_tail(ac[u], as[u], nfull, g, K, t.a[u]);
        compute_chunk<MT, NT>(t, acc);
    }

    constexpr int TILE = NT * MT * 256;
    float* mine = red + wave * TILE;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int u = 0; u < MT; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) mine[((t * MT + u) * 4 + i) * 64 + lane] = acc[t][u][i];
    __syncthreads();

    // acc[t][u][i] of lane l holds y[n0 + 16t + 4(l / 16) + i][16u + l % 16]
    constexpr int COLS = 16 * NT;
    const int rows = (int)std::min<int64_t>(M, 16 * MT);
    for (int idx = threadIdx.x; idx < rows * COLS; idx += blockDim.x) {
        const int nl = idx % COLS, ml = idx / COLS;
        const int64_t col = n0 + nl;
        if (col >= N) continue;
        const int t = nl >> 4, i = nl & 3, u = ml >> 4;
        const int pos = ((t * MT + u) * 4 + i) * 64 + ((nl >> 2) & 3) * 16 + (ml & 15);
        float s = red[pos];
        for (int w = 1; w < kw; ++w) s += red[w * TILE + pos];
        store_output(sp, ml, col, s);
    }
}

typedef void (*skinny_fn)(const uint8_t*, int64_t, const uint8_t*, int64_t, const uint8_t*, int64_t, const uint8_t*,
                          int64_t, int64_t, int64_t, int64_t, const SegParams);

// NT = 4 only for MT <= 2: with more activation tiles the operands no longer fit in registers.
template <int MT>
skinny_fn pick_nt(int nt) {
    if constexpr (MT <= 2)
        if (nt >= 4) return gemm_skinny_kernel<MT, 4>;
    if (nt >= 2) return gemm_skinny_kernel<MT, 2>;
    return gemm_skinny_kernel<MT, 1>;
}

// Waves per workgroup splitting K: depends on K alone, so the order of the additions (and so every
// output bit) is the same for any N, column tile or segment table.
int skinny_waves(int64_t K) {
    const int64_t nch = (K + CHUNK - 1) / CHUNK;
    return (int)std::min<int64_t>(4, std::max<int64_t>(1, nch / 4));
}

}  // namespace

hipError_t launch_gemm_skinny(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s,
                              const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s,
                              int64_t M, int64_t N, int64_t K, const SegParams& sp, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    if (M > SKINNY_MAX_M) return hipErrorInvalidValue;
    const int mt = (int)((M + 15) / 16);
    // widest weight tile that still leaves two workgroups per compute unit
    int nt = 1;
    while (nt < 4 && (N + 32 * nt - 1) / (32 * nt) >= 512) nt *= 2;
    if (mt >= 3) nt = std::min(nt, 2);
    const skinny_fn fn = mt == 1   ? pick_nt<1>(nt)
                         : mt == 2 ? pick_nt<2>(nt)
                         : mt == 3 ? pick_nt<3>(nt)
                                   : pick_nt<4>(nt);
    const int kw = skinny_waves(K);
    const size_t lds = (size_t)kw * nt * mt * 256 * sizeof(float);
    const int64_t blocks = (N + 16 * nt - 1) / (16 * nt);
    hipLaunchKernelGGL(fn, dim3((uint32_t)blocks), dim3(64 * kw), lds, stream, a_codes, lda_c, a_scales, lda_s,
                       w_codes, ldw_c, w_scales, ldw_s, M, N, K, sp);
    return hipGetLastError();
}

}  // namespace nvfp4
