// Block-scaled W4A4 GEMMs for decode (M <= 64 activation rows), for gfx950 (CDNA4): the skinny
// kernel for M <= 32 and the wide kernel (further down) for 32 < M <= 64.
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
//    one wave. Four consecutive lanes read one contiguous run of a row (see RowFrag), and
//    ds_bpermute then moves the data into the matrix instruction's layout. Activation rows are loaded
//    and moved the same way, so lane group g holds the same K elements of both operands, as the
//    matrix instruction requires; within a chunk the 256 elements are thus summed in a permuted
//    order, which a sum does not depend on.
//  * v_mfma_f32_16x16x32_f16 with 16 weight rows as the rows of A and 16 activation rows as the
//    columns of B; at step j (0..7) each lane feeds its elements [8j, 8j + 8). Both operands are
//    dequantized to FP16 exactly (see dequant8), products are exact in FP32 and accumulate in FP32.
//    MT = ceil(M / 16) activation tiles and NT weight tiles per wave (1 for M <= 4, else 2).
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
//
// Loads: lane l reads row l / 4 of a 16-row tile, bytes 64h + 16q (q = l % 4, h = 0, 1) of the
// chunk's 128 code bytes and bytes 4q .. 4q + 3 of its 16 scale bytes, so that each group of four
// consecutive lanes reads one contiguous run: a load whose lanes each hit another row costs the
// memory pipeline several times as much per byte (measured with loads alone: the decode kernels' loads
// took 19.7 us laid out that way, 13.6 us with four-lane runs, for the 17408 x 5120 weights and 16
// activation rows). The matrix instruction wants lane r + 16g to hold row r; to_operand moves the data there
// with ds_bpermute, after which lane (r, g) holds elements [128h + 32g, 128h + 32g + 32) of the chunk
// (h = 0, 1) in c[h] and the scale bytes of its four blocks, in order, in s. Both operands are moved
// the same way, so lane group g holds the same K elements of both, as the matrix instruction needs;
// within a chunk the 256 elements are thus summed in a permuted order.
struct RowFrag {
    u32x4 c[2];
    uint32_t s;
};

// codes/scales point at the lane's first byte of the row (row base + 16q, row base + 4q).
__device__ __forceinline__ void load_full(const uint8_t* codes, const uint8_t* scales, int64_t c, RowFrag& f) {
    const uint8_t* p = codes + c * (CHUNK / 2);
    f.c[0] = *reinterpret_cast<const u32x4*>(p);
    f.c[1] = *reinterpret_cast<const u32x4*>(p + 64);
    f.s = *reinterpret_cast<const uint32_t*>(scales + c * (CHUNK / 16));
}

// The chunk that crosses K: only bytes of elements below K are read; the rest is zero, and a zero
// scale byte makes a block contribute 0. K is a multiple of 16, so a piece is full, half or empty.
__device__ __forceinline__ void load_tail(const uint8_t* codes, const uint8_t* scales, int64_t c, int q, int64_t K,
                                          RowFrag& f) {
    const uint8_t* p = codes + c * (CHUNK / 2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t v = K / 2 - (c * (CHUNK / 2) + 64 * h + 16 * q);
        if (v >= 16) {
            f.c[h] = *reinterpret_cast<const u32x4*>(p + 64 * h);
        } else if (v >= 8) {
            const u32x2 lo = *reinterpret_cast<const u32x2*>(p + 64 * h);
            f.c[h] = u32x4{lo[0], lo[1], 0u, 0u};
        } else {
            f.c[h] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    const int64_t svalid = K / 16 - (c * (CHUNK / 16) + 4 * q);
    const uint8_t* sp = scales + c * (CHUNK / 16);
    uint32_t sv = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (i < svalid) sv |= (uint32_t)sp[i] << (8 * i);
    f.s = sv;
}

// Source lanes of this lane's operand data (byte addresses for ds_bpermute) and the byte selector
// that keeps its two scale pairs.
struct OperandLanes {
    int codes, scales0, scales1;
    uint32_t sel;
};

__device__ __forceinline__ OperandLanes operand_lanes(int lane) {
    const int r = lane & 15, g = lane >> 4;
    // codes: lane 4r + g loaded row r's bytes 64h + 16g; scales: bytes 2g, 2g + 1 of the row's 16
    // (blocks of h = 0) sit in lane 4r + g / 2, bytes 8 + 2g, 9 + 2g (h = 1) in lane 4r + 2 + g / 2
    return {4 * (4 * r + g), 4 * (4 * r + (g >> 1)), 4 * (4 * r + 2 + (g >> 1)), (g & 1) ? 0x07060302u : 0x05040100u};
}

__device__ __forceinline__ uint32_t lane_read(int src, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v);
}

__device__ __forceinline__ RowFrag to_operand(const RowFrag& f, const OperandLanes& L) {
    RowFrag o;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) o.c[h][e] = lane_read(L.codes, f.c[h][e]);
    o.s = __builtin_amdgcn_perm(lane_read(L.scales1, f.s), lane_read(L.scales0, f.s), L.sel);
    return o;
}

// The decode weight layout (nvfp4_pack_weights): 16-row tiles by 256-element chunks. Tile t, chunk c
// (of C = ceil(K / 256)) holds at (t C + c) * PK_CODES its two 1 KB code pieces already in the
// operand layout (piece h, lane r + 16g: row 16t + r, code bytes 64h + 16g .. + 15 of the chunk) and,
// after all T C of those, at (t C + c) * PK_SCALES its scale dwords (lane r + 16g: scale bytes 2g,
// 2g + 1, 8 + 2g, 9 + 2g of that row and chunk). Rows past N and bytes past K are zero, so a padded
// block has a zero scale and adds exact zeros, and the chunk that crosses K needs no special load.
// Every load of a packed operand is one contiguous 1 KB (or 256-byte) run.
constexpr int PK_CODES = 2048, PK_SCALES = 256;

// codes/scales point at the lane's bytes of chunk 0 of its tile (tile base + 16 lane, + 4 lane).
__device__ __forceinline__ void load_packed(const uint8_t* codes, const uint8_t* scales, int64_t c, RowFrag& f) {
    const uint8_t* p = codes + c * PK_CODES;
    f.c[0] = *reinterpret_cast<const u32x4*>(p);
    f.c[1] = *reinterpret_cast<const u32x4*>(p + 1024);
    f.s = *reinterpret_cast<const uint32_t*>(scales + c * PK_SCALES);
}

// A weight fragment of chunk c (the chunk that crosses K when tail): packed weights are loaded in the
// operand layout, row-major ones in the load layout.
template <bool PK>
__device__ __forceinline__ void load_w(const uint8_t* codes, const uint8_t* scales, int64_t c, bool tail, int q,
                                       int64_t K, RowFrag& f) {
    if constexpr (PK)
        load_packed(codes, scales, c, f);
    else if (tail)
        load_tail(codes, scales, c, q, K, f);
    else
        load_full(codes, scales, c, f);
}

template <bool PK>
__device__ __forceinline__ RowFrag w_operand(const RowFrag& f, const OperandLanes& L) {
    if constexpr (PK)
        return f;
    else
        return to_operand(f, L);
}

// The lane's weight pointers for weight rows n0 .. n0 + 15 (rows past N clamped to the last row; for
// packed weights, tiles past the last clamped to it): row-major in the load layout, or packed.
template <bool PK>
__device__ __forceinline__ void w_pointers(const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales,
                                           int64_t ldw_s, int64_t n0, int64_t N, int64_t K, int lane,
                                           const uint8_t*& wc, const uint8_t*& ws) {
    if constexpr (PK) {
        const int64_t C = (K + CHUNK - 1) / CHUNK;
        const int64_t tile = std::min<int64_t>(n0 / 16, (N - 1) / 16);
        wc = w_codes + tile * C * PK_CODES + 16 * lane;
        ws = w_scales + tile * C * PK_SCALES + 4 * lane;
    } else {
        const int64_t n = std::min<int64_t>(n0 + (lane >> 2), N - 1);
        wc = w_codes + n * ldw_c + 16 * (lane & 3);
        ws = w_scales + n * ldw_s + 4 * (lane & 3);
    }
}

template <int MT, int NT>
struct Frags {
    RowFrag w[NT];
    RowFrag a[MT];
};

template <int MT, int NT, bool PK>
__device__ __forceinline__ void load_full_chunk(Frags<MT, NT>& f, const uint8_t* const (&wc)[NT],
                                                const uint8_t* const (&ws)[NT], const uint8_t* const (&ac)[MT],
                                                const uint8_t* const (&as)[MT], int64_t c) {
#pragma unroll
    for (int t = 0; t < NT; ++t) load_w<PK>(wc[t], ws[t], c, false, 0, 0, f.w[t]);
#pragma unroll
    for (int u = 0; u < MT; ++u) load_full(ac[u], as[u], c, f.a[u]);
}

// One chunk's MT x NT tiles from fragments in the operand layout.
template <int MT, int NT>
__device__ __forceinline__ void mma_chunk(const RowFrag (&w)[NT], const RowFrag (&a)[MT], f32x4 (&acc)[NT][MT]) {
    half2_t sw[NT][2], sa[MT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        sw[t][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[t].s, 1.0f, false);
        sw[t][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[t].s, 1.0f, true);
    }
#pragma unroll
    for (int u = 0; u < MT; ++u) {
        sa[u][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a[u].s, 1.0f, false);
        sa[u][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a[u].s, 1.0f, true);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        // elements [8j, 8j + 8): dword j & 3 of piece j >> 2, block j >> 1
        half8_t wv[NT], av[MT];
#pragma unroll
        for (int t = 0; t < NT; ++t) wv[t] = dequant8(w[t].c[j >> 2][j & 3], sw[t][j >> 2][(j >> 1) & 1]);
#pragma unroll
        for (int u = 0; u < MT; ++u) av[u] = dequant8(a[u].c[j >> 2][j & 3], sa[u][j >> 2][(j >> 1) & 1]);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int u = 0; u < MT; ++u)
                acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv[t], av[u], acc[t][u], 0, 0, 0);
    }
}

// One chunk's tiles from fragments as loaded (activations in the load layout).
template <int MT, int NT, bool PK>
__device__ __forceinline__ void compute_chunk(const Frags<MT, NT>& f, const OperandLanes& L, f32x4 (&acc)[NT][MT]) {
    RowFrag w[NT], a[MT];
#pragma unroll
    for (int t = 0; t < NT; ++t) w[t] = w_operand<PK>(f.w[t], L);
#pragma unroll
    for (int u = 0; u < MT; ++u) a[u] = to_operand(f.a[u], L);
    mma_chunk<MT, NT>(w, a, acc);
}

template <int MT, int NT, bool PK>
__global__ __launch_bounds__(64 * MAX_WAVES) void gemm_skinny_kernel(
    const uint8_t* __restrict__ a_codes, int64_t lda_c, const uint8_t* __restrict__ a_scales, int64_t lda_s,
    const uint8_t* __restrict__ w_codes, int64_t ldw_c, const uint8_t* __restrict__ w_scales, int64_t ldw_s,
    int64_t M, int64_t N, int64_t K, const SegParams sp) {
    extern __shared__ float red[];  // [KW][NT][MT][4][64] partial sums
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, kw = blockDim.x >> 6;
    const int rl = lane >> 2, q = lane & 3;  // the row this lane loads, its piece
    const OperandLanes L = operand_lanes(lane);
    const int64_t n0 = (int64_t)blockIdx.x * (16 * NT);

    // rows past N or M are clamped to the last row: their results are never stored
    const uint8_t* wc[NT];
    const uint8_t* ws[NT];
    const uint8_t* ac[MT];
    const uint8_t* as[MT];
#pragma unroll
    for (int t = 0; t < NT; ++t) w_pointers<PK>(w_codes, ldw_c, w_scales, ldw_s, n0 + 16 * t, N, K, lane, wc[t], ws[t]);
#pragma unroll
    for (int u = 0; u < MT; ++u) {
        const int64_t m = std::min<int64_t>(16 * u + rl, M - 1);
        ac[u] = a_codes + m * lda_c + 16 * q;
        as[u] = a_scales + m * lda_s + 4 * q;
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
        for (int i = 0; i < DEPTH; ++i) load_full_chunk<MT, NT, PK>(f[i], wc, ws, ac, as, std::min(c_lo + i, c_end - 1));
        int64_t c = c_lo;
        for (; c + RING <= c_end; c += RING) {
#pragma unroll
            for (int i = 0; i < RING; ++i) {
                load_full_chunk<MT, NT, PK>(f[(i + DEPTH) % RING], wc, ws, ac, as, std::min(c + i + DEPTH, c_end - 1));
                // keep the loads ahead of this chunk's arithmetic: sunk below it they would be waited for
                __builtin_amdgcn_sched_barrier(0);
                compute_chunk<MT, NT, PK>(f[i], L, acc);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // fewer than RING chunks left, already loaded into f[0 ..]
#pragma unroll
        for (int i = 0; i < DEPTH; ++i)
            if (c + i < c_end) compute_chunk<MT, NT, PK>(f[i], L, acc);
    }
    // the chunk that crosses K, if any, is the last chunk of the last wave
    if (c_hi > nfull && c_lo <= nfull) {
        Frags<MT, NT> t;
#pragma unroll
        for (int i = 0; i < NT; ++i) load_w<PK>(wc[i], ws[i], nfull, true, q, K, t.w[i]);
#pragma unroll
        for (int u = 0; u < MT; ++u) load_tail(ac[u], as[u], nfull, q, K, t.a[u]);
        compute_chunk<MT, NT, PK>(t, L, acc);
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

    // acc[t][u][i] of lane l holds y[n0 + 16t + 4(l / 16) + i][16u + l % 16]. A thread keeps one
    // column (the workgroup size is a multiple of COLS) and walks its rows.
    constexpr int COLS = 16 * NT;
    const int rows = (int)std::min<int64_t>(M, 16 * MT);
    const int nl = threadIdx.x % COLS;
    const int64_t col = n0 + nl;
    if (col < N) {
        const ColumnOut co = column_out(sp, col);
        const int t = nl >> 4, i = nl & 3;
        for (int ml = threadIdx.x / COLS; ml < rows; ml += blockDim.x / COLS) {
            const int u = ml >> 4;
            const int pos = ((t * MT + u) * 4 + i) * 64 + ((nl >> 2) & 3) * 16 + (ml & 15);
            float s = red[pos];
            for (int w = 1; w < kw; ++w) s += red[w * TILE + pos];
            column_store(co, ml, s);
        }
    }
}

typedef void (*skinny_fn)(const uint8_t*, int64_t, const uint8_t*, int64_t, const uint8_t*, int64_t, const uint8_t*,
                          int64_t, int64_t, int64_t, int64_t, const SegParams);

template <int MT, bool PK>
skinny_fn pick_nt(int nt) {
    return nt >= 2 ? gemm_skinny_kernel<MT, 2, PK> : gemm_skinny_kernel<MT, 1, PK>;
}

// Waves per workgroup splitting K: depends on K alone, so the order of the additions (and so every
// output bit) is the same for any N, column tile or segment table.
int skinny_waves(int64_t K) {
    const int64_t nch = (K + CHUNK - 1) / CHUNK;
    return (int)std::min<int64_t>(4, std::max<int64_t>(1, nch / 4));
}

// ---------------------------------------------------------------------------------------------------
// 32 < M <= 64 ("wide" decode). With three or four activation tiles every weight tile of the kernel
// above re-reads all activation rows of its K range and dequantizes them, which is then what bounds
// it. Here a workgroup takes one range of K and 128, 80 or 64 weight rows: two "K-groups" of WPG
// waves (4, 5 or 4) with NT 16-row weight tiles each (2, 1 or 1); the shape is chosen from N and the
// split count so that the workgroups fill the CUs (wide_shape). The K-groups take alternate
// 256-element chunks of the range, so each SIMD holds two or three waves (one's dequantization
// overlaps another's matrix instructions) and twice the loads are in flight. Within a K-group each
// activation chunk is dequantized once into LDS as FP16 in the matrix instruction's operand order
// (wave u converts activation tile u, each lane the 64 elements it would hold itself; a fifth wave
// converts a clamped copy into a tile that is never read), and all waves read their B operands from
// there; a wave dequantizes only its own weight rows. Loads run two chunks ahead. The K-groups' sums are
// added in LDS (group 0 + group 1). K is split across workgroups by a count chosen from K alone: with
// one split the workgroup applies the segment epilogue itself, else it writes its partial sums (FP32,
// [split][n][64 activation rows]) to the workspace and a second kernel adds the splits in order and
// applies the epilogue. Every output bit is thus the same for any N, column group or segment table.

constexpr int WIDE_MP = 64;                  // activation rows held (M <= 64)
constexpr int WIDE_SLOTS = 3;                // register ring: K-group chunk i in slot i % 3, loads 2 chunks ahead
constexpr int WIDE_KG = 2;                   // K-groups of 4 waves per workgroup

// One K-group's FP16 activation chunk: [tile u][step j][lane] -> the 8 values lane (g, r) feeds at
// step j for activation row 16u + r (elements 128 (j / 4) + 32g + 8 (j % 4) .. + 7 of the chunk, the
// operand layout of RowFrag). A K-group of WPG waves
// has WPG tiles: tiles 0-3 hold the (at most 64) activation rows; a fifth wave's tile is written and
// never read.
template <int WPG>
using ActChunk = half8_t[WPG][8][64];

// Lane (g, r) of wave u converts its fragment of activation row 16u + r into the chunk (loaded in
// the load layout; moved to the operand layout here).
template <int WPG>
__device__ __forceinline__ void stage_act(ActChunk<WPG>& dst, const RowFrag& fl, int u, int lane) {
    const RowFrag f = to_operand(fl, operand_lanes(lane));
    half2_t sa[2];
    sa[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.s, 1.0f, false);
    sa[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.s, 1.0f, true);
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[u][j][lane] = dequant8(f.c[j >> 2][j & 3], sa[j >> 2][(j >> 1) & 1]);
}

// The MT x NT tiles of one chunk: weights dequantized here, activations read from the chunk.
template <int MT, int NT, int WPG, bool PK>
__device__ __forceinline__ void compute_lds(const RowFrag (&wl)[NT], const ActChunk<WPG>& act, int lane,
                                            f32x4 (&acc)[NT][MT]) {
    constexpr int WIDE_NT = NT;
    RowFrag w[WIDE_NT];
    const OperandLanes L = operand_lanes(lane);
#pragma unroll
    for (int t = 0; t < WIDE_NT; ++t) w[t] = w_operand<PK>(wl[t], L);
    half2_t sw[WIDE_NT][2];
#pragma unroll
    for (int t = 0; t < WIDE_NT; ++t) {
        sw[t][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[t].s, 1.0f, false);
        sw[t][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[t].s, 1.0f, true);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        half8_t wv[WIDE_NT], av[MT];
#pragma unroll
        for (int u = 0; u < MT; ++u) av[u] = act[u][j][lane];
#pragma unroll
        for (int t = 0; t < WIDE_NT; ++t) wv[t] = dequant8(w[t].c[j >> 2][j & 3], sw[t][j >> 2][(j >> 1) & 1]);
#pragma unroll
        for (int t = 0; t < WIDE_NT; ++t)
#pragma unroll
            for (int u = 0; u < MT; ++u)
                acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv[t], av[u], acc[t][u], 0, 0, 0);
    }
}

// One K-group's step i (register slot d = i % 3, LDS buffer i % 2): issue the loads of its chunk
// i + 2 (clamped to the last full chunk), wait for chunk i (converted into act[i % 2]), multiply it,
// convert the activations of chunk i + 1 into the other buffer. A chunk index at or past c_fhi (a
// repeat of the last full chunk) gets zero weight scales, which adds exact zeros. There is no branch
// in here: a load under one is issued where its value is used, or waited for at the join.
template <int MT, int NT, int WPG, bool PK, bool LOADS>
__device__ __forceinline__ void wide_step(int d, int64_t i, int64_t c, int64_t c_fhi, int64_t cl,
                                          RowFrag (&wf)[WIDE_SLOTS][NT], RowFrag (&af)[WIDE_SLOTS],
                                          ActChunk<WPG>* act, f32x4 (&acc)[NT][MT], const uint8_t* ac,
                                          const uint8_t* as, const uint8_t* const (&wc)[NT],
                                          const uint8_t* const (&ws)[NT], int u, int lane) {
    constexpr int WIDE_NT = NT;
    const int dn = (d + 2) % WIDE_SLOTS;
    if constexpr (LOADS) {
        load_full(ac, as, cl, af[dn]);
#pragma unroll
        for (int t = 0; t < WIDE_NT; ++t) load_w<PK>(wc[t], ws[t], cl, false, 0, 0, wf[dn][t]);
    }
    __builtin_amdgcn_sched_barrier(0);  // issue them before waiting for chunk c
    __syncthreads();                    // chunk c converted; every wave is done with the other buffer
    const bool live = c < c_fhi;
#pragma unroll
    for (int t = 0; t < WIDE_NT; ++t) wf[d][t].s = live ? wf[d][t].s : 0u;
    compute_lds<MT, NT, WPG, PK>(wf[d], act[i & 1], lane, acc);
    stage_act<WPG>(act[(i + 1) & 1], af[(d + 1) % WIDE_SLOTS], u, lane);
    // keep the next chunk's dequantization out of this one (it would wait for its loads)
    __builtin_amdgcn_sched_barrier(0);
}

// A workgroup is two K-groups of WPG waves, each wave NT weight tiles of 16 rows: WPG * 16 * NT
// weight rows.
template <int MT, int NT, int WPG, bool PK>
__global__ __launch_bounds__(128 * WPG) void gemm_wide_kernel(
    const uint8_t* __restrict__ a_codes, int64_t lda_c, const uint8_t* __restrict__ a_scales, int64_t lda_s,
    const uint8_t* __restrict__ w_codes, int64_t ldw_c, const uint8_t* __restrict__ w_scales, int64_t ldw_s,
    int64_t M, int64_t N, int64_t K, int64_t per, float* __restrict__ partial, const SegParams sp) {
    constexpr int WIDE_NT = NT;
    constexpr int WIDE_ROWS = WPG * 16 * NT;  // weight rows per workgroup
    constexpr int THREADS = 128 * WPG;
    // two FP16 activation buffers per K-group (32 WPG KB); reused at the end for the cross-group sum
    // and the output tile
    __shared__ ActChunk<WPG> lds[WIDE_KG][2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kg = wave / WPG, u = wave % WPG;
    const int r = lane & 15, g = lane >> 4;  // the operand layout (results)
    const int rl = lane >> 2, q = lane & 3;   // the load layout: the row this lane loads, its piece
    const int64_t groups = (N + WIDE_ROWS - 1) / WIDE_ROWS;
    const int64_t grp = blockIdx.x % groups;
    const int split = (int)(blockIdx.x / groups);
    const int64_t n0 = grp * WIDE_ROWS + u * (16 * NT);

    // weight rows past N and activation rows past M are clamped to the last row: their results are
    // never stored
    const uint8_t* wc[WIDE_NT];
    const uint8_t* ws[WIDE_NT];
#pragma unroll
    for (int t = 0; t < WIDE_NT; ++t) w_pointers<PK>(w_codes, ldw_c, w_scales, ldw_s, n0 + 16 * t, N, K, lane, wc[t], ws[t]);
    const int64_t arow = std::min<int64_t>(16 * u + rl, M - 1);
    const uint8_t* ac = a_codes + arow * lda_c + 16 * q;
    const uint8_t* as = a_scales + arow * lda_s + 4 * q;

    const int64_t nch = (K + CHUNK - 1) / CHUNK, nfull = K / CHUNK;
    const int64_t c_lo = std::min<int64_t>(nch, split * per), c_hi = std::min<int64_t>(nch, c_lo + per);
    const int64_t c_fhi = std::min(c_hi, nfull);  // full chunks of this split: [c_lo, c_fhi)
    // K-group kg takes the full chunks c_lo + 2i + kg, i < steps
    const int64_t steps = (c_fhi - c_lo + 1) / 2;
    auto chunk = [&](int64_t i) { return c_lo + 2 * i + kg; };
    auto clamped = [&](int64_t i) { return std::min(chunk(i), c_fhi - 1); };

    f32x4 acc[WIDE_NT][MT];
#pragma unroll
    for (int t = 0; t < WIDE_NT; ++t)
#pragma unroll
        for (int uu = 0; uu < MT; ++uu) acc[t][uu] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    ActChunk<WPG>* act = lds[kg];
    if (steps > 0) {
        RowFrag wf[WIDE_SLOTS][WIDE_NT], af[WIDE_SLOTS];
        // step by step, in the loop's order, so that the loop's waits count the same loads on entry
        load_full(ac, as, clamped(0), af[0]);
#pragma unroll
        for (int t = 0; t < WIDE_NT; ++t) load_w<PK>(wc[t], ws[t], clamped(0), false, 0, 0, wf[0][t]);
        load_full(ac, as, clamped(1), af[1]);
#pragma unroll
        for (int t = 0; t < WIDE_NT; ++t) load_w<PK>(wc[t], ws[t], clamped(1), false, 0, 0, wf[1][t]);
        stage_act<WPG>(act[0], af[0], u, lane);
        int64_t i0 = 0;
        for (; i0 + WIDE_SLOTS <= steps; i0 += WIDE_SLOTS) {
#pragma unroll
            for (int d = 0; d < WIDE_SLOTS; ++d)
                wide_step<MT, NT, WPG, PK, true>(d, i0 + d, chunk(i0 + d), c_fhi, clamped(i0 + d + 2), wf, af, act,
                                             acc, ac, as, wc, ws, u, lane);
        }
        // the last one or two steps: their chunks are already loaded (slots 0 and 1)
        if (i0 < steps)
            wide_step<MT, NT, WPG, PK, false>(0, i0, chunk(i0), c_fhi, 0, wf, af, act, acc, ac, as, wc, ws, u, lane);
        if (i0 + 1 < steps)
            wide_step<MT, NT, WPG, PK, false>(1, i0 + 1, chunk(i0 + 1), c_fhi, 0, wf, af, act, acc, ac, as, wc, ws, u,
                                          lane);
    }
    if (c_fhi < c_hi) {
        // the chunk that crosses K (only in the last split), multiplied by K-group 0
        __syncthreads();  // every wave is done with the activation buffers
        RowFrag twf[WIDE_NT];
        if (kg == 0) {
            RowFrag taf;
            load_tail(ac, as, c_fhi, q, K, taf);
#pragma unroll
            for (int t = 0; t < WIDE_NT; ++t) load_w<PK>(wc[t], ws[t], c_fhi, true, q, K, twf[t]);
            stage_act<WPG>(act[0], taf, u, lane);
        }
        __syncthreads();
        if (kg == 0) compute_lds<MT, NT, WPG, PK>(twf, act[0], lane, acc);
    }

    // K-group 0 + K-group 1, through LDS. acc[t][uu] of lane (g, r) holds y[n0 + 16t + 4g + e][16uu + r].
    constexpr int ACC = WIDE_NT * MT * 4;
    float* red = reinterpret_cast<float*>(&lds[0][0][0][0][0]);
    __syncthreads();  // every wave is done with the activation buffers
    if (kg == 1) {
#pragma unroll
        for (int t = 0; t < WIDE_NT; ++t)
#pragma unroll
            for (int uu = 0; uu < MT; ++uu)
#pragma unroll
                for (int e = 0; e < 4; ++e) red[(u * ACC + (t * MT + uu) * 4 + e) * 64 + lane] = acc[t][uu][e];
    }
    __syncthreads();
    if (kg == 0) {
#pragma unroll
        for (int t = 0; t < WIDE_NT; ++t)
#pragma unroll
            for (int uu = 0; uu < MT; ++uu)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[t][uu][e] += red[(u * ACC + (t * MT + uu) * 4 + e) * 64 + lane];
    }

    if (gridDim.x == groups) {
        // one split: the epilogue here, through an LDS tile [m][column] so that stores run along rows
        float(*tile)[WIDE_ROWS + 1] = reinterpret_cast<float(*)[WIDE_ROWS + 1]>(&lds[0][0][0][0][0]);
        __syncthreads();  // the group sums are read
        if (kg == 0) {
#pragma unroll
            for (int t = 0; t < WIDE_NT; ++t)
#pragma unroll
                for (int uu = 0; uu < MT; ++uu)
#pragma unroll
                    for (int e = 0; e < 4; ++e) tile[16 * uu + r][u * 16 * NT + 16 * t + 4 * g + e] = acc[t][uu][e];
        }
        __syncthreads();
        // a thread keeps one column and walks every fourth row
        const int rows = (int)std::min<int64_t>(M, 16 * MT);
        const int nl = tid % WIDE_ROWS;
        const int64_t n = grp * WIDE_ROWS + nl;
        if (n < N) {
            const ColumnOut co = column_out(sp, n);
            for (int m = tid / WIDE_ROWS; m < rows; m += THREADS / WIDE_ROWS) column_store(co, m, tile[m][nl]);
        }
    } else if (kg == 0) {
        // partial[split][n][m]
#pragma unroll
        for (int t = 0; t < WIDE_NT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t n = n0 + 16 * t + 4 * g + e;
                if (n < N) {
                    float* dst = partial + ((int64_t)split * N + n) * WIDE_MP;
#pragma unroll
                    for (int uu = 0; uu < MT; ++uu) dst[16 * uu + r] = acc[t][uu][e];
                }
            }
    }
}

// The splits added in order, then the segment epilogue. A workgroup takes 16 output columns: thread
// (column c = tid / 16, rows 4 (tid % 16) .. + 3) issues the loads of all S splits at once (float4,
// a 4 KB contiguous run per split and workgroup), adds them in split order, and the sums go through
// LDS so that the stores run along the output rows.
template <int S>
__global__ __launch_bounds__(256) void gemm_wide_reduce_kernel(const float* __restrict__ partial, int64_t M, int64_t N,
                                                               const SegParams sp) {
    __shared__ float tile[WIDE_MP][17];
    const int tid = threadIdx.x;
    const int64_t nb = (int64_t)blockIdx.x * 16;
    const int cl = tid >> 4, m4 = 4 * (tid & 15);
    const int64_t n = std::min<int64_t>(nb + cl, N - 1);
    f32x4 p[S];
#pragma unroll
    for (int s = 0; s < S; ++s) p[s] = *reinterpret_cast<const f32x4*>(partial + ((int64_t)s * N + n) * WIDE_MP + m4);
    f32x4 v = p[0];
#pragma unroll
    for (int s = 1; s < S; ++s) v += p[s];
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[m4 + e][cl] = v[e];
    __syncthreads();
    const int c = tid & 15;
    if (nb + c < N) {
        const ColumnOut co = column_out(sp, nb + c);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const int m = 16 * h + (tid >> 4);
            if (m < M) column_store(co, m, tile[m][c]);
        }
    }
}

template <int S>
void launch_reduce(const float* partial, int64_t M, int64_t N, const SegParams& sp, hipStream_t stream) {
    hipLaunchKernelGGL(gemm_wide_reduce_kernel<S>, dim3((uint32_t)((N + 15) / 16)), dim3(256), 0, stream, partial, M, N,
                       sp);
}

}  // namespace

// The decode weight layout from row-major NVFP4 weights: one thread per (tile, chunk, lane) writes the
// lane's two 16-byte code pieces and its scale dword (zeros past N and K).
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint8_t* __restrict__ w_codes, int64_t ldw_c,
                                                           const uint8_t* __restrict__ w_scales, int64_t ldw_s,
                                                           int64_t N, int64_t K, int64_t C, int64_t units,
                                                           uint8_t* __restrict__ codes_out,
                                                           uint8_t* __restrict__ scales_out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= units) return;
    const int lane = (int)(i & 63);
    const int64_t tc = i >> 6, t = tc / C, c = tc - t * C;
    const int r = lane & 15, g = lane >> 4;
    const int64_t n = 16 * t + r;
    u32x4 piece[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
    uint32_t sv = 0;
    if (n < N) {
        const uint8_t* row = w_codes + n * ldw_c;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t off = c * (CHUNK / 2) + 64 * h + 16 * g;
            const int64_t v = K / 2 - off;  // K is a multiple of 16: a piece is full, half or empty
            if (v >= 16) {
                piece[h] = *reinterpret_cast<const u32x4*>(row + off);
            } else if (v >= 8) {
                const u32x2 lo = *reinterpret_cast<const u32x2*>(row + off);
                piece[h] = u32x4{lo[0], lo[1], 0u, 0u};
            }
        }
        const uint8_t* srow = w_scales + n * ldw_s;
        const int blk[4] = {2 * g, 2 * g + 1, 8 + 2 * g, 9 + 2 * g};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t b = c * (CHUNK / 16) + blk[e];
            if (b < K / 16) sv |= (uint32_t)srow[b] << (8 * e);
        }
    }
    uint8_t* dst = codes_out + tc * PK_CODES + 16 * lane;
    *reinterpret_cast<u32x4*>(dst) = piece[0];
    *reinterpret_cast<u32x4*>(dst + 1024) = piece[1];
    *reinterpret_cast<uint32_t*>(scales_out + tc * PK_SCALES + 4 * lane) = sv;
}

// K split of the wide decode kernel, from K alone (so output bits do not depend on N): at least 11
// chunks of 256 per split, at most 8 splits, an even number of chunks per split (the two K-groups
// take alternate chunks), so the last split may be shorter. A workgroup holds a whole CU (8 waves of
// about 200 registers), so more splits than the CUs take pay a second round of workgroups.
struct WideSplit {
    int64_t per;  // chunks per split
    int splits;
};

static WideSplit wide_split(int64_t K) {
    const int64_t nch = (K + CHUNK - 1) / CHUNK;
    if (nch == 0) return {0, 1};
    const int64_t s0 = std::min<int64_t>(8, std::max<int64_t>(1, nch / 11));
    const int64_t per = ((nch + s0 - 1) / s0 + 1) / 2 * 2;
    return {per, (int)((nch + per - 1) / per)};
}

// Weight rows per workgroup of the wide kernel: 128 (4 waves of 2 tiles per K-group), 80 (5 waves of
// 1 tile) or 64 (4 waves of 1 tile), whichever gives the fewest rounds of workgroups over the CUs
// times the busiest SIMD's tiles per chunk (4, 3, 2). Only the grouping of columns changes: every
// column's sum runs in the same order in all three, so the output bits do not depend on the choice.
struct WideShape {
    int rows, wpg, nt;
};

int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

static WideShape wide_shape(int64_t N, int splits) {
    static constexpr WideShape shapes[3] = {{128, 4, 2}, {80, 5, 1}, {64, 4, 1}};
    static constexpr int load[3] = {4, 3, 2};
    const int64_t cus = device_cus();
    int best = 0;
    int64_t best_cost = -1;
    for (int s = 0; s < 3; ++s) {
        const int64_t wgs = (N + shapes[s].rows - 1) / shapes[s].rows * splits;
        const int64_t cost = (wgs + cus - 1) / cus * load[s];
        if (best_cost < 0 || cost < best_cost) {
            best = s;
            best_cost = cost;
        }
    }
    return shapes[best];
}

size_t gemm_wide_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= SKINNY_NARROW_M || M > SKINNY_MAX_M || N <= 0 || K < 0) return 0;
    const int splits = wide_split(K).splits;
    return splits > 1 ? (size_t)splits * (size_t)N * WIDE_MP * sizeof(float) : 0;
}

size_t packed_weight_bytes(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0) return 0;
    const int64_t T = (N + 15) / 16, C = (K + CHUNK - 1) / CHUNK;
    return (size_t)T * (size_t)C * (PK_CODES + PK_SCALES);
}

const uint8_t* packed_scales(const uint8_t* packed, int64_t N, int64_t K) {
    const int64_t T = (N + 15) / 16, C = (K + CHUNK - 1) / CHUNK;
    return packed + T * C * PK_CODES;
}

hipError_t launch_pack_weights(const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s,
                               int64_t N, int64_t K, uint8_t* packed, hipStream_t stream) {
    if (N <= 0 || K <= 0) return hipSuccess;
    const int64_t T = (N + 15) / 16, C = (K + CHUNK - 1) / CHUNK, units = T * C * 64;
    if ((units + 255) / 256 > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(pack_weights_kernel, dim3((uint32_t)((units + 255) / 256)), dim3(256), 0, stream, w_codes,
                       ldw_c, w_scales, ldw_s, N, K, C, units, packed, packed + T * C * PK_CODES);
    return hipGetLastError();
}

hipError_t launch_gemm_wide(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s,
                            const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s,
                            int64_t M, int64_t N, int64_t K, const SegParams& sp, void* workspace,
                            bool packed, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    const WideSplit ks = wide_split(K);
    if (M <= SKINNY_NARROW_M || M > SKINNY_MAX_M || (ks.splits > 1 && !workspace)) return hipErrorInvalidValue;
    const WideShape sh = wide_shape(N, ks.splits);
    const int64_t groups = (N + sh.rows - 1) / sh.rows;
    if (groups * ks.splits > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
    float* partial = static_cast<float*>(workspace);
    const int mt = (int)((M + 15) / 16);
    using wide_fn = void (*)(const uint8_t*, int64_t, const uint8_t*, int64_t, const uint8_t*, int64_t,
                             const uint8_t*, int64_t, int64_t, int64_t, int64_t, int64_t, float*, const SegParams);
    wide_fn fn;
    if (packed) {
        if (sh.wpg == 4 && sh.nt == 2)
            fn = mt == 3 ? gemm_wide_kernel<3, 2, 4, true> : gemm_wide_kernel<4, 2, 4, true>;
        else if (sh.wpg == 5)
            fn = mt == 3 ? gemm_wide_kernel<3, 1, 5, true> : gemm_wide_kernel<4, 1, 5, true>;
        else
            fn = mt == 3 ? gemm_wide_kernel<3, 1, 4, true> : gemm_wide_kernel<4, 1, 4, true>;
    } else {
        if (sh.wpg == 4 && sh.nt == 2)
            fn = mt == 3 ? gemm_wide_kernel<3, 2, 4, false> : gemm_wide_kernel<4, 2, 4, false>;
        else if (sh.wpg == 5)
            fn = mt == 3 ? gemm_wide_kernel<3, 1, 5, false> : gemm_wide_kernel<4, 1, 5, false>;
        else
            fn = mt == 3 ? gemm_wide_kernel<3, 1, 4, false> : gemm_wide_kernel<4, 1, 4, false>;
    }
    hipLaunchKernelGGL(fn, dim3((uint32_t)(groups * ks.splits)), dim3(128 * sh.wpg), 0, stream, a_codes, lda_c,
                       a_scales, lda_s, w_codes, ldw_c, w_scales, ldw_s, M, N, K, ks.per, partial, sp);
    if (ks.splits > 1) {
        using reduce_fn = void (*)(const float*, int64_t, int64_t, const SegParams&, hipStream_t);
        static constexpr reduce_fn reduce[8] = {launch_reduce<1>, launch_reduce<2>, launch_reduce<3>,
                                                launch_reduce<4>, launch_reduce<5>, launch_reduce<6>,
                                                launch_reduce<7>, launch_reduce<8>};
        reduce[ks.splits - 1](partial, M, N, sp, stream);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_skinny(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s,
                              const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s,
                              int64_t M, int64_t N, int64_t K, const SegParams& sp, bool packed,
                              hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    if (M > SKINNY_MAX_M) return hipErrorInvalidValue;
    const int mt = (int)((M + 15) / 16);
    // Two weight tiles per wave share each activation fragment; with one or a few activation rows
    // those loads are cheap and one tile per wave (twice the workgroups) streams the weights faster,
    // and up to 16 rows so does a grid of at least 4 one-tile workgroups per CU (MLP up 17408 x 5120:
    // 18.6 -> 15.7 us at M = 8, 20.0 -> 18.5 at M = 16; packed 15.4 -> 14.3, 16.4 -> 15.5). Measured
    // on the MLP and GDN projection shapes (N = 5120 .. 17408, K = 5120 .. 17408); N only decides how
    // columns are grouped, never the order of any sum.
    const int nt = (M <= 4 || (M <= 16 && (N + 15) / 16 >= 4 * (int64_t)device_cus())) ? 1 : 2;
    const skinny_fn fn = packed ? (mt == 1   ? pick_nt<1, true>(nt)
                                   : mt == 2 ? pick_nt<2, true>(nt)
                                   : mt == 3 ? pick_nt<3, true>(nt)
                                             : pick_nt<4, true>(nt))
                                : (mt == 1   ? pick_nt<1, false>(nt)
                                   : mt == 2 ? pick_nt<2, false>(nt)
                                   : mt == 3 ? pick_nt<3, false>(nt)
                                             : pick_nt<4, false>(nt));
    const int kw = skinny_waves(K);
    const size_t lds = (size_t)kw * nt * mt * 256 * sizeof(float);
    const int64_t blocks = (N + 16 * nt - 1) / (16 * nt);
    hipLaunchKernelGGL(fn, dim3((uint32_t)blocks), dim3(64 * kw), lds, stream, a_codes, lda_c, a_scales, lda_s,
                       w_codes, ldw_c, w_scales, ldw_s, M, N, K, sp);
    return hipGetLastError();
}

}  // namespace nvfp4
