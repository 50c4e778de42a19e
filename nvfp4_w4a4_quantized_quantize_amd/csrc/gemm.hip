// Block-scaled W4A4 GEMM with a per-segment global-scale epilogue, for gfx950 (CDNA4).
//
//   y[m, n] = g_a * g_w[seg(n)] * sum_k e2m1(qa[m,k]) sa[m,k/16] * e2m1(qw[n,k]) sw[n,k/16]
//
// The fused-module case (several separately calibrated projections in one GEMM, each output-column
// segment with its own global scale) is the repair of the global-scale mismatch of the paper
// arXiv:2609.04098 (Japanese article, "Trap 1"; English abstract); the optional gate epilogues are
// the Gated DeltaNet parameterization of "Mechanism 2".
//
// Design (a dense contraction, so it runs on the matrix cores):
//  * An E2M1 value times an E4M3 scale has at most 6 significant bits and lies in [2^-10, 2688], so
//    it is exact in FP16, and FP16 x FP16 products are exact in FP32. Both operands are dequantized
//    to FP16 in registers and fed to v_mfma_f32_32x32x16_f16 with FP32 accumulation. (The FP4
//    matrix instructions take power-of-two E8M0 scales per 32 elements, which cannot express an
//    E4M3 scale per 16 elements exactly.)
//  * Dequantization costs two VALU instructions per pair of elements: the FP4 -> FP16 conversion
//    (whose scale operand only contributes a power of two, so it runs with 1.0) and a packed FP16
//    multiply by the block scale; block scales are converted E4M3 -> FP16 two at a time.
//  * Workgroup tile 256 x 256, K chunk 256, 4 waves as 2 x 2, each wave 128 x 128 = 4 x 4 MFMA tiles
//    of 32 x 32 accumulated in 256 registers. Codes (4 bits) and scale bytes go from HBM straight
//    into LDS (global_load_lds, no register staging), double buffered (2 x 72 KB), so each chunk's
//    loads overlap the previous chunk's 256 MFMAs per wave and LDS holds 4.5 bits per element.
//    Code rows are XOR-swizzled in 16-byte pieces so the fragment reads are free of bank conflicts.
//  * Inside a 64-element sub-chunk, K is permuted identically for A and W (lane half h of the MFMA
//    takes elements [32h + 8j, 32h + 8j + 8) at step j): each lane reads its 32 codes with one
//    16-byte LDS read. A sum does not depend on the order of its terms.
//  * Tiles are ordered for the 8 XCDs (each with its own L2): workgroup b runs on XCD b % 8, so each
//    XCD gets a contiguous range of tiles, walked in groups of 8 M-tiles so that concurrently
//    running tiles share A and W panels in L2.
//  * Epilogue: accumulators are staged per wave through LDS; whole 32-column groups of a plain
//    segment are scaled and written with 16-byte stores, other columns (gates, segment boundaries,
//    the N tail) element by element.
#include "internal.h"

namespace nvfp4 {
namespace {

typedef _Float16 half_t;
typedef half_t half2_t __attribute__((ext_vector_type(2)));
typedef half_t half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 256;
constexpr int NTHREADS = 256;
constexpr int ROW_BYTES = BK / 2;          // code bytes of one tile row per chunk (8 pieces of 16)
constexpr int A_CODES = 0;
constexpr int B_CODES = A_CODES + BM * ROW_BYTES;
constexpr int A_SCALES = B_CODES + BN * ROW_BYTES;
constexpr int B_SCALES = A_SCALES + BM * 16;
constexpr int STAGE_BYTES = B_SCALES + BN * 16;  // 73728
constexpr int EP_PITCH = 36;                     // floats per row of the epilogue staging tile
constexpr int GROUP_M = 8;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ void load_lds16(const uint8_t* g, uint8_t* lds) {
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(g), (lds_ptr_t)lds, 16, 0, 0);
}

// Issue the direct-to-LDS loads of one K chunk (this wave's share: 8 + 8 code rows groups, 2 scale
// groups). Rows beyond the matrix are clamped to its last row (their products land in output rows
// or columns that are never stored); code pieces wholly beyond K are read from the row's start (their
// block scales are masked to zero when converted).
__device__ __forceinline__ void issue_chunk(uint8_t* stage, const uint8_t* __restrict__ a_codes, int64_t lda_c,
                                            const uint8_t* __restrict__ a_scales, int64_t lda_s,
                                            const uint8_t* __restrict__ w_codes, int64_t ldw_c,
                                            const uint8_t* __restrict__ w_scales, int64_t ldw_s, int64_t m0,
                                            int64_t n0, int64_t M, int64_t N, int64_t k0, int64_t K, int wave,
                                            int lane) {
    const int rsub = lane >> 3, slot = lane & 7;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int j = wave * 8 + t;  // rows 8j .. 8j+7 of the tile
        const int r = 8 * j + rsub;
        const int p = slot ^ swz(r);
        const int64_t e = k0 + 32 * p;  // first element of the piece
        const int64_t koff = (e < K) ? (e >> 1) : 0;
        const int64_t ra = m0 + r < M ? m0 + r : M - 1;
        const int64_t rb = n0 + r < N ? n0 + r : N - 1;
        load_lds16(a_codes + ra * lda_c + koff, stage + A_CODES + j * 1024);
        load_lds16(w_codes + rb * ldw_c + koff, stage + B_CODES + j * 1024);
    }
    {
        const int j = wave;  // scale rows 64j .. 64j+63
        const int r = 64 * j + lane;
        const int64_t ra = m0 + r < M ? m0 + r : M - 1;
        const int64_t rb = n0 + r < N ? n0 + r : N - 1;
        load_lds16(a_scales + ra * lda_s + (k0 >> 4), stage + A_SCALES + j * 1024);
        load_lds16(w_scales + rb * ldw_s + (k0 >> 4), stage + B_SCALES + j * 1024);
    }
}

// 8 codes (one dword) times one FP16 block scale -> 8 exact FP16 values.
__device__ __forceinline__ half8_t dequant8(uint32_t w, half_t s) {
    const half2_t ss = {s, s};
    const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
    const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
    const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
    const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
    return half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// The two E4M3 scale bytes of (sub-chunk c, lane half lh) as FP16. In the chunk that crosses K
// (kTail), blocks at or beyond K get scale 0.
template <bool kTail>
__device__ __forceinline__ half2_t scale_pair(const u32x4& s, int c, int lh, int nvalid_blocks) {
    const uint32_t word = s[c] >> (lh << 4);  // bytes 4c + 2lh, 4c + 2lh + 1
    half2_t h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false);
    if (kTail) {
        const int b0 = 4 * c + 2 * lh;
        if (b0 >= nvalid_blocks) h[0] = (half_t)0.0f;
        if (b0 + 1 >= nvalid_blocks) h[1] = (half_t)0.0f;
    }
    return h;
}

// The MFMA work of one K chunk held in LDS stage `cur`: 4 sub-chunks x 4 steps x 16 MFMAs per wave.
template <bool kTail>
__device__ __forceinline__ void compute_chunk(floatx16 (&acc)[4][4], const uint8_t* cur, const int (&a_row)[4],
                                              const int (&b_row)[4], int lh, int nvalid) {
    u32x4 ascl[4], bscl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ascl[i] = *reinterpret_cast<const u32x4*>(cur + A_SCALES + a_row[i] * 16);
        bscl[i] = *reinterpret_cast<const u32x4*>(cur + B_SCALES + b_row[i] * 16);
    }
    u32x4 araw[4], braw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        araw[i] = *reinterpret_cast<const u32x4*>(cur + A_CODES + a_row[i] * ROW_BYTES + ((lh ^ swz(a_row[i])) << 4));
        braw[i] = *reinterpret_cast<const u32x4*>(cur + B_CODES + b_row[i] * ROW_BYTES + ((lh ^ swz(b_row[i])) << 4));
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {  // 64-element sub-chunks
        u32x4 anext[4], bnext[4];
        if (c < 3) {  // prefetch the next sub-chunk's codes while this one computes
            const int q = 2 * (c + 1) + lh;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                anext[i] = *reinterpret_cast<const u32x4*>(cur + A_CODES + a_row[i] * ROW_BYTES + ((q ^ swz(a_row[i])) << 4));
                bnext[i] = *reinterpret_cast<const u32x4*>(cur + B_CODES + b_row[i] * ROW_BYTES + ((q ^ swz(b_row[i])) << 4));
            }
        }
        half2_t as2[4], bs2[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            as2[i] = scale_pair<kTail>(ascl[i], c, lh, nvalid);
            bs2[i] = scale_pair<kTail>(bscl[i], c, lh, nvalid);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // MFMA K steps of 16
            half8_t aop[4], bop[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                aop[i] = dequant8(araw[i][j], as2[i][j >> 1]);
                bop[i] = dequant8(braw[i][j], bs2[i][j >> 1]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jn = 0; jn < 4; ++jn)
                    acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[i], bop[jn], acc[i][jn], 0, 0, 0);
        }
        if (c < 3) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                araw[i] = anext[i];
                braw[i] = bnext[i];
            }
        }
    }
}

__device__ __forceinline__ float sigmoid_f32(float y) { return 1.0f / (1.0f + expf(-y)); }

__device__ __forceinline__ float softplus_f32(float z) { return fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z))); }

__device__ __forceinline__ int segment_of(const SegParams& sp, int64_t col) {
    int s = 0;
    for (int t = 1; t < sp.n_segs; ++t)
        if (col >= sp.n_begin[t]) s = t;
    return s;
}

__device__ __forceinline__ float apply_gate(float y, int epi, float a_coef, float dtb) {
    if (epi == NVFP4_EPI_SIGMOID) return sigmoid_f32(y);
    if (epi == NVFP4_EPI_GDN_DECAY) return expf(-(a_coef * softplus_f32(y + dtb)));
    return y;
}

__global__ __launch_bounds__(NTHREADS, 1) void gemm_kernel(
    const uint8_t* __restrict__ a_codes, int64_t lda_c, const uint8_t* __restrict__ a_scales, int64_t lda_s,
    const uint8_t* __restrict__ w_codes, int64_t ldw_c, const uint8_t* __restrict__ w_scales, int64_t ldw_s,
    int64_t M, int64_t N, int64_t K, int32_t tiles_m, int32_t tiles_n, const SegParams sp) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31;  // row of the MFMA fragment this lane feeds
    const int lh = lane >> 5;  // lane half: which 8-element K group of an MFMA step

    // ---- tile order: contiguous per XCD, grouped by GROUP_M M-tiles inside it -------------------
    int tm, tn;
    {
        const int T = tiles_m * tiles_n;
        const int bid = blockIdx.x;
        const int xcd = bid & 7, local = bid >> 3;
        const int q = T >> 3, rem = T & 7;
        const int vt = (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + local;
        const int per_group = GROUP_M * tiles_n;
        const int g = vt / per_group, in_g = vt - g * per_group;
        const int first_m = g * GROUP_M;
        const int gm = tiles_m - first_m < GROUP_M ? tiles_m - first_m : GROUP_M;
        tm = first_m + in_g % gm;
        tn = in_g / gm;
    }
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t nk = (K + BK - 1) / BK;
    if (nk > 0)
        issue_chunk(smem, a_codes, lda_c, a_scales, lda_s, w_codes, ldw_c, w_scales, ldw_s, m0, n0, M, N, 0, K,
                    wave, lane);

    // per-lane LDS byte offsets of the fragment rows
    int a_row[4], b_row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a_row[i] = wm * 128 + 32 * i + lr;
        b_row[i] = wn * 128 + 32 * i + lr;
    }

    // full chunks, then (if K is not a multiple of BK) the chunk that crosses K
    const int64_t nk_full = K / BK;
    for (int64_t kc = 0; kc < nk_full; ++kc) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of chunk kc landed
        __syncthreads();                                    // ... and everyone's; chunk kc-1 fully consumed
        if (kc + 1 < nk)
            issue_chunk(smem + ((kc + 1) & 1) * STAGE_BYTES, a_codes, lda_c, a_scales, lda_s, w_codes, ldw_c,
                        w_scales, ldw_s, m0, n0, M, N, (kc + 1) * BK, K, wave, lane);
        compute_chunk<false>(acc, smem + (kc & 1) * STAGE_BYTES, a_row, b_row, lh, BK / 16);
    }
    if (nk_full < nk) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        compute_chunk<true>(acc, smem + (nk_full & 1) * STAGE_BYTES, a_row, b_row, lh,
                            (int)((K - nk_full * BK) >> 4));
    }
    __syncthreads();  // all waves done with the LDS stages before the epilogue reuses them

    // ---- epilogue ---------------------------------------------------------------------------------
    float* ep = reinterpret_cast<float*>(smem) + wave * (128 * EP_PITCH);
    const int64_t row_base = m0 + wm * 128;
    const int nrows = (int)(M - row_base < 128 ? (M - row_base > 0 ? M - row_base : 0) : 128);
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                ep[(32 * i + (r >> 2) * 8 + lh * 4 + (r & 3)) * EP_PITCH + lr] = acc[i][jn][r];
        __syncthreads();
        const int64_t c0 = n0 + wn * 128 + 32 * jn;  // first column of this 32-column group
        if (c0 < N) {
            const int s0 = segment_of(sp, c0);
            const bool whole = c0 + 32 <= N && c0 + 31 < sp.n_end[s0];
            const bool vec = whole && sp.epilogue[s0] == NVFP4_EPI_NONE &&
                             ((sp.vec_mask >> s0) & 1u) != 0;
            if (vec) {
                // 16 rows x 32 columns per pass: lane -> row (lane / 4), 8 columns (lane % 4) * 8
                const float scale = sp.scale[s0];
                const int64_t j0 = c0 - sp.n_begin[s0] + (lane & 3) * 8;
                const int64_t ldo = sp.ldo[s0];
                for (int rr = lane >> 2; rr < nrows; rr += 16) {
                    const f32x4 v0 = *reinterpret_cast<const f32x4*>(ep + rr * EP_PITCH + (lane & 3) * 8);
                    const f32x4 v1 = *reinterpret_cast<const f32x4*>(ep + rr * EP_PITCH + (lane & 3) * 8 + 4);
                    const int64_t off = (row_base + rr) * ldo + j0;
                    if (sp.out_dtype[s0] == NVFP4_OUT_BF16) {
                        u32x4 packed;
                        packed[0] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)(v0[0] * scale), (__bf16)(v0[1] * scale)});
                        packed[1] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)(v0[2] * scale), (__bf16)(v0[3] * scale)});
                        packed[2] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)(v1[0] * scale), (__bf16)(v1[1] * scale)});
                        packed[3] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)(v1[2] * scale), (__bf16)(v1[3] * scale)});
                        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(sp.out[s0]) + off) = packed;
                    } else {
                        float* o = reinterpret_cast<float*>(sp.out[s0]) + off;
                        *reinterpret_cast<f32x4*>(o) = v0 * scale;
                        *reinterpret_cast<f32x4*>(o + 4) = v1 * scale;
                    }
                }
            } else {
                const int64_t col = c0 + lr;
                if (col < N) {
                    const int s = segment_of(sp, col);
                    const float scale = sp.scale[s];
                    const int epi = sp.epilogue[s];
                    const int64_t j = col - sp.n_begin[s];
                    const int64_t ldo = sp.ldo[s];
                    float a_coef = 0.0f, dtb = 0.0f;
                    if (epi == NVFP4_EPI_GDN_DECAY) {
                        a_coef = expf(sp.A_log[s][j]);
                        dtb = sp.dt_bias[s][j];
                    }
                    for (int rr = lh; rr < nrows; rr += 2) {
                        const float y = apply_gate(ep[rr * EP_PITCH + lr] * scale, epi, a_coef, dtb);
                        const int64_t off = (row_base + rr) * ldo + j;
                        if (sp.out_dtype[s] == NVFP4_OUT_F32)
                            reinterpret_cast<float*>(sp.out[s])[off] = y;
                        else
                            reinterpret_cast<__bf16*>(sp.out[s])[off] = (__bf16)y;
                    }
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s,
                       const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s,
                       int64_t M, int64_t N, int64_t K, const SegParams& sp, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    hipLaunchKernelGGL(gemm_kernel, dim3((uint32_t)(tiles_m * tiles_n)), dim3(NTHREADS), 0, stream, a_codes,
                       lda_c, a_scales, lda_s, w_codes, ldw_c, w_scales, ldw_s, M, N, K, (int32_t)tiles_m,
                       (int32_t)tiles_n, sp);
    return hipGetLastError();
}

}  // namespace nvfp4
