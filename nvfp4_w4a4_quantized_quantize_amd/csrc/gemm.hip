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
#include "device_common.h"

namespace nvfp4 {
namespace {

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

// Direct-to-LDS loads. A K chunk is 18 loads per wave ("pieces"): pieces 0-7 are A code row groups,
// 8-15 W code row groups (lane -> row 8j + lane / 8 of the tile, j = 8 wave + t, 16-byte piece
// (lane % 8) ^ swz(row)), 16 and 17 the A and W scale rows 64 wave + lane. Rows beyond the matrix are
// clamped to its last row: their products only reach output rows or columns that are never stored.
// In the chunk that crosses K, code pieces starting at or beyond K are read from the row start
// instead (in bounds); their block scales are zeroed before use.
struct Loader {
    const uint8_t* a_codes; const uint8_t* a_scales; const uint8_t* w_codes; const uint8_t* w_scales;
    int64_t lda_c, lda_s, ldw_c, ldw_s, m0, n0, M, N, K;
    int wave, lane;

    __device__ __forceinline__ void piece(uint8_t* stage, int pc, int64_t k0) const {
        const bool is_a = pc < 8 || pc == 16;
        const uint8_t* codes = is_a ? a_codes : w_codes;
        const uint8_t* scales = is_a ? a_scales : w_scales;
        const int64_t ldc = is_a ? lda_c : ldw_c, lds = is_a ? lda_s : ldw_s;
        const int64_t row0 = is_a ? m0 : n0, nrows = is_a ? M : N;
        const bool full_rows = row0 + BM <= nrows;
        if (pc < 16) {
            const int t = pc & 7;
            const int j = wave * 8 + t;  // j & 7 == t, so swz(8j + rsub) == rsub ^ t
            const int rsub = lane >> 3;
            const int p = (lane & 7) ^ rsub ^ t;
            int64_t koff = 16 * p;
            if (k0 + BK > K && k0 + 32 * p >= K) koff = -(k0 >> 1);
            const int64_t r = row0 + 8 * j + rsub;
            const int64_t row = full_rows ? r : (r < nrows ? r : nrows - 1);
            load_lds16(codes + (k0 >> 1) + row * ldc + koff, stage + (is_a ? A_CODES : B_CODES) + j * 1024);
        } else {
            const int64_t r = row0 + 64 * wave + lane;
            const int64_t row = full_rows ? r : (r < nrows ? r : nrows - 1);
            load_lds16(scales + row * lds + (k0 >> 4), stage + (is_a ? A_SCALES : B_SCALES) + wave * 1024);
        }
    }

    __device__ __forceinline__ void all(uint8_t* stage, int64_t k0) const {
#pragma unroll
        for (int pc = 0; pc < 18; ++pc) piece(stage, pc, k0);
    }
};

// The two E4M3 scale bytes of (sub-chunk c, lane half lh) as FP16.
__device__ __forceinline__ half2_t scale_pair(const u32x4& s, int c, int lh) {
    const uint32_t word = s[c] >> (lh << 4);  // bytes 4c + 2lh, 4c + 2lh + 1
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false);
}

// Codes of sub-chunk c (64 elements) for the 4 A and 4 W fragments of this lane.
__device__ __forceinline__ void read_codes(u32x4 (&ar)[4], u32x4 (&br)[4], const uint8_t* stage, const int (&a_row)[4],
                                           const int (&b_row)[4], int c, int lh) {
    const int q = 2 * c + lh;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ar[i] = *reinterpret_cast<const u32x4*>(stage + A_CODES + a_row[i] * ROW_BYTES + ((q ^ swz(a_row[i])) << 4));
        br[i] = *reinterpret_cast<const u32x4*>(stage + B_CODES + b_row[i] * ROW_BYTES + ((q ^ swz(b_row[i])) << 4));
    }
}

// Scale rows of a chunk (16 bytes each). When the chunk crosses K, bytes of blocks at or beyond K
// (nvalid of them are valid) are cleared, so that the code pieces read in their place contribute 0.
__device__ __forceinline__ void read_scales(u32x4 (&as)[4], u32x4 (&bs)[4], const uint8_t* stage, const int (&a_row)[4],
                                            const int (&b_row)[4], int nvalid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        as[i] = *reinterpret_cast<const u32x4*>(stage + A_SCALES + a_row[i] * 16);
        bs[i] = *reinterpret_cast<const u32x4*>(stage + B_SCALES + b_row[i] * 16);
    }
    if (nvalid < 16) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int nb = nvalid - 4 * d;  // valid bytes in dword d
            const uint32_t mask = nb >= 4 ? 0xffffffffu : (nb <= 0 ? 0u : (0xffffffffu >> (32 - 8 * nb)));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                as[i][d] &= mask;
                bs[i][d] &= mask;
            }
        }
    }
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

    // per-lane LDS row indices of the MFMA fragments
    int a_row[4], b_row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a_row[i] = wm * 128 + 32 * i + lr;
        b_row[i] = wn * 128 + 32 * i + lr;
    }

    // ---- main loop --------------------------------------------------------------------------------
    // Chunk kc lives in LDS stage kc % 2. One barrier per chunk, after step 11: every wave has then
    // finished reading the current stage (its last code read feeds step 12) and has waited for its
    // own loads of chunk kc + 1 (issued a whole chunk earlier), so after the barrier chunk kc + 1 is
    // visible and the current stage is free for chunk kc + 2. Steps 12-15 then prefetch chunk
    // kc + 1's scales and first codes, and step 15 dequantizes its first step, so the MFMA stream
    // runs on across the chunk boundary.
    const int64_t nk = (K + BK - 1) / BK;
    if (nk > 0) {
        auto nvalid_of = [&](int64_t kc) -> int {
            const int64_t rest = (K - kc * BK) >> 4;
            return rest >= 16 ? 16 : (int)rest;
        };
        const Loader ld{a_codes, a_scales, w_codes, w_scales, lda_c, lda_s, ldw_c, ldw_s, m0, n0, M, N, K, wave, lane};
        ld.all(smem, 0);
        // chunk 1 (or chunk 0 again when there is none): pieces 0-7 now, 8-17 during chunk 0's steps 0-4
        const int64_t k1 = nk > 1 ? BK : 0;
#pragma unroll
        for (int pc = 0; pc < 8; ++pc) ld.piece(smem + STAGE_BYTES, pc, k1);
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // the 18 loads of chunk 0 landed
        __syncthreads();

        u32x4 ascl[4], bscl[4], araw[4], braw[4], anext[4], bnext[4];
        half2_t as2[4], bs2[4];
        half8_t aop[2][4], bop[2][4];
        read_scales(ascl, bscl, smem, a_row, b_row, nvalid_of(0));
        read_codes(araw, braw, smem, a_row, b_row, 0, lh);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            as2[i] = scale_pair(ascl[i], 0, lh);
            bs2[i] = scale_pair(bscl[i], 0, lh);
            aop[0][i] = dequant8(araw[i][0], as2[i][0]);
            bop[0][i] = dequant8(braw[i][0], bs2[i][0]);
        }

        for (int64_t kc = 0; kc < nk; ++kc) {
            const uint8_t* cur = smem + (kc & 1) * STAGE_BYTES;
            uint8_t* nxt = smem + ((kc + 1) & 1) * STAGE_BYTES;
#pragma unroll
            for (int st = 0; st < 16; ++st) {
                const int c = st >> 2, j = st & 3;
                const int cb = st & 1, nb = cb ^ 1;
                // loads, two pieces per step: chunk kc + 1's pieces 8-17 at steps 0-4 (into the stage freed
                // at the previous chunk's barrier), chunk kc + 2's pieces 0-7 at steps 12-15 (into the
                // stage freed at this chunk's barrier); chunk indices clamp to the last chunk
                if (st <= 4) {
                    const int64_t k1c = (kc + 1 < nk ? kc + 1 : nk - 1) * BK;
                    ld.piece(nxt, 8 + 2 * st, k1c);
                    ld.piece(nxt, 9 + 2 * st, k1c);
                }
                if (st == 12) {
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of chunk kc + 1
                    __syncthreads();
                    read_scales(ascl, bscl, nxt, a_row, b_row, nvalid_of(kc + 1 < nk ? kc + 1 : kc));
                    read_codes(anext, bnext, nxt, a_row, b_row, 0, lh);
                } else if (j == 0) {
                    read_codes(anext, bnext, cur, a_row, b_row, c + 1, lh);  // sub-chunk c + 1
                }
                // operands of the next step (the next chunk's first step after step 15)
                const int s1 = (st + 1) & 15, c1 = s1 >> 2, j1 = s1 & 3;
                if (j1 == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        araw[i] = anext[i];
                        braw[i] = bnext[i];
                        as2[i] = scale_pair(ascl[i], c1, lh);
                        bs2[i] = scale_pair(bscl[i], c1, lh);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    aop[nb][i] = dequant8(araw[i][j1], as2[i][j1 >> 1]);
                    bop[nb][i] = dequant8(braw[i][j1], bs2[i][j1 >> 1]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int jn = 0; jn < 4; ++jn)
                        acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[cb][i], bop[cb][jn], acc[i][jn], 0, 0, 0);
                if (st >= 12) {
                    const int64_t k2c = (kc + 2 < nk ? kc + 2 : nk - 1) * BK;
                    ld.piece(const_cast<uint8_t*>(cur), 2 * (st - 12), k2c);
                    ld.piece(const_cast<uint8_t*>(cur), 2 * (st - 12) + 1, k2c);
                }
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // then four VALU
                }
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may still target the LDS
    }
    __syncthreads();  // all waves done with the LDS stages before the epilogue reuses them

    // ---- epilogue ---------------------------------------------------------------------------------
    // Each wave stages one 128 x 32 column group of its FP32 accumulators at a time in a private LDS
    // region (36-float row pitch). A group inside one plain segment is then scaled and written with
    // 16-byte stores, lane -> row lane / 4 (+16 per pass), columns (lane % 4) * 8 .. + 8; gate segments,
    // segment boundaries and the N tail go element by element, lane -> column lane % 32.
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
        // the region is private to this wave: its own LDS writes completing is enough
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int64_t c0 = n0 + wn * 128 + 32 * jn;  // first column of this 32-column group
        if (c0 < N) {
            const int s0 = segment_of(sp, c0);
            const bool vec = c0 + 32 <= N && c0 + 31 < sp.n_end[s0] && sp.epilogue[s0] == NVFP4_EPI_NONE &&
                             ((sp.vec_mask >> s0) & 1u) != 0;
            if (vec) {
                const float scale = sp.scale[s0];
                const int64_t ldo = sp.ldo[s0];
                const bool bf16 = sp.out_dtype[s0] == NVFP4_OUT_BF16;
                uint8_t* outp = reinterpret_cast<uint8_t*>(sp.out[s0]);
                const int64_t j0 = c0 - sp.n_begin[s0] + (lane & 3) * 8;
                f32x4 v[16];
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    const float* src = ep + ((lane >> 2) + 16 * p) * EP_PITCH + (lane & 3) * 8;
                    v[2 * p] = *reinterpret_cast<const f32x4*>(src);
                    v[2 * p + 1] = *reinterpret_cast<const f32x4*>(src + 4);
                }
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    const int rr = (lane >> 2) + 16 * p;
                    if (rr < nrows) {
                        const int64_t off = (row_base + rr) * ldo + j0;
                        const f32x4 y0 = v[2 * p] * scale, y1 = v[2 * p + 1] * scale;
                        if (bf16) {
                            u32x4 packed;
                            packed[0] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)y0[0], (__bf16)y0[1]});
                            packed[1] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)y0[2], (__bf16)y0[3]});
                            packed[2] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)y1[0], (__bf16)y1[1]});
                            packed[3] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)y1[2], (__bf16)y1[3]});
                            *reinterpret_cast<u32x4*>(outp + off * 2) = packed;
                        } else {
                            *reinterpret_cast<f32x4*>(outp + off * 4) = y0;
                            *reinterpret_cast<f32x4*>(outp + off * 4 + 16) = y1;
                        }
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
                    const bool f32out = sp.out_dtype[s] == NVFP4_OUT_F32;
                    uint8_t* outp = reinterpret_cast<uint8_t*>(sp.out[s]);
                    float a_coef = 0.0f, dtb = 0.0f;
                    if (epi == NVFP4_EPI_GDN_DECAY) {
                        a_coef = expf(sp.A_log[s][j]);
                        dtb = sp.dt_bias[s][j];
                    }
                    for (int rr = lh; rr < nrows; rr += 2) {
                        const float y = apply_gate(ep[rr * EP_PITCH + lr] * scale, epi, a_coef, dtb);
                        const int64_t off = (row_base + rr) * ldo + j;
                        if (f32out)
                            reinterpret_cast<float*>(outp)[off] = y;
                        else
                            reinterpret_cast<__bf16*>(outp)[off] = (__bf16)y;
                    }
                }
            }
        }
        // the next group's staging writes must not pass this group's reads
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
}

}  // namespace

hipError_t launch_gemm_tiled(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s,
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
