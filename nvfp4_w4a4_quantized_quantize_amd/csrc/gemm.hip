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
//    into LDS (buffer loads with the LDS destination, no register staging), double buffered
//    (2 x 72 KB), so each chunk's loads overlap the previous chunk's 256 MFMAs per wave and LDS holds
//    4.5 bits per element. The buffer resources cover only a tile's existing rows, so the loads need
//    no clamping: reads past the end return nothing and address only rows that are never stored.
//    Code rows are XOR-swizzled in 16-byte pieces so the fragment reads are free of bank conflicts.
//  * Inside a K chunk, K is permuted identically for A and W: at step j of sub-chunk c, lane half h
//    of the MFMA takes elements [128h + 32c + 8j, 128h + 32c + 8j + 8), so each lane reads the 32
//    codes of a sub-chunk with one 16-byte LDS read and its 8 block scales of the chunk with one
//    8-byte read. A sum does not depend on the order of its terms.
//  * In a partial last column of tiles, a wave skips the 32-column fragments that lie wholly past N
//    (no reads, dequantization or matrix instructions for them); its loads and barriers are the same.
//    A tile of at most 128 columns stacks its 4 waves along M (64 rows each), so all of them work.
//  * Tiles are ordered for the 8 XCDs (each with its own L2): workgroup b runs on XCD b % 8, so each
//    XCD gets a contiguous range of full-width tiles, walked in groups of 8 M-tiles so that
//    concurrently running tiles share A and W panels in L2; the partial column's tiles run last.
//  * When the full tiles' last round would leave CUs idle (C2's 320 tiles on 256 CUs: a second round
//    a quarter full), the trailing tile columns that make up that round run as 128- or 64-column
//    tiles instead, as many as fit one round. A narrow tile is computed exactly like the partial
//    column's (waves stacked along M), and its weight buffer resource covers only its own rows, so the
//    loads of the other rows fetch nothing. Every output's sum runs in the same order either way.
//  * Epilogue: the W fragment is the MFMA's first operand, so each lane holds runs of 4 consecutive
//    output columns of one row. Accumulators are staged per wave through LDS (one 16-byte write per
//    run), 64 columns at a time; column ranges of a plain segment are scaled and written with 16-byte
//    stores, 64 columns (whole 128-byte lines of bf16) or 32 at a time, other columns (gates,
//    segment boundaries, the N tail) element by element.
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
constexpr int EP_PITCH = 68;                     // floats per row of the epilogue staging tile
constexpr int GROUP_M = 8;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Direct-to-LDS buffer loads. A K chunk is 18 loads per wave ("pieces"): pieces 0-7 are A code row
// groups, 8-15 W code row groups (lane -> row 8j + lane / 8 of the tile, j = 8 wave + t, 16-byte piece
// (lane % 8) ^ swz(row)), 16 and 17 the A and W scale rows 64 wave + lane. Each operand's buffer
// resource covers only the tile's rows that exist, so rows beyond the matrix read outside it and
// return no data: their products only reach output rows or columns that are never stored. Code
// pieces of the chunk that crosses K read past the row's K (the next row, or outside the buffer);
// their block scales are zeroed before use.
constexpr int BUF_FLAGS = 0x00020000;  // raw buffer resource, 32-bit data format (gfx9 family)

struct Loader {
    __amdgpu_buffer_rsrc_t ra_c, rw_c, ra_s, rw_s;
    uint32_t lda_c, ldw_c, lda_s, ldw_s;
    uint32_t va_c, vw_c, va_s, vw_s;  // lane parts of the offsets: row lane / 8 (codes), row lane (scales)
    uint32_t vq;                      // 16 * ((lane % 8) ^ (lane / 8)): the lane's piece before the XOR with t
    int wave;

    __device__ __forceinline__ void piece(uint8_t* stage, int pc, uint32_t k0) const {
        const bool is_a = pc < 8 || pc == 16;
        if (pc < 16) {
            const int t = pc & 7;
            const int j = wave * 8 + t;  // j & 7 == t, so swz(8j + rsub) == rsub ^ t
            const uint32_t ldc = is_a ? lda_c : ldw_c;
            const uint32_t voff = (is_a ? va_c : vw_c) + (vq ^ (16u * t));
            const uint32_t soff = (uint32_t)(8 * j) * ldc + (k0 >> 1);
            uint8_t* dst = stage + (is_a ? A_CODES : B_CODES) + j * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? ra_c : rw_c, (lds_ptr_t)dst, 16, (int)voff, (int)soff, 0, 0);
        } else {
            const uint32_t lds = is_a ? lda_s : ldw_s;
            const uint32_t soff = (uint32_t)(64 * wave) * lds + (k0 >> 4);
            uint8_t* dst = stage + (is_a ? A_SCALES : B_SCALES) + wave * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? ra_s : rw_s, (lds_ptr_t)dst, 16, (int)(is_a ? va_s : vw_s),
                                                     (int)soff, 0, 0);
        }
    }

    __device__ __forceinline__ void all(uint8_t* stage, uint32_t k0) const {
#pragma unroll
        for (int pc = 0; pc < 18; ++pc) piece(stage, pc, k0);
    }
};

// Buffer resource over the existing rows of the tile starting at row0 (at most BM rows of ld bytes;
// the host keeps ld below 2^23, so BM * ld and every offset fit in 31 bits).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int64_t row0, int64_t nrows,
                                                            int64_t ld) {
    const int64_t rows = nrows - row0 < BM ? nrows - row0 : BM;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base + row0 * ld), (short)0, (int)(rows * ld),
                                             BUF_FLAGS);
}

// The two E4M3 scale bytes of sub-chunk c as FP16: s holds the 8 scale bytes of this lane half's
// 128 elements of the chunk, and sub-chunk c uses its bytes 2c and 2c + 1.
__device__ __forceinline__ half2_t scale_pair(const u32x2& s, int c) {
    return (c & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s[c >> 1], 1.0f, true)
                   : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s[c >> 1], 1.0f, false);
}

// Codes of sub-chunk c (64 elements) for the first NA A and the first NB W fragments of this lane.
template <int NA, int NB>
__device__ __forceinline__ void read_codes(u32x4 (&ar)[4], u32x4 (&br)[4], const uint8_t* stage, const int (&a_row)[4],
                                           const int (&b_row)[4], int c, int lh) {
    const int q = 4 * lh + c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i < NA)
            ar[i] = *reinterpret_cast<const u32x4*>(stage + A_CODES + a_row[i] * ROW_BYTES + ((q ^ swz(a_row[i])) << 4));
        if (i < NB)
            br[i] = *reinterpret_cast<const u32x4*>(stage + B_CODES + b_row[i] * ROW_BYTES + ((q ^ swz(b_row[i])) << 4));
    }
}

// This lane half's 8 scale bytes of each fragment row of a chunk (bytes 8 lh .. 8 lh + 7 of the row's
// 16). When the chunk crosses K, bytes of blocks at or beyond K (nvalid of the row's 16 are valid)
// are cleared, so that the code pieces read in their place contribute 0. (Fragments as in read_codes.)
template <int NA, int NB>
__device__ __forceinline__ void read_scales(u32x2 (&as)[4], u32x2 (&bs)[4], const uint8_t* stage, const int (&a_row)[4],
                                            const int (&b_row)[4], int lh, int nvalid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i < NA) as[i] = *reinterpret_cast<const u32x2*>(stage + A_SCALES + a_row[i] * 16 + 8 * lh);
        if (i < NB) bs[i] = *reinterpret_cast<const u32x2*>(stage + B_SCALES + b_row[i] * 16 + 8 * lh);
    }
    if (nvalid < 16) {  // only the chunk that crosses K; the asm keeps this a branch instead of selects
        asm volatile("" ::: "memory");
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const int nb = nvalid - 8 * lh - 4 * d;  // valid bytes in this lane's dword d
            const uint32_t mask = nb >= 4 ? 0xffffffffu : (nb <= 0 ? 0u : (0xffffffffu >> (32 - 8 * nb)));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i < NA) as[i][d] &= mask;
                if (i < NB) bs[i][d] &= mask;
            }
        }
    }
}

// The main loop over the nk K chunks (see the kernel) for a wave with NA row fragments and NB column
// fragments of 32: 4 x 4 in full tiles; in a partial last column of tiles the fragments past N are
// neither read, dequantized nor multiplied (4 x 2, or 2 x 2 and 2 x 4 when the tile's waves are
// stacked along M). Every wave runs the same loads and barriers.
//
// The W fragment is the MFMA's first operand, so the 32 x 32 result is the transposed output tile:
// lane l holds output row lr = l % 32 of the fragment and, in register 4 g + e, output column
// 8 g + 4 (l / 32) + e, i.e. four consecutive columns of one row per group g.
template <int NA, int NB>
__device__ __forceinline__ void main_loop(floatx16 (&acc)[4][4], uint8_t* smem, const Loader& ld, const int (&a_row)[4],
                                          const int (&b_row)[4], int lh, int64_t nk, int64_t K) {
    auto nvalid_of = [&](int64_t kc) -> int {
        const int64_t rest = (K - kc * BK) >> 4;
        return rest >= 16 ? 16 : (int)rest;
    };
    ld.all(smem, 0);
    // chunk 1 (or chunk 0 again when there is none): pieces 0-7 now, 8-17 during chunk 0's steps 0-4
    const uint32_t k1 = nk > 1 ? BK : 0;
#pragma unroll
    for (int pc = 0; pc < 8; ++pc) ld.piece(smem + STAGE_BYTES, pc, k1);
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // the 18 loads of chunk 0 landed
    __syncthreads();

    u32x2 ascl[4], bscl[4];
    u32x4 araw[4], braw[4], anext[4], bnext[4];
    half2_t as2[4], bs2[4];
    half8_t aop[2][4], bop[2][4];
    read_scales<NA, NB>(ascl, bscl, smem, a_row, b_row, lh, nvalid_of(0));
    read_codes<NA, NB>(araw, braw, smem, a_row, b_row, 0, lh);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i < NA) {
            as2[i] = scale_pair(ascl[i], 0);
            aop[0][i] = dequant8(araw[i][0], as2[i][0]);
        }
        if (i < NB) {
            bs2[i] = scale_pair(bscl[i], 0);
            bop[0][i] = dequant8(braw[i][0], bs2[i][0]);
        }
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
                const uint32_t k1c = (uint32_t)((kc + 1 < nk ? kc + 1 : nk - 1) * BK);
                ld.piece(nxt, 8 + 2 * st, k1c);
                ld.piece(nxt, 9 + 2 * st, k1c);
            }
            if (st == 12) {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of chunk kc + 1
                __syncthreads();
                read_scales<NA, NB>(ascl, bscl, nxt, a_row, b_row, lh, nvalid_of(kc + 1 < nk ? kc + 1 : kc));
                read_codes<NA, NB>(anext, bnext, nxt, a_row, b_row, 0, lh);
            } else if (j == 0) {
                read_codes<NA, NB>(anext, bnext, cur, a_row, b_row, c + 1, lh);  // sub-chunk c + 1
            }
            // operands of the next step (the next chunk's first step after step 15)
            const int s1 = (st + 1) & 15, c1 = s1 >> 2, j1 = s1 & 3;
            if (j1 == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (i < NA) {
                        araw[i] = anext[i];
                        as2[i] = scale_pair(ascl[i], c1);
                    }
                    if (i < NB) {
                        braw[i] = bnext[i];
                        bs2[i] = scale_pair(bscl[i], c1);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i < NA) aop[nb][i] = dequant8(araw[i][j1], as2[i][j1 >> 1]);
                if (i < NB) bop[nb][i] = dequant8(braw[i][j1], bs2[i][j1 >> 1]);
            }
#pragma unroll
            for (int i = 0; i < NA; ++i)
#pragma unroll
                for (int jn = 0; jn < NB; ++jn)
                    acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bop[cb][jn], aop[cb][i], acc[i][jn], 0, 0, 0);
            if (st >= 12) {
                const uint32_t k2c = (uint32_t)((kc + 2 < nk ? kc + 2 : nk - 1) * BK);
                ld.piece(const_cast<uint8_t*>(cur), 2 * (st - 12), k2c);
                ld.piece(const_cast<uint8_t*>(cur), 2 * (st - 12) + 1, k2c);
            }
#pragma unroll
            for (int t = 0; t < NA * NB; ++t) {
                // one MFMA, then its share of the (NA + NB) dequantizations of 8 VALU instructions each
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 8 * (NA + NB) / (NA * NB), 0);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may still target the LDS
}

// Writes one wave's outputs. acc[i][jn][4 g + e] is output (row0 + 32 i + lr, col0 + 32 jn + 8 g + 4 lh + e)
// (i < NA, jn < NB). Each pair of column fragments (64 columns) is staged in the wave's LDS region ep
// (32 NA rows, EP_PITCH floats apart) with one 16-byte write per group; then a pair inside one plain
// segment is scaled and written with 16-byte stores, 8 lanes per row (whole 128-byte lines of bf16),
// other 32-column fragments of a plain segment with 4 lanes per row, and gate segments, segment
// boundaries and the N tail element by element, lane -> column lr, rows of parity lh.
template <int NA, int NB>
__device__ __forceinline__ void store_tile(const floatx16 (&acc)[4][4], const SegParams& sp, int64_t row0, int64_t col0,
                                           int64_t M, int64_t N, int lane, float* ep) {
    constexpr int RW = 32 * NA;  // rows of the wave
    const int lr = lane & 31, lh = lane >> 5;
    const int nrows = (int)(M - row0 < RW ? (M - row0 > 0 ? M - row0 : 0) : RW);
    auto plain_run = [&](int64_t c0, int width) -> int {  // segment of [c0, c0 + width) if written by vector stores, else -1
        const int s0 = segment_of(sp, c0);
        const bool ok = c0 + width <= N && c0 + width - 1 < sp.n_end[s0] && sp.epilogue[s0] == NVFP4_EPI_NONE &&
                        ((sp.vec_mask >> s0) & 1u) != 0;
        return ok ? s0 : -1;
    };
    auto store8 = [&](uint8_t* outp, bool bf16, int64_t off, f32x4 y0, f32x4 y1) {
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
    };
#pragma unroll
    for (int jp = 0; jp < NB / 2; ++jp) {
        const int64_t c0 = col0 + 64 * jp;  // first column of this 64-column pair
        if (c0 >= N) break;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < NA; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<f32x4*>(ep + (32 * i + lr) * EP_PITCH + 32 * h + 8 * g + 4 * lh) =
                        f32x4{acc[i][2 * jp + h][4 * g], acc[i][2 * jp + h][4 * g + 1], acc[i][2 * jp + h][4 * g + 2],
                              acc[i][2 * jp + h][4 * g + 3]};
        // the region is private to this wave: its own LDS writes completing is enough
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int s64 = plain_run(c0, 64);
        if (s64 >= 0) {
            const float scale = sp.scale[s64];
            const int64_t ldo = sp.ldo[s64];
            const bool bf16 = sp.out_dtype[s64] == NVFP4_OUT_BF16;
            uint8_t* outp = reinterpret_cast<uint8_t*>(sp.out[s64]);
            const int64_t j0 = c0 - sp.n_begin[s64] + (lane & 7) * 8;
            if (nrows == RW && bf16) {  // full rows, bf16: no per-row masks, no per-store type test
                uint8_t* dst = outp + ((row0 + (lane >> 3)) * ldo + j0) * 2;
                const int64_t step8 = 8 * ldo * 2;  // bytes between a lane's consecutive rows
#pragma unroll
                for (int half = 0; half < RW / 64; ++half) {
                    f32x4 v[16];
#pragma unroll
                    for (int p = 0; p < 8; ++p) {
                        const float* src = ep + ((lane >> 3) + 8 * (8 * half + p)) * EP_PITCH + (lane & 7) * 8;
                        v[2 * p] = *reinterpret_cast<const f32x4*>(src);
                        v[2 * p + 1] = *reinterpret_cast<const f32x4*>(src + 4);
                    }
#pragma unroll
                    for (int p = 0; p < 8; ++p) {
                        const f32x4 y0 = v[2 * p] * scale, y1 = v[2 * p + 1] * scale;
                        u32x4 packed;
                        packed[0] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)y0[0], (__bf16)y0[1]});
                        packed[1] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)y0[2], (__bf16)y0[3]});
                        packed[2] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)y1[0], (__bf16)y1[1]});
                        packed[3] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)y1[2], (__bf16)y1[3]});
                        *reinterpret_cast<u32x4*>(dst + (8 * half + p) * step8) = packed;
                    }
                }
            } else
#pragma unroll
            for (int half = 0; half < RW / 64; ++half) {
                f32x4 v[16];
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    const float* src = ep + ((lane >> 3) + 8 * (8 * half + p)) * EP_PITCH + (lane & 7) * 8;
                    v[2 * p] = *reinterpret_cast<const f32x4*>(src);
                    v[2 * p + 1] = *reinterpret_cast<const f32x4*>(src + 4);
                }
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    const int rr = (lane >> 3) + 8 * (8 * half + p);
                    if (rr < nrows) store8(outp, bf16, (row0 + rr) * ldo + j0, v[2 * p] * scale, v[2 * p + 1] * scale);
                }
            }
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t c1 = c0 + 32 * h;  // first column of this 32-column fragment
                if (c1 >= N) break;
                const int s32 = plain_run(c1, 32);
                if (s32 >= 0) {
                    const float scale = sp.scale[s32];
                    const int64_t ldo = sp.ldo[s32];
                    const bool bf16 = sp.out_dtype[s32] == NVFP4_OUT_BF16;
                    uint8_t* outp = reinterpret_cast<uint8_t*>(sp.out[s32]);
                    const int64_t j0 = c1 - sp.n_begin[s32] + (lane & 3) * 8;
#pragma unroll
                    for (int p = 0; p < RW / 16; ++p) {
                        const int rr = (lane >> 2) + 16 * p;
                        const float* src = ep + rr * EP_PITCH + 32 * h + (lane & 3) * 8;
                        const f32x4 y0 = *reinterpret_cast<const f32x4*>(src), y1 = *reinterpret_cast<const f32x4*>(src + 4);
                        if (rr < nrows) store8(outp, bf16, (row0 + rr) * ldo + j0, y0 * scale, y1 * scale);
                    }
                } else {
                    const int64_t col = c1 + lr;
                    if (col < N) {
                        const ColumnOut c = column_out(sp, col);
                        for (int rr = lh; rr < nrows; rr += 2) column_store(c, row0 + rr, ep[rr * EP_PITCH + 32 * h + lr]);
                    }
                }
            }
        }
        // the next pair's staging writes must not pass this pair's reads
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
}

__global__ __launch_bounds__(NTHREADS, 1) void gemm_kernel(
    const uint8_t* __restrict__ a_codes, int64_t lda_c, const uint8_t* __restrict__ a_scales, int64_t lda_s,
    const uint8_t* __restrict__ w_codes, int64_t ldw_c, const uint8_t* __restrict__ w_scales, int64_t ldw_s,
    int64_t M, int64_t N, int64_t K, const TileMap tmap, const SegParams sp) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31;  // row of the MFMA fragment this lane feeds
    const int lh = lane >> 5;  // lane half: which 8-element K group of an MFMA step

    // ---- tile order ---------------------------------------------------------------------------------
    // Tiles of the first tmap.tn_wide full-width tile columns come first: contiguous per XCD, grouped
    // by GROUP_M M-tiles inside it. Then the narrow tiles, one per M-tile and narrow column: the next
    // tmap.split_cols tile columns cut into tmap.pieces columns of BN / pieces, then the partial last
    // column (fewer than BN columns of N), so that the cheaper tiles fill the final rounds.
    const int tiles_m = tmap.tiles_m;
    int tm;
    int64_t n0, n_end;  // the tile's columns [n0, n_end)
    {
        const int T = tiles_m * tmap.tn_wide;
        const int bid = blockIdx.x;
        if (bid >= T) {
            const int j = bid - T, nc = j / tiles_m, narrow = tmap.split_cols * tmap.pieces;
            tm = j - nc * tiles_m;
            if (nc < narrow) {
                const int width = BN / tmap.pieces;
                n0 = (int64_t)(tmap.tn_wide + nc / tmap.pieces) * BN + (int64_t)(nc % tmap.pieces) * width;
                n_end = n0 + width;
            } else {
                n0 = (int64_t)(tmap.tn_wide + tmap.split_cols) * BN;
                n_end = N;
            }
        } else {
            const int xcd = bid & 7, local = bid >> 3;
            const int q = T >> 3, rem = T & 7;
            const int vt = (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + local;
            const int per_group = GROUP_M * tmap.tn_wide;
            const int g = vt / per_group, in_g = vt - g * per_group;
            const int first_m = g * GROUP_M;
            const int gm = tiles_m - first_m < GROUP_M ? tiles_m - first_m : GROUP_M;
            tm = first_m + in_g % gm;
            n0 = (int64_t)(in_g / gm) * BN;
            n_end = n0 + BN;
        }
    }
    const int64_t m0 = (int64_t)tm * BM;

    // Wave layout: 2 x 2 waves of 128 x 128 in a tile with more than 128 columns; with at most 128
    // columns, 4 x 1 waves of 64 rows x 128 columns (so that all four waves have work).
    const bool stacked = n_end - n0 <= 128;
    const int wm = stacked ? wave : wave >> 1, wn = stacked ? 0 : wave & 1;
    const int64_t row0 = m0 + (stacked ? 64 : 128) * wm;  // first output row of this wave
    const int64_t col0 = n0 + 128 * wn;                    // first output column of this wave

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // per-lane LDS row indices of the MFMA fragments (stacked: only the first two A fragments are used)
    int a_row[4], b_row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a_row[i] = (int)(row0 - m0) + 32 * (stacked ? (i & 1) : i) + lr;
        b_row[i] = (int)(col0 - n0) + 32 * i + lr;
    }

    // ---- main loop --------------------------------------------------------------------------------
    // Chunk kc lives in LDS stage kc % 2. One barrier per chunk, after step 11: every wave has then
    // finished reading the current stage (its last code read feeds step 12) and has waited for its
    // own loads of chunk kc + 1 (issued a whole chunk earlier), so after the barrier chunk kc + 1 is
    // visible and the current stage is free for chunk kc + 2. Steps 12-15 then prefetch chunk
    // kc + 1's scales and first codes, and step 15 dequantizes its first step, so the MFMA stream
    // runs on across the chunk boundary.
    const int64_t nk = (K + BK - 1) / BK;
    const int64_t n_wave = n_end - col0;  // columns of this wave in the tile (> 0 in either layout)
    const uint32_t rsub = lane >> 3;
    const Loader ld{tile_rsrc(a_codes, m0, M, lda_c), tile_rsrc(w_codes, n0, n_end, ldw_c),
                    tile_rsrc(a_scales, m0, M, lda_s), tile_rsrc(w_scales, n0, n_end, ldw_s),
                    (uint32_t)lda_c, (uint32_t)ldw_c, (uint32_t)lda_s, (uint32_t)ldw_s,
                    rsub * (uint32_t)lda_c, rsub * (uint32_t)ldw_c, (uint32_t)lane * (uint32_t)lda_s,
                    (uint32_t)lane * (uint32_t)ldw_s, 16u * ((lane & 7) ^ rsub), wave};
    if (nk > 0) {
        if (stacked) {
            if (n_wave <= 64)
                main_loop<2, 2>(acc, smem, ld, a_row, b_row, lh, nk, K);
            else
                main_loop<2, 4>(acc, smem, ld, a_row, b_row, lh, nk, K);
        } else {
            if (n_wave <= 64)
                main_loop<4, 2>(acc, smem, ld, a_row, b_row, lh, nk, K);
            else
                main_loop<4, 4>(acc, smem, ld, a_row, b_row, lh, nk, K);
        }
    }

    // ---- epilogue -----------------------------------------------------------------------------------
    __syncthreads();  // all waves done with the LDS stages before the epilogue reuses them
    float* ep = reinterpret_cast<float*>(smem) + wave * (128 * EP_PITCH);
    if (stacked) {
        if (n_wave <= 64)
            store_tile<2, 2>(acc, sp, row0, col0, M, N, lane, ep);
        else
            store_tile<2, 4>(acc, sp, row0, col0, M, N, lane, ep);
    } else {
        if (n_wave <= 64)
            store_tile<4, 2>(acc, sp, row0, col0, M, N, lane, ep);
        else
            store_tile<4, 4>(acc, sp, row0, col0, M, N, lane, ep);
    }
}

}  // namespace

TileMap tile_map(int64_t M, int64_t N, int cus) {
    TileMap t{(int32_t)((M + BM - 1) / BM), (int32_t)(N / BN), 0, 1};
    const int64_t full = (int64_t)t.tiles_m * t.tn_wide, partial = N % BN ? t.tiles_m : 0;
    const int64_t rest = full % cus;  // full tiles of the last, partly occupied round
    if (rest == 0) return t;
    const int64_t cols = std::min<int64_t>(t.tn_wide, (rest + t.tiles_m - 1) / t.tiles_m);
    const int64_t fit = (cus - partial) / (cols * t.tiles_m);  // pieces per column that still fit one round
    if (fit < 2) return t;
    t.split_cols = (int32_t)cols;
    t.pieces = fit >= 4 ? 4 : 2;
    t.tn_wide -= t.split_cols;
    return t;
}

hipError_t launch_gemm_tiled(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s,
                             const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s,
                             int64_t M, int64_t N, int64_t K, const SegParams& sp, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    const TileMap t = tile_map(M, N, device_cus());
    const int64_t blocks = (int64_t)t.tiles_m * (t.tn_wide + t.split_cols * t.pieces + (N % BN ? 1 : 0));
    hipLaunchKernelGGL(gemm_kernel, dim3((uint32_t)blocks), dim3(NTHREADS), 0, stream, a_codes, lda_c, a_scales,
                       lda_s, w_codes, ldw_c, w_scales, ldw_s, M, N, K, t, sp);
    return hipGetLastError();
}

}  // namespace nvfp4
