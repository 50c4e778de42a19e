// Internal declarations shared by the HIP sources of libnvfp4.so (not installed, not part of the
// C interface in include/nvfp4.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"

namespace nvfp4 {

// Segment table as passed to the GEMM kernel by value (kernel-argument memory).
struct SegParams {
    int32_t n_segs;
    uint32_t vec_mask;                     // bit s: segment s may use 16-byte epilogue stores
    int64_t n_begin[NVFP4_MAX_SEGMENTS];
    int64_t n_end[NVFP4_MAX_SEGMENTS];     // exclusive
    float scale[NVFP4_MAX_SEGMENTS];       // RN32(g_a * g_w[s])
    int32_t epilogue[NVFP4_MAX_SEGMENTS];
    int32_t out_dtype[NVFP4_MAX_SEGMENTS];
    void* out[NVFP4_MAX_SEGMENTS];
    int64_t ldo[NVFP4_MAX_SEGMENTS];
    const float* A_log[NVFP4_MAX_SEGMENTS];
    const float* dt_bias[NVFP4_MAX_SEGMENTS];
};

// Launchers: shapes are validated by the C interface before these are called.
// Writes RN32(max |x| / divisor) to the device float g_out.
hipError_t launch_amax_scale(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, float divisor,
                             float* g_out, hipStream_t stream);
hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, float g,
                           uint8_t* codes, int64_t ldc, uint8_t* scales, int64_t lds,
                           hipStream_t stream);

// One activation row (K up to GEMV_MAX_K) runs on the weight-streaming GEMV kernel (with two rows
// its VALU dot products cost more than the matrix-core path of the skinny kernel).
constexpr int64_t GEMV_MAX_M = 1;
constexpr int64_t GEMV_MAX_K = 32 * 64 * 16;
bool gemv_supported(int64_t M, int64_t K);
hipError_t launch_gemm_gemv(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s,
                            const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s,
                            int64_t M, int64_t N, int64_t K, const SegParams& sp, hipStream_t stream);

// Activation row counts up to SKINNY_NARROW_M run on the skinny (decode) kernel, up to SKINNY_MAX_M
// on its wide variant (split K, partial sums in the workspace), larger ones on the tiled kernel.
constexpr int64_t SKINNY_NARROW_M = 32;
constexpr int64_t SKINNY_MAX_M = 64;

// CUs of the current device (a host query of its properties; it neither allocates nor synchronizes).
int device_cus();

// Grid of the tiled kernel: tiles_m tiles of 256 rows; the first tn_wide tile columns of 256 run as
// full tiles, the next split_cols as pieces columns of 256 / pieces (1, 2 or 4) each, then the
// partial last column if N is not a multiple of 256. Columns are split only when the full tiles'
// last round would leave CUs idle and the pieces of the split columns fit in one round.
struct TileMap {
    int32_t tiles_m, tn_wide, split_cols, pieces;
};
TileMap tile_map(int64_t M, int64_t N, int cus);

hipError_t launch_gemm_tiled(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s,
                             const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s,
                             int64_t M, int64_t N, int64_t K, const SegParams& sp, hipStream_t stream);
// The decode launchers take row-major weights (w_codes, ldw_c, w_scales, ldw_s), or, with packed,
// the decode weight layout: w_codes = its codes (the layout's base), w_scales = packed_scales(), the
// strides unused.
hipError_t launch_gemm_skinny(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s,
                              const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s,
                              int64_t M, int64_t N, int64_t K, const SegParams& sp, bool packed,
                              hipStream_t stream);
// SKINNY_NARROW_M < M <= SKINNY_MAX_M; workspace holds gemm_wide_workspace_bytes(M, N, K) bytes.
hipError_t launch_gemm_wide(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s,
                            const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s,
                            int64_t M, int64_t N, int64_t K, const SegParams& sp, void* workspace,
                            bool packed, hipStream_t stream);
// The decode weight layout (nvfp4_pack_weights): its size, where its scales start, and the repack.
size_t packed_weight_bytes(int64_t N, int64_t K);
const uint8_t* packed_scales(const uint8_t* packed, int64_t N, int64_t K);
hipError_t launch_pack_weights(const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s,
                               int64_t N, int64_t K, uint8_t* packed, hipStream_t stream);
// Bytes of FP32 partial sums the wide variant keeps (0 outside its range of M).
size_t gemm_wide_workspace_bytes(int64_t M, int64_t N, int64_t K);

hipError_t launch_kv_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, float s, uint8_t* q,
                              int64_t ldq, hipStream_t stream);
hipError_t launch_kv_dequantize(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, float s, uint16_t* y,
                                int64_t ldy, hipStream_t stream);
hipError_t launch_fold_scales(uint8_t* scales, int64_t rows, int64_t nblocks, int64_t lds, float ratio,
                              hipStream_t stream);
hipError_t launch_rmsnorm_quantize(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, const uint16_t* w,
                                   float eps, float g, uint8_t* codes, int64_t ldc, uint8_t* scales, int64_t lds,
                                   uint16_t* y, int64_t ldy, hipStream_t stream);

hipError_t launch_gdn_recurrence(const uint16_t* q, int64_t ldq, const uint16_t* k, int64_t ldk, const uint16_t* v,
                                 int64_t ldv, const float* alpha, int64_t lda, const float* beta, int64_t ldb,
                                 float* state, int64_t B, int64_t T, int32_t Hv, int32_t Hk, float* o, int64_t ldo,
                                 void* workspace, hipStream_t stream);
// Bytes of workspace launch_gdn_recurrence needs (the chunk factors of the chunked form; 0 below it).
size_t gdn_workspace_bytes(int64_t B, int64_t T, int32_t Hv);

}  // namespace nvfp4
