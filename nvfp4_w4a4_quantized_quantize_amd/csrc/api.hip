// C interface of libnvfp4.so: argument validation, status reporting and kernel launches.
// Every argument error is reported before anything is enqueued on the caller's stream.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "internal.h"

namespace {

// Scratch of nvfp4_gemm_noalloc: the decode kernel's split-K partial sums, for callers that cannot
// allocate. Each GPU the library runs on holds its own copy from module load until the process
// ends. In host code `scratch` is only a stand-in for the symbol: its device address on the current
// device comes from hipGetSymbolAddress (taken once per device, below) and only that address is
// ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[NVFP4_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The device address of `scratch` on the current device, looked up on the first call per device.
hipError_t scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

thread_local char g_last_error[512] = "";

nvfp4_status fail(nvfp4_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

nvfp4_status ok() {
    g_last_error[0] = '\0';
    return NVFP4_OK;
}

nvfp4_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t MAX_GEMM_LD = (int64_t)1 << 23;  // bytes per row of codes or scales, exclusive

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool good_scale(float g) { return std::isfinite(g) && g > 0.0f; }

// A [rows, K] bf16 matrix with stride ldx elements.
nvfp4_status check_bf16_matrix(const void* x, int64_t rows, int64_t K, int64_t ldx, const char* name) {
    if (rows < 0 || K < 0) return fail(NVFP4_ERR_SHAPE, "%s: negative shape [%lld, %lld]", name, (long long)rows, (long long)K);
    if (rows == 0 || K == 0) return NVFP4_OK;
    if (!x) return fail(NVFP4_ERR_NULL, "%s is NULL", name);
    if (ldx < K) return fail(NVFP4_ERR_SHAPE, "%s: row stride %lld < K = %lld", name, (long long)ldx, (long long)K);
    if (!aligned16(x) || ldx % 8 != 0)
        return fail(NVFP4_ERR_ALIGN, "%s: base must be 16-byte aligned and the row stride a multiple of 8 elements", name);
    return NVFP4_OK;
}

// An NVFP4 tensor [rows, K]: codes [rows, K/2] (stride ldc bytes) + scales [rows, K/16] (stride lds).
nvfp4_status check_nvfp4(const uint8_t* codes, int64_t ldc, const uint8_t* scales, int64_t lds, int64_t rows,
                         int64_t K, const char* name) {
    if (rows == 0 || K == 0) return NVFP4_OK;
    if (!codes || !scales) return fail(NVFP4_ERR_NULL, "%s codes or scales is NULL", name);
    if (ldc < K / 2 || lds < K / 16)
        return fail(NVFP4_ERR_SHAPE, "%s: strides (%lld, %lld) smaller than a row (%lld, %lld)", name,
                    (long long)ldc, (long long)lds, (long long)(K / 2), (long long)(K / 16));
    if (!aligned16(codes) || !aligned16(scales) || ldc % 16 != 0 || lds % 16 != 0)
        return fail(NVFP4_ERR_ALIGN, "%s: codes/scales must be 16-byte aligned with strides a multiple of 16 bytes", name);
    return NVFP4_OK;
}

}  // namespace

extern "C" {

const char* nvfp4_status_string(int status) {
    switch (status) {
        case NVFP4_OK: return "ok";
        case NVFP4_ERR_NULL: return "null pointer";
        case NVFP4_ERR_SHAPE: return "invalid shape or stride";
        case NVFP4_ERR_ALIGN: return "misaligned pointer or stride";
        case NVFP4_ERR_SEGMENTS: return "invalid segment table";
        case NVFP4_ERR_SCALE: return "global scale not finite and positive";
        case NVFP4_ERR_EPILOGUE: return "invalid epilogue or output type";
        case NVFP4_ERR_WORKSPACE: return "workspace too small";
        case NVFP4_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* nvfp4_last_error(void) { return g_last_error; }

size_t nvfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0) return 0;
    return nvfp4::gemm_wide_workspace_bytes(M, N, K);
}

nvfp4_status nvfp4_global_scale(const void* x_bf16, int64_t rows, int64_t K, int64_t ldx, float* g_out,
                                void* stream) {
    nvfp4_status st = check_bf16_matrix(x_bf16, rows, K, ldx, "x");
    if (st != NVFP4_OK) return st;
    if (!g_out) return fail(NVFP4_ERR_NULL, "g_out is NULL");
    if ((reinterpret_cast<uintptr_t>(g_out) & 3u) != 0) return fail(NVFP4_ERR_ALIGN, "g_out must be 4-byte aligned");
    return hip_status(nvfp4::launch_amax_scale(static_cast<const uint16_t*>(x_bf16), rows, K, ldx, 6.0f * 448.0f,
                                               g_out, static_cast<hipStream_t>(stream)),
                      "nvfp4_global_scale launch");
}

nvfp4_status nvfp4_quantize(const void* x_bf16, int64_t rows, int64_t K, int64_t ldx, float g, uint8_t* codes,
                            int64_t ldc, uint8_t* scales, int64_t lds, void* stream) {
    if (rows < 0 || K < 0) return fail(NVFP4_ERR_SHAPE, "negative shape");
    if (K % 16 != 0) return fail(NVFP4_ERR_SHAPE, "K = %lld is not a multiple of 16", (long long)K);
    nvfp4_status st = check_bf16_matrix(x_bf16, rows, K, ldx, "x");
    if (st != NVFP4_OK) return st;
    st = check_nvfp4(codes, ldc, scales, lds, rows, K, "output");
    if (st != NVFP4_OK) return st;
    if (!good_scale(g)) return fail(NVFP4_ERR_SCALE, "global scale g = %g must be finite and > 0", (double)g);
    if (rows == 0 || K == 0) return ok();
    if ((uint64_t)rows * (uint64_t)((K / 16 + 63) / 64) > (uint64_t)0x1FFFFFFFCull)
        return fail(NVFP4_ERR_SHAPE, "tensor too large for one launch");
    return hip_status(nvfp4::launch_quantize(static_cast<const uint16_t*>(x_bf16), rows, K, ldx, g, codes, ldc,
                                             scales, lds, static_cast<hipStream_t>(stream)),
                      "nvfp4_quantize launch");
}

}  // extern "C"

namespace {

// Validation and launch of nvfp4_gemm, nvfp4_gemm_noalloc and nvfp4_gemm_packed. With noalloc the
// workspace arguments are ignored: the partial sums go to the current device's scratch array. With
// packed the weights are w_packed, in the decode layout, and w_codes .. ldw_s are unused.
nvfp4_status gemm_entry(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s, float g_a,
                        const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s, bool packed,
                        const uint8_t* w_packed, int64_t M, int64_t N, int64_t K, const nvfp4_segment* segs,
                        const float* g_w, int32_t n_segs, void* workspace, size_t workspace_bytes, bool noalloc,
                        void* stream) {
    if (M < 0 || N < 0 || K < 0) return fail(NVFP4_ERR_SHAPE, "negative shape");
    if (K % 16 != 0) return fail(NVFP4_ERR_SHAPE, "K = %lld is not a multiple of 16", (long long)K);
    if (M > (int64_t)1 << 31 || N > (int64_t)1 << 31) return fail(NVFP4_ERR_SHAPE, "M or N too large");
    // the tiled kernel's grid indices are 32-bit
    if (M > nvfp4::SKINNY_MAX_M && ((M + 255) / 256) * ((N + 255) / 256) > (int64_t)1 << 30)
        return fail(NVFP4_ERR_SHAPE, "M = %lld, N = %lld: more than 2^30 output tiles of 256 x 256", (long long)M,
                    (long long)N);
    if (packed && M > nvfp4::SKINNY_MAX_M)
        return fail(NVFP4_ERR_SHAPE, "packed weights serve M <= %lld activation rows, M = %lld",
                    (long long)nvfp4::SKINNY_MAX_M, (long long)M);
    nvfp4_status st = check_nvfp4(a_codes, lda_c, a_scales, lda_s, M, K, "A");
    if (st != NVFP4_OK) return st;
    if (packed) {
        if (M > 0 && N > 0 && K > 0 && !w_packed) return fail(NVFP4_ERR_NULL, "w_packed is NULL");
        if (!aligned16(w_packed)) return fail(NVFP4_ERR_ALIGN, "packed weights must be 16-byte aligned");
        ldw_c = ldw_s = 0;
    } else {
        st = check_nvfp4(w_codes, ldw_c, w_scales, ldw_s, N, K, "W");
        if (st != NVFP4_OK) return st;
    }
    // the prefill kernel addresses a 256-row tile of each operand with 32-bit buffer offsets
    if (lda_c >= MAX_GEMM_LD || lda_s >= MAX_GEMM_LD || ldw_c >= MAX_GEMM_LD || ldw_s >= MAX_GEMM_LD)
        return fail(NVFP4_ERR_SHAPE, "row strides must be below %lld bytes", (long long)MAX_GEMM_LD);
    if (!segs || !g_w) return fail(NVFP4_ERR_NULL, "segment table or g_w is NULL");
    if (n_segs < 1 || n_segs > NVFP4_MAX_SEGMENTS)
        return fail(NVFP4_ERR_SEGMENTS, "n_segs = %d outside [1, %d]", n_segs, NVFP4_MAX_SEGMENTS);
    if (!good_scale(g_a)) return fail(NVFP4_ERR_SCALE, "g_a = %g must be finite and > 0", (double)g_a);

    nvfp4::SegParams sp = {};
    sp.n_segs = n_segs;
    int64_t expect = 0;
    for (int s = 0; s < n_segs; ++s) {
        const nvfp4_segment& sg = segs[s];
        if (sg.n_begin != expect || sg.n_len <= 0)
            return fail(NVFP4_ERR_SEGMENTS, "segment %d [%lld, +%lld) must start at %lld and be non-empty", s,
                        (long long)sg.n_begin, (long long)sg.n_len, (long long)expect);
        expect = sg.n_begin + sg.n_len;
        if (!good_scale(g_w[s])) return fail(NVFP4_ERR_SCALE, "g_w[%d] = %g must be finite and > 0", s, (double)g_w[s]);
        if (sg.epilogue < NVFP4_EPI_NONE || sg.epilogue > NVFP4_EPI_GDN_DECAY)
            return fail(NVFP4_ERR_EPILOGUE, "segment %d: unknown epilogue %d", s, sg.epilogue);
        if (sg.out_dtype != NVFP4_OUT_F32 && sg.out_dtype != NVFP4_OUT_BF16)
            return fail(NVFP4_ERR_EPILOGUE, "segment %d: unknown output type %d", s, sg.out_dtype);
        if (sg.epilogue != NVFP4_EPI_NONE && sg.out_dtype != NVFP4_OUT_F32)
            return fail(NVFP4_ERR_EPILOGUE, "segment %d: gate epilogues write FP32", s);
        if (sg.epilogue == NVFP4_EPI_GDN_DECAY && (!sg.A_log || !sg.dt_bias))
            return fail(NVFP4_ERR_EPILOGUE, "segment %d: GDN decay needs A_log and dt_bias", s);
        const int64_t esize = sg.out_dtype == NVFP4_OUT_F32 ? 4 : 2;
        if (M > 0) {
            if (!sg.out) return fail(NVFP4_ERR_NULL, "segment %d: out is NULL", s);
            if (sg.ldo < sg.n_len) return fail(NVFP4_ERR_SHAPE, "segment %d: ldo %lld < n_len %lld", s,
                                               (long long)sg.ldo, (long long)sg.n_len);
            if ((reinterpret_cast<uintptr_t>(sg.out) % (uintptr_t)esize) != 0)
                return fail(NVFP4_ERR_ALIGN, "segment %d: out not aligned to its element size", s);
        }
        sp.n_begin[s] = sg.n_begin;
        sp.n_end[s] = expect;
        sp.scale[s] = g_a * g_w[s];  // RN32(g_a * g_w[s])
        if (!std::isnormal(sp.scale[s]))
            return fail(NVFP4_ERR_SCALE, "segment %d: g_a * g_w = %g * %g = %g is not a normal positive float", s,
                        (double)g_a, (double)g_w[s], (double)sp.scale[s]);
        sp.epilogue[s] = sg.epilogue;
        sp.out_dtype[s] = sg.out_dtype;
        sp.out[s] = sg.out;
        sp.ldo[s] = sg.ldo;
        sp.A_log[s] = sg.A_log;
        sp.dt_bias[s] = sg.dt_bias;
        const int64_t per16 = 16 / esize;  // elements per 16 bytes
        if (sg.epilogue == NVFP4_EPI_NONE && aligned16(sg.out) && sg.ldo % per16 == 0 && sg.n_begin % per16 == 0)
            sp.vec_mask |= 1u << s;
    }
    if (expect != N) return fail(NVFP4_ERR_SEGMENTS, "segments cover [0, %lld), N = %lld", (long long)expect, (long long)N);
    const size_t need = nvfp4_gemm_workspace_bytes(M, N, K);
    if (noalloc) {
        if (need > (size_t)NVFP4_NOALLOC_SCRATCH_BYTES)
            return fail(NVFP4_ERR_WORKSPACE,
                        "nvfp4_gemm_noalloc: this shape needs %zu bytes of scratch, more than the fixed %zu bytes", need,
                        (size_t)NVFP4_NOALLOC_SCRATCH_BYTES);
        workspace = nullptr;
        if (M == 0 || N == 0) return ok();
        if (need > 0) {
            const hipError_t e = scratch_of_current_device(&workspace);
            if (e != hipSuccess) return hip_status(e, "nvfp4_gemm_noalloc: scratch address");
        }
    } else {
        if (workspace_bytes < need || (need > 0 && !workspace))
            return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
        if (need > 0 && !aligned16(workspace)) return fail(NVFP4_ERR_ALIGN, "workspace must be 16-byte aligned");
        if (M == 0 || N == 0) return ok();
    }
    const hipStream_t st_ = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (packed) {
        const uint8_t* ps = nvfp4::packed_scales(w_packed, N, K);
        if (M > nvfp4::SKINNY_NARROW_M)
            e = nvfp4::launch_gemm_wide(a_codes, lda_c, a_scales, lda_s, w_packed, 0, ps, 0, M, N, K, sp, workspace,
                                        true, st_);
        else
            e = nvfp4::launch_gemm_skinny(a_codes, lda_c, a_scales, lda_s, w_packed, 0, ps, 0, M, N, K, sp, true,
                                          st_);
        return hip_status(e, "nvfp4_gemm_packed launch");
    }
    if (M > nvfp4::SKINNY_MAX_M)
        e = nvfp4::launch_gemm_tiled(a_codes, lda_c, a_scales, lda_s, w_codes, ldw_c, w_scales, ldw_s, M, N, K, sp, st_);
    else if (M > nvfp4::SKINNY_NARROW_M)
        e = nvfp4::launch_gemm_wide(a_codes, lda_c, a_scales, lda_s, w_codes, ldw_c, w_scales, ldw_s, M, N, K, sp,
                                    workspace, false, st_);
    else if (nvfp4::gemv_supported(M, K))
        e = nvfp4::launch_gemm_gemv(a_codes, lda_c, a_scales, lda_s, w_codes, ldw_c, w_scales, ldw_s, M, N, K, sp, st_);
    else
        e = nvfp4::launch_gemm_skinny(a_codes, lda_c, a_scales, lda_s, w_codes, ldw_c, w_scales, ldw_s, M, N, K, sp,
                                      false, st_);
    return hip_status(e, noalloc ? "nvfp4_gemm_noalloc launch" : "nvfp4_gemm launch");
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_gemm(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s, float g_a,
                        const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s, int64_t M,
                        int64_t N, int64_t K, const nvfp4_segment* segs, const float* g_w, int32_t n_segs,
                        void* workspace, size_t workspace_bytes, void* stream) {
    return gemm_entry(a_codes, lda_c, a_scales, lda_s, g_a, w_codes, ldw_c, w_scales, ldw_s, false, nullptr, M, N, K,
                      segs, g_w, n_segs, workspace, workspace_bytes, false, stream);
}

size_t nvfp4_packed_weight_bytes(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0 || K % 16 != 0) return 0;
    return nvfp4::packed_weight_bytes(N, K);
}

nvfp4_status nvfp4_pack_weights(const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales, int64_t ldw_s,
                                int64_t N, int64_t K, uint8_t* packed, void* stream) {
    if (N < 0 || K < 0) return fail(NVFP4_ERR_SHAPE, "negative shape");
    if (K % 16 != 0) return fail(NVFP4_ERR_SHAPE, "K = %lld is not a multiple of 16", (long long)K);
    if (N > (int64_t)1 << 31) return fail(NVFP4_ERR_SHAPE, "N too large");
    nvfp4_status st = check_nvfp4(w_codes, ldw_c, w_scales, ldw_s, N, K, "W");
    if (st != NVFP4_OK) return st;
    if (N == 0 || K == 0) return ok();
    if (!packed) return fail(NVFP4_ERR_NULL, "packed is NULL");
    if (!aligned16(packed)) return fail(NVFP4_ERR_ALIGN, "packed must be 16-byte aligned");
    return hip_status(nvfp4::launch_pack_weights(w_codes, ldw_c, w_scales, ldw_s, N, K, packed,
                                                 static_cast<hipStream_t>(stream)),
                      "nvfp4_pack_weights launch");
}

nvfp4_status nvfp4_gemm_packed(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s,
                               float g_a, const uint8_t* w_packed, int64_t M, int64_t N, int64_t K,
                               const nvfp4_segment* segs, const float* g_w, int32_t n_segs, void* workspace,
                               size_t workspace_bytes, void* stream) {
    return gemm_entry(a_codes, lda_c, a_scales, lda_s, g_a, nullptr, 0, nullptr, 0, true, w_packed, M, N, K, segs, g_w,
                      n_segs, workspace, workspace_bytes, false, stream);
}

nvfp4_status nvfp4_gemm_noalloc(const uint8_t* a_codes, int64_t lda_c, const uint8_t* a_scales, int64_t lda_s,
                                float g_a, const uint8_t* w_codes, int64_t ldw_c, const uint8_t* w_scales,
                                int64_t ldw_s, int64_t M, int64_t N, int64_t K, const nvfp4_segment* segs,
                                const float* g_w, int32_t n_segs, void* stream) {
    return gemm_entry(a_codes, lda_c, a_scales, lda_s, g_a, w_codes, ldw_c, w_scales, ldw_s, false, nullptr, M, N, K,
                      segs, g_w, n_segs, nullptr, 0, true, stream);
}

nvfp4_status nvfp4_kv_scale(const void* x_bf16, int64_t rows, int64_t cols, int64_t ldx, float* s_out,
                            void* stream) {
    nvfp4_status st = check_bf16_matrix(x_bf16, rows, cols, ldx, "x");
    if (st != NVFP4_OK) return st;
    if (!s_out) return fail(NVFP4_ERR_NULL, "s_out is NULL");
    if ((reinterpret_cast<uintptr_t>(s_out) & 3u) != 0) return fail(NVFP4_ERR_ALIGN, "s_out must be 4-byte aligned");
    return hip_status(nvfp4::launch_amax_scale(static_cast<const uint16_t*>(x_bf16), rows, cols, ldx, 448.0f, s_out,
                                               static_cast<hipStream_t>(stream)),
                      "nvfp4_kv_scale launch");
}

namespace {

// An FP8 byte matrix [rows, cols] with stride ldq: 16-byte aligned base and stride.
nvfp4_status check_fp8_matrix(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const char* name) {
    if (rows == 0 || cols == 0) return NVFP4_OK;
    if (!q) return fail(NVFP4_ERR_NULL, "%s is NULL", name);
    if (ldq < cols) return fail(NVFP4_ERR_SHAPE, "%s: row stride %lld < cols = %lld", name, (long long)ldq, (long long)cols);
    if (!aligned16(q) || ldq % 16 != 0)
        return fail(NVFP4_ERR_ALIGN, "%s: base must be 16-byte aligned and the row stride a multiple of 16", name);
    return NVFP4_OK;
}

nvfp4_status check_kv_shape(int64_t rows, int64_t cols, float s) {
    if (rows < 0 || cols < 0) return fail(NVFP4_ERR_SHAPE, "negative shape");
    if (cols % 16 != 0) return fail(NVFP4_ERR_SHAPE, "cols = %lld is not a multiple of 16", (long long)cols);
    if (!good_scale(s)) return fail(NVFP4_ERR_SCALE, "KV scale s = %g must be finite and > 0", (double)s);
    return NVFP4_OK;
}

}  // namespace

nvfp4_status nvfp4_kv_quantize(const void* x_bf16, int64_t rows, int64_t cols, int64_t ldx, float s, uint8_t* q,
                               int64_t ldq, void* stream) {
    nvfp4_status st = check_kv_shape(rows, cols, s);
    if (st != NVFP4_OK) return st;
    if ((st = check_bf16_matrix(x_bf16, rows, cols, ldx, "x")) != NVFP4_OK) return st;
    if ((st = check_fp8_matrix(q, rows, cols, ldq, "q")) != NVFP4_OK) return st;
    if (rows == 0 || cols == 0) return ok();
    return hip_status(nvfp4::launch_kv_quantize(static_cast<const uint16_t*>(x_bf16), rows, cols, ldx, s, q, ldq,
                                                static_cast<hipStream_t>(stream)),
                      "nvfp4_kv_quantize launch");
}

nvfp4_status nvfp4_kv_dequantize(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, float s, void* y_bf16,
                                 int64_t ldy, void* stream) {
    nvfp4_status st = check_kv_shape(rows, cols, s);
    if (st != NVFP4_OK) return st;
    if ((st = check_fp8_matrix(q, rows, cols, ldq, "q")) != NVFP4_OK) return st;
    if ((st = check_bf16_matrix(y_bf16, rows, cols, ldy, "y")) != NVFP4_OK) return st;
    if (rows == 0 || cols == 0) return ok();
    return hip_status(nvfp4::launch_kv_dequantize(q, rows, cols, ldq, s, static_cast<uint16_t*>(y_bf16), ldy,
                                                  static_cast<hipStream_t>(stream)),
                      "nvfp4_kv_dequantize launch");
}

nvfp4_status nvfp4_fold_scales(uint8_t* scales, int64_t rows, int64_t nblocks, int64_t lds, float ratio,
                               void* stream) {
    if (rows < 0 || nblocks < 0) return fail(NVFP4_ERR_SHAPE, "negative shape");
    if (!good_scale(ratio)) return fail(NVFP4_ERR_SCALE, "ratio = %g must be finite and > 0", (double)ratio);
    if (rows == 0 || nblocks == 0) return ok();
    if (!scales) return fail(NVFP4_ERR_NULL, "scales is NULL");
    if (lds < nblocks) return fail(NVFP4_ERR_SHAPE, "row stride %lld < nblocks = %lld", (long long)lds, (long long)nblocks);
    return hip_status(nvfp4::launch_fold_scales(scales, rows, nblocks, lds, ratio, static_cast<hipStream_t>(stream)),
                      "nvfp4_fold_scales launch");
}

nvfp4_status nvfp4_fold_group(uint8_t* w_scales, int64_t ldw_s, int64_t K, const int64_t* seg_rows, const float* g_w,
                              int32_t n_segs, float* g_common, void* stream) {
    if (!seg_rows || !g_w || !g_common) return fail(NVFP4_ERR_NULL, "seg_rows, g_w or g_common is NULL");
    if (K < 0 || K % 16 != 0) return fail(NVFP4_ERR_SHAPE, "K = %lld is not a non-negative multiple of 16", (long long)K);
    if (n_segs < 1 || n_segs > NVFP4_MAX_SEGMENTS)
        return fail(NVFP4_ERR_SEGMENTS, "n_segs = %d outside [1, %d]", n_segs, NVFP4_MAX_SEGMENTS);
    // pass 1: validate everything (rows, scales, every ratio, the scale buffer) before touching any
    // output, so that an error leaves the weights and *g_common as they were
    float G = 0.0f;
    int64_t total_rows = 0;
    for (int s = 0; s < n_segs; ++s) {
        if (seg_rows[s] < 0) return fail(NVFP4_ERR_SEGMENTS, "segment %d has %lld rows", s, (long long)seg_rows[s]);
        if (!good_scale(g_w[s])) return fail(NVFP4_ERR_SCALE, "g_w[%d] = %g must be finite and > 0", s, (double)g_w[s]);
        if (g_w[s] > G) G = g_w[s];
        total_rows += seg_rows[s];
    }
    float ratio[NVFP4_MAX_SEGMENTS];
    for (int s = 0; s < n_segs; ++s) {
        ratio[s] = g_w[s] / G;  // RN32
        if (!good_scale(ratio[s]))
            return fail(NVFP4_ERR_SCALE, "ratio g_w[%d] / G = %g / %g underflows to 0", s, (double)g_w[s], (double)G);
    }
    const int64_t nblocks = K / 16;
    if (total_rows > 0 && nblocks > 0) {
        if (!w_scales) return fail(NVFP4_ERR_NULL, "w_scales is NULL");
        if (ldw_s < nblocks)
            return fail(NVFP4_ERR_SHAPE, "row stride %lld < nblocks = %lld", (long long)ldw_s, (long long)nblocks);
    }
    // pass 2: every argument is valid; enqueue the folds
    *g_common = G;
    int64_t row0 = 0;
    for (int s = 0; s < n_segs; ++s) {
        nvfp4_status st = nvfp4_fold_scales(w_scales + row0 * ldw_s, seg_rows[s], nblocks, ldw_s, ratio[s], stream);
        if (st != NVFP4_OK) return st;  // only a launch failure can remain here
        row0 += seg_rows[s];
    }
    return ok();
}

nvfp4_status nvfp4_rmsnorm_quantize(const void* x_bf16, int64_t rows, int64_t K, int64_t ldx, const void* w_bf16,
                                    float eps, float g, uint8_t* codes, int64_t ldc, uint8_t* scales, int64_t lds,
                                    void* y_bf16, int64_t ldy, void* stream) {
    if (rows < 0 || K < 0) return fail(NVFP4_ERR_SHAPE, "negative shape");
    if (K % 16 != 0) return fail(NVFP4_ERR_SHAPE, "K = %lld is not a multiple of 16", (long long)K);
    nvfp4_status st = check_bf16_matrix(x_bf16, rows, K, ldx, "x");
    if (st != NVFP4_OK) return st;
    if ((st = check_nvfp4(codes, ldc, scales, lds, rows, K, "output")) != NVFP4_OK) return st;
    if (y_bf16 && (st = check_bf16_matrix(y_bf16, rows, K, ldy, "y")) != NVFP4_OK) return st;
    if (!good_scale(g)) return fail(NVFP4_ERR_SCALE, "global scale g = %g must be finite and > 0", (double)g);
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(NVFP4_ERR_SCALE, "eps = %g must be finite and >= 0", (double)eps);
    if (rows == 0 || K == 0) return ok();
    if (!w_bf16) return fail(NVFP4_ERR_NULL, "w is NULL");
    if (!aligned16(w_bf16)) return fail(NVFP4_ERR_ALIGN, "w must be 16-byte aligned");
    return hip_status(nvfp4::launch_rmsnorm_quantize(static_cast<const uint16_t*>(x_bf16), rows, K, ldx,
                                                     static_cast<const uint16_t*>(w_bf16), eps, g, codes, ldc, scales,
                                                     lds, static_cast<uint16_t*>(y_bf16), ldy,
                                                     static_cast<hipStream_t>(stream)),
                      "nvfp4_rmsnorm_quantize launch");
}

size_t nvfp4_gdn_workspace_bytes(int64_t B, int64_t T, int32_t Hv, int32_t Hk, int32_t D) {
    if (B <= 0 || T <= 0 || D != 128 || Hv < 1 || Hk < 1 || Hv % Hk != 0) return 0;
    return nvfp4::gdn_workspace_bytes(B, T, Hv);
}

nvfp4_status nvfp4_gdn_recurrence(const void* q_bf16, int64_t ldq, const void* k_bf16, int64_t ldk, const void* v_bf16,
                                  int64_t ldv, const float* alpha, int64_t lda, const float* beta, int64_t ldb,
                                  float* state, int64_t B, int64_t T, int32_t Hv, int32_t Hk, int32_t D, float* o,
                                  int64_t ldo, void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 0 || T < 0) return fail(NVFP4_ERR_SHAPE, "negative shape");
    if (D != 128) return fail(NVFP4_ERR_SHAPE, "head dimension D = %d is not supported (128)", D);
    if (Hv < 1 || Hk < 1 || Hv % Hk != 0) return fail(NVFP4_ERR_SHAPE, "Hv = %d must be a positive multiple of Hk = %d", Hv, Hk);
    if (B == 0 || T == 0) return ok();
    if (!q_bf16 || !k_bf16 || !v_bf16 || !alpha || !beta || !state || !o)
        return fail(NVFP4_ERR_NULL, "a GDN recurrence buffer is NULL");
    if (ldq < (int64_t)Hk * D || ldk < (int64_t)Hk * D || ldv < (int64_t)Hv * D || lda < Hv || ldb < Hv ||
        ldo < (int64_t)Hv * D)
        return fail(NVFP4_ERR_SHAPE, "a row stride is smaller than its row");
    if (!aligned16(q_bf16) || !aligned16(k_bf16) || ldq % 8 != 0 || ldk % 8 != 0)
        return fail(NVFP4_ERR_ALIGN, "q and k must be 16-byte aligned with strides a multiple of 8 elements");
    if ((reinterpret_cast<uintptr_t>(v_bf16) & 1u) || (reinterpret_cast<uintptr_t>(alpha) & 3u) ||
        (reinterpret_cast<uintptr_t>(beta) & 3u) || (reinterpret_cast<uintptr_t>(o) & 3u))
        return fail(NVFP4_ERR_ALIGN, "v, alpha, beta and o must be aligned to their element size");
    if (!aligned16(state)) return fail(NVFP4_ERR_ALIGN, "state must be 16-byte aligned");
    if (ldq >= (1 << 23) || ldk >= (1 << 23) || ldv >= (1 << 23) || ldo >= (1 << 23))
        return fail(NVFP4_ERR_SHAPE, "q, k, v and o row strides must be below 2^23 elements");
    const size_t need = nvfp4_gdn_workspace_bytes(B, T, Hv, Hk, D);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    if (need > 0 && !aligned16(workspace)) return fail(NVFP4_ERR_ALIGN, "workspace must be 16-byte aligned");
    return hip_status(nvfp4::launch_gdn_recurrence(static_cast<const uint16_t*>(q_bf16), ldq,
                                                   static_cast<const uint16_t*>(k_bf16), ldk,
                                                   static_cast<const uint16_t*>(v_bf16), ldv, alpha, lda, beta, ldb,
                                                   state, B, T, Hv, Hk, o, ldo, workspace,
                                                   static_cast<hipStream_t>(stream)),
                      "nvfp4_gdn_recurrence launch");
}

}  // extern "C"
