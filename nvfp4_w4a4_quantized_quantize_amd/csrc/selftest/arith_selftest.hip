// Device self-checks of the arithmetic the NVFP4 quantizer and the FP8 KV codec rely on, built as
// libnvfp4_selftest.so for the test suite only (libnvfp4.so neither contains nor exports it).
//
// The quantizer takes every rounding decision of the format (E2M1 elements with an E4M3 scale per
// 16 elements, per the Japanese article's "Mechanism 1" and its FAQ "What is NVFP4?") in IEEE
// binary32, but computes two of its steps with faster gfx950 instructions. These kernels exercise
// exactly the helpers of quant_common.h that the product kernels call:
//  * quotient_fast (reciprocal + one exact-residual correction) against the IEEE division
//    __fdiv_rn, for every finite non-negative bf16 numerator against every binary32 significand of
//    the divisor, in a set of divisor binades spanning quotient_fast_ok's range: equal whenever a
//    quotient reaches 2^-11, and giving the same E2M1 code and E4M3 byte everywhere;
//  * e4m3_rne_sat (clamp + hardware FP8 conversion) over every non-negative binary32 input and
//    +infinity: the result is a finite E4M3FN byte and never decreases as the input grows;
//  * put_e2m1_pair (hardware FP4 conversion) over every non-negative binary32 input and
//    +infinity: the magnitude code never decreases as the input grows, the negated input gives the
//    same magnitude with the sign bit, and the other bytes of the packed word are left untouched.
// A monotone function that agrees with the oracle's nearest-even rounding at every grid point,
// every rounding midpoint and both binary32 neighbours of each is equal to it everywhere; the test
// suite takes those points to the oracle through the point-evaluation entries below.
#include "quant_common.h"

namespace nvfp4 {
namespace {

// Adds a per-lane count into *dst with one atomic per wave (same-address atomics serialize in L2).
__device__ __forceinline__ void wave_add(unsigned long long* dst, uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0 && v) atomicAdd(dst, (unsigned long long)v);
}

// counters: [0] pairs checked, [1] pairs whose quotients differ while one of them is 2^-11 or more,
// [2] pairs whose quotients differ below 2^-11, [3] pairs whose E2M1 code or E4M3 byte differ.
// first: numerator and divisor bits of the first pair counted in [1] or [3].
__global__ __launch_bounds__(256) void quotient_scan_kernel(uint32_t s_exp_field, unsigned long long* counters,
                                                            uint32_t* first) {
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;  // divisor significand, grid covers [0, 2^23)
    const uint32_t s_bits = (s_exp_field << 23) | t;
    const float S = __uint_as_float(s_bits);
    const float y = __builtin_amdgcn_rcpf(S);
    uint32_t checked = 0, bad_big = 0, diff_small = 0, bad_code = 0;
    for (uint32_t ab = 0; ab < 0x7F80u; ++ab) {  // every finite non-negative bf16 pattern
        const float a = __uint_as_float(ab << 16);
        if (!quotient_fast_ok(S, a)) continue;
        ++checked;
        const float qf = quotient_fast(a, S, y);
        const float qi = __fdiv_rn(a, S);
        bool bad = false;
        if (__float_as_uint(qf) != __float_as_uint(qi)) {
            if (fmaxf(qf, qi) >= 0x1p-11f) {
                ++bad_big;
                bad = true;
            } else {
                ++diff_small;
            }
        }
        if ((put_e2m1_pair<0>(0u, qf, qf) & 0xffu) != (put_e2m1_pair<0>(0u, qi, qi) & 0xffu) ||
            e4m3_rne_sat(qf) != e4m3_rne_sat(qi)) {
            ++bad_code;
            bad = true;
        }
        if (bad && atomicCAS(first + 2, 0u, 1u) == 0u) {
            first[0] = ab << 16;
            first[1] = s_bits;
        }
    }
    wave_add(counters + 0, checked);
    wave_add(counters + 1, bad_big);
    wave_add(counters + 2, diff_small);
    wave_add(counters + 3, bad_code);
}

constexpr uint32_t POS_END = 0x7F800001u;  // binary32 patterns [0, +inf]
constexpr uint32_t PER_THREAD = 1024;

// counters: [0] inputs checked, [1] outputs that are not a finite non-negative E4M3FN byte,
// [2] places where the output decreases.
__global__ __launch_bounds__(256) void e4m3_scan_kernel(unsigned long long* counters) {
    const uint64_t start0 = ((uint64_t)blockIdx.x * 256u + threadIdx.x) * PER_THREAD;
    const uint64_t start = start0 < POS_END ? start0 : POS_END;  // lanes past the end check nothing
    const uint32_t end = (uint32_t)(start + PER_THREAD < POS_END ? start + PER_THREAD : POS_END);
    uint32_t prev = start == 0 ? 0u : e4m3_rne_sat(__uint_as_float((uint32_t)start - 1u));
    uint32_t checked = 0, bad_range = 0, bad_order = 0;
    for (uint32_t b = (uint32_t)start; b < end; ++b) {
        const uint32_t e = e4m3_rne_sat(__uint_as_float(b));
        ++checked;
        if (e > 0x7Eu) ++bad_range;
        if (e < prev) ++bad_order;
        prev = e;
    }
    wave_add(counters + 0, checked);
    wave_add(counters + 1, bad_range);
    wave_add(counters + 2, bad_order);
}

// counters: [0] inputs checked, [1] positive inputs whose code has the sign bit, [2] places where
// the magnitude code decreases, [3] negated inputs not giving code | 8, [4] packed words whose other
// bytes changed or whose two nibbles disagree with the single conversions.
__global__ __launch_bounds__(256) void e2m1_scan_kernel(unsigned long long* counters) {
    const uint64_t start0 = ((uint64_t)blockIdx.x * 256u + threadIdx.x) * PER_THREAD;
    const uint64_t start = start0 < POS_END ? start0 : POS_END;  // lanes past the end check nothing
    const uint32_t end = (uint32_t)(start + PER_THREAD < POS_END ? start + PER_THREAD : POS_END);
    auto code = [](float v) -> uint32_t { return put_e2m1_pair<0>(0u, v, v) & 0xfu; };
    uint32_t prev = start == 0 ? 0u : code(__uint_as_float((uint32_t)start - 1u));
    uint32_t checked = 0, bad_sign = 0, bad_order = 0, bad_neg = 0, bad_pack = 0;
    for (uint32_t b = (uint32_t)start; b < end; ++b) {
        const float v = __uint_as_float(b);
        const uint32_t c = code(v);
        ++checked;
        if (c & 8u) ++bad_sign;
        if (c < prev) ++bad_order;
        prev = c;
        const uint32_t cn = code(-v);
        if (cn != (c | 8u)) ++bad_neg;
        // the pair lands in byte (b & 3) with v in the low nibble and -v in the high one; the other
        // bytes of the word keep their values
        const uint32_t old = 0x9C5A3E71u ^ b;
        uint32_t w;
        switch (b & 3u) {
            case 0: w = put_e2m1_pair<0>(old, v, -v); break;
            case 1: w = put_e2m1_pair<1>(old, v, -v); break;
            case 2: w = put_e2m1_pair<2>(old, v, -v); break;
            default: w = put_e2m1_pair<3>(old, v, -v); break;
        }
        const uint32_t sh = 8u * (b & 3u);
        const uint32_t keep = ~(0xffu << sh);
        if ((w & keep) != (old & keep) || ((w >> sh) & 0xffu) != (c | (cn << 4))) ++bad_pack;
    }
    wave_add(counters + 0, checked);
    wave_add(counters + 1, bad_sign);
    wave_add(counters + 2, bad_order);
    wave_add(counters + 3, bad_neg);
    wave_add(counters + 4, bad_pack);
}

__global__ void eval_kernel(const float* v, const float* S, int64_t n, uint8_t* e4m3, uint8_t* e2m1, float* q_ieee,
                            float* q_fast) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float x = v[i];
    e4m3[i] = (uint8_t)(x >= 0.0f ? e4m3_rne_sat(x) : 0xffu);
    e2m1[i] = (uint8_t)(put_e2m1_pair<0>(0u, x, x) & 0xfu);
    const float a = fabsf(x), s = S[i];
    q_ieee[i] = __fdiv_rn(a, s);
    q_fast[i] = quotient_fast(a, s, __builtin_amdgcn_rcpf(s));
}

}  // namespace
}  // namespace nvfp4

extern "C" {

// All pointers are device pointers; each call runs on the null stream and returns the hipError_t of
// its launch (the caller synchronizes before reading the results).

// Divisors with binary32 exponent field s_exp_field (1..254) and every significand, against every
// finite non-negative bf16 numerator. counters: 4 zeroed uint64; first: 3 zeroed uint32.
int nvfp4_selftest_quotient_scan(uint32_t s_exp_field, unsigned long long* counters, uint32_t* first) {
    if (s_exp_field < 1 || s_exp_field > 254 || !counters || !first) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(nvfp4::quotient_scan_kernel, dim3((1u << 23) / 256u), dim3(256), 0, nullptr, s_exp_field,
                       counters, first);
    return (int)hipGetLastError();
}

// Every binary32 pattern in [0, +inf] through e4m3_rne_sat. counters: 3 zeroed uint64.
int nvfp4_selftest_e4m3_scan(unsigned long long* counters) {
    if (!counters) return (int)hipErrorInvalidValue;
    const uint64_t threads = ((uint64_t)nvfp4::POS_END + nvfp4::PER_THREAD - 1) / nvfp4::PER_THREAD;
    hipLaunchKernelGGL(nvfp4::e4m3_scan_kernel, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, nullptr,
                       counters);
    return (int)hipGetLastError();
}

// Every binary32 pattern in [0, +inf] and its negation through put_e2m1_pair. counters: 5 zeroed uint64.
int nvfp4_selftest_e2m1_scan(unsigned long long* counters) {
    if (!counters) return (int)hipErrorInvalidValue;
    const uint64_t threads = ((uint64_t)nvfp4::POS_END + nvfp4::PER_THREAD - 1) / nvfp4::PER_THREAD;
    hipLaunchKernelGGL(nvfp4::e2m1_scan_kernel, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, nullptr,
                       counters);
    return (int)hipGetLastError();
}

// Point evaluation: for each i, e4m3[i] = e4m3_rne_sat(v[i]) (0xff for negative v), e2m1[i] = the
// signed code of v[i], q_ieee[i] = __fdiv_rn(|v[i]|, S[i]), q_fast[i] = quotient_fast(|v[i]|, S[i]).
int nvfp4_selftest_eval(const float* v, const float* S, int64_t n, uint8_t* e4m3, uint8_t* e2m1, float* q_ieee,
                        float* q_fast) {
    if (n < 0 || (n > 0 && (!v || !S || !e4m3 || !e2m1 || !q_ieee || !q_fast))) return (int)hipErrorInvalidValue;
    if (n == 0) return 0;
    hipLaunchKernelGGL(nvfp4::eval_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, nullptr, v, S, n, e4m3,
                       e2m1, q_ieee, q_fast);
    return (int)hipGetLastError();
}

}  // extern "C"
