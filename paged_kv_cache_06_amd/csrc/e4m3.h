// e4m3.h: fp16 -> E4M3 (FP8) codes, the quantizer of every write into an
// E4M3 pool (kv_append_fp8 and kv_scatter_prefill_fp8 in blockops.hip, the
// fused append in decode_kernel.h), so that all store the same byte for the
// same input.
// Internal to libpagedattn.

#pragma once

#include <hip/hip_runtime.h>

namespace pa_e4m3 {

// The correctly rounded fp32 quotient x / s for s in [2^-96, 2^96], given
// y = RN(1/s) (computed once, on the host): q0 = RN(x*y) is within an ulp,
// and one correction step with a fused multiply-add (Markstein's:
// r = x - q0*s, exact, then RN(q0 + r*y)) makes it the correctly rounded
// quotient (the CPU test of this construction compares it with IEEE division
// for every finite fp16 x across that range of scales); zeros keep their sign
// (the sign of the quotient is x's, s > 0), infinities and NaN pass through.
__device__ __forceinline__ float quotient(float x, float s, float y) {
    const float q0 = x * y;
    const float r = __builtin_fmaf(-q0, s, x);
    const float q = __builtin_copysignf(__builtin_fmaf(r, y, q0), x);
    return __builtin_isinf(x) ? x : q;
}

// The stored codes of two fp16 elements a, b of a pool with scale s
// (y = RN(1/s)), byte 0 for a and byte 1 for b: E4M3 (OCP 8-bit float, bias
// 7, 3 mantissa bits, no infinity) of the correctly rounded fp32 quotients
// x / s, rounded to nearest with ties to the even mantissa by the hardware
// converter (v_cvt_pk_fp8_f32); magnitudes from 448 up (infinity included)
// are clamped to 448 first, so the converter's own result past the largest
// code never matters; a NaN quotient gives 0x7f; signs are kept (a negative
// value that rounds to zero gives 0x80). The GPU tests compare the codes of
// every fp16 bit pattern with the oracle's.
__device__ __forceinline__ unsigned quantize2(_Float16 a, _Float16 b, float s, float y) {
    const float qa = quotient((float)a, s, y), qb = quotient((float)b, s, y);
    unsigned w = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fminf(__builtin_fmaxf(qa, -448.0f), 448.0f),
                                                           __builtin_fminf(__builtin_fmaxf(qb, -448.0f), 448.0f),
                                                           0, false) & 0xffffu;
    if (__builtin_isnan(qa)) w = (w & 0xff00u) | 0x7fu;
    if (__builtin_isnan(qb)) w = (w & 0x00ffu) | 0x7f00u;
    return w;
}

}  // namespace pa_e4m3
