// e4m3.h: fp32 -> E4M3 (FP8) code, the quantizer of every append into an
// E4M3 pool (kv_append_fp8 in blockops.hip, the fused append in
// decode_kernel.h), so that both store the same byte for the same input.
// Internal to libpagedattn.

#pragma once

#include <hip/hip_runtime.h>

namespace pa_e4m3 {

// fp32 -> E4M3 code (OCP 8-bit float, bias 7, 3 mantissa bits, no
// infinity): round to nearest, ties to even mantissa; magnitudes from 448 up
// (infinity included) saturate to 448; NaN gives 0x7f; the sign bit is kept.
__device__ __forceinline__ unsigned rne_sat(float t) {
    const unsigned u = __float_as_uint(t);
    const unsigned sign = (u >> 24) & 0x80u;
    const unsigned a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return 0x7fu;          // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;  // |t| >= 448
    if (a < 0x3c800000u) {                      // |t| < 2^-6: multiples of 2^-9 (the product is exact)
        const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);  // 0..8; 8 is the code of 2^-6
        return sign | (unsigned)m;
    }
    // normal: round the 20 dropped mantissa bits to nearest even; a carry
    // moves into the exponent, and |t| < 448 keeps the result at most 448
    const unsigned r = a + 0x7ffffu + ((a >> 20) & 1u);
    return sign | ((((r >> 23) - 120u) << 3) | ((r >> 20) & 7u));
}

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

// The stored code of an fp16 element x of a pool with scale s (y = RN(1/s)):
// the code of the correctly rounded fp32 quotient x / s.
__device__ __forceinline__ unsigned quantize(_Float16 x, float s, float y) { return rne_sat(quotient((float)x, s, y)); }

}  // namespace pa_e4m3
