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

// The stored code of an fp16 element x of a pool with scale s: the code of
// the fp32 quotient x / s (one correctly rounded division).
__device__ __forceinline__ unsigned quantize(_Float16 x, float s) { return rne_sat((float)x / s); }

}  // namespace pa_e4m3
