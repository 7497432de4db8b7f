// CPU oracle for paged KV-cache decode attention.
//
// TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
// cpu_baseline leg of bench.py may load this library. The product path
// (libpagedattn, HIP) never calls, links or includes anything here, and this
// file includes nothing from the product. It is plain, slow, obviously
// correct C++: loops in the order the definition reads, fp32 accumulation
// (the precision the method statement fixes), built with -O2
// -ffp-contract=off and no fast-math so every product and sum is rounded
// exactly as written.
//
// Sources (page title, section):
//   [Paged attention]  danielfleming.xyz/writing/inference/paged
//   [PagedAttention]   deepconcepts.dev/c/llm-paged-attention
//   [SLM paged attention] aicassindra.com/blogs/slm/slm_paged_attention.html
//
// What is computed. A request's keys and values live in fixed-size blocks of
// one shared pool; its block table maps logical block n = position / block_size
// to a physical block id [SLM paged attention, "The architecture: every piece
// explained"]; [PagedAttention, intro]. The decode kernel reads, for each row,
// only the blocks its table lists, at the row's own true length [Paged
// attention, "What changed"]. Paging changes where the bytes live and nothing
// about the numbers: the result is exact softmax attention over the row's
// tokens [PagedAttention, intro and "Sharing is the part that pays twice"].
// So the attention oracle is the textbook definition, evaluated with a plain
// two-pass softmax (max first, then exponentials), never the online/blockwise
// form the GPU uses. Two key/value heads serve twelve attention heads
// [Paged attention, "What a small pool does"]; query head h reads KV head
// h / (Hq / Hkv) (contiguous groups, a reading the pages leave open).
//
// Pool layout (the same bytes the GPU library reads; written out here
// independently):
//   K element (blk, g, t, d) at ((blk*Hkv + g)*(D/8) + d/8)*bs*8 + t*8 + d%8
//   V element (blk, g, t, d) at ((blk*Hkv + g)*D + d)*bs + t
// with blk a physical block id, g a KV head, t the slot in the block, d the
// channel. fp16 values are passed as uint16_t bit patterns. FP8 pools (E4M3
// bytes) use K at ((blk*Hkv + g)*(D/16) + d/16)*bs*16 + t*16 + d%16 and V at
// the fp16 V index, one byte each.
//
// Pins (tests/test_oracle_pins.py): dense float64 attention and torch's
// scaled_dot_product_attention on the numpy-gathered sequence; closed forms
// (L = 1 gives v_0; constant V gives the constant; q = 0 gives the mean of V;
// two tokens give the logistic weight); bit-exact invariance under physical
// block permutation, free-list history, batch position and block size;
// kv_append against a numpy scatter; fp16 conversions against numpy over
// every half pattern; E4M3 decoding of all 256 codes and encoding against
// torch's float8_e4m3fn and the format's closed-form values, the
// quantization error bound, and the FP8 attention against the fp16 oracle
// on pools whose dequantized values are exact in fp16.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// IEEE binary16 -> binary32, exact for every pattern.
float half_bits_to_float(uint16_t h) {
    const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    const uint32_t expo = (h >> 10) & 0x1fu;
    const uint32_t mant = h & 0x3ffu;
    uint32_t bits;
    if (expo == 0) {
        if (mant == 0) {
            bits = sign;
        } else {
            // subnormal: mant * 2^-24, exact in binary32
            float v = (float)mant * 5.9604644775390625e-08f;
            std::memcpy(&bits, &v, 4);
            bits |= sign;
        }
    } else if (expo == 31) {
        bits = sign | 0x7f800000u | (mant << 13);
    } else {
        bits = sign | ((expo - 15 + 127) << 23) | (mant << 13);
    }
    float f;
    std::memcpy(&f, &bits, 4);
    return f;
}

// binary32 -> binary16, round to nearest, ties to even.
uint16_t float_to_half_bits_rne(float f) {
    uint32_t x;
    std::memcpy(&x, &f, 4);
    const uint32_t sign = (x >> 16) & 0x8000u;
    const uint32_t ax = x & 0x7fffffffu;
    if (ax > 0x7f800000u) return (uint16_t)(sign | 0x7e00u | ((ax >> 13) & 0x3ffu));  // NaN
    if (ax >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);  // >= 65520 rounds to inf
    if (ax >= 0x38800000u) {                                    // normal half range
        const uint32_t mant = ax & 0x7fffffu;
        const uint32_t e = (ax >> 23) - 127 + 15;
        uint32_t h = (e << 10) | (mant >> 13);
        const uint32_t rem = mant & 0x1fffu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1;
        return (uint16_t)(sign | h);
    }
    if (ax < 0x33000000u) return (uint16_t)sign;  // below 2^-25: rounds to zero
    const uint32_t e = ax >> 23;
    const uint32_t m = (ax & 0x7fffffu) | 0x800000u;
    const uint32_t shift = 126 - e;  // value = m * 2^(e-150) = (m >> shift) units of 2^-24
    uint32_t h = m >> shift;
    const uint32_t rem = m & ((1u << shift) - 1u);
    const uint32_t halfway = 1u << (shift - 1);
    if (rem > halfway || (rem == halfway && (h & 1u))) h += 1;
    return (uint16_t)(sign | h);
}

inline size_t k_index(int64_t blk, int g, int t, int d, int Hkv, int D, int bs) {
    return ((size_t)(blk * Hkv + g) * (size_t)(D / 8) + (size_t)(d / 8)) * (size_t)bs * 8 + (size_t)t * 8 +
           (size_t)(d % 8);
}

inline size_t v_index(int64_t blk, int g, int t, int d, int Hkv, int D, int bs) {
    return ((size_t)(blk * Hkv + g) * (size_t)D + (size_t)d) * (size_t)bs + (size_t)t;
}

// 8-bit floating point, E4M3 in the OCP 8-bit floating point specification
// (the "fn" variant: finite values and NaN only): sign bit, 4 exponent bits
// with bias 7, 3 mantissa bits. Exponent field 0 holds zero and the
// subnormals (m/8) * 2^-6; exponent field 15 is an ordinary binade except for
// mantissa 7, which is NaN; there is no infinity, and the largest finite
// magnitude is 1.75 * 2^8 = 448. Every value is exact in fp32.
float fp8_bits_to_float(uint8_t c) {
    const int e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    const float mag = e == 0 ? std::ldexp((float)m, -9) : std::ldexp((float)(8 + m), e - 10);
    return (c & 0x80) ? -mag : mag;
}

// fp32 -> E4M3: the nearest finite code by direct search over the magnitudes,
// a tie going to the code with even mantissa; magnitudes at or above 448
// (infinity included) saturate to 448, NaN gives code 0x7f, and the sign bit
// is kept (a negative value that rounds to zero gives 0x80).
uint8_t float_to_fp8_bits(float x) {
    if (std::isnan(x)) return 0x7f;
    const uint8_t sign = std::signbit(x) ? 0x80 : 0;
    const double a = std::fabs((double)x);
    if (a >= 448.0) return sign | 0x7e;
    int best = 0;
    for (int c = 1; c <= 0x7e; ++c) {
        const double dc = std::fabs((double)fp8_bits_to_float((uint8_t)c) - a);
        const double db = std::fabs((double)fp8_bits_to_float((uint8_t)best) - a);
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;
    }
    return (uint8_t)(sign | best);
}

// The stored code of an fp16 value x in a pool quantized with scale s:
// E4M3 of the fp32 quotient x / s (one correctly rounded fp32 division, then
// the rounding above). Its value is code * s.
uint8_t quantize_fp8(uint16_t x, float s) { return float_to_fp8_bits(half_bits_to_float(x) / s); }

// fp8 pool layout: K element (blk, g, t, d) at
// ((blk*Hkv + g)*(D/16) + d/16)*bs*16 + t*16 + d%16 (16 channels = 16 bytes
// per slot and chunk); V as in the fp16 pool, one byte per element.
inline size_t k_index8(int64_t blk, int g, int t, int d, int Hkv, int D, int bs) {
    return ((size_t)(blk * Hkv + g) * (size_t)(D / 16) + (size_t)(d / 16)) * (size_t)bs * 16 + (size_t)t * 16 +
           (size_t)(d % 16);
}

// Attention for one query head over L tokens whose K/V elements (as fp32
// values) are fetched by the callbacks. Two-pass softmax in fp32, ascending
// sums.
template <class KAt, class VAt>
void attend_one_head(float *o, const uint16_t *qh, int L, int D, float scale, KAt k_at, VAt v_at) {
    if (L <= 0) {
        for (int d = 0; d < D; ++d) o[d] = 0.0f;
        return;
    }
    std::vector<float> s((size_t)L), p((size_t)L);
    for (int t = 0; t < L; ++t) {
        float dot = 0.0f;
        for (int d = 0; d < D; ++d) dot += half_bits_to_float(qh[d]) * k_at(t, d);
        s[(size_t)t] = scale * dot;
    }
    float m = s[0];
    for (int t = 1; t < L; ++t)
        if (s[(size_t)t] > m) m = s[(size_t)t];
    float l = 0.0f;
    for (int t = 0; t < L; ++t) {
        p[(size_t)t] = std::exp(s[(size_t)t] - m);
        l += p[(size_t)t];
    }
    for (int d = 0; d < D; ++d) {
        float acc = 0.0f;
        for (int t = 0; t < L; ++t) acc += p[(size_t)t] * v_at(t, d);
        o[d] = acc / l;
    }
}

bool dims_ok(int B, int Hq, int Hkv, int D, int bs, int W) {
    return B >= 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0 && D > 0 && D % 8 == 0 && bs > 0 && W > 0;
}

// Driver shared by the paged attention entry points: the checks, then one
// (row, query head) item at a time, split over `nthreads` std::threads (the
// arithmetic of an item does not depend on the split). k_at(table, g, t, d)
// and v_at(...) return the fp32 value of element (t, d) of KV head g of the
// row whose block table is `table`.
template <class KAt, class VAt>
int paged_attend(float *out_f32, uint16_t *out_f16, const uint16_t *q, const int32_t *block_tables,
                 const int32_t *seq_lens, int B, int Hq, int Hkv, int D, int bs, int W, int N, float scale,
                 int nthreads, KAt k_at, VAt v_at) {
    const size_t cap = (size_t)W * bs;
    for (int b = 0; b < B; ++b) {
        const int L = seq_lens[b];
        if (L < 0 || (size_t)L > cap) return -2;
        for (int j = 0; j < (L + bs - 1) / bs; ++j) {
            const int32_t blk = block_tables[(size_t)b * W + j];
            if (blk < 0 || blk >= N) return -2;
        }
    }
    const int nrep = Hq / Hkv;
    auto work = [&](int64_t item) {
        const int b = (int)(item / Hq), h = (int)(item % Hq), g = h / nrep;
        const int32_t *table = block_tables + (size_t)b * W;
        float *o = out_f32 + ((size_t)b * Hq + h) * D;
        attend_one_head(o, q + ((size_t)b * Hq + h) * D, seq_lens[b], D, scale,
                        [&](int t, int d) { return k_at(table, g, t, d); },
                        [&](int t, int d) { return v_at(table, g, t, d); });
        if (out_f16)
            for (int d = 0; d < D; ++d) out_f16[((size_t)b * Hq + h) * D + d] = float_to_half_bits_rne(o[d]);
    };
    const int64_t items = (int64_t)B * Hq;
    if (nthreads <= 1) {
        for (int64_t i = 0; i < items; ++i) work(i);
    } else {
        std::vector<std::thread> pool;
        for (int w = 0; w < nthreads; ++w)
            pool.emplace_back([&, w] {
                for (int64_t i = w; i < items; i += nthreads) work(i);
            });
        for (auto &th : pool) th.join();
    }
    return 0;
}

}  // namespace

extern "C" {

// Round-trip helpers exported so the tests can pin the conversions against
// numpy over every bit pattern.
void oracle_half_to_float(float *out, const uint16_t *in, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = half_bits_to_float(in[i]);
}

void oracle_float_to_half(uint16_t *out, const float *in, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = float_to_half_bits_rne(in[i]);
}

// E4M3 conversions exported so the tests can pin them against torch's
// float8_e4m3fn and the format's closed-form values.
void oracle_fp8_to_float(float *out, const uint8_t *in, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = fp8_bits_to_float(in[i]);
}

void oracle_float_to_fp8(uint8_t *out, const float *in, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = float_to_fp8_bits(in[i]);
}

void oracle_quantize_fp8(uint8_t *out, const uint16_t *in, int64_t n, float scale) {
    for (int64_t i = 0; i < n; ++i) out[i] = quantize_fp8(in[i], scale);
}

// Append one decode step's K/V: row b's new token sits at position
// seq_lens[b] - 1 (seq_lens counts the token being appended), in the row's
// last listed block at slot position % bs [SLM paged attention, "End-to-end
// flow"; "The architecture: every piece explained"]. A pure bit copy; every
// other pool byte is left as it was. Rows with seq_len < 1 are skipped.
// Returns 0, or -1 on bad dimensions, or -2 if a row's target block id is
// outside [0, N) or its position outside the table (nothing is written for
// such a row).
int oracle_kv_append(const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool, uint16_t *v_pool,
                     const int32_t *block_tables, const int32_t *seq_lens, int B, int Hkv, int D, int bs, int W,
                     int N) {
    if (!dims_ok(B, Hkv, Hkv, D, bs, W) || N <= 0) return -1;
    int rc = 0;
    for (int b = 0; b < B; ++b) {
        const int L = seq_lens[b];
        if (L < 1) continue;
        const int pos = L - 1;
        const int logical = pos / bs;
        if (logical >= W) {
            rc = -2;
            continue;
        }
        const int32_t blk = block_tables[(size_t)b * W + logical];
        if (blk < 0 || blk >= N) {
            rc = -2;
            continue;
        }
        const int slot = pos % bs;
        for (int g = 0; g < Hkv; ++g) {
            for (int d = 0; d < D; ++d) {
                k_pool[k_index(blk, g, slot, d, Hkv, D, bs)] = k_new[((size_t)b * Hkv + g) * D + d];
                v_pool[v_index(blk, g, slot, d, Hkv, D, bs)] = v_new[((size_t)b * Hkv + g) * D + d];
            }
        }
    }
    return rc;
}

// The same append into an FP8 pool. A KV pool in 8-bit floats holds half the
// bytes per token of an fp16 one; the dtype is one of the terms that set
// bytes per token, which paging leaves alone [PagedAttention, "Three wastes
// wearing one name" and "Checking it on a real system"]. The pages fix no
// format or scaling; the reading taken here: E4M3 codes with one fp32 scale
// for all of K and one for all of V, each new element stored as
// quantize_fp8(x, scale). Same skips and return codes as oracle_kv_append.
int oracle_kv_append_fp8(const uint16_t *k_new, const uint16_t *v_new, uint8_t *k_pool, uint8_t *v_pool,
                         const int32_t *block_tables, const int32_t *seq_lens, int B, int Hkv, int D, int bs, int W,
                         int N, float k_scale, float v_scale) {
    if (!dims_ok(B, Hkv, Hkv, D, bs, W) || D % 16 || N <= 0) return -1;
    int rc = 0;
    for (int b = 0; b < B; ++b) {
        const int L = seq_lens[b];
        if (L < 1) continue;
        const int pos = L - 1;
        if (pos / bs >= W) {
            rc = -2;
            continue;
        }
        const int32_t blk = block_tables[(size_t)b * W + pos / bs];
        if (blk < 0 || blk >= N) {
            rc = -2;
            continue;
        }
        for (int g = 0; g < Hkv; ++g)
            for (int d = 0; d < D; ++d) {
                const size_t i = ((size_t)b * Hkv + g) * D + d;
                k_pool[k_index8(blk, g, pos % bs, d, Hkv, D, bs)] = quantize_fp8(k_new[i], k_scale);
                v_pool[v_index(blk, g, pos % bs, d, Hkv, D, bs)] = quantize_fp8(v_new[i], v_scale);
            }
    }
    return rc;
}

// Copy whole blocks for copy-on-write: for each pair i in order, block dst[i]
// takes block src[i]'s keys and values, every KV head and every slot. A block
// shared by several rows is cloned before one of them writes into it, and
// only that writer's table entry is repointed [SLM paged attention, "The
// architecture: every piece explained" and "End-to-end flow"; PagedAttention,
// "Sharing is the part that pays twice"]. A bit copy; no other block changes.
// Returns 0, -1 on bad dimensions, or -2 if a pair names a block outside
// [0, N) (that pair is skipped).
int oracle_kv_copy_blocks(uint16_t *k_pool, uint16_t *v_pool, const int32_t *src, const int32_t *dst, int n,
                          int Hkv, int D, int bs, int N) {
    if (n < 0 || Hkv <= 0 || D <= 0 || D % 8 || bs <= 0 || N <= 0) return -1;
    int rc = 0;
    for (int i = 0; i < n; ++i) {
        const int32_t s = src[i], t = dst[i];
        if (s < 0 || s >= N || t < 0 || t >= N) {
            rc = -2;
            continue;
        }
        for (int g = 0; g < Hkv; ++g)
            for (int slot = 0; slot < bs; ++slot)
                for (int d = 0; d < D; ++d) {
                    k_pool[k_index(t, g, slot, d, Hkv, D, bs)] = k_pool[k_index(s, g, slot, d, Hkv, D, bs)];
                    v_pool[v_index(t, g, slot, d, Hkv, D, bs)] = v_pool[v_index(s, g, slot, d, Hkv, D, bs)];
                }
    }
    return rc;
}

// The same block copies in FP8 pools (E4M3 codes, K groups of 16
// channels): a byte copy of every KV head and slot of each block. Same
// return codes as oracle_kv_copy_blocks.
int oracle_kv_copy_blocks_fp8(uint8_t *k_pool, uint8_t *v_pool, const int32_t *src, const int32_t *dst, int n,
                              int Hkv, int D, int bs, int N) {
    if (n < 0 || Hkv <= 0 || D <= 0 || D % 16 || bs <= 0 || N <= 0) return -1;
    int rc = 0;
    for (int i = 0; i < n; ++i) {
        const int32_t s = src[i], t = dst[i];
        if (s < 0 || s >= N || t < 0 || t >= N) {
            rc = -2;
            continue;
        }
        for (int g = 0; g < Hkv; ++g)
            for (int slot = 0; slot < bs; ++slot)
                for (int d = 0; d < D; ++d) {
                    k_pool[k_index8(t, g, slot, d, Hkv, D, bs)] = k_pool[k_index8(s, g, slot, d, Hkv, D, bs)];
                    v_pool[v_index(t, g, slot, d, Hkv, D, bs)] = v_pool[v_index(s, g, slot, d, Hkv, D, bs)];
                }
    }
    return rc;
}

// Scatter a prefill group's keys and values into the rows' blocks. The group
// was run left padded to its widest prompt (width S), so row b's prompt of
// length P = prompt_lens[b] sits at positions S-P .. S-1 of its [S][D] rows
// of k_src / v_src ([B][Hkv][S][D]); its token t goes to block
// block_tables[b][t / bs], slot t % bs, and the padding is dropped [Paged
// attention, "What changed"]. A bit copy; slots past P and blocks no row
// lists are untouched. Returns 0, -1 on bad dimensions, or -2 if a row's
// length exceeds S or W*bs (the row is skipped) or it lists a block outside
// [0, N) (that block's tokens are skipped).
int oracle_kv_scatter_prefill(const uint16_t *k_src, const uint16_t *v_src, uint16_t *k_pool, uint16_t *v_pool,
                              const int32_t *block_tables, const int32_t *prompt_lens, int B, int Hkv, int D,
                              int bs, int W, int N, int S) {
    if (!dims_ok(B, Hkv, Hkv, D, bs, W) || N <= 0 || S <= 0) return -1;
    int rc = 0;
    for (int b = 0; b < B; ++b) {
        const int P = prompt_lens[b];
        if (P <= 0) continue;
        if (P > S || (int64_t)P > (int64_t)W * bs) {
            rc = -2;
            continue;
        }
        for (int t = 0; t < P; ++t) {
            const int32_t blk = block_tables[(size_t)b * W + t / bs];
            if (blk < 0 || blk >= N) {
                rc = -2;
                continue;
            }
            const size_t s = (size_t)(S - P + t);
            for (int g = 0; g < Hkv; ++g)
                for (int d = 0; d < D; ++d) {
                    const size_t i = (((size_t)b * Hkv + g) * S + s) * D + d;
                    k_pool[k_index(blk, g, t % bs, d, Hkv, D, bs)] = k_src[i];
                    v_pool[v_index(blk, g, t % bs, d, Hkv, D, bs)] = v_src[i];
                }
        }
    }
    return rc;
}

// The post-prefill scatter into FP8 pools: as oracle_kv_scatter_prefill,
// each element stored as quantize_fp8(x, k_scale) (keys) or
// quantize_fp8(x, v_scale) (values) in the E4M3 layouts. Same skips and
// return codes; D % 16 == 0.
int oracle_kv_scatter_prefill_fp8(const uint16_t *k_src, const uint16_t *v_src, uint8_t *k_pool, uint8_t *v_pool,
                                  const int32_t *block_tables, const int32_t *prompt_lens, int B, int Hkv, int D,
                                  int bs, int W, int N, int S, float k_scale, float v_scale) {
    if (!dims_ok(B, Hkv, Hkv, D, bs, W) || D % 16 || N <= 0 || S <= 0) return -1;
    int rc = 0;
    for (int b = 0; b < B; ++b) {
        const int P = prompt_lens[b];
        if (P <= 0) continue;
        if (P > S || (int64_t)P > (int64_t)W * bs) {
            rc = -2;
            continue;
        }
        for (int t = 0; t < P; ++t) {
            const int32_t blk = block_tables[(size_t)b * W + t / bs];
            if (blk < 0 || blk >= N) {
                rc = -2;
                continue;
            }
            for (int g = 0; g < Hkv; ++g)
                for (int d = 0; d < D; ++d) {
                    const size_t i = (((size_t)b * Hkv + g) * S + (size_t)(S - P + t)) * D + d;
                    k_pool[k_index8(blk, g, t % bs, d, Hkv, D, bs)] = quantize_fp8(k_src[i], k_scale);
                    v_pool[v_index(blk, g, t % bs, d, Hkv, D, bs)] = quantize_fp8(v_src[i], v_scale);
                }
        }
    }
    return rc;
}

// Copy each row's first seq_len tokens out of the pool into contiguous
// [B][Hkv][W*bs][D] arrays, walking the table; positions >= seq_len are left
// untouched. This is the "read the same blocks" debug path [Paged attention,
// "What changed"] written as plain loops.
int oracle_gather_kv(uint16_t *k_out, uint16_t *v_out, const uint16_t *k_pool, const uint16_t *v_pool,
                     const int32_t *block_tables, const int32_t *seq_lens, int B, int Hkv, int D, int bs, int W,
                     int N) {
    if (!dims_ok(B, Hkv, Hkv, D, bs, W) || N <= 0) return -1;
    const size_t cap = (size_t)W * bs;
    for (int b = 0; b < B; ++b) {
        const int L = seq_lens[b];
        if (L < 0 || (size_t)L > cap) return -2;
        for (int t = 0; t < L; ++t) {
            const int32_t blk = block_tables[(size_t)b * W + t / bs];
            if (blk < 0 || blk >= N) return -2;
            for (int g = 0; g < Hkv; ++g)
                for (int d = 0; d < D; ++d) {
                    const size_t o = (((size_t)b * Hkv + g) * cap + (size_t)t) * D + d;
                    k_out[o] = k_pool[k_index(blk, g, t % bs, d, Hkv, D, bs)];
                    v_out[o] = v_pool[v_index(blk, g, t % bs, d, Hkv, D, bs)];
                }
        }
    }
    return 0;
}

// Paged decode attention: out[b][h][:] = softmax_t(scale * q[b][h] . k_t) . v_t
// over the row's tokens t = 0 .. seq_lens[b]-1, k_t and v_t read from block
// block_tables[b][t / bs], slot t % bs, KV head h / (Hq/Hkv) [Paged attention,
// "What changed"; PagedAttention, intro; SLM paged attention, "The
// architecture: every piece explained"]. out_f32 receives the unrounded
// result, out_f16 (if not null) its round-to-nearest-even fp16 bits. A row of
// length 0 gets zeros. Work is split over `nthreads` std::threads by
// (row, head) item; the arithmetic of each item does not depend on it.
// Returns 0, -1 on bad dimensions, -2 on a table entry outside [0, N) or a
// length outside [0, W*bs] (outputs are then unspecified).
int oracle_paged_decode_attn(float *out_f32, uint16_t *out_f16, const uint16_t *q, const uint16_t *k_pool,
                             const uint16_t *v_pool, const int32_t *block_tables, const int32_t *seq_lens, int B,
                             int Hq, int Hkv, int D, int bs, int W, int N, float scale, int nthreads) {
    if (!dims_ok(B, Hq, Hkv, D, bs, W) || N <= 0) return -1;
    auto k_at = [&](const int32_t *table, int g, int t, int d) {
        return half_bits_to_float(k_pool[k_index(table[t / bs], g, t % bs, d, Hkv, D, bs)]);
    };
    auto v_at = [&](const int32_t *table, int g, int t, int d) {
        return half_bits_to_float(v_pool[v_index(table[t / bs], g, t % bs, d, Hkv, D, bs)]);
    };
    return paged_attend(out_f32, out_f16, q, block_tables, seq_lens, B, Hq, Hkv, D, bs, W, N, scale, nthreads, k_at,
                        v_at);
}

// Paged decode attention over an FP8 pool: as oracle_paged_decode_attn with
// key element value fp8(code) * k_scale and value element fp8(code) * v_scale
// (each an fp32 product), q fp16. Same checks and return codes.
int oracle_paged_decode_attn_fp8(float *out_f32, uint16_t *out_f16, const uint16_t *q, const uint8_t *k_pool,
                                 const uint8_t *v_pool, const int32_t *block_tables, const int32_t *seq_lens, int B,
                                 int Hq, int Hkv, int D, int bs, int W, int N, float scale, float k_scale,
                                 float v_scale, int nthreads) {
    if (!dims_ok(B, Hq, Hkv, D, bs, W) || D % 16 || N <= 0) return -1;
    auto k_at = [&](const int32_t *table, int g, int t, int d) {
        return fp8_bits_to_float(k_pool[k_index8(table[t / bs], g, t % bs, d, Hkv, D, bs)]) * k_scale;
    };
    auto v_at = [&](const int32_t *table, int g, int t, int d) {
        return fp8_bits_to_float(v_pool[v_index(table[t / bs], g, t % bs, d, Hkv, D, bs)]) * v_scale;
    };
    return paged_attend(out_f32, out_f16, q, block_tables, seq_lens, B, Hq, Hkv, D, bs, W, N, scale, nthreads, k_at,
                        v_at);
}

// The same two-pass attention for one row over a contiguous sequence:
// q [Hq][D], k and v [L][Hkv][D]. No table, no block size.
int oracle_dense_attn(float *out_f32, const uint16_t *q, const uint16_t *k, const uint16_t *v, int L, int Hq,
                      int Hkv, int D, float scale) {
    if (!dims_ok(1, Hq, Hkv, D, 1, 1) || L < 0) return -1;
    const int nrep = Hq / Hkv;
    for (int h = 0; h < Hq; ++h) {
        const int g = h / nrep;
        auto k_at = [&](int t, int d) { return half_bits_to_float(k[((size_t)t * Hkv + g) * D + d]); };
        auto v_at = [&](int t, int d) { return half_bits_to_float(v[((size_t)t * Hkv + g) * D + d]); };
        attend_one_head(out_f32 + (size_t)h * D, q + (size_t)h * D, L, D, scale, k_at, v_at);
    }
    return 0;
}

// Checks the preconditions the GPU library assumes but does not verify on
// the device. Returns a bit set:
//   1  a table entry at logical index < ceil(L/bs) is outside [0, N)
//   2  a length is negative or exceeds W*bs
//   4  two rows append into the same (block, slot)
//   8  a row appends into a block that another row's live table lists
//      (copy-on-write would be required [SLM paged attention, "The
//      architecture: every piece explained"])
//  16  a row lists the same physical block twice
// `check_append` = 0 skips bits 4 and 8 (decode-only batches may share the
// block that holds their last token).
int oracle_validate(const int32_t *block_tables, const int32_t *seq_lens, int B, int bs, int W, int N,
                    int check_append) {
    int flags = 0;
    std::vector<int> refs((size_t)(N > 0 ? N : 0), 0);
    for (int b = 0; b < B; ++b) {
        const int L = seq_lens[b];
        if (L < 0 || (int64_t)L > (int64_t)W * bs) {
            flags |= 2;
            continue;
        }
        const int nblk = (L + bs - 1) / bs;
        for (int j = 0; j < nblk; ++j) {
            const int32_t blk = block_tables[(size_t)b * W + j];
            if (blk < 0 || blk >= N) {
                flags |= 1;
                continue;
            }
            for (int i = 0; i < j; ++i)
                if (block_tables[(size_t)b * W + i] == blk) flags |= 16;
            refs[(size_t)blk] += 1;
        }
    }
    if (check_append) {
        for (int b = 0; b < B; ++b) {
            const int L = seq_lens[b];
            if (L < 1 || (int64_t)L > (int64_t)W * bs) continue;
            const int32_t blk = block_tables[(size_t)b * W + (L - 1) / bs];
            if (blk < 0 || blk >= N) continue;
            if (refs[(size_t)blk] > 1) flags |= 8;
            for (int c = 0; c < b; ++c) {
                const int Lc = seq_lens[c];
                if (Lc < 1 || (int64_t)Lc > (int64_t)W * bs) continue;
                if (block_tables[(size_t)c * W + (Lc - 1) / bs] == blk && (Lc - 1) % bs == (L - 1) % bs)
                    flags |= 4;
            }
        }
    }
    return flags;
}

}  // extern "C"
