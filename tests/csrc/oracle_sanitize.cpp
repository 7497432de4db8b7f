// Exercises every entry point of the CPU oracle (oracle/oracle.cpp, linked
// into this program) on small seeded cases, valid and invalid, so that a
// build with the address and undefined-behaviour sanitizers checks the
// oracle's own memory accesses and arithmetic. Exit status 0 when every
// call returned the status the case expects; the sanitizers abort on any
// fault they find.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

extern "C" {
void oracle_half_to_float(float *, const uint16_t *, int64_t);
void oracle_float_to_half(uint16_t *, const float *, int64_t);
void oracle_fp8_to_float(float *, const uint8_t *, int64_t);
void oracle_float_to_fp8(uint8_t *, const float *, int64_t);
void oracle_quantize_fp8(uint8_t *, const uint16_t *, int64_t, float);
int oracle_kv_append(const uint16_t *, const uint16_t *, uint16_t *, uint16_t *, const int32_t *, const int32_t *,
                     int, int, int, int, int, int);
int oracle_kv_append_fp8(const uint16_t *, const uint16_t *, uint8_t *, uint8_t *, const int32_t *, const int32_t *,
                         int, int, int, int, int, int, float, float);
int oracle_kv_copy_blocks(uint16_t *, uint16_t *, const int32_t *, const int32_t *, int, int, int, int, int);
int oracle_kv_copy_blocks_fp8(uint8_t *, uint8_t *, const int32_t *, const int32_t *, int, int, int, int, int);
int oracle_kv_scatter_prefill(const uint16_t *, const uint16_t *, uint16_t *, uint16_t *, const int32_t *,
                              const int32_t *, int, int, int, int, int, int, int);
int oracle_kv_scatter_prefill_fp8(const uint16_t *, const uint16_t *, uint8_t *, uint8_t *, const int32_t *,
                                  const int32_t *, int, int, int, int, int, int, int, float, float);
int oracle_gather_kv(uint16_t *, uint16_t *, const uint16_t *, const uint16_t *, const int32_t *, const int32_t *,
                     int, int, int, int, int, int);
int oracle_paged_decode_attn(float *, uint16_t *, const uint16_t *, const uint16_t *, const uint16_t *,
                             const int32_t *, const int32_t *, int, int, int, int, int, int, int, float, int);
int oracle_paged_decode_attn_fp8(float *, uint16_t *, const uint16_t *, const uint8_t *, const uint8_t *,
                                 const int32_t *, const int32_t *, int, int, int, int, int, int, int, float, float,
                                 float, int);
int oracle_dense_attn(float *, const uint16_t *, const uint16_t *, const uint16_t *, int, int, int, int, float);
int oracle_validate(const int32_t *, const int32_t *, int, int, int, int, int);
}

static uint64_t g_state = 88172645463325252ULL;
static uint32_t next_u32() {
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return (uint32_t)g_state;
}
static int uniform(int lo, int hi) { return lo + (int)(next_u32() % (uint32_t)(hi - lo + 1)); }
static uint16_t random_half() {  // finite fp16 of moderate magnitude
    return (uint16_t)((next_u32() & 0x8000u) | (uint32_t)uniform(0x2000, 0x4800));
}

static int failures = 0;
static void expect(int got, int want, const char *what, int c) {
    if (got != want) {
        std::printf("case %d: %s returned %d, expected %d\n", c, what, got, want);
        ++failures;
    }
}

int main() {
    for (int c = 0; c < 40; ++c) {
        const int Hkv = uniform(1, 2), nrep = uniform(1, 3), Hq = Hkv * nrep;
        const int D = 16 * uniform(1, 4), bs = 8 * uniform(1, 2), B = uniform(1, 5), W = uniform(1, 4);
        std::vector<int32_t> lens(B), tables((size_t)B * W, -1);
        int N = 0;
        for (int b = 0; b < B; ++b) {
            lens[b] = uniform(0, W * bs);
            for (int j = 0; j < (lens[b] + bs - 1) / bs; ++j) tables[(size_t)b * W + j] = N++;
        }
        N += uniform(1, 3);
        const size_t pool = (size_t)N * Hkv * D * bs;
        std::vector<uint16_t> kp(pool), vp(pool), q((size_t)B * Hq * D), kn((size_t)B * Hkv * D), vn(kn.size());
        for (auto *v : {&kp, &vp, &q, &kn, &vn})
            for (auto &x : *v) x = random_half();
        std::vector<uint8_t> k8(pool), v8(pool);
        for (size_t i = 0; i < pool; ++i) {
            k8[i] = (uint8_t)(next_u32() & 0xf7u);  // never the NaN pattern
            v8[i] = (uint8_t)(next_u32() & 0xf7u);
        }
        std::vector<float> out((size_t)B * Hq * D);
        std::vector<uint16_t> out16(out.size());
        const float scale = 1.0f / std::sqrt((float)D);

        expect(oracle_validate(tables.data(), lens.data(), B, bs, W, N, 1), 0, "validate", c);
        expect(oracle_kv_append(kn.data(), vn.data(), kp.data(), vp.data(), tables.data(), lens.data(), B, Hkv, D, bs,
                                W, N), 0, "kv_append", c);
        expect(oracle_kv_append_fp8(kn.data(), vn.data(), k8.data(), v8.data(), tables.data(), lens.data(), B, Hkv, D,
                                    bs, W, N, 0.25f, 0.5f), 0, "kv_append_fp8", c);
        expect(oracle_paged_decode_attn(out.data(), out16.data(), q.data(), kp.data(), vp.data(), tables.data(),
                                        lens.data(), B, Hq, Hkv, D, bs, W, N, scale, 1 + c % 3), 0, "decode", c);
        expect(oracle_paged_decode_attn_fp8(out.data(), out16.data(), q.data(), k8.data(), v8.data(), tables.data(),
                                            lens.data(), B, Hq, Hkv, D, bs, W, N, scale, 0.25f, 0.5f, 1 + c % 2), 0,
               "decode_fp8", c);
        std::vector<uint16_t> ko((size_t)B * Hkv * W * bs * D), vo(ko.size());
        expect(oracle_gather_kv(ko.data(), vo.data(), kp.data(), vp.data(), tables.data(), lens.data(), B, Hkv, D, bs,
                                W, N), 0, "gather", c);
        if (lens[0] > 0) {  // dense attention over row 0, gathered into [L][Hkv][D]
            const int L = lens[0];
            std::vector<uint16_t> kd((size_t)L * Hkv * D), vd(kd.size());
            for (int t = 0; t < L; ++t)
                for (int g = 0; g < Hkv; ++g)
                    for (int d = 0; d < D; ++d) {
                        kd[((size_t)t * Hkv + g) * D + d] = ko[(((size_t)0 * Hkv + g) * W * bs + t) * D + d];
                        vd[((size_t)t * Hkv + g) * D + d] = vo[(((size_t)0 * Hkv + g) * W * bs + t) * D + d];
                    }
            expect(oracle_dense_attn(out.data(), q.data(), kd.data(), vd.data(), L, Hq, Hkv, D, scale), 0, "dense", c);
        }
        // copies, with one pair outside the pool
        std::vector<int32_t> src = {0, N - 1, N}, dst = {N - 1, 0, 0};
        expect(oracle_kv_copy_blocks(kp.data(), vp.data(), src.data(), dst.data(), 3, Hkv, D, bs, N), -2, "copy", c);
        expect(oracle_kv_copy_blocks_fp8(k8.data(), v8.data(), src.data(), dst.data(), 3, Hkv, D, bs, N), -2,
               "copy_fp8", c);
        // prefill scatter of a left-padded group, one row wider than the group
        const int S = W * bs;
        std::vector<uint16_t> ks((size_t)B * Hkv * S * D), vs(ks.size());
        for (size_t i = 0; i < ks.size(); ++i) {
            ks[i] = random_half();
            vs[i] = random_half();
        }
        std::vector<int32_t> prompts(lens);
        prompts[0] = S + 1;
        expect(oracle_kv_scatter_prefill(ks.data(), vs.data(), kp.data(), vp.data(), tables.data(), prompts.data(), B,
                                         Hkv, D, bs, W, N, S), -2, "scatter", c);
        expect(oracle_kv_scatter_prefill_fp8(ks.data(), vs.data(), k8.data(), v8.data(), tables.data(), prompts.data(),
                                             B, Hkv, D, bs, W, N, S, 0.1f, 0.2f), -2, "scatter_fp8", c);
        // a table entry outside the pool
        std::vector<int32_t> bad(tables);
        int row = -1;
        for (int b = 0; b < B && row < 0; ++b)
            if (lens[b] > 0) row = b;
        if (row >= 0) {
            bad[(size_t)row * W] = N + 5;
            expect(oracle_paged_decode_attn(out.data(), nullptr, q.data(), kp.data(), vp.data(), bad.data(),
                                            lens.data(), B, Hq, Hkv, D, bs, W, N, scale, 1), -2, "decode bad id", c);
            expect(oracle_kv_append(kn.data(), vn.data(), kp.data(), vp.data(), bad.data(), lens.data(), B, Hkv, D,
                                    bs, W, N), lens[row] <= bs ? -2 : 0, "append bad id", c);
            expect(oracle_validate(bad.data(), lens.data(), B, bs, W, N, 0) & 1, 1, "validate bad id", c);
        }
    }
    // conversions over every pattern
    std::vector<uint16_t> h(65536);
    std::vector<float> f(65536);
    for (int i = 0; i < 65536; ++i) h[i] = (uint16_t)i;
    oracle_half_to_float(f.data(), h.data(), 65536);
    oracle_float_to_half(h.data(), f.data(), 65536);
    std::vector<uint8_t> e(65536);
    oracle_quantize_fp8(e.data(), h.data(), 65536, 0.3f);
    oracle_float_to_fp8(e.data(), f.data(), 65536);
    std::vector<float> g(256);
    std::vector<uint8_t> codes(256);
    for (int i = 0; i < 256; ++i) codes[i] = (uint8_t)i;
    oracle_fp8_to_float(g.data(), codes.data(), 256);
    std::printf("%s: %d failures\n", failures ? "FAIL" : "ok", failures);
    return failures ? 1 : 0;
}
