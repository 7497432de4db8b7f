// libpagedattn, block operations: the pool writes and copies around the
// decode step, all of them bit copies bound by memory latency or bandwidth:
//
//   append_kernel           kv_append: one decode step's K/V into each row's
//                           last block [SLM paged attention, "End-to-end flow"]
//   copy_blocks_kernel      kv_copy_blocks: whole-block copies for
//                           copy-on-write [SLM paged attention, "The
//                           architecture: every piece explained"]
//   scatter_prefill_kernel  kv_scatter_prefill: a left-padded prefill group's
//                           K/V into the rows' blocks, padding dropped [Paged
//                           attention, "What changed"]
//   append_fp8_kernel       kv_append_fp8: the same append into E4M3 (FP8)
//                           pools, quantizing [PagedAttention, "Checking it
//                           on a real system": FP8 KV halves bytes per token]
//   scatter_prefill_fp8_kernel  kv_scatter_prefill_fp8: the same scatter into
//                           E4M3 pools, quantizing
//   gather_kernel           paged_gather_kv: the debug path, the blocks a row
//                           lists copied out contiguously [Paged attention,
//                           "What changed"]
//
// Pool layouts (include/pagedattn.h): K [N][Hkv][D/8][bs][8], V [N][Hkv][D][bs];
// E4M3 pools K [N][Hkv][D/16][bs][16], V [N][Hkv][D][bs], one byte each.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "e4m3.h"
#include "pagedattn.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// E4M3 pool scales: finite, in [2^-96, 2^96] (the range in which the kernels'
// quotient x / scale is exact, see e4m3.h).
bool fp8_scale_ok(float s) { return std::isfinite(s) && s >= 0x1p-96f && s <= 0x1p96f; }

__device__ __forceinline__ int clamp_block(int blk, int N) {
    return (unsigned)blk < (unsigned)N ? blk : 0;
}

// One wave per (row, KV head): lanes 0..D/8-1 copy the 16-byte K groups,
// every lane copies D/64 (or fewer) V channels. The new token's K and V are
// requested before the row's length and table entry, which they do not depend
// on, so the call costs two dependent memory round trips instead of three.
__global__ void __launch_bounds__(64) append_kernel(const uint16_t* __restrict__ k_new,
                                                    const uint16_t* __restrict__ v_new,
                                                    uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool,
                                                    const int32_t* __restrict__ tables,
                                                    const int32_t* __restrict__ seq_lens, int Hkv, int D, int BS,
                                                    int W, int N) {
    constexpr int kMaxV = 8;  // V channels per lane held in registers (D <= 512)
    const int bg = blockIdx.x;
    const int b = bg / Hkv, g = bg % Hkv;
    const int lane = threadIdx.x;
    const uint16_t* ksrc = k_new + ((size_t)b * Hkv + g) * D;
    const uint16_t* vsrc = v_new + ((size_t)b * Hkv + g) * D;
    const bool fast = D <= 64 * kMaxV;
    // Issued from assembly, at clamped (always valid) addresses, so that the
    // compiler neither sinks them below the length and table reads nor waits
    // for them early; the wait comes right before the stores.
    u32x4 kx;
    unsigned vx[kMaxV];
    asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(kx) : "v"(ksrc + 8 * min(lane, D / 8 - 1)) : "memory");
#pragma unroll
    for (int i = 0; i < kMaxV; ++i)
        asm volatile("global_load_ushort %0, %1, off" : "=v"(vx[i]) : "v"(vsrc + min(lane + 64 * i, D - 1)) : "memory");
    const int L = seq_lens[b];
    const bool live = L >= 1 && (long long)L <= (long long)W * BS;
    const int pos = live ? L - 1 : 0;
    const int blk = tables[(size_t)b * W + pos / BS];
    asm volatile("s_waitcnt vmcnt(0)"  // the loads above have landed (also before leaving early)
                 : "+v"(kx), "+v"(vx[0]), "+v"(vx[1]), "+v"(vx[2]), "+v"(vx[3]), "+v"(vx[4]), "+v"(vx[5]),
                   "+v"(vx[6]), "+v"(vx[7])::"memory");
    if (!live || blk < 0 || blk >= N) return;
    const int slot = pos % BS;
    const size_t base = (size_t)blk * Hkv + g;
    if (fast) {
        if (lane < D / 8) *reinterpret_cast<u32x4*>(k_pool + ((base * (D / 8) + lane) * BS + slot) * 8) = kx;
#pragma unroll
        for (int i = 0; i < kMaxV; ++i)
            if (lane + 64 * i < D) v_pool[(base * D + lane + 64 * i) * BS + slot] = (uint16_t)vx[i];
        return;
    }
    for (int j = lane; j < D / 8; j += 64) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(ksrc + 8 * j);
        *reinterpret_cast<u32x4*>(k_pool + ((base * (D / 8) + j) * BS + slot) * 8) = x;
    }
    for (int d = lane; d < D; d += 64) v_pool[(base * D + d) * BS + slot] = vsrc[d];
}

// One workgroup per (row, KV head, logical block); thread per (token, channel).
// One wave per (row, KV head): each lane quantizes channels lane, lane+64, ...
// of the new token's K and V (code of x / scale, the quotient correctly
// rounded in fp32) and stores the bytes into the row's last block.
__global__ void __launch_bounds__(64) append_fp8_kernel(const uint16_t* __restrict__ k_new,
                                                        const uint16_t* __restrict__ v_new,
                                                        uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                                                        const int32_t* __restrict__ tables,
                                                        const int32_t* __restrict__ seq_lens, int Hkv, int D, int BS,
                                                        int W, int N, float k_scale, float v_scale, float k_inv,
                                                        float v_inv) {
    const int bg = blockIdx.x;
    const int b = bg / Hkv, g = bg % Hkv;
    const int lane = threadIdx.x;
    const int L = seq_lens[b];
    if (L < 1 || (long long)L > (long long)W * BS) return;
    const int pos = L - 1;
    const int blk = tables[(size_t)b * W + pos / BS];
    if (blk < 0 || blk >= N) return;
    const int slot = pos % BS;
    const size_t base = (size_t)blk * Hkv + g;
    const _Float16* ks = reinterpret_cast<const _Float16*>(k_new) + ((size_t)b * Hkv + g) * D;
    const _Float16* vs = reinterpret_cast<const _Float16*>(v_new) + ((size_t)b * Hkv + g) * D;
    for (int d = lane; d < D; d += 64) {
        k_pool[((base * (D / 16) + d / 16) * BS + slot) * 16 + d % 16] =
            (uint8_t)pa_e4m3::quantize2(ks[d], ks[d], k_scale, k_inv);
        v_pool[(base * D + d) * BS + slot] = (uint8_t)pa_e4m3::quantize2(vs[d], vs[d], v_scale, v_inv);
    }
}

__global__ void __launch_bounds__(256) gather_kernel(uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out,
                                                     const uint16_t* __restrict__ k_pool,
                                                     const uint16_t* __restrict__ v_pool,
                                                     const int32_t* __restrict__ tables,
                                                     const int32_t* __restrict__ seq_lens, int Hkv, int D, int BS,
                                                     int W, int N) {
    const int j = blockIdx.x % W;
    const int bg = blockIdx.x / W;
    const int b = bg / Hkv, g = bg % Hkv;
    const int cap = W * BS;
    int L = seq_lens[b];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int t_lo = j * BS;
    if (t_lo >= L) return;
    const int n = min(BS, L - t_lo);
    const int blk = clamp_block(tables[(size_t)b * W + j], N);
    const size_t base = (size_t)blk * Hkv + g;
    for (int e = threadIdx.x; e < n * D; e += blockDim.x) {
        const int t = e / D, d = e % D;
        const size_t o = (((size_t)bg * cap) + t_lo + t) * D + d;
        k_out[o] = k_pool[((base * (D / 8) + d / 8) * BS + t) * 8 + d % 8];
        v_out[o] = v_pool[(base * D + d) * BS + t];
    }
}

// Copy-on-write block copy: workgroup (pair, layer, pool) copies one block of
// the K pool (z = 0) or the V pool (z = 1). A block is Hkv*D*bs contiguous
// halves in both layouts; each thread moves eight 16-byte pieces per round
// (a whole 32 KiB block at the Qwen shape), all loads in flight before the
// stores, which are non-temporal: the copy is not read again by this launch.
__global__ void __launch_bounds__(256) copy_blocks_kernel(uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool,
                                                          const int32_t* __restrict__ src,
                                                          const int32_t* __restrict__ dst, int N,
                                                          long long block_elems, long long layer_stride) {
    const int s = src[blockIdx.x], t = dst[blockIdx.x];
    if ((unsigned)s >= (unsigned)N || (unsigned)t >= (unsigned)N || s == t) return;
    uint16_t* base = (blockIdx.z ? v_pool : k_pool) + (long long)blockIdx.y * layer_stride;
    const u32x4* from = reinterpret_cast<const u32x4*>(base + (long long)s * block_elems);
    u32x4* to = reinterpret_cast<u32x4*>(base + (long long)t * block_elems);
    const int n16 = (int)(block_elems / 8);
    constexpr int kU = 8;
    for (int i0 = threadIdx.x; i0 < n16; i0 += 256 * kU) {
        u32x4 x[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (i0 + u * 256 < n16) x[u] = from[i0 + u * 256];
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (i0 + u * 256 < n16) __builtin_nontemporal_store(x[u], &to[i0 + u * 256]);
    }
}

// Post-prefill scatter: workgroup (x, KV head g, row b) moves the keys (x < W:
// logical block j = x) or the values (x >= W: j = x - W) of the row's tokens
// j*bs .. j*bs+bs-1 from the left-padded prefill group
// ([B][Hkv][S][D], token-major; row b's prompt right-aligned) into physical
// block block_tables[b][j]. Both pool layouts want a transpose of the
// token-major source (K: [D/8][bs][8], V: [D][bs]), done through LDS so that
// the global reads run along the channels and the writes along the slots:
// K in 16-byte units (row stride bs+1 units, conflict-free), then V in halves
// (row stride bs+8 halves), the writes 16 bytes per lane where eight whole
// slots are present and 2 bytes per slot at a partial end; the 16-byte writes
// are non-temporal (nothing in this launch reads them).
__global__ void __launch_bounds__(256) scatter_prefill_kernel(
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src, uint16_t* __restrict__ k_pool,
    uint16_t* __restrict__ v_pool, const int32_t* __restrict__ tables, const int32_t* __restrict__ prompt_lens,
    int Hkv, int D, int BS, int W, int N, int S) {
    extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];
    const bool vpart = (int)blockIdx.x >= W;
    const int j = vpart ? blockIdx.x - W : blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int P = prompt_lens[b];
    const int t0 = j * BS;
    if (P <= 0 || P > S || (long long)P > (long long)W * BS || t0 >= P) return;
    const int blk = tables[(size_t)b * W + j];
    if ((unsigned)blk >= (unsigned)N) return;
    const int n = min(BS, P - t0);  // tokens of this block
    const int C = D / 8;             // 16-byte channel groups per token
    const size_t src0 = (((size_t)b * Hkv + g) * S + (size_t)(S - P + t0)) * D;  // the block's first token
    const size_t dst0 = ((size_t)blk * Hkv + g) * (size_t)D * BS;             // the (block, head) slab, both pools

    if (!vpart) {  // ---- K: [token][D] -> [D/8][bs][8]
        u32x4* sk = reinterpret_cast<u32x4*>(s_raw);  // [C][BS + 1]
        for (int u = threadIdx.x; u < n * C; u += 256) {
            const int i = u / C, c = u - i * C;
            sk[c * (BS + 1) + i] = *reinterpret_cast<const u32x4*>(k_src + src0 + (size_t)i * D + 8 * c);
        }
        __syncthreads();
        for (int u = threadIdx.x; u < n * C; u += 256) {
            const int c = u / n, i = u - c * n;
            __builtin_nontemporal_store(sk[c * (BS + 1) + i], reinterpret_cast<u32x4*>(k_pool + dst0 + ((size_t)c * BS + i) * 8));
        }
        return;
    }

    // ---- V: [token][D] -> [D][bs]
    uint16_t* sv = reinterpret_cast<uint16_t*>(s_raw);  // [D][BS + 8]
    const int R = BS + 8;
    for (int u = threadIdx.x; u < n * C; u += 256) {
        const int i = u / C, c = u - i * C;
        const u32x4 x = *reinterpret_cast<const u32x4*>(v_src + src0 + (size_t)i * D + 8 * c);
        const unsigned w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            sv[(8 * c + 2 * k) * R + i] = (uint16_t)(w4[k] & 0xffffu);
            sv[(8 * c + 2 * k + 1) * R + i] = (uint16_t)(w4[k] >> 16);
        }
    }
    __syncthreads();
    const int n8 = (BS % 8 == 0) ? n / 8 : 0;  // whole 8-slot groups (16-byte aligned in the pool)
    for (int u = threadIdx.x; u < D * n8; u += 256) {
        const int d = u / n8, q = u - d * n8;
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(sv + d * R + 8 * q),
                                    reinterpret_cast<u32x4*>(v_pool + dst0 + (size_t)d * BS + 8 * q));
    }
    const int rest = n - 8 * n8;  // slots past the last whole group
    for (int u = threadIdx.x; u < D * rest; u += 256) {
        const int d = u / rest, i = 8 * n8 + (u - d * rest);
        v_pool[dst0 + (size_t)d * BS + i] = sv[d * R + i];
    }
}

// Post-prefill scatter into E4M3 pools: the same grid as scatter_prefill_kernel
// (keys or values of one logical block of one row and KV head per
// workgroup), each element quantized (code of x / scale) on its way through
// LDS. Keys: codes staged token-major ([token][D + 16] bytes), then written
// 16 bytes per lane along the slots of each 16-channel group ([D/16][bs][16]).
// Values: codes staged channel-major ([D][bs + 16] bytes), then written 16
// slots (16 bytes) per lane along each channel row ([D][bs]), single bytes
// for the slots past the last whole 16 of a partial block.
__global__ void __launch_bounds__(256) scatter_prefill_fp8_kernel(
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src, uint8_t* __restrict__ k_pool,
    uint8_t* __restrict__ v_pool, const int32_t* __restrict__ tables, const int32_t* __restrict__ prompt_lens,
    int Hkv, int D, int BS, int W, int N, int S, float k_scale, float v_scale, float k_inv, float v_inv) {
    extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];
    const bool vpart = (int)blockIdx.x >= W;
    const int j = vpart ? blockIdx.x - W : blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int P = prompt_lens[b];
    const int t0 = j * BS;
    if (P <= 0 || P > S || (long long)P > (long long)W * BS || t0 >= P) return;
    const int blk = tables[(size_t)b * W + j];
    if ((unsigned)blk >= (unsigned)N) return;
    const int n = min(BS, P - t0);  // tokens of this block
    const int C = D / 8;             // 16-byte groups of 8 fp16 channels per source token
    const size_t src0 = (((size_t)b * Hkv + g) * S + (size_t)(S - P + t0)) * D;
    const size_t dst0 = ((size_t)blk * Hkv + g) * (size_t)D * BS;  // the (block, head) slab, bytes, both pools
    const uint16_t* src = vpart ? v_src : k_src;
    const float scale = vpart ? v_scale : k_scale, inv = vpart ? v_inv : k_inv;

    if (!vpart) {  // ---- K: [token][D] -> codes [D/16][bs][16]
        const int RK = D + 16;  // staging row stride, bytes
        for (int u = threadIdx.x; u < n * C; u += 256) {
            const int i = u / C, c = u - i * C;
            const u32x4 x = *reinterpret_cast<const u32x4*>(src + src0 + (size_t)i * D + 8 * c);
            const _Float16* h = reinterpret_cast<const _Float16*>(&x);
            unsigned w0 = 0, w1 = 0;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                w0 |= pa_e4m3::quantize2(h[2 * k], h[2 * k + 1], scale, inv) << (16 * k);
                w1 |= pa_e4m3::quantize2(h[4 + 2 * k], h[5 + 2 * k], scale, inv) << (16 * k);
            }
            *reinterpret_cast<uint2*>(s_raw + i * RK + 8 * c) = make_uint2(w0, w1);
        }
        __syncthreads();
        const int C16 = D / 16;
        for (int u = threadIdx.x; u < n * C16; u += 256) {
            const int c = u / n, i = u - c * n;
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(s_raw + i * RK + 16 * c),
                                        reinterpret_cast<u32x4*>(k_pool + dst0 + ((size_t)c * BS + i) * 16));
        }
        return;
    }

    // ---- V: [token][D] -> codes [D][bs]
    const int RV = BS + 16;  // staging row stride, bytes
    for (int u = threadIdx.x; u < n * C; u += 256) {
        const int i = u / C, c = u - i * C;
        const u32x4 x = *reinterpret_cast<const u32x4*>(src + src0 + (size_t)i * D + 8 * c);
        const _Float16* h = reinterpret_cast<const _Float16*>(&x);
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
            const unsigned w = pa_e4m3::quantize2(h[k], h[k + 1], scale, inv);
            s_raw[(8 * c + k) * RV + i] = (unsigned char)(w & 0xffu);
            s_raw[(8 * c + k + 1) * RV + i] = (unsigned char)(w >> 8);
        }
    }
    __syncthreads();
    const int n16 = n / 16;  // whole 16-slot groups (16-byte aligned in the pool: BS % 16 == 0)
    for (int u = threadIdx.x; u < D * n16; u += 256) {
        const int d = u / n16, q = u - d * n16;
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(s_raw + d * RV + 16 * q),
                                    reinterpret_cast<u32x4*>(v_pool + dst0 + (size_t)d * BS + 16 * q));
    }
    const int rest = n - 16 * n16;
    for (int u = threadIdx.x; u < D * rest; u += 256) {
        const int d = u / rest, i = 16 * n16 + (u - d * rest);
        v_pool[dst0 + (size_t)d * BS + i] = s_raw[d * RV + i];
    }
}

// Streaming-read probe: every 16-byte unit of the buffer read once, in
// coalesced grid-stride order, folded into one XOR per lane so the loads are
// not dropped; one word per workgroup is written. The bandwidth a plain read
// of a given byte count reaches, launch and ramp included: the reference a
// kernel that reads that many bytes can be held against.
__global__ void __launch_bounds__(256) probe_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
    constexpr int kU = 4;
    u32x4 acc = {0u, 0u, 0u, 0u};
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + (kU - 1) * stride < n16; i += kU * stride) {
        u32x4 x[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) x[u] = __builtin_nontemporal_load(&src[i + u * stride]);
#pragma unroll
        for (int u = 0; u < kU; ++u) acc ^= x[u];
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(&src[i]);
    const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
    // keep the loads live: one store per workgroup (the XOR of lane 0; its value does not matter)
    if (threadIdx.x == 0) sink[blockIdx.x] = v;
}

}  // namespace

extern "C" {

pa_status kv_append(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_pool, uint16_t* v_pool,
                    const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                    void* stream) {
    if (num_seqs < 0 || num_kv_heads <= 0 || head_dim <= 0 || head_dim % 8 || block_size <= 0 ||
        max_blocks_per_seq <= 0 || num_blocks <= 0)
        return PA_ERR_INVALID_ARG;
    if (num_seqs == 0) return PA_OK;
    if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !seq_lens) return PA_ERR_INVALID_ARG;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
        return PA_ERR_INVALID_ARG;
    if ((long long)num_seqs * num_kv_heads > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(append_kernel, dim3(num_seqs * num_kv_heads), dim3(64), 0, (hipStream_t)stream, k_new,
                       v_new, k_pool, v_pool, block_tables, seq_lens, num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, num_blocks);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status kv_append_fp8(const uint16_t* k_new, const uint16_t* v_new, uint8_t* k_pool, uint8_t* v_pool,
                        const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                        int32_t num_blocks, float k_scale, float v_scale, void* stream) {
    if (num_seqs < 0 || num_kv_heads <= 0 || head_dim <= 0 || head_dim % 16 || block_size <= 0 ||
        max_blocks_per_seq <= 0 || num_blocks <= 0)
        return PA_ERR_INVALID_ARG;
    if (!fp8_scale_ok(k_scale) || !fp8_scale_ok(v_scale)) return PA_ERR_INVALID_ARG;
    if (num_seqs == 0) return PA_OK;
    if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !seq_lens) return PA_ERR_INVALID_ARG;
    if ((long long)num_seqs * num_kv_heads > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(append_fp8_kernel, dim3(num_seqs * num_kv_heads), dim3(64), 0, (hipStream_t)stream, k_new,
                       v_new, k_pool, v_pool, block_tables, seq_lens, num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, num_blocks, k_scale, v_scale, 1.0f / k_scale, 1.0f / v_scale);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status kv_copy_blocks(uint16_t* k_pool, uint16_t* v_pool, const int32_t* src, const int32_t* dst, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                         int32_t num_layers, int64_t layer_stride, void* stream) {
    if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || head_dim % 8 || block_size <= 0 || num_blocks <= 0 ||
        num_layers <= 0 || num_layers > 65535)
        return PA_ERR_INVALID_ARG;
    const long long block_elems = (long long)num_kv_heads * head_dim * block_size;
    if (num_layers > 1 && (layer_stride < block_elems * num_blocks || layer_stride % 8)) return PA_ERR_INVALID_ARG;
    if (num_pairs == 0) return PA_OK;
    if (!k_pool || !v_pool || !src || !dst) return PA_ERR_INVALID_ARG;
    if (!aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_INVALID_ARG;
    const long long stride = num_layers > 1 ? (long long)layer_stride : 0;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)num_pairs, (unsigned)num_layers, 2), dim3(256), 0,
                       (hipStream_t)stream, k_pool, v_pool, src, dst, num_blocks, block_elems, stride);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status kv_copy_blocks_fp8(uint8_t* k_pool, uint8_t* v_pool, const int32_t* src, const int32_t* dst,
                             int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t num_layers, int64_t layer_stride, void* stream) {
    // the fp16 copy kernel moves 16-byte units: an E4M3 block is Hkv*D*bs bytes, i.e. Hkv*(D/2)*bs halves
    if (head_dim <= 0 || head_dim % 16 || (num_layers > 1 && layer_stride % 2)) return PA_ERR_INVALID_ARG;
    return kv_copy_blocks(reinterpret_cast<uint16_t*>(k_pool), reinterpret_cast<uint16_t*>(v_pool), src, dst,
                          num_pairs, num_kv_heads, head_dim / 2, block_size, num_blocks, num_layers,
                          layer_stride / 2, stream);
}

pa_status kv_scatter_prefill(const uint16_t* k_src, const uint16_t* v_src, uint16_t* k_pool, uint16_t* v_pool,
                             const int32_t* block_tables, const int32_t* prompt_lens, int32_t num_seqs,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                             int32_t num_blocks, int32_t padded_len, void* stream) {
    if (num_seqs < 0 || num_seqs > 65535 || num_kv_heads <= 0 || num_kv_heads > 65535 || head_dim <= 0 ||
        head_dim % 8 || block_size <= 0 || block_size > 1024 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
        padded_len <= 0)
        return PA_ERR_INVALID_ARG;
    if (num_seqs == 0) return PA_OK;
    if (!k_src || !v_src || !k_pool || !v_pool || !block_tables || !prompt_lens) return PA_ERR_INVALID_ARG;
    if (!aligned16(k_src) || !aligned16(v_src) || !aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_INVALID_ARG;
    // LDS: the larger of the K tile ([D/8][bs+1] x 16 B) and the V tile ([D][bs+8] x 2 B)
    const size_t lds = std::max<size_t>((size_t)(head_dim / 8) * (block_size + 1) * 16,
                                        (size_t)head_dim * (block_size + 8) * 2);
    if (lds > 64 * 1024) return PA_ERR_UNSUPPORTED;
    if ((long long)max_blocks_per_seq * 2 > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(scatter_prefill_kernel, dim3((unsigned)max_blocks_per_seq * 2, (unsigned)num_kv_heads,
                                                    (unsigned)num_seqs),
                       dim3(256), lds, (hipStream_t)stream, k_src, v_src, k_pool, v_pool, block_tables, prompt_lens,
                       num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, padded_len);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status kv_scatter_prefill_fp8(const uint16_t* k_src, const uint16_t* v_src, uint8_t* k_pool, uint8_t* v_pool,
                                 const int32_t* block_tables, const int32_t* prompt_lens, int32_t num_seqs,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t max_blocks_per_seq, int32_t num_blocks, int32_t padded_len, float k_scale,
                                 float v_scale, void* stream) {
    if (num_seqs < 0 || num_seqs > 65535 || num_kv_heads <= 0 || num_kv_heads > 65535 || head_dim <= 0 ||
        head_dim % 16 || block_size <= 0 || block_size % 16 || block_size > 1024 || max_blocks_per_seq <= 0 ||
        num_blocks <= 0 || padded_len <= 0)
        return PA_ERR_INVALID_ARG;
    if (!fp8_scale_ok(k_scale) || !fp8_scale_ok(v_scale)) return PA_ERR_INVALID_ARG;
    if (num_seqs == 0) return PA_OK;
    if (!k_src || !v_src || !k_pool || !v_pool || !block_tables || !prompt_lens) return PA_ERR_INVALID_ARG;
    if (!aligned16(k_src) || !aligned16(v_src) || !aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_INVALID_ARG;
    // LDS: the larger of the K staging ([bs][D+16] bytes) and the V staging ([D][bs+16] bytes)
    const size_t lds = std::max<size_t>((size_t)block_size * (head_dim + 16), (size_t)head_dim * (block_size + 16));
    if (lds > 64 * 1024) return PA_ERR_UNSUPPORTED;
    if ((long long)max_blocks_per_seq * 2 > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(scatter_prefill_fp8_kernel, dim3((unsigned)max_blocks_per_seq * 2, (unsigned)num_kv_heads,
                                                        (unsigned)num_seqs),
                       dim3(256), lds, (hipStream_t)stream, k_src, v_src, k_pool, v_pool, block_tables, prompt_lens,
                       num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, padded_len, k_scale,
                       v_scale, 1.0f / k_scale, 1.0f / v_scale);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_probe_read(const void* src, size_t bytes, uint32_t* sink, int32_t num_workgroups, void* stream) {
    if (!src || !sink || bytes == 0 || bytes % 16 || !aligned16(src) || num_workgroups <= 0) return PA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)num_workgroups), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const u32x4*>(src), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status paged_gather_kv(uint16_t* k_out, uint16_t* v_out, const uint16_t* k_pool, const uint16_t* v_pool,
                          const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                          int32_t num_blocks, void* stream) {
    if (num_seqs < 0 || num_kv_heads <= 0 || head_dim <= 0 || head_dim % 8 || block_size <= 0 ||
        max_blocks_per_seq <= 0 || num_blocks <= 0)
        return PA_ERR_INVALID_ARG;
    if (num_seqs == 0) return PA_OK;
    if (!k_out || !v_out || !k_pool || !v_pool || !block_tables || !seq_lens) return PA_ERR_INVALID_ARG;
    const long long grid = (long long)num_seqs * num_kv_heads * max_blocks_per_seq;
    if (grid > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, k_out, v_out, k_pool,
                       v_pool, block_tables, seq_lens, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                       num_blocks);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
