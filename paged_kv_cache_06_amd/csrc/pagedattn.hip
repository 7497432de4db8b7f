// libpagedattn: paged KV-cache decode attention for MI355X (gfx950).
//
// Sources (page title, section):
//   [Paged attention]     danielfleming.xyz/writing/inference/paged
//   [PagedAttention]      deepconcepts.dev/c/llm-paged-attention
//   [SLM paged attention] aicassindra.com/blogs/slm/slm_paged_attention.html
//
// Three kernels sit behind the C ABI declared in include/pagedattn.h:
//
//   append_kernel   one decode step's K/V scattered into each row's last block
//                   [SLM paged attention, "End-to-end flow"].
//   decode_kernel   one query token per row; the row's table is walked, its
//                   blocks gathered at its own length [Paged attention, "What
//                   changed"], and softmax attention computed for the query
//                   heads of one KV group at once.
//   gather_kernel   debug path: the same blocks copied out contiguously.
//
// decode_kernel design (CDNA4: 64-lane waves, 4 SIMDs per CU, fp16 dot2 on
// the vector ALU, no matrix cores -- decode attention is a matrix-vector
// product per KV group and HBM-bound):
//
//  * Work item = (row b, KV head g, partition p). A row's tokens are cut into
//    64-token tiles; a partition is `chunk` consecutive tiles. Every
//    workgroup reads seq_lens, sizes `chunk` so the launch yields about
//    `target_wgs` items, and finds its own item by prefix sum -- no host
//    sync, no empty work for short rows. The split over the sequence is exact
//    because partial softmax results are rescaled and combined exactly
//    [PagedAttention, "Sharing is the part that pays twice"].
//  * A workgroup is 4 waves; wave w takes tiles w, w+4, ... of the
//    partition. Per tile every lane issues 16-byte loads: with the K pool
//    in [D/8][bs][8] order, load j of lane l is the 8 channels 8j..8j+7 of
//    token l, so one load instruction covers 1 KiB of contiguous K and a
//    lane ends up owning one token's whole key. With V in [D][bs] order,
//    load jj of lane l is 8 consecutive tokens (8*(l%8)..) of channel row
//    8*jj' + l/8, again 1 KiB contiguous per instruction.
//  * QK: lane = token, dot products with v_dot2_f32_f16 against the query
//    heads of the group (the same query bits for every lane, read through the
//    scalar unit), so no cross-lane reduction is needed for scores.
//  * Online softmax per tile: wave max by DPP row permutes plus the gfx950
//    permlane16/32 swaps; p = exp2(s*scale*log2e - m) rounded to fp16 and
//    passed through LDS to the V layout; l accumulated per lane.
//  * PV: lane (l%8 = token chunk, l/8 = channel offset) accumulates
//    p[t..t+7] . v[d][t..t+7] with dot2 into fp32 accumulators that persist
//    across tiles. The V rows a lane loads are permuted (jj' = jj ^ f(l%8))
//    so that the final reduction over the 8 lanes sharing a channel row is a
//    transposing butterfly costing one DPP add per output.
//  * The 4 waves merge through LDS; a one-partition row writes fp16 output
//    directly. Otherwise the partition writes (max, sum, unnormalised
//    output) to the workspace, and the last partition to arrive (atomic
//    ticket) merges all of them in partition order, then resets the ticket.
//
// Stale slots and unlisted blocks may hold NaN: scores of tokens past the
// row's length are replaced (not multiplied) by -inf, and their V halves are
// zeroed before the dot products.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "pagedattn.h"

namespace {

constexpr int kLanes = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kLanes * kWaves;
constexpr int kTile = 64;  // tokens per tile (one lane per token in QK)

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// wave-level helpers
// ---------------------------------------------------------------------------

// DPP controls (gfx9 encoding).
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowMirror = 0x140;   // lane i <-> 15-i within 16
constexpr int kHalfMirror = 0x141;  // lane i <-> 7-i within 8

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Combine lanes i and i^16, then i and i^32, with the gfx950 permlane swaps.
template <class Op>
__device__ __forceinline__ float cross_rows(float x, Op op) {
    auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return op(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<kQuadXor1>(x));
    x = fmaxf(x, dpp<kQuadXor2>(x));
    x = fmaxf(x, dpp<kHalfMirror>(x));
    x = fmaxf(x, dpp<kRowMirror>(x));
    return cross_rows(x, [](float a, float b) { return fmaxf(a, b); });
}

__device__ __forceinline__ float wave_sum(float x) {
    x += dpp<kQuadXor1>(x);
    x += dpp<kQuadXor2>(x);
    x += dpp<kHalfMirror>(x);
    x += dpp<kRowMirror>(x);
    return cross_rows(x, [](float a, float b) { return a + b; });
}

__device__ __forceinline__ half2_t as_h2(unsigned int u) { return __builtin_bit_cast(half2_t, u); }

// c + a.b over 8 fp16 pairs, fp32 accumulate (v_dot2_f32_f16).
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, float c) {
    c = __builtin_amdgcn_fdot2(as_h2(a.x), as_h2(b.x), c, false);
    c = __builtin_amdgcn_fdot2(as_h2(a.y), as_h2(b.y), c, false);
    c = __builtin_amdgcn_fdot2(as_h2(a.z), as_h2(b.z), c, false);
    c = __builtin_amdgcn_fdot2(as_h2(a.w), as_h2(b.w), c, false);
    return c;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ int clamp_block(int blk, int N) {
    return (unsigned)blk < (unsigned)N ? blk : 0;
}

// Row order of the V loads: register jj of a lane whose token chunk is c
// holds channel rows 8*(jj ^ vrow_twist(c)) + l/8. The twist is linear in c
// with twist(7) = NJ/2, twist(2) = NJ/4, twist(1) = NJ/8, matching the
// partners of the three butterfly steps (lane c^7 by row_half_mirror, c^2 and
// c^1 by quad permutes).
template <int NJ>
__device__ __forceinline__ int vrow_twist(int c) {
    static_assert(NJ == 8 || NJ == 16, "head_dim 64 or 128");
    const int t1 = NJ / 8, t2 = NJ / 4, t4 = (NJ / 2) ^ (NJ / 4) ^ (NJ / 8);
    return ((c & 1) ? t1 : 0) ^ ((c & 2) ? t2 : 0) ^ ((c & 4) ? t4 : 0);
}

// ---------------------------------------------------------------------------
// work decomposition shared by all workgroups of one decode launch
// ---------------------------------------------------------------------------

struct Item {
    int b, g, p, np, chunk, L;
    bool valid;
};

__device__ __forceinline__ int row_len(const int32_t* __restrict__ seq_lens, int b, int cap) {
    int L = seq_lens[b];
    return L < 0 ? 0 : (L > cap ? cap : L);
}

// Every workgroup computes the same decomposition from seq_lens: the tile
// count of all rows, the partition size `chunk` (a multiple of kWaves tiles),
// the prefix sum of partitions per row, and from that its own item.
__device__ Item find_item(const int32_t* __restrict__ seq_lens, int B, int Hkv, int cap, int target_wgs) {
    __shared__ int s_red[kWaves];
    __shared__ int s_item[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (B + kThreads - 1) / kThreads;  // contiguous rows per thread
    const int r0 = tid * per, r1 = min(B, r0 + per);

    if (tid == 0) s_item[0] = -1;  // stays -1 unless some thread owns this item
    int tiles = 0;
    for (int r = r0; r < r1; ++r) tiles += (row_len(seq_lens, r, cap) + kTile - 1) / kTile;
    // block sum of tiles
    int t = tiles;
    for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o);
    if (lane == 0) s_red[wave] = t;
    __syncthreads();
    const int total = (s_red[0] + s_red[1] + s_red[2] + s_red[3]) * Hkv;
    const int tpw = max(1, (total + kWaves * target_wgs - 1) / (kWaves * target_wgs));
    const int chunk = kWaves * tpw;

    int parts = 0;
    for (int r = r0; r < r1; ++r) parts += max(1, ((row_len(seq_lens, r, cap) + kTile - 1) / kTile + chunk - 1) / chunk);
    // inclusive scan of parts over threads
    int incl = parts;
    for (int o = 1; o < 64; o <<= 1) {
        int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
    }
    __syncthreads();  // s_red reuse
    if (lane == 63) s_red[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += s_red[w];
    const int P_total = s_red[0] + s_red[1] + s_red[2] + s_red[3];
    const int excl = before + incl - parts;

    const int item = blockIdx.x;
    Item it;
    it.chunk = chunk;
    it.valid = item < P_total * Hkv;
    if (!it.valid) return it;
    it.g = item / P_total;
    const int r = item - it.g * P_total;
    if (r >= excl && r < excl + parts) {
        int acc = excl;
        for (int row = r0; row < r1; ++row) {
            const int L = row_len(seq_lens, row, cap);
            const int np = max(1, ((L + kTile - 1) / kTile + chunk - 1) / chunk);
            if (r < acc + np) {
                s_item[0] = row;
                s_item[1] = r - acc;
                s_item[2] = np;
                s_item[3] = L;
                break;
            }
            acc += np;
        }
    }
    __syncthreads();
    it.b = uniform(s_item[0]);
    if (it.b < 0 || it.b >= B) {
        it.valid = false;
        return it;
    }
    it.p = uniform(s_item[1]);
    it.np = uniform(s_item[2]);
    it.L = uniform(s_item[3]);
    it.g = uniform(it.g);
    return it;
}

// ---------------------------------------------------------------------------
// decode kernel
// ---------------------------------------------------------------------------

template <int BS, int D, int NREP>
__global__ void __launch_bounds__(kThreads) decode_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ tables, const int32_t* __restrict__ seq_lens,
    int32_t* __restrict__ counters, float* __restrict__ part_ml, float* __restrict__ part_acc, int B, int Hkv,
    int W, int N, int max_parts, int target_wgs, float scale_log2) {
    constexpr int NJ = D / 8;      // 16-byte loads per lane per tile, for K and for V
    constexpr int NR = NJ / 8;     // channel rows per lane after the butterfly
    constexpr int TPB = BS >= kTile ? 1 : kTile / BS;  // blocks per tile
    static_assert(BS % 16 == 0, "block size must be a multiple of 16");

    __shared__ __attribute__((aligned(16))) _Float16 s_p[kWaves][NREP][kTile];
    __shared__ float s_m[kWaves][NREP];
    __shared__ float s_l[kWaves][NREP];
    __shared__ float s_acc[kWaves][NREP][D];
    __shared__ int s_last;
    __shared__ u32x4 s_q[D / 8][NREP];

    const int cap = W * BS;
    const Item it = find_item(seq_lens, B, Hkv, cap, target_wgs);
    if (!it.valid) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int b = it.b, g = it.g, L = it.L;
    const int Hq = Hkv * NREP;
    uint16_t* __restrict__ orow = out + ((size_t)b * Hq + (size_t)g * NREP) * D;

    if (L == 0) {
        for (int o = tid; o < NREP * D; o += kThreads) orow[o] = 0;
        return;
    }

    const int ntiles = (L + kTile - 1) / kTile;
    const int nblk = (L + BS - 1) / BS;
    const int t_begin = it.p * it.chunk;
    const int t_end = min(ntiles, t_begin + it.chunk);
    const int32_t* __restrict__ trow = tables + (size_t)b * W;
    const u32x4* __restrict__ qv = reinterpret_cast<const u32x4*>(q + ((size_t)b * Hq + (size_t)g * NREP) * D);

    const int c = lane & 7;        // token chunk of this lane in the PV layout
    const int drow = lane >> 3;    // channel offset within each group of 8 rows
    const int twist = vrow_twist<NJ>(c);

    // query heads of the group, regrouped as [channel group][head] in LDS
    for (int i = tid; i < NREP * NJ; i += kThreads) s_q[i % NJ][i / NJ] = qv[i];
    __syncthreads();

    float m[NREP], lsum[NREP], acc[NREP][NJ];
#pragma unroll
    for (int h = 0; h < NREP; ++h) {
        m[h] = -INFINITY;
        lsum[h] = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[h][j] = 0.f;
    }

    for (int tile = t_begin + wave; tile < t_end; tile += kWaves) {
        const int t0 = tile * kTile;
        const int tk = t0 + lane;     // token of this lane's K row
        const int tv = t0 + 8 * c;    // first of this lane's 8 V tokens
        u32x4 kr[NJ], vr[NJ];
        // ---- table walk and 16-byte loads of the K and V tiles
        if constexpr (TPB == 1) {
            // the whole tile lies in one block: its id is wave-uniform
            const int phys = uniform(clamp_block(trow[uniform(t0 / BS)], N));
            const uint16_t* kb = k_pool + ((size_t)phys * Hkv + g) * (size_t)(D * BS);
            const uint16_t* vb = v_pool + ((size_t)phys * Hkv + g) * (size_t)(D * BS);
            const uint32_t koff = (uint32_t)((t0 % BS) + lane) * 8;
            const uint32_t voff = (uint32_t)(drow * BS + (t0 % BS) + 8 * c);
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                kr[j] = *reinterpret_cast<const u32x4*>(kb + koff + (uint32_t)(j * BS * 8));
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj)
                vr[jj] = *reinterpret_cast<const u32x4*>(vb + voff + (uint32_t)((jj ^ twist) * 8 * BS));
        } else {
            const int first = t0 / BS;
            int kbi = tk / BS, vbi = tv / BS;
            if (kbi >= nblk) kbi = first;  // never read table entries past the row's last block
            if (vbi >= nblk) vbi = first;
            const int kphys = clamp_block(trow[kbi], N);
            const int vphys = clamp_block(trow[vbi], N);
            const uint16_t* kb = k_pool + ((size_t)kphys * Hkv + g) * (size_t)(D * BS) + (size_t)(tk % BS) * 8;
            const uint16_t* vb = v_pool + ((size_t)vphys * Hkv + g) * (size_t)(D * BS) + (size_t)(drow * BS + tv % BS);
#pragma unroll
            for (int j = 0; j < NJ; ++j) kr[j] = *reinterpret_cast<const u32x4*>(kb + (uint32_t)(j * BS * 8));
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj)
                vr[jj] = *reinterpret_cast<const u32x4*>(vb + (uint32_t)((jj ^ twist) * 8 * BS));
        }

        // ---- scores (lane = token); the query of the group is broadcast from LDS
        float s[NREP];
#pragma unroll
        for (int h = 0; h < NREP; ++h) s[h] = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int h = 0; h < NREP; ++h) s[h] = dot8(s_q[j][h], kr[j], s[h]);
        const bool live = tk < L;
#pragma unroll
        for (int h = 0; h < NREP; ++h) s[h] = live ? s[h] * scale_log2 : -INFINITY;

        // ---- online softmax
        float alpha[NREP];
        bool rescale = false;
#pragma unroll
        for (int h = 0; h < NREP; ++h) {
            const float mt = wave_max(s[h]);
            const float mn = fmaxf(m[h], mt);
            alpha[h] = __builtin_amdgcn_exp2f(m[h] - mn);
            rescale |= alpha[h] != 1.0f;
            m[h] = mn;
            const _Float16 ph = (_Float16)__builtin_amdgcn_exp2f(s[h] - mn);
            lsum[h] = lsum[h] * alpha[h] + (float)ph;
            s_p[wave][h][lane] = ph;
        }
        if (__builtin_amdgcn_readfirstlane((int)rescale)) {
#pragma unroll
            for (int h = 0; h < NREP; ++h)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[h][j] *= alpha[h];
        }
        __builtin_amdgcn_wave_barrier();

        // ---- zero V halves of tokens past the row's end (they may be NaN)
        if (t0 + kTile > L) {
            u32x4 mask;
            const int n = L - tv;  // live tokens among tv .. tv+7
            mask.x = (n > 0 ? 0xffffu : 0u) | (n > 1 ? 0xffff0000u : 0u);
            mask.y = (n > 2 ? 0xffffu : 0u) | (n > 3 ? 0xffff0000u : 0u);
            mask.z = (n > 4 ? 0xffffu : 0u) | (n > 5 ? 0xffff0000u : 0u);
            mask.w = (n > 6 ? 0xffffu : 0u) | (n > 7 ? 0xffff0000u : 0u);
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) vr[jj] &= mask;
        }

        // ---- PV: p for this lane's 8 tokens comes back from LDS, one head at a time
#pragma unroll
        for (int h = 0; h < NREP; ++h) {
            const u32x4 pp = *reinterpret_cast<const u32x4*>(&s_p[wave][h][8 * c]);
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) acc[h][jj] = dot8(pp, vr[jj], acc[h][jj]);
        }
        __builtin_amdgcn_wave_barrier();
    }

    // ---- per-wave epilogue: sums over lanes
#pragma unroll
    for (int h = 0; h < NREP; ++h) lsum[h] = wave_sum(lsum[h]);
#pragma unroll
    for (int h = 0; h < NREP; ++h) {
#pragma unroll
        for (int r = 0; r < NJ / 2; ++r) acc[h][r] += dpp<kHalfMirror>(acc[h][r + NJ / 2]);
#pragma unroll
        for (int r = 0; r < NJ / 4; ++r) acc[h][r] += dpp<kQuadXor2>(acc[h][r + NJ / 4]);
#pragma unroll
        for (int r = 0; r < NJ / 8; ++r) acc[h][r] += dpp<kQuadXor1>(acc[h][r + NJ / 8]);
    }
#pragma unroll
    for (int h = 0; h < NREP; ++h) {
#pragma unroll
        for (int r = 0; r < NR; ++r) s_acc[wave][h][8 * (r ^ twist) + drow] = acc[h][r];
        if (lane == 0) {
            s_m[wave][h] = m[h];
            s_l[wave][h] = lsum[h];
        }
    }
    __syncthreads();

    // ---- merge the 4 waves
    const bool single = it.np == 1;
    const size_t bg = (size_t)b * Hkv + g;
    float* pacc = part_acc + (bg * max_parts + it.p) * (size_t)(NREP * D);
    float* pml = part_ml + (bg * max_parts + it.p) * (size_t)(NREP * 2);
    for (int o = tid; o < NREP * D; o += kThreads) {
        const int h = o / D, d = o % D;
        float M = s_m[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = __builtin_amdgcn_exp2f(s_m[w][h] - M);
            num += f * s_acc[w][h][d];
            den += f * s_l[w][h];
        }
        if (single) {
            orow[o] = __builtin_bit_cast(uint16_t, (_Float16)(num / den));
        } else {
            pacc[o] = num;
            if (d == 0) {
                pml[2 * h] = M;
                pml[2 * h + 1] = den;
            }
        }
    }
    if (single) return;

    // ---- split-sequence reduction: the last partition to arrive merges
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&counters[bg], 1) == it.np - 1;
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const float* acc0 = part_acc + bg * max_parts * (size_t)(NREP * D);
    const float* ml0 = part_ml + bg * max_parts * (size_t)(NREP * 2);
    for (int o = tid; o < NREP * D; o += kThreads) {
        const int h = o / D;
        float M = -INFINITY;
        for (int p = 0; p < it.np; ++p) M = fmaxf(M, ml0[p * NREP * 2 + 2 * h]);
        float num = 0.f, den = 0.f;
        for (int p = 0; p < it.np; ++p) {
            const float f = __builtin_amdgcn_exp2f(ml0[p * NREP * 2 + 2 * h] - M);
            num += f * acc0[p * NREP * D + o];
            den += f * ml0[p * NREP * 2 + 2 * h + 1];
        }
        orow[o] = __builtin_bit_cast(uint16_t, (_Float16)(num / den));
    }
    if (tid == 0) atomicExch(&counters[bg], 0);
}

// ---------------------------------------------------------------------------
// kv_append, gather, workspace fill
// ---------------------------------------------------------------------------

// One wave per (row, KV head): lanes 0..D/8-1 copy the 16-byte K groups,
// every lane copies D/64 (or fewer) V channels.
__global__ void __launch_bounds__(64) append_kernel(const uint16_t* __restrict__ k_new,
                                                    const uint16_t* __restrict__ v_new,
                                                    uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool,
                                                    const int32_t* __restrict__ tables,
                                                    const int32_t* __restrict__ seq_lens, int Hkv, int D, int BS,
                                                    int W, int N) {
    const int bg = blockIdx.x;
    const int b = bg / Hkv, g = bg % Hkv;
    const int L = seq_lens[b];
    if (L < 1 || (long long)L > (long long)W * BS) return;
    const int pos = L - 1;
    const int blk = tables[(size_t)b * W + pos / BS];
    if (blk < 0 || blk >= N) return;
    const int slot = pos % BS;
    const size_t base = (size_t)blk * Hkv + g;
    const uint16_t* ksrc = k_new + ((size_t)b * Hkv + g) * D;
    const uint16_t* vsrc = v_new + ((size_t)b * Hkv + g) * D;
    for (int j = threadIdx.x; j < D / 8; j += 64) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(ksrc + 8 * j);
        *reinterpret_cast<u32x4*>(k_pool + ((base * (D / 8) + j) * BS + slot) * 8) = x;
    }
    for (int d = threadIdx.x; d < D; d += 64) v_pool[(base * D + d) * BS + slot] = vsrc[d];
}

// One workgroup per (row, KV head, logical block); thread per (token, channel).
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

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

typedef void (*DecodeFn)(uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, const int32_t*,
                         const int32_t*, int32_t*, float*, float*, int, int, int, int, int, int, float);

template <int BS, int D>
DecodeFn pick_nrep(int nrep) {
    switch (nrep) {
        case 1: return decode_kernel<BS, D, 1>;
        case 2: return decode_kernel<BS, D, 2>;
        case 4: return decode_kernel<BS, D, 4>;
        case 6: return decode_kernel<BS, D, 6>;
        case 8: return decode_kernel<BS, D, 8>;
        default: return nullptr;
    }
}

template <int BS>
DecodeFn pick_d(int D, int nrep) {
    switch (D) {
        case 64: return pick_nrep<BS, 64>(nrep);
        case 128: return pick_nrep<BS, 128>(nrep);
        default: return nullptr;
    }
}

DecodeFn pick_decode(int bs, int D, int nrep) {
    switch (bs) {
        case 16: return pick_d<16>(D, nrep);
        case 32: return pick_d<32>(D, nrep);
        case 64: return pick_d<64>(D, nrep);
        case 128: return pick_d<128>(D, nrep);
        default: return nullptr;
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int max_parts_for(int bs, int W) {
    const long long tiles = ((long long)W * bs + kTile - 1) / kTile;
    return (int)((tiles + kWaves - 1) / kWaves);
}

size_t counters_bytes(int B, int Hkv) { return (((size_t)B * Hkv * 4) + 255) / 256 * 256; }

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        g_cu_count[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
    switch (status) {
        case PA_OK: return "PA_OK";
        case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG: null pointer, bad size or misaligned buffer";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: block_size/head_dim/group size not compiled in";
        case PA_ERR_HIP: return "PA_ERR_HIP: kernel launch failed";
        case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
        default: return "unknown pa_status";
    }
}

int paged_decode_supported(int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size) {
    if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads) return 0;
    return pick_decode(block_size, head_dim, num_heads / num_kv_heads) != nullptr;
}

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

size_t paged_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t max_blocks_per_seq) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads || head_dim <= 0 ||
        block_size <= 0 || max_blocks_per_seq <= 0)
        return 0;
    const size_t parts = (size_t)max_parts_for(block_size, max_blocks_per_seq);
    const size_t rows = (size_t)(num_seqs > 0 ? num_seqs : 1);
    return counters_bytes((int)rows, num_kv_heads) + rows * parts * (size_t)num_heads * (head_dim + 2) * 4;
}

pa_status paged_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 3u) || workspace_bytes % 4) return PA_ERR_INVALID_ARG;
    const size_t n = workspace_bytes / 4;
    if (n == 0) return PA_OK;
    const unsigned blocks = (unsigned)std::min<size_t>(1024, (n + 255) / 256);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (uint32_t*)workspace, n);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status paged_decode_attn(uint16_t* out, const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                            const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t max_blocks_per_seq, int32_t num_blocks, float scale, void* workspace,
                            size_t workspace_bytes, void* stream) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads || head_dim <= 0 ||
        block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || !std::isfinite(scale))
        return PA_ERR_INVALID_ARG;
    const int nrep = num_heads / num_kv_heads;
    DecodeFn fn = pick_decode(block_size, head_dim, nrep);
    if (!fn) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    if (!out || !q || !k_pool || !v_pool || !block_tables || !seq_lens) return PA_ERR_INVALID_ARG;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_INVALID_ARG;
    if ((long long)max_blocks_per_seq * block_size > 0x7fffffffLL / 2) return PA_ERR_INVALID_ARG;
    const size_t need = paged_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                                    max_blocks_per_seq);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return PA_ERR_WORKSPACE;
    const int max_parts = max_parts_for(block_size, max_blocks_per_seq);
    const int target = 2 * cu_count();
    const long long grid = (long long)target + (long long)num_seqs * num_kv_heads;
    if (grid > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
    char* ws = static_cast<char*>(workspace);
    int32_t* counters = reinterpret_cast<int32_t*>(ws);
    float* part_ml = reinterpret_cast<float*>(ws + counters_bytes(num_seqs, num_kv_heads));
    float* part_acc = part_ml + (size_t)num_seqs * max_parts * num_heads * 2;
    const float scale_log2 = scale * 1.4426950408889634f;
    int W = max_blocks_per_seq, Hkv = num_kv_heads, B = num_seqs, N = num_blocks;
    float sl2 = scale_log2;
    void* args[] = {&out, (void*)&q, (void*)&k_pool, (void*)&v_pool, (void*)&block_tables, (void*)&seq_lens,
                    &counters, &part_ml, &part_acc, &B, &Hkv, &W, &N, (void*)&max_parts, (void*)&target, &sl2};
    if (hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)grid), dim3(kThreads), args, 0,
                        (hipStream_t)stream) != hipSuccess)
        return PA_ERR_HIP;
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
