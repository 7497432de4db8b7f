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
#include <type_traits>
#include <utility>

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

// Scores of one 16-byte K chunk (channel pairs 4j..4j+3) against HPW query
// heads: a[k][h] += q_h[pair 4j+k] . k[pair k], the query pair taken from
// lane L0+k of this lane's 16-lane row by DPP row_newbcast. The compiler
// cannot see inside the asm, so the block carries its own wait states: two
// before it (a VALU result read by a DPP instruction) and three after it (a
// dot result read by a different VALU instruction). Within a block every
// accumulator is written once, so the dots need no spacing between them.
template <int L0>
__device__ __forceinline__ void score_block(float (&a)[4][1], const unsigned (&q)[1], const u32x4& k) {
    asm("s_nop 1\n\t"
        "v_dot2c_f32_f16_dpp %0, %4, %5 row_newbcast:%9 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %1, %4, %6 row_newbcast:%10 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %2, %4, %7 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %3, %4, %8 row_newbcast:%12 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 2\n\t"
        : "+v"(a[0][0]), "+v"(a[1][0]), "+v"(a[2][0]), "+v"(a[3][0])
        : "v"(q[0]), "v"(k.x), "v"(k.y), "v"(k.z), "v"(k.w), "n"(L0), "n"(L0 + 1), "n"(L0 + 2), "n"(L0 + 3));
}
template <int L0>
__device__ __forceinline__ void score_block(float (&a)[4][2], const unsigned (&q)[2], const u32x4& k) {
    asm("s_nop 1\n\t"
        "v_dot2c_f32_f16_dpp %0, %8, %10 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %1, %9, %10 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %2, %8, %11 row_newbcast:%15 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %3, %9, %11 row_newbcast:%15 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %4, %8, %12 row_newbcast:%16 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %5, %9, %12 row_newbcast:%16 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %6, %8, %13 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %7, %9, %13 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 2\n\t"
        : "+v"(a[0][0]), "+v"(a[0][1]), "+v"(a[1][0]), "+v"(a[1][1]), "+v"(a[2][0]), "+v"(a[2][1]), "+v"(a[3][0]), "+v"(a[3][1])
        : "v"(q[0]), "v"(q[1]), "v"(k.x), "v"(k.y), "v"(k.z), "v"(k.w), "n"(L0), "n"(L0 + 1), "n"(L0 + 2), "n"(L0 + 3));
}
template <int L0>
__device__ __forceinline__ void score_block(float (&a)[4][3], const unsigned (&q)[3], const u32x4& k) {
    asm("s_nop 1\n\t"
        "v_dot2c_f32_f16_dpp %0, %12, %15 row_newbcast:%19 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %1, %13, %15 row_newbcast:%19 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %2, %14, %15 row_newbcast:%19 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %3, %12, %16 row_newbcast:%20 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %4, %13, %16 row_newbcast:%20 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %5, %14, %16 row_newbcast:%20 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %6, %12, %17 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %7, %13, %17 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %8, %14, %17 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %9, %12, %18 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %10, %13, %18 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %11, %14, %18 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 2\n\t"
        : "+v"(a[0][0]), "+v"(a[0][1]), "+v"(a[0][2]), "+v"(a[1][0]), "+v"(a[1][1]), "+v"(a[1][2]), "+v"(a[2][0]), "+v"(a[2][1]), "+v"(a[2][2]), "+v"(a[3][0]), "+v"(a[3][1]), "+v"(a[3][2])
        : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(k.x), "v"(k.y), "v"(k.z), "v"(k.w), "n"(L0), "n"(L0 + 1), "n"(L0 + 2), "n"(L0 + 3));
}
template <int L0>
__device__ __forceinline__ void score_block(float (&a)[4][4], const unsigned (&q)[4], const u32x4& k) {
    asm("s_nop 1\n\t"
        "v_dot2c_f32_f16_dpp %0, %16, %20 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %1, %17, %20 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %2, %18, %20 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %3, %19, %20 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %4, %16, %21 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %5, %17, %21 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %6, %18, %21 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %7, %19, %21 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %8, %16, %22 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %9, %17, %22 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %10, %18, %22 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %11, %19, %22 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %12, %16, %23 row_newbcast:%27 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %13, %17, %23 row_newbcast:%27 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %14, %18, %23 row_newbcast:%27 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %15, %19, %23 row_newbcast:%27 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 2\n\t"
        : "+v"(a[0][0]), "+v"(a[0][1]), "+v"(a[0][2]), "+v"(a[0][3]), "+v"(a[1][0]), "+v"(a[1][1]), "+v"(a[1][2]), "+v"(a[1][3]), "+v"(a[2][0]), "+v"(a[2][1]), "+v"(a[2][2]), "+v"(a[2][3]), "+v"(a[3][0]), "+v"(a[3][1]), "+v"(a[3][2]), "+v"(a[3][3])
        : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(k.x), "v"(k.y), "v"(k.z), "v"(k.w), "n"(L0), "n"(L0 + 1), "n"(L0 + 2), "n"(L0 + 3));
}

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

// Relaxed agent-scope atomic accesses compile to plain global loads/stores
// with the sc1 bit: coherent across the GPU's L2 slices without a cache
// writeback or invalidate. The split-sequence partials travel this way.
__device__ __forceinline__ void store_coherent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kMaxSplit = 16;  // partitions per (row, KV head), hard cap

// ---------------------------------------------------------------------------
// decode kernel
// ---------------------------------------------------------------------------

// s_waitcnt immediate that waits until at most `n` vector-memory operations of
// this wave are outstanding and does not wait on LDS/scalar or export counts
// (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int n>
__device__ __forceinline__ void wait_vmem() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) alone: this wave's LDS (and scalar) accesses are done.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

typedef __attribute__((address_space(3))) void* lds_ptr;

// Workgroup barrier without a memory fence. Inside the tile loop the only
// data shared between waves are tiles written by direct-to-LDS loads, whose
// completion each wave establishes itself with wait_vmem before arriving; a
// fenced __syncthreads would also wait for the next tile's loads, which must
// stay in flight. The signal fences keep the compiler from moving LDS
// accesses across the barrier.
__device__ __forceinline__ void tile_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One 16-byte load per lane from global memory straight into LDS: lane i's
// bytes land at dst + 16*i (dst is wave-uniform).
__device__ __forceinline__ void load16_to_lds(const void* src, void* dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_ptr)dst, 16, 0, 0);
}

// Work item of a workgroup: (row b, KV head g, partition p) straight from the
// block index. Partition p covers tiles [p*chunk, (p+1)*chunk) of the row;
// `chunk` and the partition count `parts` are fixed by the host from the
// table width, so a workgroup knows its tiles without reading any length.
// Partitions that start past the row's end exit at once.
//
// Each tile stream of the workgroup (a pair of waves, or one wave when the
// group has an odd number of query heads) owns an LDS K buffer and an LDS V
// buffer holding the 64-token tile it is computing on; both waves of a pair
// read the shared copy, each for its half of the query heads. The next tile
// is requested into registers at the top of an iteration, every wave loading
// its half with 16-byte loads, and written into the LDS buffers at the bottom,
// after the current tile is consumed:
//   request tile i+1 -> barrier -> scores, softmax, PV on tile i -> barrier
//   -> wait for tile i+1, write it to LDS
// So a tile is always in flight while the previous one is computed, held in
// the register file, whose capacity (not the LDS's) then bounds the bytes in
// flight per compute unit. The first tile goes straight into LDS.
template <int BS, int D, int NREP>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) decode_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ tables, const int32_t* __restrict__ seq_lens,
    int32_t* __restrict__ counters, float* __restrict__ part_ml, float* __restrict__ part_acc, int Hkv, int W,
    int N, int chunk, int parts, float scale_log2) {
    constexpr int NJ = D / 8;                       // 1 KiB load instructions per K (and per V) tile
    constexpr int WPT = (NREP % 2 == 0) ? 2 : 1;   // waves sharing one tile, each with part of the heads
    constexpr int HPW = NREP / WPT;                 // query heads per wave
    constexpr int TS = kWaves / WPT;                // tile streams per workgroup
    constexpr int LPW = NJ / WPT;                   // load instructions per wave per K (or V) tile
    constexpr int TPB = BS >= kTile ? 1 : kTile / BS;  // blocks per tile
    constexpr int TILE = kTile * D;                 // halves per K (or V) tile
    static_assert(BS % 16 == 0, "block size must be a multiple of 16");

    __shared__ __attribute__((aligned(16))) uint16_t s_kv[TS][2][TILE];
    __shared__ __attribute__((aligned(16))) _Float16 s_p[kWaves][HPW][kTile];
    __shared__ float s_m[TS][NREP];
    __shared__ float s_l[TS][NREP];
    __shared__ float s_w[kMaxSplit][NREP];
    __shared__ float s_pm[kMaxSplit][NREP];
    __shared__ float s_pl[kMaxSplit][NREP];
    __shared__ float s_den[NREP];
    __shared__ int s_last;
    // after the tile loop the tile buffers hold the per-stream partial outputs
    float(*s_acc)[NREP][D] = reinterpret_cast<float(*)[NREP][D]>(&s_kv[0][0][0]);
    static_assert(sizeof(float) * TS * NREP * D <= sizeof(uint16_t) * TS * 2 * TILE, "s_acc alias");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int stream = wave / WPT;        // which tiles this wave walks
    const int wip = wave % WPT;           // position of the wave in its pair
    const int h0 = wip * HPW;             // its first query head within the group
    const int bg = blockIdx.x / parts;
    const int p = blockIdx.x - bg * parts;
    const int b = bg / Hkv, g = bg - b * Hkv;
    const int Hq = Hkv * NREP;
    const int cap = W * BS;
    const int wtiles = (cap + kTile - 1) / kTile;
    const int t_begin = p * chunk;
    const int32_t* __restrict__ trow = tables + (size_t)b * W;
    uint16_t* __restrict__ orow = out + ((size_t)b * Hq + (size_t)g * NREP) * D;
    const u32x4* __restrict__ qv = reinterpret_cast<const u32x4*>(q + ((size_t)b * Hq + (size_t)g * NREP) * D);
    const int c = lane & 7;        // token chunk of this lane in the V layout
    const int drow = lane >> 3;    // channel row offset within each group of 8
    uint16_t* kbuf = &s_kv[stream][0][0];
    uint16_t* vbuf = &s_kv[stream][1][0];

    // table entries of a tile: the block of this lane's K token and of its V
    // chunk. A block past the row's last block is replaced by the tile's first
    // block (its values are masked), so no unlisted entry is ever used.
    auto k_block = [&](int t) { return TPB == 1 ? (t * kTile) / BS : (t * kTile + lane) / BS; };
    auto v_block = [&](int t) { return (t * kTile + 8 * c) / BS; };

    // ---- one round trip: the row's length, the query, the first table entry
    int tile0 = t_begin + stream;
    int kent = 0, vent = 0;
    if (tile0 < wtiles) {  // inside the table row; used only if the tile is live
        kent = TPB == 1 ? uniform(trow[k_block(tile0)]) : trow[min(k_block(tile0), W - 1)];
        if constexpr (TPB > 1) vent = trow[min(v_block(tile0), W - 1)];
    }
    // this wave's query heads: pair p of head h at lane p % 16 (every row) of qr[h][p / 16]
    constexpr int QR = NJ / 4;
    unsigned qr[HPW][QR];
    {
        const unsigned* qw = reinterpret_cast<const unsigned*>(qv) + (size_t)h0 * (D / 2);
#pragma unroll
        for (int h = 0; h < HPW; ++h)
#pragma unroll
            for (int i = 0; i < QR; ++i) qr[h][i] = qw[h * (D / 2) + 16 * i + (lane & 15)];
    }
    int L = seq_lens[b];
    L = uniform(L < 0 ? 0 : (L > cap ? cap : L));
    const int ntiles = (L + kTile - 1) / kTile;
    if (t_begin >= ntiles && !(L == 0 && p == 0)) return;  // partition past the row's end
    if (L == 0) {
        for (int o = tid; o < NREP * D; o += kThreads) orow[o] = 0;
        return;
    }
    const int nblk = (L + BS - 1) / BS;
    const int t_end = min(ntiles, t_begin + chunk);
    const int np = (ntiles + chunk - 1) / chunk;  // live partitions of this row
    const int n_iter = (t_end - t_begin + TS - 1) / TS;

    auto fix_entries = [&](int t, int& ke, int& ve) {
        if constexpr (TPB > 1) {
            const int first = (t * kTile) / BS;
            if (k_block(t) >= nblk) ke = trow[first];
            if (v_block(t) >= nblk) ve = trow[first];
        }
    };
    auto next_entries = [&](int t, int& ke, int& ve) {
        if constexpr (TPB == 1) {
            ke = uniform(trow[k_block(t)]);
        } else {
            const int first = (t * kTile) / BS;
            ke = trow[k_block(t) < nblk ? k_block(t) : first];
            ve = trow[v_block(t) < nblk ? v_block(t) : first];
        }
    };
    // This wave's half of a tile's 16-byte loads, straight into LDS.
    auto issue_k = [&](int t, int ent) {
        const int phys = clamp_block(ent, N);
        const uint16_t* src = k_pool + ((size_t)phys * Hkv + g) * (size_t)(D * BS) +
                              (size_t)((t * kTile + lane) % BS) * 8;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int j = i * WPT + wip;
            load16_to_lds(src + (size_t)j * (BS * 8), kbuf + j * (kTile * 8));
        }
    };
    auto issue_v = [&](int t, int ent) {
        const int phys = clamp_block(ent, N);
        const uint16_t* src = v_pool + ((size_t)phys * Hkv + g) * (size_t)(D * BS) +
                              (size_t)(drow * BS + (t * kTile + 8 * c) % BS);
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int jj = i * WPT + wip;
            load16_to_lds(src + (size_t)jj * (8 * BS), vbuf + jj * (kTile * 8));
        }
    };


    float m[HPW], lsum[HPW], acc[HPW][NJ];
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        m[h] = -INFINITY;
        lsum[h] = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[h][j] = 0.f;
    }

    // The query registers must have landed before any tile load is in flight,
    // so the compiler never has to wait for those loads to read them.
    wait_vmem<0>();
    if (tile0 < t_end) {
        fix_entries(tile0, kent, vent);
        issue_k(tile0, kent);
        issue_v(tile0, TPB == 1 ? kent : vent);
    }
    // entries of the next tile of this stream
    int kent_n = 0, vent_n = 0;
    if (tile0 + TS < t_end) next_entries(tile0 + TS, kent_n, vent_n);

    for (int it = 0; it < n_iter; ++it) {
        const int tile = tile0 + it * TS;
        const int t0 = tile * kTile;
        const bool act = tile < t_end;             // this stream has a tile in this round
        const bool more = tile + TS < t_end;       // ... and another after it
        if (it == 0) {
            wait_vmem<0>();                        // the first tile, loaded straight into LDS
        } else {
            wait_lds();  // this wave's LDS writes of the tile
        }
        // ---- request the next tile into registers (this wave's half of its loads)
        u32x4 kst[LPW], vst[LPW];
        if (more) {
            const int nt = tile + TS;
            const int kphys = clamp_block(kent_n, N);
            const int vphys = clamp_block(TPB == 1 ? kent_n : vent_n, N);
            const uint16_t* ksrc = k_pool + ((size_t)(TPB == 1 ? uniform(kphys) : kphys) * Hkv + g) * (size_t)(D * BS) +
                                   (size_t)((nt * kTile + lane) % BS) * 8;
            const uint16_t* vsrc = v_pool + ((size_t)(TPB == 1 ? uniform(vphys) : vphys) * Hkv + g) * (size_t)(D * BS) +
                                   (size_t)(drow * BS + (nt * kTile + 8 * c) % BS);
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                const int j = i * WPT + wip;
                kst[i] = *reinterpret_cast<const u32x4*>(ksrc + (size_t)j * (BS * 8));
            }
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                const int jj = i * WPT + wip;
                vst[i] = *reinterpret_cast<const u32x4*>(vsrc + (size_t)jj * (8 * BS));
            }
            if (tile + 2 * TS < t_end) next_entries(tile + 2 * TS, kent_n, vent_n);
        }
        tile_barrier();  // tile i is in LDS for both waves of every pair

        if (act) {
            // ---- scores: lane = token, query pairs broadcast across lanes by DPP
            float s[HPW];
            u32x4 kj[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) kj[j] = *reinterpret_cast<const u32x4*>(kbuf + j * (kTile * 8) + lane * 8);
            float a4[4][HPW];
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int h = 0; h < HPW; ++h) a4[k][h] = 0.f;
            [&]<int... J>(std::integer_sequence<int, J...>) {
                ([&] {
                    unsigned qj[HPW];
#pragma unroll
                    for (int h = 0; h < HPW; ++h) qj[h] = qr[h][J / 4];
                    score_block<4 * (J % 4)>(a4, qj, kj[J]);
                }(), ...);
            }(std::make_integer_sequence<int, NJ>{});
#pragma unroll
            for (int h = 0; h < HPW; ++h) s[h] = (a4[0][h] + a4[1][h]) + (a4[2][h] + a4[3][h]);
            const bool live = t0 + lane < L;
#pragma unroll
            for (int h = 0; h < HPW; ++h) s[h] = live ? s[h] * scale_log2 : -INFINITY;
            // ---- online softmax
            float alpha[HPW];
            bool rescale = false;
#pragma unroll
            for (int h = 0; h < HPW; ++h) {
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
                for (int h = 0; h < HPW; ++h)
#pragma unroll
                    for (int j = 0; j < NJ; ++j) acc[h][j] *= alpha[h];
            }
            __builtin_amdgcn_wave_barrier();
            // ---- PV: p of this lane's 8 tokens, V of its 8 tokens and channel rows
            u32x4 mask = {~0u, ~0u, ~0u, ~0u};
            if (t0 + kTile > L) {  // tokens past the row's end may hold NaN
                const int n = L - (t0 + 8 * c);
                mask.x = (n > 0 ? 0xffffu : 0u) | (n > 1 ? 0xffff0000u : 0u);
                mask.y = (n > 2 ? 0xffffu : 0u) | (n > 3 ? 0xffff0000u : 0u);
                mask.z = (n > 4 ? 0xffffu : 0u) | (n > 5 ? 0xffff0000u : 0u);
                mask.w = (n > 6 ? 0xffffu : 0u) | (n > 7 ? 0xffff0000u : 0u);
            }
            u32x4 pp[HPW];
#pragma unroll
            for (int h = 0; h < HPW; ++h) pp[h] = *reinterpret_cast<const u32x4*>(&s_p[wave][h][8 * c]);
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) {
                const u32x4 vj = *reinterpret_cast<const u32x4*>(vbuf + jj * (kTile * 8) + lane * 8) & mask;
#pragma unroll
                for (int h = 0; h < HPW; ++h) acc[h][jj] = dot8(pp[h], vj, acc[h][jj]);
            }
        }
        tile_barrier();  // every wave is done reading tile i
        if (more) {
            // ---- tile i+1 into the LDS buffers (the compiler waits for the loads)
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                const int j = i * WPT + wip;
                *reinterpret_cast<u32x4*>(kbuf + j * (kTile * 8) + lane * 8) = kst[i];
                *reinterpret_cast<u32x4*>(vbuf + j * (kTile * 8) + lane * 8) = vst[i];
            }
        }
    }

    // ---- per-wave epilogue: l over all lanes, acc over the 8 lanes of a channel row
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        lsum[h] = wave_sum(lsum[h]);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            float x = acc[h][j];
            x += dpp<kQuadXor1>(x);
            x += dpp<kQuadXor2>(x);
            x += dpp<kHalfMirror>(x);
            acc[h][j] = x;
        }
    }
    // (the last loop barrier guarantees the tile buffers are no longer read)
    if (c == 0) {
#pragma unroll
        for (int h = 0; h < HPW; ++h)
#pragma unroll
            for (int j = 0; j < NJ; ++j) s_acc[stream][h0 + h][8 * j + drow] = acc[h][j];
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
            s_m[stream][h0 + h] = m[h];
            s_l[stream][h0 + h] = lsum[h];
        }
    }
    __syncthreads();

    // ---- merge the tile streams of this workgroup
    const bool single = np == 1;
    float* pacc = part_acc + ((size_t)bg * parts + p) * (size_t)(NREP * D);
    float* pml = part_ml + ((size_t)bg * parts + p) * (size_t)(NREP * 2);
    for (int o = tid; o < NREP * D; o += kThreads) {
        const int h = o / D, d = o % D;
        float M = s_m[0][h];
#pragma unroll
        for (int w = 1; w < TS; ++w) M = fmaxf(M, s_m[w][h]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < TS; ++w) {
            const float f = __builtin_amdgcn_exp2f(s_m[w][h] - M);
            num += f * s_acc[w][h][d];
            den += f * s_l[w][h];
        }
        if (single) {
            orow[o] = __builtin_bit_cast(uint16_t, (_Float16)(num / den));
        } else {
            store_coherent(pacc + o, num);
            if (d == 0) {
                store_coherent(pml + 2 * h, M);
                store_coherent(pml + 2 * h + 1, den);
            }
        }
    }
    if (single) return;

    // ---- split-sequence reduction: the last partition to arrive merges all
    // partitions in partition order. Partials were written coherently; the
    // wait makes them complete before this workgroup's ticket is taken.
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (tid == 0)
        s_last = __hip_atomic_fetch_add(&counters[bg], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == np - 1;
    __syncthreads();
    if (!s_last) return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const float* acc0 = part_acc + (size_t)bg * parts * (size_t)(NREP * D);
    const float* ml0 = part_ml + (size_t)bg * parts * (size_t)(NREP * 2);
    // every partial is requested at once: one round trip, not one per partition
    for (int e = tid; e < np * NREP; e += kThreads) {
        const int pp = e / NREP, h = e - pp * NREP;
        s_pm[pp][h] = load_coherent(ml0 + pp * NREP * 2 + 2 * h);
        s_pl[pp][h] = load_coherent(ml0 + pp * NREP * 2 + 2 * h + 1);
    }
    constexpr int OPT = (NREP * D + kThreads - 1) / kThreads;  // outputs per thread
    float part[OPT][kMaxSplit];
#pragma unroll
    for (int i = 0; i < OPT; ++i) {
        const int o = tid + i * kThreads;
        const int oc = o < NREP * D ? o : 0;
#pragma unroll
        for (int pp = 0; pp < kMaxSplit; ++pp)  // partitions past np re-read the last one (unused)
            part[i][pp] = load_coherent(acc0 + (pp < np ? pp : np - 1) * NREP * D + oc);
    }
    __syncthreads();
    if (tid < NREP) {
        const int h = tid;
        float M = -INFINITY;
        for (int pp = 0; pp < np; ++pp) M = fmaxf(M, s_pm[pp][h]);
        float den = 0.f;
        for (int pp = 0; pp < np; ++pp) {
            const float f = __builtin_amdgcn_exp2f(s_pm[pp][h] - M);
            s_w[pp][h] = f;
            den += f * s_pl[pp][h];
        }
        s_den[h] = den;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < OPT; ++i) {
        const int o = tid + i * kThreads;
        if (o >= NREP * D) break;
        const int h = o / D;
        float num = 0.f;
#pragma unroll
        for (int pp = 0; pp < kMaxSplit; ++pp)
            if (pp < np) num += s_w[pp][h] * part[i][pp];
        orow[o] = __builtin_bit_cast(uint16_t, (_Float16)(num / s_den[h]));
    }
    if (tid == 0) __hip_atomic_store(&counters[bg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
                         const int32_t*, int32_t*, float*, float*, int, int, int, int, int, float);

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

// Partitions per (row, KV head) the workspace must hold: a partition has at
// least two tiles (one per tile stream of a workgroup) and there are never
// more than kMaxSplit of them.
int max_parts_for(int bs, int W) {
    const long long tiles = ((long long)W * bs + kTile - 1) / kTile;
    return (int)std::min<long long>(kMaxSplit, (tiles + 1) / 2);
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
    // Partition plan, fixed from the table width: tiles of 64 tokens, `chunk`
    // tiles per partition (a multiple of the workgroup's tile streams), sized
    // so that B*Hkv*parts workgroups give about two per compute unit, with at
    // most kMaxSplit partitions per row.
    const int ts = (nrep % 2 == 0) ? kWaves / 2 : kWaves;
    const long long wtiles = ((long long)max_blocks_per_seq * block_size + kTile - 1) / kTile;
    const long long target = 2LL * cu_count();
    const long long rows = (long long)num_seqs * num_kv_heads;
    long long tpw = std::max(1LL, (rows * wtiles + ts * target - 1) / (ts * target));
    long long chunk = ts * tpw;
    long long parts = (wtiles + chunk - 1) / chunk;
    if (parts > kMaxSplit) {
        const long long need = (wtiles + kMaxSplit - 1) / kMaxSplit;
        chunk = ((need + ts - 1) / ts) * ts;
        parts = (wtiles + chunk - 1) / chunk;
    }
    const long long grid = rows * parts;
    if (grid > 0x7fffffffLL || parts > max_parts_for(block_size, max_blocks_per_seq)) return PA_ERR_INVALID_ARG;
    const int max_parts = max_parts_for(block_size, max_blocks_per_seq);
    char* ws = static_cast<char*>(workspace);
    int32_t* counters = reinterpret_cast<int32_t*>(ws);
    float* part_ml = reinterpret_cast<float*>(ws + counters_bytes(num_seqs, num_kv_heads));
    float* part_acc = part_ml + (size_t)num_seqs * max_parts * num_heads * 2;
    int Hkv = num_kv_heads, W = max_blocks_per_seq, N = num_blocks, ck = (int)chunk, np = (int)parts;
    float sl2 = scale * 1.4426950408889634f;
    void* args[] = {&out, (void*)&q, (void*)&k_pool, (void*)&v_pool, (void*)&block_tables, (void*)&seq_lens,
                    &counters, &part_ml, &part_acc, &Hkv, &W, &N, &ck, &np, &sl2};
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
