// decode_kernel.h: the paged decode attention kernel and its launch table,
// included by the translation units that instantiate it (pagedattn.hip: fp16
// pools; pagedattn_fp8.hip: E4M3 pools). Internal to libpagedattn; the C ABI
// is include/pagedattn.h.
//
// Sources (page title, section):
//   [Paged attention]     danielfleming.xyz/writing/inference/paged
//   [PagedAttention]      deepconcepts.dev/c/llm-paged-attention
//   [SLM paged attention] aicassindra.com/blogs/slm/slm_paged_attention.html

// decode_kernel: one query token per row; the row's block table is walked,
// its blocks gathered at its own length [Paged attention, "What changed";
// PagedAttention, "What the block table costs"], and softmax attention
// computed for the query heads of one KV group at once; long rows are split
// over workgroups and their partial results merged exactly [PagedAttention,
// "Sharing is the part that pays twice"]. With k_new / v_new it also performs
// the step's kv_append [SLM paged attention, "End-to-end flow"]. Pools hold
// fp16 or E4M3 (FP8) elements (template argument F8); E4M3 tiles are widened
// to fp16 in registers as they are used, exactly, and the pool's K and V
// scales are folded into the score scale and the output.
//
// Both products of a tile run on the matrix cores (16x16x32 fp16, fp32
// accumulate) with the group's query heads as the 16-wide side: scores as
// K.Q^T, one 16-token block per product, and the output as V^T.P^T, 32
// tokens per product. The kernel stays bound by HBM bandwidth; the matrix
// cores take the instruction issue of the products off the vector ALU, so the
// compute waves keep pace with the loads at a fraction of a tile's load time.
// The design (persistent workgroups over balanced tile ranges, a load wave
// issuing direct-to-LDS loads, two compute waves splitting each tile's tokens,
// the merge by the last partition to arrive) is described above decode_kernel.
//
// Stale slots and unlisted blocks may hold NaN: scores of tokens past the
// row's length are replaced (not multiplied) by -inf, and their V values are
// zeroed before the products (fp16: in registers; E4M3: in LDS, by the load
// wave, and in registers).

#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <type_traits>
#include <utility>

#include "e4m3.h"

namespace pa_detail {

// A decode kernel instance and its workgroup size.
struct DecodeFn {
    const void* fn;
    int threads;
    explicit operator bool() const { return fn != nullptr; }
};

// The E4M3-pool instances live in their own translation unit.
DecodeFn pick_decode_fp8(int bs, int D, int nrep);

}  // namespace pa_detail

namespace {

using pa_detail::DecodeFn;

// Tokens per tile: 64 for fp16 pools, 128 for E4M3 pools, so that a tile is
// 16 KiB of K and 16 KiB of V at head_dim 128 in either format (the bytes a
// workgroup keeps in flight set its share of the bandwidth). The load wave
// moves K one token per lane for each 64-token half of a tile.
constexpr int tile_tokens(bool f8) { return f8 ? 128 : 64; }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// wave-level helpers
// ---------------------------------------------------------------------------

// Combine lanes i and i^16, then i and i^32, with the gfx950 permlane swaps.
template <class Op>
__device__ __forceinline__ float cross_rows(float x, Op op) {
    auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return op(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Two E4M3 bytes of w (bytes 0-1, or 2-3 with HI) as an fp16 pair, first
// byte in the low half: exact, every E4M3 value is an fp16 value (the
// converter's scale operand is 1). NaN codes give NaN.
template <bool HI>
__device__ __forceinline__ unsigned f8x2(unsigned w) {
    return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}
// Half H (bytes 8H..8H+7) of a 16-byte chunk of E4M3 values as 8 fp16.
template <int H>
__device__ __forceinline__ u32x4 widen8(const u32x4& r) {
    const unsigned a = H ? r.z : r.x, b = H ? r.w : r.y;
    return u32x4{f8x2<false>(a), f8x2<true>(a), f8x2<false>(b), f8x2<true>(b)};
}
// Mask that keeps the first n (0..16 after clamping) bytes of a 16-byte chunk.
__device__ __forceinline__ u32x4 keep_first_bytes(int n) {
    auto word = [n](int w) {
        const int k = n - 4 * w;  // bytes of this word to keep
        return k >= 4 ? 0xffffffffu : (k <= 0 ? 0u : (1u << (8 * k)) - 1u);
    };
    return u32x4{word(0), word(1), word(2), word(3)};
}

// ---------------------------------------------------------------------------
// matrix-core helpers
// ---------------------------------------------------------------------------

// v_mfma_f32_16x16x32_f16, C += A.B with A 16x32, B 32x16, fp32 accumulate.
// Operands as 8 fp16 per lane: lane l holds A[l%16][8(l/16) .. 8(l/16)+7]
// and B[8(l/16) .. 8(l/16)+7][l%16]; result element i of lane l is
// C[4(l/16)+i][l%16].
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c,
                                                  0, 0, 0);
}
// fp16 ones in every operand slot (0x3c00 = 1.0)
constexpr u32x4 kOnes = {0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};
__device__ __forceinline__ unsigned pack_h2(_Float16 lo, _Float16 hi) {
    return (unsigned)__builtin_bit_cast(uint16_t, lo) | ((unsigned)__builtin_bit_cast(uint16_t, hi) << 16);
}
// Mask of the fp16 pair (first, first+1) of a run whose first n values are kept.
__device__ __forceinline__ unsigned keep2(int n, int first) {
    return (n > first ? 0xffffu : 0u) | (n > first + 1 ? 0xffff0000u : 0u);
}

// ---------------------------------------------------------------------------
// memory helpers
// ---------------------------------------------------------------------------

// s_waitcnt immediate that waits until at most `n` vector-memory operations of
// this wave are outstanding and does not wait on LDS/scalar or export counts
// (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int n>
__device__ __forceinline__ void wait_vmem() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The same with a wave-uniform run-time count (a scalar branch tree over the
// immediate forms). Counts above 63 wait for 63, which is stricter.
template <int LO, int HI>
__device__ __forceinline__ void wait_vmem_range(int n) {
    if constexpr (LO == HI) {
        wait_vmem<LO>();
    } else {
        constexpr int MID = (LO + HI) / 2;
        if (n <= MID)
            wait_vmem_range<LO, MID>(n);
        else
            wait_vmem_range<MID + 1, HI>(n);
    }
}
__device__ __forceinline__ void wait_vmem_dyn(int n) { wait_vmem_range<0, 63>(n < 0 ? 0 : (n > 63 ? 63 : n)); }

typedef __attribute__((address_space(3))) void* lds_ptr;

// Workgroup barrier without a memory fence. Inside the tile loop the only
// data shared between waves are tiles written by direct-to-LDS loads, whose
// completion each wave establishes itself with a vmcnt wait before arriving;
// a fenced __syncthreads would also wait for the next tiles' loads, which
// must stay in flight. The signal fences keep the compiler from moving LDS
// accesses across the barrier.
__device__ __forceinline__ void tile_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait for this wave's LDS operations only (lgkmcnt 0; vector-memory and
// export counts left alone), before a barrier that publishes LDS writes.
__device__ __forceinline__ void wait_lds() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((unsigned)reinterpret_cast<size_t>((lds_ptr)p));
}

// The tile loop's vector-memory instructions are all issued from inline
// assembly, so that the wave itself knows exactly how many are in flight: the
// waits for a tile are counted from that (vm_count in the kernel), and the
// compiler, which cannot see these instructions, inserts no waits of its own
// for them. (Vector-memory operations of a wave complete in issue order on
// this architecture, loads and stores alike, so "at most n outstanding"
// means "everything issued before the last n has completed".)

// One 16-byte load per lane from global memory straight into LDS: lane i's
// bytes land at dst + 16*i (dst wave-uniform, passed in M0). One wait state
// separates the compiler's write of M0 from the load that reads it.
__device__ __forceinline__ void dma16(const void* src, unsigned dst) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(dst) : "memory");
}
// The same with the non-temporal (streaming) cache policy, for the K/V tiles,
// which a launch reads once: measured 9 % faster at uniform 4096 (134 MB per
// launch), 7 % on the 95-row pool, 4 % at uniform 1024; ~1 % slower on the
// 28-layer step, whose rows that share a prefix re-read its blocks.
__device__ __forceinline__ void dma16_nt(const void* src, unsigned dst) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "{m0}"(dst) : "memory");
}
// Device-coherent (sc1) stores of the split-sequence partials.
__device__ __forceinline__ void st_f32x4_sc1(float* p, f32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void st_2f32_sc1(float* p, float a, float b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    f32x2 v = {a, b};
    asm volatile("global_store_dwordx2 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
// Device-coherent (sc1) loads of the partials for the merge: buffer loads
// over one (row, KV head)'s partials, cache policy sc1 (the same coherence as
// a relaxed agent-scope atomic load), 8 or 16 bytes per lane.
constexpr int kCoherent = 16;                     // cache-policy bits: sc1
constexpr int kRawBufferFormat = 0x00020000;      // dword3 of a raw 32-bit buffer resource
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Stores of the output and of the fused append's new K/V: written through
// (sc1) like the partials, so that the launch leaves no dirty L2 lines for the
// release at its end to write back (measured 0.2-0.3 us faster at uniform
// 1024 and on the mixed batch, ~0.2 us slower on the 95-row pool with
// 16-token blocks).
__device__ __forceinline__ void st_b64(void* p, unsigned lo, unsigned hi) {
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    u32x2 v = {lo, hi};
    asm volatile("global_store_dwordx2 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void st_u16(uint16_t* p, uint16_t v) {
    asm volatile("global_store_short %0, %1, off sc1" ::"v"(p), "v"((unsigned)v) : "memory");
}
__device__ __forceinline__ void st_b128(void* p, u32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void st_u8(void* p, unsigned v) {
    asm volatile("global_store_byte %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}

__device__ __forceinline__ int clamp_block(int blk, int N) {
    return (unsigned)blk < (unsigned)N ? blk : 0;
}

// ---------------------------------------------------------------------------
// decode kernel
// ---------------------------------------------------------------------------

constexpr int kMaxRows = 256;    // rows per launch (longer batches are split by the host)
constexpr int kMaxParts = 64;    // partitions per (row, KV head)
constexpr int kMaxPending = 4;   // split runs one workgroup may finish (at most its first and last)
// int32 words between two arrival counters: one counter per 128-byte line, since
// device-scope atomics on one line are performed one after another
constexpr int kCounterStride = 32;
constexpr int kLenMask = 0x3fffffff;     // row length held in LDS ...
constexpr int kLenNoSlot = 0x40000000;   // ... and a flag: the length exceeds the table, no slot to append into

// Work decomposition. A row of length L has nt = ceil(L/64) tiles of 64
// tokens per KV head (an empty row counts one tile, without data, so that its
// zero output is written by someone). All tiles of the batch are numbered
// row by row, KV head by KV head; workgroup w of the G' busy ones takes the
// contiguous range [w*T/G', (w+1)*T/G') of the T tiles, so every workgroup has
// the same work to within one tile whatever the length mix. Every workgroup
// reads seq_lens at start and builds the prefix count of tiles per row in
// LDS, so it finds its tiles without any host-side plan.
//
// A run is the part of one (row, KV head) inside one workgroup's range. A
// (row, KV head) covered by a single workgroup is finished by it; otherwise
// each covering workgroup stores one partial (max, sum, unnormalised output)
// and the last to arrive merges them. G' is capped so that a workgroup gets
// at least C tiles, which bounds the partials of a (row, KV head) by the
// workspace's P.
struct Pos {
    // Packed so that the positions in flight take few scalar registers:
    //   tf:  tile index within the row (bits 0-23; rows hold at most 2^30 tokens),
    //        flags first (24) and last (25) tile of the run, ap (26): the row takes
    //        this step's new token (fused append; L >= 1, within the table), nw (27):
    //        this tile holds that token, kp (28): parity of the run's ordinal in
    //        this workgroup (it picks the query buffer)
    //   bgn: row (bits 0-7, < kMaxRows), KV head (8-20), partitions np of the
    //        (row, KV head) (21-27, <= kMaxParts)
    int t;               // tile number in the batch; >= this workgroup's range end means none
    int L;               // row length (0: an empty row's only, data-less tile)
    int nt;              // tiles of the row (>= 1)
    int tf, bgn;
    int slot;            // this workgroup's index among the np
    int e0, e1, e2, e3;  // physical blocks of the tile (e1.. used when blocks are shorter than a tile)
    int e4, e5, e6, e7;
    int enew;            // physical block of the new token (read by the wave that stores it)
    __device__ bool valid(int t_end) const { return t < t_end; }
    __device__ bool has_tile() const { return L > 0; }
    __device__ int tile() const { return tf & 0xffffff; }
    __device__ int first() const { return (tf >> 24) & 1; }
    __device__ int last() const { return (tf >> 25) & 1; }
    __device__ int ap() const { return (tf >> 26) & 1; }
    __device__ int nw() const { return (tf >> 27) & 1; }
    __device__ int kp() const { return (tf >> 28) & 1; }
    __device__ int b() const { return bgn & 0xff; }
    __device__ int g() const { return (bgn >> 8) & 0x1fff; }
    __device__ int np() const { return (bgn >> 21) & 0x7f; }
};
static_assert(kMaxRows <= 256 && kMaxParts < 128, "Pos field widths");

// Row of tile u: the last row whose prefix count is <= u, by two rounds of a
// 64-lane search over the LDS prefix array pre[0..B].
__device__ __forceinline__ int find_row(const int* pre, int B, int u, int lane) {
    const int S = (B + 63) / 64;  // rows per first-round lane
    const int i1 = min(lane * S, B);
    const unsigned long long m1 = __ballot(pre[i1] <= u && lane * S <= B);
    const int r1 = (64 - __clzll(m1) - 1) * S;  // highest lane whose start is <= u
    const int i2 = min(r1 + lane, B);
    const unsigned long long m2 = __ballot(lane < S && pre[i2] <= u);
    return __builtin_amdgcn_readfirstlane(r1 + (64 - __clzll(m2) - 1));
}

template <int BS, int D, int NREP, bool F8>
struct Cfg {
    static constexpr int E = F8 ? 1 : 2;                   // bytes per pool element (E4M3 or fp16)
    static constexpr int G16 = 16 / E;                     // K channels per 16-byte group; V tokens per 16 bytes
    static constexpr int TT = tile_tokens(F8);             // tokens per tile
    static constexpr int HALVES = TT / 64;                 // 64-token halves of a tile
    static constexpr int NJ = D / 8;                       // 1 KiB load instructions per K (and per V) tile
    static constexpr int NJH = NJ / HALVES;                // K load instructions per half (one per channel group)
    static constexpr int NH = D / 64;                      // 64-channel halves (PV: lane = channel)
    static constexpr int CW = 2;                           // compute waves: each takes half of every tile's tokens
    static constexpr int NB = TT / 16, KS = D / 32, CB = D / 16, PS = TT / 32;  // matrix-core product shapes
    static constexpr int TPB = BS >= TT ? 1 : TT / BS;     // blocks per tile
    static constexpr int TILE = TT * D * E / 2;            // LDS halves per K (or V) tile
    static constexpr int QC = NREP * D / 8;                // 16-byte chunks of a group's queries
    static constexpr int QI = (QC + 63) / 64;              // q load instructions
    static constexpr int QBUF = QI * 64 * 8;               // halves per q buffer
    static constexpr int THREADS = 64 * (CW + 1);          // the compute waves and one load wave
    static_assert(TPB <= 8, "block size of at least 16 tokens");
};

// decode_kernel: persistent, one workgroup per slot: two compute waves and
// one load wave (wave 2) that issues every tile load and waits for it. A wave
// that issues a load stalls whenever the memory system is saturated; keeping
// all loads in their own wave keeps those stalls off the compute waves.
//
// Tile pipeline (step j computes tile position P_j; buffers alternate by j):
//   prologue:  load wave issues K(P0), V(P0)
//   step j:    load wave waits for K(P_j) -> barrier A -> load wave issues
//              [j = 0: K(P1)] V(P_{j+1}) into the V buffer freed by step j-1
//              and waits for V(P_j) while compute waves do QK + softmax on
//              K(P_j) -> barrier B -> load wave issues K(P_{j+2}) into the K
//              buffer just read while compute waves do PV on V(P_j) and, if
//              P_j ends its unit, store the unit's result
// so 1.5 tiles of loads are in flight during every compute phase, across unit
// boundaries as well. The query of a unit is loaded into LDS with the K tile
// of its first position.
//
// Token split: compute wave w takes the w-th half of every tile's tokens
// (16-token score blocks w*NB/2 .., 32-token output steps w*PS/2 ..) and
// keeps its own online softmax state (max, sum, output) for all of the
// group's query heads. At the end of a run of tiles of one (row, KV head),
// wave 1 hands its state to wave 0 through LDS, and wave 0 rescales both to
// the common max and adds them: the exact two-way merge of partial softmax
// results.
//
// Register layouts (query head hq = lane % 16, lane group lg = lane / 16):
// a score block's result holds tokens 4lg .. 4lg+3 of the block for head hq,
// so a head's running max lives in lanes hq, hq+16, hq+32, hq+48 (combined
// with the permlane swaps); the fp16 probabilities of a 32-token output step
// are already the B operand of V^T.P^T in the lanes that computed them; the
// output accumulators hold head hq, channels 16cb + 4lg .. 16cb + 4lg + 3; and
// the sum of the weights is one more product of the same step, a row of ones
// times P^T, so it adds exactly the fp16-rounded weights the output adds, in
// fp32, and every element of that accumulator holds head hq's sum.
//
// LDS tile layouts (fp16 pools, 64-token tiles): K is [NJ][64 tokens][8 ch],
// so the A operand of a score product (token, 8 channels) is one 16-byte
// read; V is [NJ row blocks][8 chunks][8 rows][8 tokens], loaded so that a
// load instruction still covers eight whole 128-byte rows of V, and the A
// operand of an output product (channel, 4 + 4 tokens) is two 8-byte reads.
// E4M3 pools, 128-token tiles: K is [2 halves][D/16][64 tokens][16 ch] bytes,
// one 16-byte read serving two score products after widening; V's bytes sit
// exactly as an fp16 tile's, each 16-byte unit now 16 tokens of one row.
//
// Probabilities enter the output product as 2^15 * exp2(s - max) in fp16:
// the factor cancels between output and sum. Weights down to 2^-29 of the
// row's largest stay normal fp16 numbers (relative precision 2^-11), those
// down to 2^-39 are subnormals, and smaller ones are 0; a plain
// exp2(s - max) would already turn subnormal below 2^-14.
//
// Results: a one-partition row writes fp16 output directly; otherwise the
// partition writes (max, sum, unnormalised output) with coherent stores and is
// listed; at exit the workgroup adds one to the arrival counter of each
// (row, KV head) it holds a partition of, and merges every pair whose count
// it completed, in partition order.
template <int BS, int D, int NREP, bool F8>
__global__ void __launch_bounds__((Cfg<BS, D, NREP, F8>::THREADS)) decode_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, uint16_t* k_pool, uint16_t* v_pool,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ seq_lens, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, int32_t* __restrict__ counters, float* __restrict__ part_ml,
    float* __restrict__ part_acc, int B, int Hkv, int W, int N, int C, int P, float scale_log2, int width, float k_scale, float v_scale,
    float k_inv, float v_inv) {
    using K = Cfg<BS, D, NREP, F8>;
    constexpr int NJ = K::NJ, NH = K::NH, CW = K::CW, TPB = K::TPB;
    constexpr int NB = K::NB, KS = K::KS, CB = K::CB, PS = K::PS;
    constexpr int E = K::E, G16 = K::G16, TT = K::TT, HALVES = K::HALVES, NJH = K::NJH;
    constexpr int TILE = K::TILE, QC = K::QC, QI = K::QI, QBUF = K::QBUF, THREADS = K::THREADS;
    static_assert(BS % 16 == 0, "block size must be a multiple of 16");

    __shared__ __attribute__((aligned(16))) uint16_t s_k[2][TILE];
    __shared__ __attribute__((aligned(16))) uint16_t s_v[2][TILE];
    __shared__ __attribute__((aligned(16))) uint16_t s_q[2][QBUF];
    __shared__ __attribute__((aligned(16))) float s_xacc[K::CB * 4 * 64];  // wave 1's state at a run's end
    __shared__ float s_xml[2 * 16];
    __shared__ __attribute__((aligned(16))) uint16_t s_kn[2][D];  // fused append: the new token's K ...
    __shared__ __attribute__((aligned(16))) uint16_t s_vn[2][D];  // ... and V, staged with the tile holding it
    __shared__ int s_len[kMaxRows];
    __shared__ int s_pre[kMaxRows + 1];
    __shared__ int s_pend[kMaxPending];  // (row*Hkv + g) of split partitions finished here
    __shared__ int s_pend_np[kMaxPending];
    __shared__ int s_npend;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wip = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index in the workgroup
    const bool loader = wip == CW;                              // the load wave
    const int Hq = Hkv * NREP;
    const int G = gridDim.x;
    const int cap = W * BS;
    // V load lane: row (channel) among the instruction's 8, and chunk of G16 tokens (8 chunks per tile)
    const int drow = lane & 7, vc = lane >> 3;
    const bool append = k_new != nullptr;  // fused kv_append: this step's K/V enter the pool here

    // ---- tile list: lengths and the prefix count of tiles per row
    for (int r = tid; r < B; r += THREADS) {
        int L = seq_lens[r];
        const int noslot = L > cap ? kLenNoSlot : 0;
        L = L < 0 ? 0 : (L > cap ? cap : L);
        s_len[r] = L | noslot;
    }
    if (tid == 0) s_npend = 0;
    __syncthreads();
    if (wip == 0) {
        // serial over 64-row chunks, a wave-wide inclusive scan within each
        int carry = 0;
        for (int r0 = 0; r0 < B; r0 += 64) {
            const int r = r0 + lane;
            const int Lr = r < B ? (s_len[r] & kLenMask) : 0;
            // width > 0 (the masked-width contrast): every non-empty row spans max(width, L) tokens
            const int nt = r < B ? Hkv * max(1, ((width > 0 && Lr > 0 ? max(width, Lr) : Lr) + TT - 1) / TT) : 0;
            int x = nt;
#pragma unroll
            for (int sh = 1; sh < 64; sh <<= 1) {
                const int y = __shfl_up(x, sh);
                if (lane >= sh) x += y;
            }
            if (r < B) s_pre[r + 1] = carry + x;
            carry += __shfl(x, 63);
        }
        if (lane == 0) s_pre[0] = 0;
    }
    __syncthreads();
    const int T = __builtin_amdgcn_readfirstlane(s_pre[B]);
    const int Gb = min(G, max(1, T / C));  // busy workgroups: each gets at least C tiles
    const int w = blockIdx.x;
    const int t_begin = w < Gb ? (int)(((long long)w * T) / Gb) : 0;
    const int t_end = w < Gb ? (int)(((long long)(w + 1) * T) / Gb) : 0;
    auto owner = [&](int a) {  // the workgroup whose range holds tile a
        return (int)((((long long)a + 1) * Gb + T - 1) / T) - 1;
    };
    wait_vmem<0>();  // nothing of the prologue is left in flight: the count below starts at zero
    int vm_count = 0;

    // table entries of a position's tile (scalar loads; entries past the
    // row's last block are replaced by the tile's first, whose data is masked)
    auto load_entries = [&](Pos& s) {
        s.e0 = s.e1 = s.e2 = s.e3 = s.e4 = s.e5 = s.e6 = s.e7 = 0;
        if (!loader || !s.valid(t_end) || !s.has_tile()) return;
        const int32_t* trow = tables + (size_t)s.b() * W;
        const int n0 = (s.tile() * TT) / BS;
        const int nblk = ((width > 0 ? max(s.L, width) : s.L) + BS - 1) / BS;
        auto at = [&](int i) { return trow[n0 + i < nblk ? n0 + i : n0]; };
        s.e0 = trow[n0];
        if constexpr (TPB > 1) s.e1 = at(1);
        if constexpr (TPB > 2) {
            s.e2 = at(2);
            s.e3 = at(3);
        }
        if constexpr (TPB > 4) {
            s.e4 = at(4);
            s.e5 = at(5);
            s.e6 = at(6);
            s.e7 = at(7);
        }
    };
    // the partitions of a run's (row, KV head) and this workgroup's index among them
    auto split_of = [&](Pos& s) {
        const int a0 = s.t - s.tile();  // the (row, KV head)'s first tile
        const int w0 = owner(a0);
        const int np = owner(a0 + s.nt - 1) - w0 + 1;
        s.slot = w - w0;
        s.bgn = (s.bgn & 0x1fffff) | (np << 21);
    };
    // the position of tile t (prev: the position before it in this range); with
    // defer, the start of a run leaves np and slot to split_of
    auto pos_at = [&](int t, const Pos& prev, bool has_prev, bool defer = false) {
        Pos s;
        if (t >= t_end) {
            s = prev;
            s.t = t_end;
            return s;
        }
        int tile, first, ap, kp;
        if (has_prev && prev.tile() + 1 < prev.nt) {  // the same run goes on
            s = prev;
            s.t = t;
            tile = prev.tile() + 1;
            first = 0;
            ap = prev.ap();
            kp = prev.kp();
        } else {
            s.t = t;
            const int b = find_row(s_pre, B, t, lane);
            const int lf = __builtin_amdgcn_readfirstlane(s_len[b]);
            s.L = lf & kLenMask;
            ap = append && s.L > 0 && !(lf & kLenNoSlot);
            s.nt = max(1, ((width > 0 && s.L > 0 ? max(width, s.L) : s.L) + TT - 1) / TT);
            const int r = t - __builtin_amdgcn_readfirstlane(s_pre[b]);
            const int g = r / s.nt;
            tile = r - g * s.nt;
            s.bgn = b | (g << 8);
            if (!defer) split_of(s);
            kp = has_prev ? prev.kp() ^ 1 : 0;
            first = 1;
        }
        const int last = (t + 1 == t_end) || (tile + 1 == s.nt);
        const int nw = ap && tile == (s.L - 1) / TT;
        s.tf = tile | (first << 24) | (last << 25) | (ap << 26) | (nw << 27) | (kp << 28);
        s.enew = 0;
        if (wip == 0 && nw) s.enew = tables[(size_t)s.b() * W + (s.L - 1) / BS];
        load_entries(s);
        return s;
    };
    auto entry_for = [&](const Pos& s, int idx) {  // idx = block of the tile (0..TPB-1), wave-divergent
        if constexpr (TPB == 1) {
            return s.e0;
        } else if constexpr (TPB == 2) {
            return idx == 0 ? s.e0 : s.e1;
        } else if constexpr (TPB == 4) {
            return idx == 0 ? s.e0 : (idx == 1 ? s.e1 : (idx == 2 ? s.e2 : s.e3));
        } else {
            const int lo = idx == 0 ? s.e0 : (idx == 1 ? s.e1 : (idx == 2 ? s.e2 : s.e3));
            const int hi = idx == 4 ? s.e4 : (idx == 5 ? s.e5 : (idx == 6 ? s.e6 : s.e7));
            return idx < 4 ? lo : hi;
        }
    };

    // ---- loads into LDS (issued by the load wave only); LDS byte addresses
    const unsigned lds_k = lds_addr(&s_k[0][0]), lds_v = lds_addr(&s_v[0][0]), lds_q = lds_addr(&s_q[0][0]);
    const unsigned lds_kn = lds_addr(&s_kn[0][0]), lds_vn = lds_addr(&s_vn[0][0]);
    // the new token's K (or V) of a tile that holds it, staged in LDS ahead of the tile's own loads
    auto issue_new = [&](const Pos& s, const uint16_t* src, unsigned dst) {
        if (lane < D / 8) dma16(src + ((size_t)s.b() * Hkv + s.g()) * D + 8 * lane, dst);
        vm_count += 1;
    };
    auto issue_q = [&](const Pos& s) {
        const uint16_t* qrow = q + ((size_t)s.b() * Hq + (size_t)s.g() * NREP) * D;
#pragma unroll
        for (int i = 0; i < QI; ++i) {
            const int c = i * 64 + lane;
            dma16(qrow + 8 * min(c, QC - 1), lds_q + (unsigned)(((s.kp()) * QBUF + i * 512) * 2));
        }
        vm_count += QI;
    };
    auto issue_k = [&](const Pos& s, int buf) {
        if (s.nw()) issue_new(s, k_new, lds_kn + (unsigned)(buf * D * 2));
#pragma unroll
        for (int hf = 0; hf < HALVES; ++hf) {  // lane = token of the half; one instruction per channel group
            const int tok = s.tile() * TT + 64 * hf + lane;
            const int phys = clamp_block(entry_for(s, TPB == 1 ? 0 : (64 * hf + lane) / BS), N);
            const char* src = reinterpret_cast<const char*>(k_pool) +
                              ((size_t)phys * Hkv + s.g()) * (size_t)(D * BS) * E + (size_t)(tok % BS) * 16;
#pragma unroll
            for (int j = 0; j < NJH; ++j)
                dma16_nt(src + (size_t)j * (BS * 16), lds_k + (unsigned)((buf * TILE + (hf * NJH + j) * 512) * 2));
        }
        vm_count += NJ;
    };
    auto issue_v = [&](const Pos& s, int buf) {
        if (s.nw()) issue_new(s, v_new, lds_vn + (unsigned)(buf * D * 2));
        const int tok = s.tile() * TT + G16 * vc;
        const int phys = clamp_block(entry_for(s, TPB == 1 ? 0 : (G16 * vc) / BS), N);
        const char* src = reinterpret_cast<const char*>(v_pool) +
                          (((size_t)phys * Hkv + s.g()) * (size_t)(D * BS) + (size_t)drow * BS + (size_t)(tok % BS)) * E;
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)  // rows 8jj .. 8jj+7
            dma16_nt(src + (size_t)jj * (8 * BS) * E, lds_v + (unsigned)((buf * TILE + jj * 512) * 2));
        vm_count += NJ;
    };

    // ---- per-unit state of a compute wave (query head hq = lane % 16, lane group lg = lane / 16)
    const int hq = lane & 15, lg = lane >> 4;
    u32x4 qb[KS];
    f32x4 acc[CB];
    u32x4 pb[PS / 2];  // this tile's probabilities (this wave's tokens) as the output product's operand
    float m = -INFINITY;
    f32x4 accl = {0.f, 0.f, 0.f, 0.f};  // the run's sum of weights for head hq (every element), kept by the matrix cores

    // The first tile is requested as soon as its table entries are in; the
    // entries of the next positions are requested after it.
    const Pos none = {};
    Pos P0 = pos_at(t_begin, none, false, true);
    int mk0 = 0, mk1 = 0, mv0 = 0, mv1 = 0;  // vm_count after each buffer's last load
    if (loader && P0.valid(t_end) && P0.has_tile()) {
        issue_q(P0);
        issue_k(P0, 0);
        mk0 = vm_count;
        issue_v(P0, 0);
        mv0 = vm_count;
    }
    if (P0.valid(t_end)) split_of(P0);  // after the first request: not needed for it
    Pos P1 = pos_at(t_begin + 1, P0, true);
    // With every slot busy, the second K tile is requested in the prologue as well
    // (with some slots idle, the first tiles land sooner without it).
    const bool k1_early = Gb == G && P0.valid(t_end) && P0.has_tile();
    if (loader && k1_early && P1.valid(t_end) && P1.has_tile()) {
        if (P1.first()) issue_q(P1);
        issue_k(P1, 1);
        mk1 = vm_count;
    }
    Pos P2 = pos_at(t_begin + 2, P1, true);

    for (int j = 0; P0.valid(t_end); ++j) {
        const int buf = j & 1;
        const bool tile = P0.has_tile();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (loader && tile) wait_vmem_dyn(vm_count - (buf ? mk1 : mk0));
        // the new token's 16-byte K group `lane` in the tile: instruction (half, group), slot tn % 64
        auto new_k_slot = [&](int tn) {
            return reinterpret_cast<u32x4*>(&s_k[buf][((tn >> 6) * NJH + lane) * 512 + (tn & 63) * 8]);
        };
        if (loader && tile && P0.nw()) {  // fused append: the new token's K into its slot of the tile
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            const int tn = P0.L - 1 - P0.tile() * TT;
            if constexpr (!F8) {
                if (lane < D / 8) *new_k_slot(tn) = *reinterpret_cast<const u32x4*>(&s_kn[buf][lane * 8]);
            } else {  // quantized, one channel per lane and half: byte c%16 of group c/16
                const _Float16* x = reinterpret_cast<const _Float16*>(&s_kn[buf][0]);
                uint8_t* kt = reinterpret_cast<uint8_t*>(&s_k[buf][0]) + (tn & 63) * 16;
                const unsigned w = pa_e4m3::quantize2(x[lane], x[NH > 1 ? 64 + lane : lane], k_scale, k_inv);
#pragma unroll
                for (int hv = 0; hv < NH; ++hv) {
                    const int c = hv * 64 + lane;
                    kt[((tn >> 6) * NJH + (c >> 4)) * 1024 + (c & 15)] = (uint8_t)(w >> (8 * hv));
                }
            }
            wait_lds();
        }
        tile_barrier();  // K(P_j) is in LDS for every wave; PV of step j-1 is done everywhere
        if (wip == 0 && tile && P0.nw() && (unsigned)P0.enew < (unsigned)N && lane < D / G16) {
            // fused append: the new token's K into the pool (nothing in this launch reads it back)
            const size_t base = (size_t)P0.enew * Hkv + P0.g();
            const int tn = P0.L - 1 - P0.tile() * TT;
            st_b128(reinterpret_cast<char*>(k_pool) + ((base * (D / G16) + lane) * BS + (P0.L - 1) % BS) * 16,
                    *new_k_slot(tn));
        }
        if (loader && P1.valid(t_end) && P1.has_tile()) {
            if (j == 0 && !k1_early) {  // the second K tile, unless the prologue requested it
                if (P1.first()) issue_q(P1);
                issue_k(P1, 1);
                mk1 = vm_count;
            }
            issue_v(P1, buf ^ 1);
            if (buf) mv0 = vm_count; else mv1 = vm_count;
        }
        // the position after P2: its table entries are requested a whole step
        // before anything waits on them
        const Pos P3 = pos_at(P2.t + 1, P2, true);
        if (!loader && tile) {
            if (P0.first()) {
                // the query operand: head hq, channels c0(ks) .. c0(ks)+7 (zero past the group's heads)
                const uint16_t* qh = &s_q[P0.kp()][min(hq, NREP - 1) * D];  // rows past NREP: read, then zeroed
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int c0 = F8 ? 64 * (ks >> 1) + 16 * lg + 8 * (ks & 1) : 32 * ks + 8 * lg;
                    const u32x4 x = *reinterpret_cast<const u32x4*>(qh + c0);
                    qb[ks] = hq < NREP ? x : u32x4{0u, 0u, 0u, 0u};
                }
                m = -INFINITY;
                accl = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            // ---- scores: S^T = K . Q^T per 16-token block. Every operand read of the
            // tile is issued first (they complete in order), then the products, the
            // blocks' chains interleaved.
            constexpr int NB2 = NB / 2;   // this wave's 16-token blocks: wip*NB2 ..
            constexpr int PS2 = PS / 2;   // and output steps: wip*PS2 ..
            const int nb0 = wip * NB2;
            f32x4 sc[NB2];
#pragma unroll
            for (int nb = 0; nb < NB2; ++nb) sc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (!F8) {
                u32x4 kr[KS][NB2];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int nb = 0; nb < NB2; ++nb)
                        kr[ks][nb] = *reinterpret_cast<const u32x4*>(
                            &s_k[buf][((4 * ks + lg) * 64 + 16 * (nb0 + nb) + hq) * 8]);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int nb = 0; nb < NB2; ++nb) sc[nb] = mfma16(kr[ks][nb], qb[ks], sc[nb]);
                // all operand reads first, then the products
                __builtin_amdgcn_sched_group_barrier(0x100, KS * NB2, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, KS * NB2, 0);
            } else {
                // token 16(nb%4) + hq of 64-token half nb/4; one 16-byte read serves steps 2kp, 2kp+1
                const char* kt = reinterpret_cast<const char*>(&s_k[buf][0]);
                u32x4 kr[KS / 2][NB2];
#pragma unroll
                for (int kp = 0; kp < KS / 2; ++kp)
#pragma unroll
                    for (int nb = 0; nb < NB2; ++nb)
                        kr[kp][nb] = *reinterpret_cast<const u32x4*>(
                            kt + ((nb0 + nb) >> 2) * (D * 64) + ((4 * kp + lg) * 64 + 16 * ((nb0 + nb) & 3) + hq) * 16);
#pragma unroll
                for (int kp = 0; kp < KS / 2; ++kp)
#pragma unroll
                    for (int nb = 0; nb < NB2; ++nb) {
                        sc[nb] = mfma16(widen8<0>(kr[kp][nb]), qb[2 * kp], sc[nb]);
                        sc[nb] = mfma16(widen8<1>(kr[kp][nb]), qb[2 * kp + 1], sc[nb]);
                    }
            }
            // ---- online softmax (exp2 domain): max over the lane's 4*NB tokens, then over the
            // four lanes of the head
            const int t0 = P0.tile() * TT + 16 * nb0 + 4 * lg;  // token of element 0 of this wave's block 0
            float smax = -INFINITY;
            if (P0.tile() * TT + TT <= P0.L) {  // a full tile: no token to mask
#pragma unroll
                for (int nb = 0; nb < NB2; ++nb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sc[nb][i] *= scale_log2;
                        smax = fmaxf(smax, sc[nb][i]);
                    }
            } else {
#pragma unroll
                for (int nb = 0; nb < NB2; ++nb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x = t0 + 16 * nb + i < P0.L ? sc[nb][i] * scale_log2 : -INFINITY;
                        sc[nb][i] = x;
                        smax = fmaxf(smax, x);
                    }
            }
            const float mn = fmaxf(m, cross_rows(smax, [](float a, float b) { return fmaxf(a, b); }));
            const float mref = mn == -INFINITY ? 0.f : mn;  // no live token yet (a masked tile): p and alpha are 0
            const float alpha = __builtin_amdgcn_exp2f(m - mref);
            m = mn;
            const float mb = mref - 15.f;  // p enters the products as 2^15 * exp2(s - max)
#pragma unroll
            for (int q2 = 0; q2 < PS2; ++q2) {
                _Float16 ph[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) ph[i] = (_Float16)__builtin_amdgcn_exp2f(sc[2 * q2 + (i >> 2)][i & 3] - mb);
                pb[q2] = u32x4{pack_h2(ph[0], ph[1]), pack_h2(ph[2], ph[3]), pack_h2(ph[4], ph[5]),
                               pack_h2(ph[6], ph[7])};
            }
            if (__builtin_amdgcn_readfirstlane((int)(__ballot(alpha != 1.0f) != 0))) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) acc[cb] *= alpha;
                accl *= alpha;
            }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (loader && tile) wait_vmem_dyn(vm_count - (buf ? mv1 : mv0));
        if (!F8 && loader && tile && P0.nw()) {  // fused append: the new token's V into its slot of the tile
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            const int tn = P0.L - 1 - P0.tile() * TT;
#pragma unroll
            for (int hv = 0; hv < NH; ++hv) {
                const int c = hv * 64 + lane;
                s_v[buf][(c >> 3) * 512 + (tn >> 3) * 64 + (c & 7) * 8 + (tn & 7)] = s_vn[buf][c];
            }
            wait_lds();
        }
        // byte of channel c, tile token tn in an E4M3 V tile: instruction c/8, chunk tn/16, row c%8
        auto v8_at = [&](int c, int tn) {
            return reinterpret_cast<uint8_t*>(&s_v[buf][0]) + (c >> 3) * 1024 + ((tn >> 4) * 8 + (c & 7)) * 16 +
                   (tn & 15);
        };
        if (F8 && loader && tile && (P0.tile() * TT + TT > P0.L || P0.nw())) {
            // an E4M3 tile past the row's end: its dead slots may hold NaN
            // codes; they are zeroed in LDS here (lane = chunk*8 + row, one
            // 16-byte unit per instruction), so PV needs no masking; then
            // the fused append's new token (quantized) goes into its slot
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (P0.tile() * TT + TT > P0.L) {
                const u32x4 mask = keep_first_bytes(P0.L - (P0.tile() * TT + 16 * vc));
                char* vt = reinterpret_cast<char*>(&s_v[buf][0]) + 16 * lane;
#pragma unroll
                for (int jj = 0; jj < NJ; ++jj) *reinterpret_cast<u32x4*>(vt + jj * 1024) &= mask;
            }
            if (P0.nw()) {
                const int tn = P0.L - 1 - P0.tile() * TT;
                const _Float16* x = reinterpret_cast<const _Float16*>(&s_vn[buf][0]);
                const unsigned w = pa_e4m3::quantize2(x[lane], x[NH > 1 ? 64 + lane : lane], v_scale, v_inv);
#pragma unroll
                for (int hv = 0; hv < NH; ++hv) *v8_at(hv * 64 + lane, tn) = (uint8_t)(w >> (8 * hv));
            }
            wait_lds();
        }
        tile_barrier();  // V(P_j) is in LDS for every wave; every wave is done with K(P_j)
        if (wip == 0 && tile && P0.nw() && (unsigned)P0.enew < (unsigned)N) {
            // fused append: the new token's V into the pool
            const size_t base = (size_t)P0.enew * Hkv + P0.g();
            const int slot = (P0.L - 1) % BS;
#pragma unroll
            for (int hv = 0; hv < NH; ++hv) {
                const int c = hv * 64 + lane;
                if constexpr (!F8)
                    st_u16(v_pool + (base * D + c) * BS + slot, s_vn[buf][c]);
                else
                    st_u8(reinterpret_cast<uint8_t*>(v_pool) + (base * D + c) * BS + slot,
                          *v8_at(c, P0.L - 1 - P0.tile() * TT));
            }
        }
        if (loader && P2.valid(t_end) && P2.has_tile()) {
            if (P2.first()) issue_q(P2);
            issue_k(P2, buf);
            if (buf) mk1 = vm_count; else mk0 = vm_count;
        }
        if (!loader && tile) {
            // ---- output: O^T += V^T . P^T per 16-channel block, 32 tokens a step; lane l reads
            // channel 16cb + hq, tokens 32ps + 4lg + 0..3 and 32ps + 16 + 4lg + 0..3
            const int c7 = hq & 7;
            if constexpr (!F8) {
                // halves of (channel c, token t): (c/8)*512 + (t/8)*64 + (c%8)*8 + t%8
                constexpr int PS2 = PS / 2;
                const int q0 = wip * PS2;
                const int tl = P0.L - P0.tile() * TT - 32 * q0 - 4 * lg;  // live tokens from this lane's first one
                const bool ragged = P0.tile() * TT + TT > P0.L;
                uint2 vr[PS2][CB][2];
#pragma unroll
                for (int q2 = 0; q2 < PS2; ++q2)
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        const uint16_t* v = &s_v[buf][(2 * cb + (hq >> 3)) * 512 + (4 * (q0 + q2) + (lg >> 1)) * 64 +
                                                      c7 * 8 + 4 * (lg & 1)];
                        vr[q2][cb][0] = *reinterpret_cast<const uint2*>(v);
                        vr[q2][cb][1] = *reinterpret_cast<const uint2*>(v + 128);
                    }
                if (ragged) {  // tokens past the row's end may hold NaN: zero their V
#pragma unroll
                    for (int q2 = 0; q2 < PS2; ++q2) {
                        const unsigned mlo0 = keep2(tl - 32 * q2, 0), mlo1 = keep2(tl - 32 * q2, 2);
                        const unsigned mhi0 = keep2(tl - 32 * q2 - 16, 0), mhi1 = keep2(tl - 32 * q2 - 16, 2);
#pragma unroll
                        for (int cb = 0; cb < CB; ++cb) {
                            vr[q2][cb][0].x &= mlo0;
                            vr[q2][cb][0].y &= mlo1;
                            vr[q2][cb][1].x &= mhi0;
                            vr[q2][cb][1].y &= mhi1;
                        }
                    }
                }
#pragma unroll
                for (int q2 = 0; q2 < PS2; ++q2) {
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
                        acc[cb] = mfma16(u32x4{vr[q2][cb][0].x, vr[q2][cb][0].y, vr[q2][cb][1].x, vr[q2][cb][1].y},
                                         pb[q2], acc[cb]);
                    accl = mfma16(kOnes, pb[q2], accl);  // the weights' sum: a row of ones times P^T
                }
            } else {
                // bytes of (channel c, token t): (c/8)*1024 + (t/16)*128 + (c%8)*16 + t%16; the
                // codes of tokens past the row's end are already zero (the load wave cleared them
                // in LDS before barrier B)
                const char* vt = reinterpret_cast<const char*>(&s_v[buf][0]);
                constexpr int PS2 = PS / 2;
                const int q0 = wip * PS2;
                unsigned vr[PS2][CB][2];
#pragma unroll
                for (int q2 = 0; q2 < PS2; ++q2)
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        const char* v = vt + (2 * cb + (hq >> 3)) * 1024 + (2 * (q0 + q2)) * 128 + c7 * 16 + 4 * lg;
                        vr[q2][cb][0] = *reinterpret_cast<const unsigned*>(v);
                        vr[q2][cb][1] = *reinterpret_cast<const unsigned*>(v + 128);
                    }
#pragma unroll
                for (int q2 = 0; q2 < PS2; ++q2) {
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        const unsigned w0 = vr[q2][cb][0], w1 = vr[q2][cb][1];
                        acc[cb] = mfma16(u32x4{f8x2<false>(w0), f8x2<true>(w0), f8x2<false>(w1), f8x2<true>(w1)},
                                         pb[q2], acc[cb]);
                    }
                    accl = mfma16(kOnes, pb[q2], accl);  // the weights' sum: a row of ones times P^T
                }
            }
        }
        float lt = 0.f;
        if (P0.last()) {
            // ---- the two compute waves' states of this run combined (wave 1 -> LDS -> wave 0)
            if (!loader) lt = tile ? accl[0] : 0.f;
            if (wip == 1) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
                    *reinterpret_cast<f32x4*>(&s_xacc[(cb * 64 + lane) * 4]) = tile ? acc[cb] : f32x4{0.f, 0.f, 0.f, 0.f};
                if (lg == 0) {
                    s_xml[hq] = tile ? m : -INFINITY;
                    s_xml[16 + hq] = lt;
                }
            }
            __syncthreads();
            if (wip == 0 && tile) {
                const float m1 = s_xml[hq], l1 = s_xml[16 + hq];
                const float mn = fmaxf(m, m1);
                const float mr = mn == -INFINITY ? 0.f : mn;
                const float a0 = __builtin_amdgcn_exp2f(m - mr), a1 = __builtin_amdgcn_exp2f(m1 - mr);
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
                    acc[cb] = acc[cb] * a0 + *reinterpret_cast<const f32x4*>(&s_xacc[(cb * 64 + lane) * 4]) * a1;
                lt = lt * a0 + l1 * a1;
                m = mn;
            }
        }
        if (wip == 0 && P0.last()) {
            // ---- the unit's result: head hq, channels 16cb + 4lg + 0..3
            const int b = P0.b(), g = P0.g();
            if (!tile) lt = 1.f;
            if (P0.np() == 1) {
                if (hq < NREP) {
                    uint16_t* orow = out + ((size_t)b * Hq + (size_t)g * NREP + hq) * D + 4 * lg;
                    const float r = v_scale / lt;
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        const f32x4 o = tile ? acc[cb] * r : f32x4{0.f, 0.f, 0.f, 0.f};
                        st_b64(orow + 16 * cb, pack_h2((_Float16)o[0], (_Float16)o[1]),
                               pack_h2((_Float16)o[2], (_Float16)o[3]));
                    }
                }
            } else {
                const size_t slot = ((size_t)(b * Hkv + g) * P + P0.slot) * NREP + hq;
                if (hq < NREP) {
                    float* pa = part_acc + slot * D + 4 * lg;
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) st_f32x4_sc1(pa + 16 * cb, tile ? acc[cb] : f32x4{0.f, 0.f, 0.f, 0.f});
                    if (lg == 0) st_2f32_sc1(part_ml + slot * 2, m, lt);
                }
                if (lane == 0) {
                    const int n = s_npend;
                    if (n < kMaxPending) {
                        s_pend[n] = b * Hkv + g;
                        s_pend_np[n] = P0.np();
                        s_npend = n + 1;
                    }
                }
            }
        }
        P0 = P1;
        P1 = P2;
        P2 = P3;
    }

    // ---- tickets and merges of split (row, KV head)s
    __builtin_amdgcn_s_waitcnt(0);  // every partial of this workgroup is stored
    __syncthreads();
    const int npend = __builtin_amdgcn_readfirstlane(s_npend);
    for (int e = tid; e < npend; e += THREADS) {
        const int t = __hip_atomic_fetch_add(&counters[s_pend[e] * kCounterStride], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_pend_np[e] = (t + 1 == s_pend_np[e]) ? s_pend_np[e] : -s_pend_np[e];  // > 0: this workgroup merges
    }
    __syncthreads();
    // Merge: every thread owns 4-channel chunks of the group's output and
    // combines the partitions in partition order, eight at a time with all
    // their loads in flight together (running max, rescaled sums).
    constexpr int NC4 = NREP * D / 4;
    constexpr int CPT = (NC4 + THREADS - 1) / THREADS;  // chunks per thread
    constexpr int MB = 8;                               // partitions per round trip
    for (int e = 0; e < npend; ++e) {
        const int np = __builtin_amdgcn_readfirstlane(s_pend_np[e]);
        if (np <= 0) continue;
        const int bg = __builtin_amdgcn_readfirstlane(s_pend[e]);
        const float* ml0 = part_ml + (size_t)bg * P * NREP * 2;
        const float* acc0 = part_acc + (size_t)bg * P * NREP * D;
        const __amdgpu_buffer_rsrc_t rml =
            __builtin_amdgcn_make_buffer_rsrc((void*)ml0, 0, np * NREP * 2 * 4, kRawBufferFormat);
        const __amdgpu_buffer_rsrc_t racc =
            __builtin_amdgcn_make_buffer_rsrc((void*)acc0, 0, np * NREP * D * 4, kRawBufferFormat);
        uint16_t* orow = out + (size_t)bg * NREP * D;  // (b*Hq + g*NREP)*D with bg = b*Hkv + g
        float M[CPT], den[CPT];
        f32x4 num[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            M[i] = -INFINITY;
            den[i] = 0.f;
            num[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        for (int p0 = 0; p0 < np; p0 += MB) {
            float mv[CPT][MB], lv[CPT][MB];
            f32x4 av[CPT][MB];
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int c4 = min(tid + i * THREADS, NC4 - 1);
                const int h = (4 * c4) / D;
#pragma unroll
                for (int k = 0; k < MB; ++k) {
                    const int pp = min(p0 + k, np - 1);  // past np: a repeat, weighted 0 below
                    const f32x2 ml = __builtin_bit_cast(
                        f32x2, __builtin_amdgcn_raw_buffer_load_b64(rml, (pp * NREP + h) * 8, 0, kCoherent));
                    mv[i][k] = ml.x;
                    lv[i][k] = ml.y;
                    av[i][k] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(racc, (pp * NREP * D + 4 * c4) * 4, 0, kCoherent));
                }
            }
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                float mb = M[i];
#pragma unroll
                for (int k = 0; k < MB; ++k)
                    if (p0 + k < np) mb = fmaxf(mb, mv[i][k]);
                const float r = __builtin_amdgcn_exp2f(M[i] - mb);  // 0 on the first batch (M = -inf)
                den[i] *= r;
                num[i] *= r;
#pragma unroll
                for (int k = 0; k < MB; ++k) {
                    const float w = (p0 + k < np) ? __builtin_amdgcn_exp2f(mv[i][k] - mb) : 0.f;
                    den[i] += w * lv[i][k];
                    num[i] += w * av[i][k];
                }
                M[i] = mb;
            }
        }
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c4 = tid + i * THREADS;
            if (c4 < NC4) {
                const f32x4 o = num[i] / den[i] * v_scale;
                st_b64(orow + 4 * c4, pack_h2((_Float16)o.x, (_Float16)o.y), pack_h2((_Float16)o.z, (_Float16)o.w));
            }
        }
        if (tid == 0) __hip_atomic_store(&counters[bg * kCounterStride], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// launch table
// ---------------------------------------------------------------------------



template <bool F8, int BS, int D, int NREP>
DecodeFn make_fn() {
    return {reinterpret_cast<const void*>(decode_kernel<BS, D, NREP, F8>), Cfg<BS, D, NREP, F8>::THREADS};
}

template <bool F8, int BS, int D>
DecodeFn pick_nrep(int nrep) {
    switch (nrep) {
        case 1: return make_fn<F8, BS, D, 1>();
        case 2: return make_fn<F8, BS, D, 2>();
        case 4: return make_fn<F8, BS, D, 4>();
        case 6: return make_fn<F8, BS, D, 6>();
        case 8: return make_fn<F8, BS, D, 8>();
        default: return {nullptr, 0};
    }
}

template <bool F8, int BS>
DecodeFn pick_d(int D, int nrep) {
    switch (D) {
        case 64: return pick_nrep<F8, BS, 64>(nrep);
        case 128: return pick_nrep<F8, BS, 128>(nrep);
        default: return {nullptr, 0};
    }
}

// The compiled set: block sizes 16..256, head_dim 64 and 128, 1..8 query heads per KV head.
template <bool F8>
DecodeFn pick_decode_t(int bs, int D, int nrep) {
    switch (bs) {
        case 16: return pick_d<F8, 16>(D, nrep);
        case 32: return pick_d<F8, 32>(D, nrep);
        case 64: return pick_d<F8, 64>(D, nrep);
        case 128: return pick_d<F8, 128>(D, nrep);
        case 256: return pick_d<F8, 256>(D, nrep);
        default: return {nullptr, 0};
    }
}

}  // namespace
