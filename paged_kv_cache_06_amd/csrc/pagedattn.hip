// libpagedattn, decode attention: paged KV-cache decode attention for MI355X
// (gfx950). The block operations (kv_append, kv_copy_blocks,
// kv_scatter_prefill, paged_gather_kv and their E4M3-pool forms) live in
// blockops.hip; the files build into one library behind the C ABI of
// include/pagedattn.h.
//
// Sources (page title, section):
//   [Paged attention]     danielfleming.xyz/writing/inference/paged
//   [PagedAttention]      deepconcepts.dev/c/llm-paged-attention
//   [SLM paged attention] aicassindra.com/blogs/slm/slm_paged_attention.html
//
// This file holds the host side of decode attention (argument checks, the
// split plan, the workspace, launches) and the fp16-pool instances of
// decode_kernel; the kernel itself is in decode_kernel.h, and the E4M3-pool
// instances are in pagedattn_fp8.hip.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "decode_kernel.h"
#include "pagedattn.h"

namespace {

// ---------------------------------------------------------------------------
// workspace fill
// ---------------------------------------------------------------------------

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

DecodeFn pick_decode(int bs, int D, int nrep) { return pick_decode_t<false>(bs, D, nrep); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Split bounds, fixed on the host from sizes alone (no device value is read):
// at most P = min(kMaxParts, tiles of a full row) partials per (row, KV head),
// which holds when every busy workgroup takes at least C tiles. Tiles are
// tt tokens (tile_tokens of the pool format); the workspace is sized with
// the fp16 pools' 64-token tiles, which give the larger P.
struct Plan {
    long long wtiles;  // tiles of a full-width row
    int rows;          // rows per launch
    int C;             // tiles per busy workgroup, at least
    int P;             // partials per (row, KV head), at most
};

// Arrival counters: a fixed region at the start of the workspace, one int32
// per (row, KV head) of a launch, each on a 128-byte line of its own (the
// arrivals of different (row, KV head)s do not queue behind one another at the
// memory's atomic unit: measured 13.1 against 13.7 us at uniform 1024, 12.0
// against 12.4 on the mixed batch). Launches of one call run in order on one
// stream and each leaves its counters at zero, so they share the region.
constexpr int kCounterSlots = 8192;
constexpr size_t kCounterBytes = (size_t)kCounterSlots * kCounterStride * 4;  // 1 MiB

Plan make_plan(int B, int Hkv, int bs, int W, int tt) {
    Plan pl;
    pl.wtiles = ((long long)W * bs + tt - 1) / tt;
    pl.rows = std::max(1, std::min({B, kMaxRows, kCounterSlots / Hkv}));
    pl.P = (int)std::min<long long>(kMaxParts, pl.wtiles);
    // a (row, KV head) of nt tiles meets at most 1 + ceil((nt-1)/C) ranges of >= C tiles
    pl.C = pl.P > 1 ? (int)((pl.wtiles - 1 + pl.P - 2) / (pl.P - 1)) : 1;
    return pl;
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }
size_t partials_bytes(int B, int Hq, int D, int P) { return round256((size_t)B * P * Hq * (D + 2) * 4); }

// Workspace layout: the arrival counters in a fixed region at the start
// (kCounterBytes), then the fp32 partials of one launch's rows: (max, sum)
// per query head of every partition, then the unnormalised outputs. The
// counter region does not depend on the call's sizes, so no call's partials
// ever reach any call's counters, and a workspace sized for a shape serves
// every call whose partials fit in it.

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

// Resident workgroups per compute unit for a decode kernel, cached per
// (kernel, device) under a lock: the query is made once, and a reader never
// sees one kernel's entry with another's count.
int blocks_per_cu(const DecodeFn& f) {
    static std::mutex mu;
    static std::map<std::pair<const void*, int>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    const std::pair<const void*, int> key{f.fn, dev};
    std::lock_guard<std::mutex> lock(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, f.fn, f.threads, 0) != hipSuccess || occ <= 0) occ = 1;
    cache.emplace(key, occ);
    return occ;
}

// Scratch of paged_decode_attn_noalloc: the decode's workspace (arrival
// counters, then partials) in a static device array, so that the call
// allocates nothing. Every GPU the library runs on holds its own copy for
// the life of the process. In host code `scratch` only names the symbol: its
// device address on the current GPU comes from hipGetSymbolAddress, kept per
// device, and only that address is handed to kernels.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, guarded by g_scratch_mu

// The current device's scratch address. On the first call on a device its
// counter region is zero-filled by a kernel on `stream`, ahead of the
// caller's launch on the same stream; every later call finds the counters
// at zero, since each decode leaves them so.
pa_status scratch_for_current_device(void** ptr, hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PA_ERR_HIP;
        const size_t words = kCounterBytes / 4;
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                           static_cast<uint32_t*>(p), words);
        if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return PA_OK;
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
        case PA_ERR_SCRATCH:
            return "PA_ERR_SCRATCH: the call needs more workspace than the 32 MiB static scratch of "
                   "paged_decode_attn_noalloc holds";
        default: return "unknown pa_status";
    }
}

int paged_decode_supported(int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size) {
    if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads) return 0;
    return pick_decode(block_size, head_dim, num_heads / num_kv_heads).fn != nullptr;
}

size_t paged_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t max_blocks_per_seq) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_kv_heads > kCounterSlots ||
        num_heads % num_kv_heads || head_dim <= 0 || block_size <= 0 || max_blocks_per_seq <= 0)
        return 0;
    const Plan pl = make_plan(std::max(num_seqs, 1), num_kv_heads, block_size, max_blocks_per_seq, tile_tokens(false));
    // partials for min(B, kMaxRows) rows, a bound on a launch's rows that does not
    // depend on num_kv_heads, so that the size never shrinks when an argument grows
    return kCounterBytes + partials_bytes(std::min(std::max(num_seqs, 1), kMaxRows), num_heads, head_dim, pl.P);
}

pa_status paged_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 3u) || workspace_bytes % 4) return PA_ERR_INVALID_ARG;
    const size_t n = workspace_bytes / 4;
    if (n == 0) return PA_OK;
    const unsigned blocks = (unsigned)std::min<size_t>(1024, (n + 255) / 256);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (uint32_t*)workspace, n);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"

namespace {

// The pool's element format and its scales (E4M3 pools only; fp16 pools
// use fp8 = false and scales of 1).
struct PoolFormat {
    bool fp8;
    float k_scale, v_scale;
};
constexpr PoolFormat kFp16Pool = {false, 1.0f, 1.0f};

// paged_decode_attn, and with k_new/v_new (non-null) the same launch with
// kv_append of the step's K/V fused in (quantized for E4M3 pools).
pa_status launch_decode(uint16_t* out, const uint16_t* q, void* k_pool, void* v_pool, const int32_t* block_tables,
                        const int32_t* seq_lens, const uint16_t* k_new, const uint16_t* v_new, int32_t num_seqs,
                        int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t max_blocks_per_seq, int32_t num_blocks, float scale, void* workspace,
                        size_t workspace_bytes, void* stream, int32_t width = 0, PoolFormat fmt = kFp16Pool) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_kv_heads > kCounterSlots ||
        num_heads % num_kv_heads || head_dim <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
        !std::isfinite(scale))
        return PA_ERR_INVALID_ARG;
    auto scale_ok = [&](float x) { return std::isfinite(x) && (fmt.fp8 ? x >= 0x1p-96f && x <= 0x1p96f : x > 0.f); };
    if (!scale_ok(fmt.k_scale) || !scale_ok(fmt.v_scale)) return PA_ERR_INVALID_ARG;
    const int nrep = num_heads / num_kv_heads;
    DecodeFn fn = fmt.fp8 ? pa_detail::pick_decode_fp8(block_size, head_dim, nrep) : pick_decode(block_size, head_dim, nrep);
    if (!fn) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    if (!out || !q || !k_pool || !v_pool || !block_tables || !seq_lens) return PA_ERR_INVALID_ARG;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_INVALID_ARG;
    if ((k_new == nullptr) != (v_new == nullptr)) return PA_ERR_INVALID_ARG;
    if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return PA_ERR_INVALID_ARG;
    if ((long long)max_blocks_per_seq * block_size > 0x7fffffffLL / 2) return PA_ERR_INVALID_ARG;
    if (width < 0 || (long long)width > (long long)max_blocks_per_seq * block_size) return PA_ERR_INVALID_ARG;
    const size_t need = paged_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                                    max_blocks_per_seq);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return PA_ERR_WORKSPACE;
    const Plan pl = make_plan(num_seqs, num_kv_heads, block_size, max_blocks_per_seq, tile_tokens(fmt.fp8));
    const int slots = blocks_per_cu(fn) * cu_count();
    char* ws = static_cast<char*>(workspace);
    int32_t* counters = reinterpret_cast<int32_t*>(ws);
    float* part_ml = reinterpret_cast<float*>(ws + kCounterBytes);
    float* part_acc = part_ml + (size_t)pl.rows * pl.P * num_heads * 2;
    float sl2 = scale * fmt.k_scale * 1.4426950408889634f;
    float ksc = fmt.k_scale, vsc = fmt.v_scale, kinv = 1.0f / fmt.k_scale, vinv = 1.0f / fmt.v_scale;
    int Hkv = num_kv_heads, W = max_blocks_per_seq, N = num_blocks, C = pl.C, P = pl.P;
    // Rows are processed pl.rows at a time (the workgroups keep the rows'
    // lengths in LDS); each launch covers its own rows of q, out, the tables
    // and the new tokens, and reuses the counters and partials of the one
    // before it, which it follows on the stream.
    for (int r0 = 0; r0 < num_seqs; r0 += pl.rows) {
        int Bc = std::min(pl.rows, num_seqs - r0);
        const long long grid = std::min<long long>(slots, (long long)Bc * Hkv * pl.wtiles);
        uint16_t* o = out + (size_t)r0 * num_heads * head_dim;
        const uint16_t* qq = q + (size_t)r0 * num_heads * head_dim;
        const int32_t* tt = block_tables + (size_t)r0 * max_blocks_per_seq;
        const int32_t* ll = seq_lens + r0;
        const uint16_t* kn = k_new ? k_new + (size_t)r0 * num_kv_heads * head_dim : nullptr;
        const uint16_t* vn = v_new ? v_new + (size_t)r0 * num_kv_heads * head_dim : nullptr;
        int32_t* cc = counters;
        float* pm = part_ml;
        float* pa = part_acc;
        void* args[] = {&o, (void*)&qq, (void*)&k_pool, (void*)&v_pool, (void*)&tt, (void*)&ll, (void*)&kn,
                        (void*)&vn, &cc, &pm, &pa, &Bc, &Hkv, &W, &N, &C, &P, &sl2, &width, &ksc, &vsc, &kinv, &vinv};
        if (hipLaunchKernel(fn.fn, dim3((unsigned)grid), dim3(fn.threads), args, 0, (hipStream_t)stream) !=
            hipSuccess)
            return PA_ERR_HIP;
    }
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" {

pa_status paged_decode_attn(uint16_t* out, const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                            const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t max_blocks_per_seq, int32_t num_blocks, float scale, void* workspace,
                            size_t workspace_bytes, void* stream) {
    // the pools are only read on this path (no k_new: nothing is stored into them)
    return launch_decode(out, q, const_cast<uint16_t*>(k_pool), const_cast<uint16_t*>(v_pool), block_tables,
                         seq_lens, nullptr, nullptr, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                         max_blocks_per_seq, num_blocks, scale, workspace, workspace_bytes, stream);
}

pa_status paged_decode_attn_noalloc(uint16_t* out, const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                                    const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                                    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t max_blocks_per_seq, int32_t num_blocks, float scale, void* stream) {
    const size_t need = paged_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                                    max_blocks_per_seq);
    if (need == 0) return PA_ERR_INVALID_ARG;
    if (need > kScratchBytes) return PA_ERR_SCRATCH;
    void* ws = nullptr;
    const pa_status st = scratch_for_current_device(&ws, (hipStream_t)stream);
    if (st != PA_OK) return st;
    return launch_decode(out, q, const_cast<uint16_t*>(k_pool), const_cast<uint16_t*>(v_pool), block_tables,
                         seq_lens, nullptr, nullptr, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                         max_blocks_per_seq, num_blocks, scale, ws, kScratchBytes, stream);
}

pa_status paged_decode_attn_masked(uint16_t* out, const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                                   const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                                   int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t max_blocks_per_seq, int32_t num_blocks, float scale, int32_t width,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    if (width <= 0) return PA_ERR_INVALID_ARG;
    return launch_decode(out, q, const_cast<uint16_t*>(k_pool), const_cast<uint16_t*>(v_pool), block_tables,
                         seq_lens, nullptr, nullptr, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                         max_blocks_per_seq, num_blocks, scale, workspace, workspace_bytes, stream, width);
}

pa_status paged_decode_attn_fp8(uint16_t* out, const uint16_t* q, const uint8_t* k_pool, const uint8_t* v_pool,
                                const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                                int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int32_t max_blocks_per_seq, int32_t num_blocks, float scale, float k_scale,
                                float v_scale, void* workspace, size_t workspace_bytes, void* stream) {
    return launch_decode(out, q, const_cast<uint8_t*>(k_pool), const_cast<uint8_t*>(v_pool), block_tables, seq_lens,
                         nullptr, nullptr, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                         max_blocks_per_seq, num_blocks, scale, workspace, workspace_bytes, stream, 0,
                         PoolFormat{true, k_scale, v_scale});
}

pa_status paged_decode_attn_append_fp8(uint16_t* out, const uint16_t* q, const uint16_t* k_new,
                                       const uint16_t* v_new, uint8_t* k_pool, uint8_t* v_pool,
                                       const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                       int32_t max_blocks_per_seq, int32_t num_blocks, float scale, float k_scale,
                                       float v_scale, void* workspace, size_t workspace_bytes, void* stream) {
    if (num_seqs > 0 && (!k_new || !v_new)) return PA_ERR_INVALID_ARG;
    return launch_decode(out, q, k_pool, v_pool, block_tables, seq_lens, k_new, v_new, num_seqs, num_heads,
                         num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale, workspace,
                         workspace_bytes, stream, 0, PoolFormat{true, k_scale, v_scale});
}

pa_status paged_decode_attn_append(uint16_t* out, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                                   uint16_t* k_pool, uint16_t* v_pool, const int32_t* block_tables,
                                   const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t max_blocks_per_seq, int32_t num_blocks, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    if (num_seqs > 0 && (!k_new || !v_new)) return PA_ERR_INVALID_ARG;
    return launch_decode(out, q, k_pool, v_pool, block_tables, seq_lens, k_new, v_new, num_seqs, num_heads,
                         num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale, workspace,
                         workspace_bytes, stream);
}

}  // extern "C"
