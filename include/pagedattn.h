/*
 * libpagedattn -- paged KV-cache decode attention for AMD Instinct MI355X
 * (gfx950), behind a C ABI.
 *
 * Sources (page title, section):
 *   [Paged attention]     danielfleming.xyz/writing/inference/paged
 *   [PagedAttention]      deepconcepts.dev/c/llm-paged-attention
 *   [SLM paged attention] aicassindra.com/blogs/slm/slm_paged_attention.html
 *
 * The problem. Keys and values of every sequence live in one preallocated
 * pool cut into equal blocks of `block_size` tokens [SLM paged attention,
 * "The architecture: every piece explained"]. Each sequence owns a block
 * table: entry n is the physical block that holds its tokens
 * n*block_size .. (n+1)*block_size-1 [PagedAttention, intro; SLM paged
 * attention, same section]. A decode step appends the new token's K/V into
 * the sequence's last block, a fresh block having been appended to the table
 * by the host when the previous one filled [SLM paged attention, "End-to-end
 * flow"], and then attends, for each sequence, over only the blocks its table
 * lists, at its own true length [Paged attention, "What changed"]. The result
 * is exact softmax attention; splitting the sum over blocks does not change
 * it [PagedAttention, "Sharing is the part that pays twice"]. Several query
 * heads share one KV head (grouped-query attention: 12 query heads over 2 KV
 * heads for Qwen2.5-1.5B [Paged attention, "What a small pool does"]).
 *
 * ---------------------------------------------------------------------------
 * Conventions shared by every call
 * ---------------------------------------------------------------------------
 *  - All data pointers are DEVICE pointers (hipMalloc / torch CUDA tensors)
 *    owned by the caller. The library allocates nothing and keeps no state
 *    between calls except per-device caches of the compute-unit count and
 *    of each decode kernel's resident workgroups per compute unit.
 *  - fp16 data is passed as uint16_t bit patterns (IEEE binary16).
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *    enqueues work on it and returns; there is no host synchronisation and
 *    no device value is read on the host.
 *  - Shapes (row-major, innermost last):
 *      q, out         [B][Hq][D]
 *      k_new, v_new   [B][Hkv][D]
 *      k_pool         [N][Hkv][D/8][block_size][8]   (8 channels = 16 bytes,
 *                                                     token-minor)
 *      v_pool         [N][Hkv][D][block_size]        (tokens contiguous)
 *      block_tables   [B][W] int32, W = max_blocks_per_seq
 *      seq_lens       [B]    int32
 *    B = num_seqs, Hq = num_heads, Hkv = num_kv_heads, D = head_dim,
 *    N = num_blocks. Query head h reads KV head h / (Hq / Hkv).
 *  - seq_lens[b] is the row's length INCLUDING the token of this step: the
 *    append writes position seq_lens[b]-1 and attention covers positions
 *    0 .. seq_lens[b]-1. A row with seq_lens[b] == 0 is skipped by
 *    kv_append and gets zeros from paged_decode_attn.
 *  - Table entries at index >= ceil(seq_lens[b] / block_size) are never
 *    read and may hold anything (e.g. -1). Pool slots outside every row's
 *    live range may hold anything, including NaN.
 *  - Device-data preconditions (not checked on the host, since checking
 *    would need a device read): live table entries lie in [0, N);
 *    seq_lens[b] <= W * block_size; in kv_append no two rows target the
 *    same slot and no row appends into a block another row also lists.
 *    Violations give unspecified results but never an out-of-bounds access:
 *    the kernels clamp block ids into [0, N) and lengths into [0, W*bs].
 *
 * Errors: every call returns PA_OK, or a status before anything is
 * enqueued (PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE), or
 * PA_ERR_HIP if the launch itself failed. pa_status_string() names them.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, Hq % Hkv != 0, misalignment */
    PA_ERR_UNSUPPORTED = 2, /* (block_size, head_dim, Hq/Hkv) combination not compiled in */
    PA_ERR_HIP = 3,         /* the kernel launch failed */
    PA_ERR_WORKSPACE = 4,   /* workspace null or smaller than paged_decode_workspace_size() */
    PA_ERR_SCRATCH = 5      /* paged_decode_attn_noalloc: the call needs more than its 32 MiB scratch */
} pa_status;

/* Static string naming a status. Never NULL. */
const char *pa_status_string(int status);

/* 1 if paged_decode_attn has a kernel for this shape, else 0.
 * Compiled in: block_size in {16, 32, 64, 128, 256}, head_dim in {64, 128},
 * num_heads / num_kv_heads in {1, 2, 4, 6, 8}. */
int paged_decode_supported(int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size);

/*
 * kv_append -- write one decode step's new key and value of every row into
 * the row's last block [SLM paged attention, "End-to-end flow": a sequence
 * grows one block at a time, the host appending a fresh block from the free
 * list when the current one fills; "The architecture: every piece
 * explained": logical block index = position / block_size].
 *
 * For each row b with L = seq_lens[b] >= 1: pos = L-1,
 * blk = block_tables[b][pos / block_size], slot = pos % block_size, and for
 * every KV head g and channel d
 *     K[blk][g][d/8][slot][d%8] = k_new[b][g][d]
 *     V[blk][g][d][slot]        = v_new[b][g][d]
 * A pure bit copy; no other pool byte changes. Rows whose target block id is
 * outside [0, N) or whose L exceeds W*block_size are skipped.
 * k_new, v_new: 16-byte aligned. Supported: head_dim % 8 == 0, any
 * block_size >= 1 (block_size % 8 == 0 not required).
 */
pa_status kv_append(const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool, uint16_t *v_pool,
                    const int32_t *block_tables, const int32_t *seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                    void *stream);

/*
 * Bytes of device workspace paged_decode_attn needs for these sizes: a fixed
 * region of 1 MiB at the start holding the int32 arrival counters of the
 * split-sequence reduction (one per (row, KV head) of a launch, each on a
 * 128-byte line of its own), then the
 * fp32 partial results (max, sum, unnormalised output per query head) of up
 * to P = min(64, T) sequence partitions per (row, KV head) of min(num_seqs,
 * 256) rows, T = ceil(W*block_size/64) being the number of 64-token tiles
 * of a full row, rounded up to 256 bytes. A launch covers
 * min(num_seqs, 256, 8192 / num_kv_heads) rows; larger batches run as
 * several launches in order on the stream, which reuse the same counters
 * and partials. The value never decreases when any argument grows. The same
 * size serves the E4M3-pool calls (their 128-token tiles give at most as
 * many partitions). Returns 0 for invalid sizes (num_kv_heads > 8192
 * included).
 */
size_t paged_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t max_blocks_per_seq);

/*
 * Zero a workspace with a device fill kernel (no memset, so it may be
 * captured in a HIP graph). A workspace must be all-zero before its first
 * paged_decode_attn call. The counters sit in a region of fixed size at its
 * start that no partial result ever overlaps, and every completed call
 * leaves its counters at zero again, so one init per allocation suffices
 * for any sequence of calls whose workspace size the allocation covers
 * (e.g. sized with the largest num_seqs and max_blocks_per_seq used).
 */
pa_status paged_decode_workspace_init(void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_decode_attn -- one query token per row, grouped-query softmax
 * attention over the row's own blocks at its true length [Paged attention,
 * "What changed"; PagedAttention, "What the block table costs": read the
 * table, resolve each logical block to a physical one, gather;
 * PagedAttention, "Sharing is the part that pays twice": block-wise softmax
 * rescaled and combined exactly].
 *
 *   out[b][h][:] = sum_t softmax_t(scale * q[b][h] . k_t) v_t,
 *   t = 0 .. seq_lens[b]-1, k_t / v_t from block block_tables[b][t/bs],
 *   slot t % bs, KV head h / (Hq/Hkv).
 *
 * fp32 accumulation, fp16 output (round to nearest even). Long rows are
 * split into partitions whose partial (max, sum, output) are merged in
 * partition order by the last partition to finish, so results are
 * bit-identical from run to run.
 * q, out, k_pool, v_pool: 16-byte aligned. workspace: at least
 * paged_decode_workspace_size() bytes, 256-byte aligned, zeroed once by
 * paged_decode_workspace_init() (or any zero fill) before first use. Calls
 * that are in flight at the same time must use different workspaces.
 * Unsupported shapes (see paged_decode_supported) return PA_ERR_UNSUPPORTED.
 */
pa_status paged_decode_attn(uint16_t *out, const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                            const int32_t *block_tables, const int32_t *seq_lens, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t max_blocks_per_seq, int32_t num_blocks, float scale, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * paged_decode_attn_noalloc -- paged_decode_attn for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments,
 * conventions, results (bit-identical, same kernel) and errors as
 * paged_decode_attn, without the workspace arguments: the workspace is a
 * static device array inside the library, 32 MiB per GPU, held by every GPU
 * the library runs on until the process ends. The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); it only enqueues
 * the decode on `stream`, and on its first call on a device also a small
 * zero fill of the array's counter region ahead of it.
 * Limit: calls whose paged_decode_workspace_size() exceeds 32 MiB return
 * PA_ERR_SCRATCH before anything is enqueued (e.g. 32 rows of 12/2/128 heads
 * with tables of up to 300 blocks of 64 tokens need 13.2 MiB).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: two calls in flight at the same time on one GPU (different
 * streams, or a graph replayed concurrently with a direct call) race on it
 * and give unspecified results. Calls in order on one stream are safe.
 */
pa_status paged_decode_attn_noalloc(uint16_t *out, const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                    const int32_t *block_tables, const int32_t *seq_lens, int32_t num_seqs,
                                    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t max_blocks_per_seq, int32_t num_blocks, float scale, void *stream);

/*
 * paged_decode_attn_append -- kv_append followed by paged_decode_attn, in one
 * launch: a decode step's two calls [SLM paged attention, "End-to-end flow":
 * the new token's K/V enter the row's last block, then attention runs over the
 * row's blocks at its new length]. The results are bit-identical to
 *     kv_append(k_new, v_new, k_pool, v_pool, ...);
 *     paged_decode_attn(out, q, k_pool, v_pool, ...);
 * on the same stream: the pools end up with the same bytes and `out` holds
 * the same values. Inside the launch the workgroup that owns a row's last tile
 * takes the new token's K/V straight from k_new / v_new (staged in LDS), so no
 * read depends on the write, and stores them into the pool for later steps.
 * Same arguments, alignment, workspace and errors as paged_decode_attn, plus
 * k_new, v_new: [num_seqs][num_kv_heads][head_dim] fp16, 16-byte aligned,
 * non-null. The append side follows kv_append: nothing is written for rows
 * with L < 1, L > W*block_size or a target block id outside [0, N) (for the
 * last, the attention result is unspecified, as is paged_decode_attn's for an
 * invalid table entry). Appending into a block that another row reads in the
 * same call (a shared block) is outside the contract, as for kv_append.
 */
pa_status paged_decode_attn_append(uint16_t *out, const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                                   uint16_t *k_pool, uint16_t *v_pool, const int32_t *block_tables,
                                   const int32_t *seq_lens, int32_t num_seqs, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t max_blocks_per_seq, int32_t num_blocks, float scale, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * paged_decode_attn_masked -- the contrast of the earlier contiguous engine:
 * the same result as paged_decode_attn, computed the way a cache of one
 * fixed-width slot per row computes it [Paged attention, "What changed": the
 * earlier engine reserved the widest row's width for every row and masked
 * the unused columns, which hid the data but not the work; Continuous
 * batching, "What changed": a mask tells the decode which cache columns
 * belong to which row]. Every
 * row with seq_lens[b] >= 1 reads and scores max(width, seq_lens[b]) tokens
 * (its table must list that many tokens' worth of valid blocks), and positions at or past
 * seq_lens[b] are masked out of the softmax and the output. With an identity
 * table (row b's blocks b*W .. b*W+W-1) it is the contiguous layout. For
 * measurement only; results equal paged_decode_attn's to the same tolerance.
 * Same arguments, workspace and errors as paged_decode_attn, plus
 * 1 <= width <= max_blocks_per_seq * block_size (else PA_ERR_INVALID_ARG).
 */
pa_status paged_decode_attn_masked(uint16_t *out, const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                   const int32_t *block_tables, const int32_t *seq_lens, int32_t num_seqs,
                                   int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t max_blocks_per_seq, int32_t num_blocks, float scale, int32_t width,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * kv_copy_blocks -- whole-block copies for copy-on-write: for every i <
 * num_pairs, block dst[i] of both pools takes the contents of block src[i]
 * (every KV head and every slot, K and V; a bit copy) [SLM paged attention,
 * "The architecture: every piece explained": the manager clones the one
 * shared block a sequence must write into and repoints that sequence's table
 * entry, leaving the readers untouched; "End-to-end flow"; PagedAttention,
 * "Sharing is the part that pays twice": a shared block counts its readers,
 * and only the one that a row starts to change is copied for that row]. Which
 * blocks to copy is the caller's bookkeeping
 * (paged_kv_cache_06_amd.blocks.plan_copy_on_write does it on the
 * host); run the copies before the step's kv_append.
 *
 * src, dst: device int32 [num_pairs]. A pair with an id outside [0, N), or
 * with src == dst, is skipped. No dst may appear twice or also be a src in
 * the same call (the copies run concurrently; such a call has no defined
 * result). k_pool, v_pool: 16-byte aligned, layouts as for kv_append. With
 * num_layers > 1 the pools hold num_layers layers of N blocks each,
 * layer_stride halves apart (a multiple of 8, at least N*Hkv*D*block_size),
 * the same block ids in every layer, and every layer is copied; with
 * num_layers == 1 layer_stride is ignored. num_pairs == 0 returns PA_OK.
 */
pa_status kv_copy_blocks(uint16_t *k_pool, uint16_t *v_pool, const int32_t *src, const int32_t *dst, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                         int32_t num_layers, int64_t layer_stride, void *stream);

/*
 * kv_scatter_prefill -- after a prefill, move each row's prompt K/V into its
 * blocks [Paged attention, "What changed": requests admitted together run
 * one prefill, their prompts padded on the left to the longest of them; each
 * row's keys and values then go into its own blocks without the padding].
 *
 * k_src, v_src: [num_seqs][Hkv][S][D] fp16 (S = padded_len, token-major rows
 * of D channels), 16-byte aligned; row b's prompt of length P =
 * prompt_lens[b] occupies positions S-P .. S-1. For t < P:
 *     K[block_tables[b][t/bs]][g][d/8][t%bs][d%8] = k_src[b][g][S-P+t][d]
 *     V[block_tables[b][t/bs]][g][d][t%bs]        = v_src[b][g][S-P+t][d]
 * A bit copy; slots past P and unlisted blocks are untouched. Rows with P <= 0
 * are skipped, and so are rows with P > S or P > W*block_size; a table entry
 * outside [0, N) skips that block's tokens. Host checks: head_dim % 8 == 0,
 * num_seqs and num_kv_heads <= 65535, block_size <= 1024, and the LDS
 * transpose tile (max of D/8*(bs+1)*16 and D*(bs+8)*2 bytes) within 64 KiB,
 * else PA_ERR_UNSUPPORTED. The tables must give each row private blocks for
 * its prompt (no two rows writing one slot).
 */
pa_status kv_scatter_prefill(const uint16_t *k_src, const uint16_t *v_src, uint16_t *k_pool, uint16_t *v_pool,
                             const int32_t *block_tables, const int32_t *prompt_lens, int32_t num_seqs,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                             int32_t num_blocks, int32_t padded_len, void *stream);

/*
 * FP8 pools. A pool of 8-bit floats holds half the bytes per token of an
 * fp16 pool; the dtype is one of the terms that set bytes per token, which
 * paging itself leaves alone [PagedAttention, "Three wastes wearing one
 * name"; "Checking it on a real system": FP8 KV]. The pages fix neither the
 * format nor the scaling; this library takes E4M3 as in the OCP 8-bit
 * floating point specification (bias 7, 3 mantissa bits, no infinity, NaN
 * = 0x7f/0xff, largest finite 448) with one fp32 scale for every K element
 * of the pool and one for every V element: element value = code * scale.
 * Every FP8 call takes the scales finite and within [2^-96, 2^96]
 * (else PA_ERR_INVALID_ARG): over that range the kernels' quotient x / scale
 * is the correctly rounded one.
 *   k_pool  [N][Hkv][D/16][block_size][16] bytes (16 channels = 16 bytes,
 *                                                token-minor)
 *   v_pool  [N][Hkv][D][block_size]        bytes (tokens contiguous)
 * head_dim must be a multiple of 16; block_size, head_dim and Hq/Hkv as for
 * the fp16 pools (paged_decode_supported).
 */

/*
 * kv_append_fp8 -- kv_append into FP8 pools: the new token's K and V
 * elements x (fp16) are stored as the E4M3 code of x / scale, the quotient
 * rounded to fp32 (one correctly rounded division), then to the nearest
 * code with ties to the even mantissa; magnitudes from 448 up saturate to
 * 448, NaN stays NaN (0x7f) and the sign is kept. Same rows skipped and same
 * preconditions as kv_append. k_scale, v_scale: finite, in [2^-96, 2^96],
 * else PA_ERR_INVALID_ARG; head_dim % 16 != 0 is PA_ERR_INVALID_ARG.
 */
pa_status kv_append_fp8(const uint16_t *k_new, const uint16_t *v_new, uint8_t *k_pool, uint8_t *v_pool,
                        const int32_t *block_tables, const int32_t *seq_lens, int32_t num_seqs,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                        int32_t num_blocks, float k_scale, float v_scale, void *stream);

/*
 * paged_decode_attn_fp8 -- paged_decode_attn over FP8 pools: the attention
 * of q (fp16) over key values code * k_scale and value values code *
 * v_scale. Codes are widened to fp16 exactly; k_scale is folded into the
 * score scale and v_scale applied to the output. Arguments, workspace
 * (paged_decode_workspace_size) and errors as paged_decode_attn, plus
 * k_scale, v_scale finite and in [2^-96, 2^96] (else PA_ERR_INVALID_ARG);
 * k_pool and v_pool 16-byte aligned.
 */
pa_status paged_decode_attn_fp8(uint16_t *out, const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                                const int32_t *block_tables, const int32_t *seq_lens, int32_t num_seqs,
                                int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int32_t max_blocks_per_seq, int32_t num_blocks, float scale, float k_scale,
                                float v_scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_decode_attn_append_fp8 -- kv_append_fp8 followed by
 * paged_decode_attn_fp8 in one launch, as paged_decode_attn_append is for
 * fp16 pools: the pools and the output are bit-identical to the two calls'.
 * The new token's codes are written into the tile in LDS and into the pool
 * by the workgroup that reads the row's last tile. k_new, v_new: [B][Hkv][D]
 * fp16, 16-byte aligned, non-null when num_seqs > 0. Arguments, workspace
 * and errors otherwise as paged_decode_attn_fp8; the preconditions of
 * kv_append hold.
 */
pa_status paged_decode_attn_append_fp8(uint16_t *out, const uint16_t *q, const uint16_t *k_new,
                                       const uint16_t *v_new, uint8_t *k_pool, uint8_t *v_pool,
                                       const int32_t *block_tables, const int32_t *seq_lens, int32_t num_seqs,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                       int32_t max_blocks_per_seq, int32_t num_blocks, float scale, float k_scale,
                                       float v_scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * kv_copy_blocks_fp8 -- kv_copy_blocks for FP8 pools (copy-on-write of
 * shared E4M3 blocks): block dst[i] of both pools takes block src[i]'s
 * bytes, every KV head and slot. Same pair rules and errors as
 * kv_copy_blocks; head_dim % 16 == 0; with num_layers > 1, layer_stride is
 * in bytes (a multiple of 16, at least N*Hkv*D*block_size).
 */
pa_status kv_copy_blocks_fp8(uint8_t *k_pool, uint8_t *v_pool, const int32_t *src, const int32_t *dst,
                             int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t num_layers, int64_t layer_stride, void *stream);

/*
 * kv_scatter_prefill_fp8 -- kv_scatter_prefill into FP8 pools: token t of
 * row b goes to block block_tables[b][t/bs], slot t%bs, every element
 * quantized as in kv_append_fp8 (the code of x / scale, k_scale for keys,
 * v_scale for values), in the E4M3 layouts. Same row and block skips as
 * kv_scatter_prefill. Host checks: head_dim % 16 == 0 and block_size % 16 ==
 * 0 (else PA_ERR_INVALID_ARG), scales as for every FP8 call, the staging tile
 * (max of bs*(D+16) and D*(bs+16) bytes) within 64 KiB (else
 * PA_ERR_UNSUPPORTED).
 */
pa_status kv_scatter_prefill_fp8(const uint16_t *k_src, const uint16_t *v_src, uint8_t *k_pool, uint8_t *v_pool,
                                 const int32_t *block_tables, const int32_t *prompt_lens, int32_t num_seqs,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t max_blocks_per_seq, int32_t num_blocks, int32_t padded_len, float k_scale,
                                 float v_scale, void *stream);

/*
 * pa_probe_read -- measurement aid, not part of the decode path: reads
 * `bytes` bytes of device memory at `src` once (16 bytes per lane,
 * grid-stride, non-temporal), so that the time of a plain read of a byte
 * count (launch and ramp included) can be set beside a kernel that reads
 * that many bytes. sink: device uint32 [num_workgroups], overwritten with
 * values of no meaning. src 16-byte aligned, bytes a positive multiple of 16,
 * num_workgroups > 0 (else PA_ERR_INVALID_ARG).
 */
pa_status pa_probe_read(const void *src, size_t bytes, uint32_t *sink, int32_t num_workgroups, void *stream);

/*
 * paged_gather_kv -- debug path that reads the same blocks the decode kernel
 * reads and writes them out contiguously [Paged attention, "What changed":
 * the block machinery was first checked through a path that reads the same
 * blocks with the earlier dense kernel].
 *   k_out[b][g][t][d] = K[block_tables[b][t/bs]][g][d/8][t%bs][d%8]
 *   v_out[b][g][t][d] = V[block_tables[b][t/bs]][g][d][t%bs]
 * for t < seq_lens[b]; k_out / v_out are [B][Hkv][W*block_size][D] and their
 * positions t >= seq_lens[b] are left untouched.
 */
pa_status paged_gather_kv(uint16_t *k_out, uint16_t *v_out, const uint16_t *k_pool, const uint16_t *v_pool,
                          const int32_t *block_tables, const int32_t *seq_lens, int32_t num_seqs,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                          int32_t num_blocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
