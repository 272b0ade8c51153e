/*
 * pagedkv.h -- C ABI of libpagedkv: single-token decode attention over a paged
 * KV cache on AMD Instinct MI355X (gfx950).
 *
 * What the operations are (from the pages this library follows):
 *  - The cache keeps, for every layer and every token, one key and one value
 *    vector per KV head; each decode step appends the new token's K and V and
 *    then attends over the whole cache, the new token included
 *    ("KV cache and PagedAttention", askaiml.pages.dev, §1 "The setup";
 *    "Memoizing Context via KV Caching", blog.sanjeevnode.in).
 *  - Storage is a pool of fixed-size pages; each request owns a table of page
 *    indices and the attention kernel gathers K/V through it; pages are
 *    uniform so handing one out is O(1); requests with a common prefix may map
 *    the same pages (askaiml page, §4 "PagedAttention"; "KV Cache" glossary,
 *    inferensys.com, PagedAttention block management).
 *  - Several query heads may share one KV head (GQA; MQA when there is a single
 *    KV head) ("KV Cache" glossary, GQA and MQA entries).
 *  - The cache may be held in fp8 E4M3 or INT8 to halve its bytes (askaiml page, §7
 *    "KV cache quantisation").
 *
 * Conventions for every function:
 *  - Every status-returning function returns a kv_status; nothing aborts or
 *    throws.  On a non-OK return, kv_last_error() gives a message for the
 *    calling thread.  Host-side state is unchanged by a failed call unless the
 *    function says otherwise.
 *  - Exhausted host memory is reported as KV_E_INVALID with a "host memory"
 *    message.  kv_pool_create then creates nothing, and the batch
 *    reservations and kv_window_release change nothing (they allocate before
 *    they change any state).  After such an error from kv_prefix_match,
 *    kv_prefix_insert or kv_prefix_evict, the prefix cache and the
 *    reference counts it holds are unspecified.
 *  - Device pointers are HIP device addresses on the current device; host
 *    pointers are ordinary process memory.  The library never allocates,
 *    frees or copies device memory itself: the caller owns every buffer, and
 *    the buffers given to kv_pool_create must outlive the pool.
 *  - Device work is enqueued on the caller's HIP stream (`hip_stream`, a
 *    hipStream_t; NULL means the default stream) and is asynchronous; argument
 *    checks are synchronous.  A failed launch returns KV_E_HIP.
 *  - Values stored in device memory (block-table entries, context lengths,
 *    slot mappings) are a caller contract: they are not bounds-checked by the
 *    kernels.  Every table entry a decode reads must name a block in
 *    [0, num_blocks); every slot must be -1 or lie in [0, num_blocks*block_size).
 *  - Host functions are not thread-safe for one pool (one scheduler thread).
 *
 * Pool layout in device memory, one array for K and one for V, each indexed
 *   K: [num_layers][num_blocks][num_kv_heads][block_size][head_dim]  token-major
 *   V: [num_layers][num_blocks][num_kv_heads][head_dim][block_size]  dim-major
 * Element type: float (KV_F32), bfloat16 (KV_BF16), E4M3 code bytes
 * (KV_FP8_E4M3) or symmetric int8 codes (KV_INT8).  Each (block, kv-head) tile
 * of K and of V is contiguous.
 * fp8 and int8 pools also take two fp32 scale arrays [num_layers][num_blocks][num_kv_heads],
 * one for K and one for V; a stored element means decode(code) * scale.
 * Supported: block_size 16, head_dim 64 or 128.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kv_pool kv_pool; /* opaque; holds host allocator state only */

typedef enum { KV_F32 = 0, KV_BF16 = 1, KV_FP8_E4M3 = 2, KV_INT8 = 3 } kv_dtype;

typedef enum {
  KV_OK = 0,
  KV_E_INVALID = -1,     /* bad argument (null pointer, size, range)          */
  KV_E_UNSUPPORTED = -2, /* shape or dtype not built into the library          */
  KV_E_NO_BLOCKS = -3,   /* the free list is empty                             */
  KV_E_BAD_BLOCK = -4,   /* block id out of range, or not currently allocated  */
  KV_E_SHARED = -5,      /* write into a block mapped by more than one table   */
  KV_E_WORKSPACE = -6,   /* workspace missing or smaller than required         */
  KV_E_HIP = -7          /* a HIP runtime call or kernel launch failed         */
} kv_status;

typedef struct {
  int32_t num_layers;   /* >= 1                                     */
  int32_t num_blocks;   /* physical pages per layer, >= 1           */
  int32_t block_size;   /* tokens per page; must be 16              */
  int32_t num_kv_heads; /* >= 1                                     */
  int32_t head_dim;     /* 64 or 128                                */
  int32_t cache_dtype;  /* a kv_dtype                               */
} kv_pool_desc;

/* ---------------------------------------------------------------- sizes -- */

/* Bytes of K plus V one token occupies across all layers:
 * 2 * num_layers * num_kv_heads * head_dim * element bytes (fp8 / int8 scales not
 * included) -- the per-token memory formula of the askaiml page, §2
 * "Memory cost".  Returns -1 for an invalid descriptor. */
int64_t kv_bytes_per_token(const kv_pool_desc* desc);

/* Pages needed for n tokens: ceil(n / block_size) (askaiml page, §4: a
 * 17-token request holds 2 pages of 16).  Returns -1 if n < 0 or
 * block_size <= 0. */
int32_t kv_blocks_for_tokens(int32_t n, int32_t block_size);

/* Bytes the caller must allocate for the K array (the V array is the same
 * size) and for each scale array (fp8 and int8 pools; 0 otherwise).  Either output
 * pointer may be NULL. */
int kv_pool_buffer_bytes(const kv_pool_desc* desc, int64_t* cache_bytes, int64_t* scale_bytes);

/* ----------------------------------------------------------------- pool -- */

/* Create a pool over caller-owned device arrays (layout above).  k_scale and
 * v_scale are device fp32 arrays for fp8 and int8 pools and must be NULL otherwise.
 * initial_free_order: host array of num_blocks distinct ids (a permutation of
 * 0..num_blocks-1) giving the order in which a fresh pool hands blocks out
 * (first kv_block_alloc returns initial_free_order[0]); NULL means 0,1,2,...
 * The pool copies what it needs from the descriptor and the order array. */
int kv_pool_create(const kv_pool_desc* desc, void* k_cache, void* v_cache, float* k_scale,
                   float* v_scale, const int32_t* initial_free_order, kv_pool** out);

/* Release the host state.  The device arrays are untouched. NULL is accepted. */
int kv_pool_destroy(kv_pool* pool);

/* ------------------------------------------------------------ allocator -- */
/* O(1) free-list allocator with reference counts (askaiml page, §4: uniform
 * pages, O(1) allocation, prefix pages shared between requests).  Free blocks
 * form a LIFO stack: a released block is the next one handed out. */

/* Pop a free block into *block and set its count to 1.  KV_E_NO_BLOCKS when
 * none is free. */
int kv_block_alloc(kv_pool* pool, int32_t* block);

/* Add one mapping to an allocated block (another block table now lists it).
 * KV_E_BAD_BLOCK if out of range or free. */
int kv_block_retain(kv_pool* pool, int32_t block);

/* Drop one mapping; at zero the block is pushed on the free stack.
 * KV_E_BAD_BLOCK if out of range or already free (double release). */
int kv_block_release(kv_pool* pool, int32_t block);

/* Retain, or release, each of the n blocks of `blocks` (host array) in order:
 * one mapping more (or less) per entry, as when a request that shares a
 * prefix is admitted (or retired).  On an error the entries already processed
 * are undone in reverse order, so counts and the free stack are exactly as
 * before the call, and the status of the failing entry is returned. */
int kv_block_retain_n(kv_pool* pool, const int32_t* blocks, int32_t n);
int kv_block_release_n(kv_pool* pool, const int32_t* blocks, int32_t n);

/* Current reference count (0 for a free block).  KV_E_BAD_BLOCK if out of range. */
int kv_block_refcount(const kv_pool* pool, int32_t block, int32_t* rc);

/* Number of free blocks. */
int kv_num_free_blocks(const kv_pool* pool, int32_t* n);

/* Number of blocks whose reference count is at least 2: pages that several
 * block tables, or a table and the prefix cache, map (askaiml page, §4 and
 * §6: shared prefix pages).  The decode reads K/V with the non-temporal cache
 * hint while this is 0, and with plain loads otherwise, so that the caches
 * serve the repeated reads of a shared page. */
int kv_num_shared_blocks(const kv_pool* pool, int32_t* n);

/* --------------------------------------------------------- slot mapping -- */

/* Host: slots_out[i] = table_row[positions[i] / block_size] * block_size
 *                      + positions[i] % block_size,
 * the physical slot that position i of a request writes (askaiml page, §4:
 * per-request page table).  table_row: host [n_table]; positions, slots_out:
 * host [n].  Errors: KV_E_INVALID for a negative position or one beyond the
 * table; KV_E_BAD_BLOCK if the block is out of range or free; KV_E_SHARED if
 * it is mapped more than once (a shared page is never written in place).
 * slots_out is unspecified after an error. */
int kv_slot_mapping(const kv_pool* pool, const int32_t* table_row, int32_t n_table,
                    const int32_t* positions, int32_t n, int32_t* slots_out);

/* Host: the allocator and slot-mapping half of one decode step for a batch.
 * For each request b in [0, B): it currently holds lens[b] tokens and will
 * append n_new[b] more.  Blocks that positions lens[b] .. lens[b]+n_new[b]-1
 * need and that the request does not hold yet are allocated (in request
 * order, then block order) and written into table[b * max_blocks + j]; the
 * slots of those positions are written to slots_out, request after request
 * (sum of n_new entries); lens[b] is advanced by n_new[b].
 * table, lens: host, read and written; n_new: host [B]; slots_out: host.
 * Errors: KV_E_INVALID (negative sizes, a request outgrowing max_blocks),
 * KV_E_NO_BLOCKS, KV_E_BAD_BLOCK / KV_E_SHARED for a held last block that is
 * free or shared.  On error every block allocated by this call is released
 * again in reverse order (the free stack is exactly as before) and table and
 * lens are restored. */
int kv_batch_reserve(kv_pool* pool, int32_t B, int32_t* table, int32_t max_blocks, int32_t* lens,
                     const int32_t* n_new, int32_t* slots_out);

/* ---------------------------------------------------- prefix sharing -- */

/* Host: the prefix cache ("KV cache and PagedAttention", askaiml §6 "Prefix
 * caching": the engine hashes a prompt prefix, keeps its KV pages under that
 * key and reuses them for a later request with the same prefix; the key
 * carries the tenant so tenants never share).  Granularity is one whole page:
 * page i of a prompt is keyed by (tenant, the entry of page i-1, its 16
 * token ids), compared exactly (a 64-bit FNV-1a-style hash over the key's
 * 32-bit words only locates keys), so a page is reused only after an
 * identical prefix.  The cache holds one reference on every cached page.  Every match or insert touch stamps the
 * entry with the next value of a counter.  All host functions, no device work.
 *
 * kv_prefix_match: walks the whole pages of tokens[0, n_tokens) from the
 * start, stopping at the first page without an entry or after max_blocks;
 * writes the cached pages to blocks_out (host [max_blocks]) and their number
 * to *n_matched.  Each matched page gains one reference (the caller's table
 * now maps it; kv_block_release it when the request ends). */
int kv_prefix_match(kv_pool* pool, int64_t tenant, const int32_t* tokens, int32_t n_tokens,
                    int32_t* blocks_out, int32_t max_blocks, int32_t* n_matched);

/* kv_prefix_insert: once table_row's pages hold the KV of tokens[0, n_tokens),
 * enters its whole pages: a page whose key is already cached keeps the
 * existing entry (table_row's page stays private to its request); otherwise
 * table_row[i] becomes the entry and gains one reference.  *n_added = new
 * entries.  KV_E_INVALID if n_table < n_tokens / 16; KV_E_BAD_BLOCK (nothing
 * changed) if any of those table entries is out of range or free. */
int kv_prefix_insert(kv_pool* pool, int64_t tenant, const int32_t* tokens, int32_t n_tokens,
                     const int32_t* table_row, int32_t n_table, int32_t* n_added);

/* kv_prefix_evict: frees up to n_wanted cached pages, least recently touched
 * first, among entries whose page no request maps (refcount 1) and that no
 * other entry continues (removing one may make its parent eligible).  The
 * freed pages go on the free stack in that order and, if blocks_freed is not
 * NULL (host [n_wanted]), are listed there; *n_freed = how many. */
int kv_prefix_evict(kv_pool* pool, int32_t n_wanted, int32_t* blocks_freed, int32_t* n_freed);

/* Number of cache entries (cached pages). */
int kv_prefix_num_entries(const kv_pool* pool, int32_t* n);

/* Host: kv_batch_reserve with copy-on-write.  Same arguments and effect, except
 * that a request about to write into its partly filled last page while that
 * page is shared (refcount > 1, e.g. after a fork for parallel sampling or
 * beam search: copy the table row and kv_block_retain_n its pages) gets a
 * fresh page in its table instead.  The old page loses that reference and the
 * pair is listed in copy_src / copy_dst (host, capacity B; *n_copies pairs)
 * for kv_block_copy, which must run before the new tokens are appended.  Per
 * request the copy's page is allocated before the request's new pages.  On
 * error nothing changes (stack, counts, table, lens as before). */
int kv_batch_reserve_cow(kv_pool* pool, int32_t B, int32_t* table, int32_t max_blocks, int32_t* lens,
                         const int32_t* n_new, int32_t* slots_out, int32_t* copy_src, int32_t* copy_dst,
                         int32_t* n_copies);

/* Device: copy page src[i] to page dst[i] for i < n, every layer, K and V, and
 * for fp8 and int8 pools both scales.  src, dst: device int32 [n]; pairs with an id out
 * of [0, num_blocks), or src == dst, are skipped.  Destinations must be
 * distinct and not also sources (the copies run concurrently). */
int kv_block_copy(kv_pool* pool, const int32_t* src, const int32_t* dst, int32_t n, void* hip_stream);

/* --------------------------------------------------------------- append -- */

/* Device: write T new tokens into layer `layer` of the pool.
 * k_new, v_new: device [T][num_kv_heads][head_dim], float for KV_F32 pools and
 * bfloat16 for KV_BF16, KV_FP8_E4M3 and KV_INT8 pools.  slot_mapping: device int32 [T];
 * token t goes to block slot/block_size, offset slot%block_size; -1 skips it.
 * f32 and bf16 pools store the bits unchanged.  fp8 and int8 pools quantise per
 * (block, kv-head) tile, separately for K and V: the tokens of one call that
 * land in one tile (which must be consecutive tokens of the call, at
 * increasing offsets) form a run; a run starting at offset 0 starts a fresh
 * tile (old scale ignored), otherwise s0 is the stored scale; the new scale is
 * s1 = max(s0, max|x| / M) in fp32 (M = 448 for fp8, 127 for int8); when
 * s1 != s0 the codes already below the run's first offset are re-encoded from
 * decode(code)*s0; each new code encodes x * (1/s1): fp8, the E4M3 encoding
 * (round to nearest even, saturating at 448); int8, round half to even then
 * clamp to [-127, 127] (askaiml §7 names INT8 next to fp8 with no details;
 * this symmetric form reuses the fp8 tile rule).  All codes 0 when s1 == 0.
 * Two tokens of one call must not share a slot.  T == 0 is a no-op. */
int kv_append(kv_pool* pool, int32_t layer, const void* k_new, const void* v_new,
              const int32_t* slot_mapping, int32_t T, void* hip_stream);

/* ------------------------------------------------------------ attention -- */

/* Workspace bytes paged_attention_decode needs for this batch shape, -1 on
 * invalid arguments.  fp32 caches: 0 when one partition covers max_ctx.
 * bf16, fp8 and int8 caches: always > 0: 256 KiB of piece-arrival counters,
 * then the split states, then B + 1 integers.  The workspace is caller-owned
 * device memory, 16-byte aligned.
 * bf16 / fp8 / int8 workspaces: the first 256 KiB must be zero before the
 * workspace's first decode call (paged_attention_workspace_init, or memory
 * the caller zeroed); every decode call leaves them zero, so one workspace
 * serves any number of later calls of any shape that fits it.  Two calls
 * that run at the same time need two workspaces. */
int64_t paged_attention_workspace_bytes(const kv_pool* pool, int32_t B, int32_t h_q,
                                        int32_t max_ctx, int32_t partition_tokens);

/* Device: zero the counter region of a bf16 / fp8 / int8 decode workspace
 * (its first 256 KiB) on hip_stream, with a fill kernel (no memset node, so
 * it may be captured in a graph).  Nothing to do for f32 pools or
 * workspace_bytes == 0.  KV_E_INVALID for a NULL pool or workspace, a
 * negative size or a workspace not 16-byte aligned; KV_E_WORKSPACE when
 * workspace_bytes is below 256 KiB. */
int paged_attention_workspace_init(const kv_pool* pool, void* workspace, int64_t workspace_bytes,
                                   void* hip_stream);

/* Device: one decode step of attention for B requests in layer `layer`.
 * For request b and query head h (group g = h / (h_q / num_kv_heads)), with
 * n = context_lens[b] tokens cached (the token appended this step included):
 *   out[b][h] = sum_t softmax_t(scale * <q[b][h], K_t>) * V_t  over t < n,
 * K_t, V_t read through block_tables[b][t / block_size]; n == 0 gives zeros
 * (the attention step of "Memoizing Context via KV Caching" and of the askaiml
 * page, §1, over the paged layout of its §4).
 * q: device [B][h_q][head_dim] of q_dtype (KV_F32 with f32 pools, KV_BF16 with
 * bf16, fp8 and int8 pools); out: device, same shape and dtype as q.
 * block_tables: device int32 [B][max_blocks_per_seq]; context_lens: device
 * int32 [B]; max_ctx: host bound, <= max_blocks_per_seq * block_size.  Each
 * context length is clamped to [0, max_ctx] before use, so a length beyond
 * the bound is truncated, never read past the table or the workspace.
 * h_q must be a multiple of num_kv_heads.
 * Work split (partition_tokens, a multiple of block_size):
 *  - fp32 caches: partitions of partition_tokens tokens (0 = 512) per request
 *    and kv-head; with more than one, their (max, sum, weighted sum) states go
 *    to the workspace and a second kernel merges them.
 *  - bf16, fp8 and int8 caches (B <= 8192): 0 splits the blocks of the whole batch
 *    evenly over the kernel's waves; otherwise each piece covers at most
 *    partition_tokens tokens.  Pieces that do not cover a whole request leave
 *    states in the workspace, merged in piece order: by the last piece of the
 *    request to finish, inside the same kernel, when requests have few pieces
 *    (at most 16 on average and B * num_kv_heads * ceil(h_q / num_kv_heads /
 *    16) <= 65536), else by a second kernel.
 * Results depend on the context lengths of the batch (through the split) but
 * not on which physical blocks hold the data, nor on the cache hint of the
 * K/V loads (non-temporal while kv_num_shared_blocks is 0).  Accumulation is
 * fp32; the result is rounded to nearest even into out. */
int paged_attention_decode(kv_pool* pool, int32_t layer, void* out, const void* q, int32_t q_dtype,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t B, int32_t h_q, int32_t max_ctx,
                           float scale, int32_t partition_tokens, void* workspace,
                           int64_t workspace_bytes, void* hip_stream);

/* Device: one whole decode step of layer `layer`: the append of one new token
 * per request followed by the attention over the context that includes it
 * (the order of §1 of the askaiml page: the new token's K and V join the
 * cache, then attention reads all of it).  Same result as
 *   kv_append(pool, layer, k_new, v_new, slot_mapping, B, stream);
 *   paged_attention_decode(pool, layer, out, q, ...);
 * with these added arguments:
 * k_new, v_new: device [B][num_kv_heads][head_dim] (bf16 for bf16, fp8 and int8
 * pools, float for f32 pools), the new token of each request; slot_mapping:
 * device int32 [B], the slot of position context_lens[b] - 1 of request b
 * (as kv_slot_mapping / kv_batch_reserve give it), or -1 when request b
 * appends nothing this step.  The slot's block must be mapped by request b
 * alone (kv_slot_mapping refuses shared blocks).
 * bf16 pools run it as one kernel: the attention takes the last position from
 * k_new / v_new while the same launch stores them into the slot, so the step
 * costs no separate append launch (outputs agree with the two calls to the
 * bf16 rounding of the weights).  fp8 and int8 pools with at most 16 query
 * heads per kv head also run one kernel: the wave that owns a request's last
 * tile re-quantises it as kv_append does (cache bytes identical) before it
 * reads it.  f32 pools, and 8-bit pools with more query heads per kv head,
 * launch the append kernel and then the decode.  Errors and workspace are those of paged_attention_decode, plus
 * KV_E_INVALID for a NULL k_new, v_new or slot_mapping. */
int paged_attention_decode_append(kv_pool* pool, int32_t layer, void* out, const void* q,
                                  int32_t q_dtype, const void* k_new, const void* v_new,
                                  const int32_t* slot_mapping, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t B,
                                  int32_t h_q, int32_t max_ctx, float scale, int32_t partition_tokens,
                                  void* workspace, int64_t workspace_bytes, void* hip_stream);

/* Device: paged_attention_decode_append without a caller workspace, for
 * callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation).  Arguments,
 * kernels and results are those of paged_attention_decode_append; the
 * workspace is a fixed 24 MiB array inside the library, one per device,
 * looked up on the first call on that device (the device of hip_stream) and
 * held until the process ends.  Nothing is allocated.  KV_E_WORKSPACE when
 * the batch needs more than 24 MiB (paged_attention_workspace_bytes tells;
 * e.g. any Llama-3-8B or -70B shaped batch of up to 8192 requests with the
 * default split fits).  Every call on a device shares its array: calls that
 * overlap on one device race and must not be issued; calls in one stream
 * order are fine. */
int paged_attention_decode_append_noalloc(kv_pool* pool, int32_t layer, void* out, const void* q,
                                          int32_t q_dtype, const void* k_new, const void* v_new,
                                          const int32_t* slot_mapping, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t B,
                                          int32_t h_q, int32_t max_ctx, float scale, int32_t partition_tokens,
                                          void* hip_stream);

/* --------------------------------------------------------------- prefill -- */

/* Device: causal attention of each request's new tokens over its paged cache
 * (the prompt pass of "KV cache and PagedAttention", askaiml §1, computed in
 * tiles as the glossary's FlashAttention entry describes).  Request b's
 * queries are rows query_start[b] .. query_start[b+1]-1 of q; they are the
 * last n_q = query_start[b+1] - query_start[b] of its n = context_lens[b]
 * cached positions (their K and V appended first, e.g. by kv_append), so
 * query i sits at position n - n_q + i and
 *   out[row][h] = sum_{t <= n - n_q + i} softmax_t(scale * <q[row][h], K_t>) V_t
 * with query head h reading kv head h / (h_q / num_kv_heads).  Positions
 * before the new tokens (a cached prefix, earlier chunks) are read as they
 * are.  n_q <= n is required.
 * q, out: device bf16 [total rows][h_q][head_dim]; query_start: device int32
 * [B+1], non-decreasing from 0; block_tables, context_lens as for
 * paged_attention_decode; max_q_len: host bound on every n_q (sizes the grid);
 * max_ctx: host bound on context_lens (<= max_blocks_per_seq * block_size).
 * Any finite scale (a negative one negates q exactly inside the call, zero
 * gives equal weights).  bf16 pools and queries only, at most 128 query heads
 * per kv head (KV_E_UNSUPPORTED otherwise).  No workspace: one workgroup
 * covers all keys of its query tile. */
int paged_attention_prefill(kv_pool* pool, int32_t layer, void* out, const void* q, int32_t q_dtype,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, const int32_t* query_start, int32_t B, int32_t h_q,
                            int32_t max_q_len, int32_t max_ctx, float scale, void* hip_stream);

/* ------------------------------------------------------ sliding window -- */

/* Device: paged_attention_decode for a model with sliding-window attention
 * and attention sinks ("KV cache and PagedAttention", askaiml §8: only the
 * last W tokens are needed, and keeping the first few tokens as well steadies
 * long generations).  For a request of n = context_lens[b] tokens the output
 * is the attention over positions t < sink_tokens and n - window_tokens <= t
 * < n, positions keeping their index.  Only pages holding such positions are
 * read, so their table entries must be valid and the others may be -1 or
 * released (kv_window_release).  sink_tokens >= 0, window_tokens >= 1; bf16,
 * fp8 and int8 pools (KV_E_UNSUPPORTED for f32).  All other arguments, the
 * workspace and errors are those of paged_attention_decode. */
int paged_attention_decode_window(kv_pool* pool, int32_t layer, void* out, const void* q, int32_t q_dtype,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t B, int32_t h_q, int32_t max_ctx,
                                  float scale, int32_t sink_tokens, int32_t window_tokens,
                                  int32_t partition_tokens, void* workspace, int64_t workspace_bytes,
                                  void* hip_stream);

/* Device: one windowed decode step with the step's append: the same result as
 *   kv_append(pool, layer, k_new, v_new, slot_mapping, B, stream);
 *   paged_attention_decode_window(pool, layer, out, q, ...);
 * (askaiml §1: the new token's K and V join the cache, then attention reads
 * it; §8: through the window and the sinks).  k_new, v_new and slot_mapping
 * are those of paged_attention_decode_append: slot_mapping[b] is the slot of
 * position context_lens[b] - 1, or -1 when request b appends nothing.  bf16
 * pools run one kernel, which takes the last position from k_new / v_new
 * while the same launch stores it (outputs agree with the two calls to the
 * bf16 rounding of the weights); fp8 and int8 pools launch the append kernel
 * and then the windowed decode.  The other arguments, the workspace and the
 * errors are those of paged_attention_decode_window, plus KV_E_INVALID for a
 * NULL k_new, v_new or slot_mapping. */
int paged_attention_decode_window_append(kv_pool* pool, int32_t layer, void* out, const void* q,
                                         int32_t q_dtype, const void* k_new, const void* v_new,
                                         const int32_t* slot_mapping, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t B,
                                         int32_t h_q, int32_t max_ctx, float scale, int32_t sink_tokens,
                                         int32_t window_tokens, int32_t partition_tokens, void* workspace,
                                         int64_t workspace_bytes, void* hip_stream);

/* Host: give back the pages no later windowed decode of these requests reads.
 * The window only moves forward, so logical page j of a request of lens[b]
 * tokens is dead when 16 j >= sink_tokens and 16 (j + 1) <= lens[b] -
 * window_tokens.  Each dead page's table entry loses its reference (pushed on
 * the free stack at zero, request by request, page by page) and becomes -1;
 * entries already -1 are skipped.  table: host [B][max_blocks], edited;
 * lens: host [B].  *n_released = pages dropped.  KV_E_INVALID for bad sizes,
 * KV_E_BAD_BLOCK if a dead entry is free, out of range or dropped more often
 * than it is mapped; nothing changes on an error. */
int kv_window_release(kv_pool* pool, int32_t B, int32_t* table, int32_t max_blocks, const int32_t* lens,
                      int32_t sink_tokens, int32_t window_tokens, int32_t* n_released);

/* -------------------------------------------------------------- errors -- */

/* Static name of a status code. */
const char* kv_status_string(int status);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* kv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
