/*
 * pagedkv.h — C ABI of the paged KV cache and paged decode attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * The method: each sequence's KV cache is cut into fixed blocks of tokens
 * (16 by default; 32 and 64 are supported too) that live anywhere in one
 * shared physical pool; a per-sequence block table
 * maps logical block -> physical block, and the attention of one new query
 * token per sequence reads its context through that table
 * ("PagedAttention — 把 KV cache 当虚拟内存页来管理", 是什么 and 实践案例 / 案例 2;
 * "One Deep Concept #01 — PagedAttention: From Operating System Virtual Memory
 * to Large Language Model Memory Systems", §4 Core Innovation).
 *
 * Conventions for every call
 * --------------------------
 * - Return value: PA_OK (0) or a negative pa_status. No call throws or
 *   aborts. pa_last_error() gives a text for the last failing call of the
 *   calling thread.
 * - Ownership: the caller allocates every device buffer (pools, scales, q,
 *   out, tables, slots, workspace). The library never allocates or frees
 *   device memory; it only keeps small host descriptors.
 * - Asynchrony: device calls validate their host-visible arguments, enqueue
 *   kernels on the caller's stream and return. On a validation error nothing
 *   is enqueued. A launch failure returns PA_ERR_HIP.
 * - Device-side indices (table entries, slots, copy pairs) are range-checked
 *   in the kernels: an out-of-range entry is skipped (a table entry is
 *   treated as masked, a slot or pair is not written) and a bit is set in the
 *   pool's own sticky device error word; pa_check_errors(pool, ...) reads and
 *   clears that word alone, atomically. Calls tied to no pool
 *   (pa_decode_contiguous) flag a word of their own, read with pool = NULL.
 * - Layouts (all row-major, element type given by the pool dtype):
 *     K, V pools    [num_blocks][num_heads][block_size][head_dim]
 *                   (PA_I4: [...][head_dim / 2] bytes, two codes per byte)
 *     int8/int4 scales [num_blocks][num_heads] fp16 (one per block and head)
 *     q, out        [num_seqs][num_heads][head_dim]
 *     new K, V rows [n][num_heads][head_dim]
 *     block tables  int32 [num_seqs][max_blocks], logical order
 *     context lens  int32 [num_seqs]
 *     slot mapping  int64 [n], slot = physical_block * block_size + offset
 * - Supported geometry: block_size 16, 32 or 64, head_dim 64 or 128,
 *   num_heads >= 1. Pages of 16, 32 or 64 tokens are the sizes "KV Cache与长上
 *   下文管理" lists (the section on the second problem paging solves); the
 *   study note "PagedAttention — 把 KV cache 当虚拟内存页来管理" (踩过的坑) calls
 *   16 the default compromise between table-lookup and copy overhead and
 *   fragmentation. A pool, its block manager and its tables share one size.
 *
 * The block manager (pa_bm_*) is host-only: it touches no device memory and
 * needs no GPU.
 */
#ifndef PAGEDKV_H_
#define PAGEDKV_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* An opaque stream handle: a hipStream_t (NULL = the default stream). */
typedef void* pa_stream;

typedef int32_t pa_status;
enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,   /* null pointer, negative size, bad combination   */
  PA_ERR_UNSUPPORTED = -2,   /* geometry or dtype outside the supported set    */
  PA_ERR_OUT_OF_BLOCKS = -3, /* block manager: the free list cannot serve it   */
  PA_ERR_OUT_OF_RANGE = -4,  /* an index or capacity out of range              */
  PA_ERR_STATE = -5,         /* unknown / duplicate sequence, double free      */
  PA_ERR_HIP = -6            /* a HIP runtime call failed                      */
};

/* PA_I4: int4 codes in [-7, 7], two per byte: dim 2j of a row in the low
 * nibble of byte j and dim 2j+1 in the high nibble, each nibble holding
 * code + 8 (so a row of head_dim values takes head_dim / 2 bytes). Like
 * PA_I8, one fp16 scale per (block, head) for K and one for V. */
typedef enum { PA_F32 = 0, PA_F16 = 1, PA_I8 = 2, PA_I4 = 3 } pa_dtype;

/* Device error word bits, reported by pa_check_errors(). */
enum {
  PA_DEV_BAD_TABLE_ENTRY = 1,  /* a table entry outside [0, num_blocks)        */
  PA_DEV_BAD_SLOT = 2,         /* a slot outside the pool                      */
  PA_DEV_BAD_PAIR = 4,         /* a copy pair outside the pool                 */
  PA_DEV_BAD_CONTEXT = 8,      /* context_lens[s] < 0 or > the stated maximum  */
  PA_DEV_BAD_RUN = 16          /* int8/int4 write: one block hit by duplicate
                                  slots, by more than block_size rows, or by
                                  two runs of rows that are not adjacent     */
};

/* Text of the last failing call on this thread ("" if none). Never NULL. */
const char* pa_last_error(void);

/* Library version as 10000*major + 100*minor + patch. */
int32_t pa_version(void);

/* ----------------------------------------------------------------------------
 * Pool descriptor.
 *
 * The pool is the shared physical block store of the method ("One Deep
 * Concept #01", §4 Core Innovation: logical KV blocks -> block table ->
 * physical GPU blocks). K and V are separate arrays; int8 and int4 pools carry
 * one fp16 scale per (block, head) for K and one for V.
 * ------------------------------------------------------------------------- */
typedef struct pa_pool pa_pool;

/* Bytes the caller must allocate for one of K or V (*kv_bytes) and for one of
 * the scale arrays (*scale_bytes, 0 unless kv_dtype is PA_I8 or PA_I4).
 * Errors: PA_ERR_INVALID_ARG (null outputs, non-positive sizes),
 * PA_ERR_UNSUPPORTED (block_size not 16/32/64, head_dim not 64/128). */
pa_status pa_pool_bytes(int32_t num_blocks, int32_t block_size, int32_t num_heads,
                        int32_t head_dim, pa_dtype kv_dtype, int64_t* kv_bytes,
                        int64_t* scale_bytes);

/* Create a descriptor over caller-owned device buffers. k_cache / v_cache must
 * each hold pa_pool_bytes(...)->kv_bytes and be 16-byte aligned; k_scale /
 * v_scale must be given for PA_I8 and PA_I4 and NULL otherwise. The buffers stay owned
 * by the caller and must outlive the descriptor. *out receives the handle.
 * The pool belongs to the device current at this call, and takes one of the
 * library's 4095 device error words (cleared here, with a synchronous copy)
 * until pa_free_pool; every later call on the pool must run with that device
 * current.
 * In a process that sees no GPU the descriptor is still made, without an
 * error word, so that host-side validation can be exercised; any of its
 * calls that reaches a kernel launch then fails with PA_ERR_HIP.
 * Errors: as pa_pool_bytes, plus PA_ERR_INVALID_ARG for null or misaligned
 * buffers and scales given for a float pool, PA_ERR_OUT_OF_RANGE if 4095
 * pools are alive, PA_ERR_HIP. */
pa_status pa_alloc_pool(int32_t num_blocks, int32_t block_size, int32_t num_heads,
                        int32_t head_dim, pa_dtype kv_dtype, void* k_cache, void* v_cache,
                        void* k_scale, void* v_scale, pa_pool** out);

/* Destroy the descriptor (never the buffers) and return its error word.
 * Kernels enqueued on the pool must have completed. NULL is accepted. */
pa_status pa_free_pool(pa_pool* pool);

/* ----------------------------------------------------------------------------
 * Write new K/V rows into their slots (reshape-and-cache).
 *
 * Row i of k_new / v_new ([n][num_heads][head_dim], dtype src_dtype, PA_F32
 * or PA_F16) is stored at slot_mapping[i] (device int64): block
 * slot / block_size, offset slot % block_size — the lookup of "PagedAttention
 * — 把 KV cache 当虚拟内存页来管理", 实践案例 / 案例 2. A negative slot skips the
 * row. Float pools store the row rounded to nearest even.
 *
 * int8 pools quantise on write (the FP16 -> INT8 compression listed in "KV
 * Cache与长上下文管理", section 二.3; the scheme is this library's): rows of one
 * call that land in one (block, head) form a group with a = max|x|;
 * s_new = fp16(a / 127); s_old = 0 if the group writes offset 0, else the
 * stored scale; s = max(s_old, s_new). If s > s_old > 0 the block's rows not
 * written by the call are re-coded as clamp(rne(q * s_old / s), -127, 127);
 * new rows are clamp(rne(x / s), -127, 127) (0 if s == 0); the stored scale
 * becomes s. All arithmetic is IEEE fp32 with correctly rounded division.
 * int4 pools (INT4, the next step of the same page's list) follow the same
 * rule with 7 in place of 127, codes stored as in the PA_I4 layout.
 * Precondition for int8 and int4 pools: the entries of slot_mapping that hit
 * one block are adjacent and distinct, at most block_size of them (true for
 * decode, one row per sequence, and for a sequence's prefill in token order).
 * A call that breaks it flags PA_DEV_BAD_RUN; the content of that block is
 * then unspecified (never out of bounds). Checking two runs costs the wave of
 * each run leader (head 0, K) a read of the slots before it.
 * Float pools: duplicate slots in one call leave one of the rows (which one
 * is unspecified).
 * n == 0 is a no-op. Errors: PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_HIP.
 */
pa_status pa_write_kv(pa_pool* pool, const void* k_new, const void* v_new, pa_dtype src_dtype,
                      const int64_t* slot_mapping, int32_t n, pa_stream stream);

/* ----------------------------------------------------------------------------
 * Copy whole blocks (copy-on-write).
 *
 * For every pair p < n of pairs ([n][2] device int32, {src, dst}) copies
 * K[src] -> K[dst] and V[src] -> V[dst] over all heads and offsets, plus the
 * two scales of an int8 or int4 pool. The unit of the copy is one block, as in
 * "PagedAttention — 把 KV cache 当虚拟内存页来管理", 实践案例 / 案例 3. Pairs are
 * independent: no dst may appear twice or also be a src in the same call.
 * n == 0 is a no-op. Errors: PA_ERR_INVALID_ARG, PA_ERR_HIP.
 */
pa_status pa_copy_blocks(pa_pool* pool, const int32_t* pairs, int32_t n, pa_stream stream);

/* ----------------------------------------------------------------------------
 * Copy whole blocks between the device pool and a host pool (swap).
 *
 * Page-by-page swapping to host memory and back is what paging makes
 * possible ("KV Cache与长上下文管理", the fourth point). The host pool is
 * caller-owned pinned host memory (hipHostMalloc, or a pinned tensor) with
 * the pool's per-block layout: host_k / host_v [num_host_blocks][num_heads]
 * [block_size][head_dim] of the pool's dtype, 16-byte aligned; host_k_scale /
 * host_v_scale [num_host_blocks][num_heads] fp16 for int8 and int4 pools, NULL
 * otherwise. pairs ([n][2] device int32): PA_SWAP_OUT copies device block
 * pairs[i][0] to host block pairs[i][1]; PA_SWAP_IN copies host block
 * pairs[i][0] to device block pairs[i][1] (K, V and the scales). One kernel
 * reads or writes the host pool directly over the host link; no destination
 * may appear twice in one call. An id outside its pool flags
 * PA_DEV_BAD_PAIR and the pair is skipped. The host sees swapped-out data
 * once the stream has reached the end of the call.
 * n == 0 is a no-op. Errors: PA_ERR_INVALID_ARG (NULL, misaligned, memory
 * that is not pinned host memory, scales given or missing, bad direction,
 * n > 65535), PA_ERR_HIP. */
enum { PA_SWAP_OUT = 0, PA_SWAP_IN = 1 };
pa_status pa_swap_blocks(pa_pool* pool, void* host_k, void* host_v, void* host_k_scale,
                         void* host_v_scale, int32_t num_host_blocks, const int32_t* pairs, int32_t n,
                         int32_t direction, pa_stream stream);

/* ----------------------------------------------------------------------------
 * Paged decode attention.
 *
 * For each sequence s and head h, with ctx = context_lens[s] and
 * k_t = K[table[s][t / B]][h][t % B] with B = the pool's block_size (int8 and
 * int4: code * scale[block][h]):
 *     out[s][h] = sum_{t < ctx} softmax_t(q[s][h] . k_t * sm_scale) v_t
 * ("One Deep Concept #01", §2 Background: softmax(Q K^T / sqrt(d)) V; the
 * table indirection of "PagedAttention — 把 KV cache 当虚拟内存页来管理",
 * 实践案例 / 案例 2). Accumulation is fp32; out is stored in q_dtype (round to
 * nearest even for PA_F16). ctx == 0 gives zeros. Only the first
 * ceil(ctx / B) table entries of a row are read; tokens at t >= ctx are
 * never used, whatever the pool holds there.
 *
 * q_dtype: PA_F32 or PA_F16 (q and out). sm_scale <= 0 selects 1/sqrt(head_dim).
 * partition_tokens == 0: one workgroup per (sequence, head) covers the whole
 * context (single pass; workspace may be NULL).
 * partition_tokens  > 0 (a multiple of B): split-K. Every (sequence, head,
 * partition of partition_tokens tokens) is decoded on its own and writes its
 * partial (m, l, o) into workspace; a second kernel merges them by
 * log-sum-exp. Sequences with a single partition are written directly.
 * max_context_len bounds every context_lens[s] (larger values are clamped and
 * flagged with PA_DEV_BAD_CONTEXT); max_blocks is the row stride of
 * block_tables and must be >= ceil(max_context_len / B).
 * Errors: PA_ERR_INVALID_ARG (null pointers, bad sizes, workspace too small),
 * PA_ERR_UNSUPPORTED, PA_ERR_HIP.
 */
pa_status pa_decode_workspace_bytes(const pa_pool* pool, int32_t num_seqs,
                                    int32_t max_context_len, int32_t partition_tokens,
                                    int64_t* bytes);

pa_status pa_decode(pa_pool* pool, const void* q, pa_dtype q_dtype, void* out,
                    const int32_t* block_tables, int32_t max_blocks,
                    const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                    float sm_scale, int32_t partition_tokens, void* workspace,
                    int64_t workspace_bytes, pa_stream stream);

/* pa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels, but the split-K workspace is the library's own static
 * device scratch of 32 MiB (one per GPU, held until the process ends) instead
 * of a caller buffer, and nothing is allocated or freed. Arguments are
 * pa_decode's without workspace / workspace_bytes; batch order, PA_SCHED_HEADS.
 * The scratch keeps the last call's partials; every (sequence, head,
 * partition) a call reads is written by that same call first, so nothing is
 * cleared. Calls that overlap on one GPU (other streams, other threads) share
 * the scratch and race: serialise them. Single pass (partition_tokens == 0)
 * uses no scratch.
 * Errors: PA_ERR_OUT_OF_RANGE when the split-K partials, pa_decode_workspace_bytes
 * of the call, exceed 32 MiB (checked before anything is launched); otherwise
 * as pa_decode. */
pa_status pa_decode_noalloc(pa_pool* pool, const void* q, pa_dtype q_dtype, void* out,
                            const int32_t* block_tables, int32_t max_blocks,
                            const int32_t* context_lens, int32_t num_seqs,
                            int32_t max_context_len, float sm_scale, int32_t partition_tokens,
                            pa_stream stream);

/* Dispatch schedules for an ordered decode (seq_order not NULL):
 * PA_SCHED_HEADS  — ranks one after the other, all heads of a rank together
 *                   (each XCD takes 4 adjacent heads: 4 adjacent tiles of each
 *                   block); the faster one when sequences share no blocks.
 * PA_SCHED_SHARED — ranks in groups of 4, a group head by head (each XCD
 *                   takes one head of 4 adjacent ranks), so samples that share
 *                   blocks and sit next to each other in the order read them
 *                   through one L2 at about the same time. */
enum { PA_SCHED_HEADS = 0, PA_SCHED_SHARED = 1 };

/* pa_decode with a schedule: seq_order (device int32 [num_seqs], a
 * permutation of the batch, or NULL for batch order) is the order in which
 * sequences are dispatched; schedule is a PA_SCHED_* value (ignored without
 * an order). Passing the batch sorted by decreasing context length (longest
 * first) shortens the tail of a single-pass launch, whose per-sequence work
 * is proportional to the context. Results do not depend on the order or the
 * schedule. An entry outside [0, num_seqs) flags PA_DEV_BAD_CONTEXT and that
 * work is skipped. */
pa_status pa_decode_ordered(pa_pool* pool, const void* q, pa_dtype q_dtype, void* out,
                            const int32_t* block_tables, int32_t max_blocks,
                            const int32_t* context_lens, const int32_t* seq_order, int32_t schedule,
                            int32_t num_seqs,
                            int32_t max_context_len, float sm_scale, int32_t partition_tokens,
                            void* workspace, int64_t workspace_bytes, pa_stream stream);

/* Several new tokens per sequence attending at once (a prompt, or a chunk of
 * one). The attention formula of "One Deep Concept #01" (§2 Background) takes
 * a matrix of queries, and each generated token attends to every earlier
 * token and itself ("PagedAttention的终极用途", part 一). So when the last
 * n_s = query_start[s+1] - query_start[s] tokens of sequence s are processed
 * together, row query_start[s] + i (position p = context_lens[s] - n_s + i)
 * gets exactly its own decode over tokens 0..p:
 *     out[r][h] = sum_{t <= p} softmax_t(q[r][h] . k_t * sm_scale) v_t
 * Their K and V must already be in the pool (pa_write_kv with the slots of
 * positions ctx - n_s .. ctx - 1); K and V are read through block_tables as
 * in pa_decode.
 *
 * q, out: device fp16 [num_rows][num_heads][head_dim], 16-byte aligned; rows
 * of a sequence are contiguous and in position order. query_start: device
 * int32 [num_seqs + 1], non-decreasing, query_start[num_seqs] <= num_rows.
 * block_tables, context_lens, max_blocks, max_context_len: as pa_decode.
 * max_query_len bounds every n_s. q_dtype must be PA_F16 and the pool PA_F16,
 * PA_I8 or PA_I4 (the products run on the matrix cores in fp16 with fp32
 * accumulation; int8 and int4 codes are dequantised to fp16 as code * scale,
 * rounded once; the softmax weights are rounded to fp16 before they meet V). sm_scale <= 0
 * selects 1/sqrt(head_dim). n_s == 0 writes nothing. On the device, n_s < 0,
 * n_s > context_lens[s], n_s > max_query_len, context_lens[s] >
 * max_context_len or rows outside [0, num_rows) flag PA_DEV_BAD_CONTEXT and
 * leave that sequence's rows unwritten; a table entry outside the pool flags
 * PA_DEV_BAD_TABLE_ENTRY and block 0 is read in its place.
 * Errors: PA_ERR_INVALID_ARG (null pointers, misalignment, bad sizes),
 * PA_ERR_UNSUPPORTED (fp32 pool, non-fp16 q, a pool of more than 2^32
 * token-head rows, num_blocks * num_heads * block_size: the kernel indexes
 * rows with 32 bits), PA_ERR_HIP. */
pa_status pa_prefill(pa_pool* pool, const void* q, pa_dtype q_dtype, void* out,
                     const int32_t* query_start, int32_t num_rows, const int32_t* block_tables,
                     int32_t max_blocks, const int32_t* context_lens, int32_t num_seqs,
                     int32_t max_query_len, int32_t max_context_len, float sm_scale,
                     pa_stream stream);

/* pa_prefill with a dispatch order: seq_order (device int32 [num_seqs]) is
 * a permutation of the batch and sequences are dispatched in that order
 * (callers pass them longest first, so a long sequence does not stretch the
 * launch's tail); NULL is batch order. Results are identical to pa_prefill's
 * whatever the order. An entry outside [0, num_seqs) flags
 * PA_DEV_BAD_CONTEXT and that work is skipped. Otherwise as pa_prefill. */
pa_status pa_prefill_ordered(pa_pool* pool, const void* q, pa_dtype q_dtype, void* out,
                             const int32_t* query_start, int32_t num_rows, const int32_t* block_tables,
                             int32_t max_blocks, const int32_t* context_lens, const int32_t* seq_order,
                             int32_t num_seqs, int32_t max_query_len, int32_t max_context_len, float sm_scale,
                             pa_stream stream);

/* pa_write_kv followed by pa_decode_ordered, in one launch, for float pools:
 * row s of k_new / v_new ([num_seqs][num_heads][head_dim], src_dtype PA_F32
 * or PA_F16) is sequence s's newest token and slot_mapping[s] (device int64)
 * its slot, i.e. the slot of token context_lens[s] - 1 (what a decode step's
 * append returns). The workgroup that reads a sequence's last block stores
 * the row there and uses it directly, so the step needs no separate write
 * launch. The pool ends up byte-identical to pa_write_kv's result and out
 * identical to the two calls. A negative slot writes nothing; a slot that is
 * not the newest token's flags PA_DEV_BAD_SLOT and is not written.
 * Errors: PA_ERR_UNSUPPORTED for int8 and int4 pools (their quantisation works
 * on whole blocks: use pa_write_kv), otherwise as pa_decode. */
pa_status pa_write_decode(pa_pool* pool, const void* k_new, const void* v_new, pa_dtype src_dtype,
                          const int64_t* slot_mapping, const void* q, pa_dtype q_dtype, void* out,
                          const int32_t* block_tables, int32_t max_blocks,
                          const int32_t* context_lens, const int32_t* seq_order, int32_t schedule,
                          int32_t num_seqs, int32_t max_context_len, float sm_scale,
                          int32_t partition_tokens, void* workspace, int64_t workspace_bytes,
                          pa_stream stream);

/* Layout of the split-K workspace, for callers that inspect partials: with
 * P = ceil(max_context_len / partition_tokens) and n = num_seqs * num_heads * P,
 * the workspace holds
 *   m [num_seqs][num_heads][P] fp32   largest logit of the partition (natural units)
 *   l [num_seqs][num_heads][P] fp32   sum of exp(logit - m)
 *   o [num_seqs][num_heads][P][head_dim] fp32  attention over the partition alone
 * in that order, m and l each padded to a multiple of 4 floats (n rounded up)
 * so that o is 16-byte aligned. Entries of partitions past a sequence's
 * context are not written. */

/* Upload a step's small host data (slots, table rows, context lengths, ...)
 * with a compute kernel that reads pinned host memory directly: host_src must
 * come from hipHostMalloc (or another pinned, device-mapped allocation) and
 * stay unchanged until the copy has run; dst is device memory. bytes is a
 * multiple of 16 and both pointers are 16-byte aligned. Unlike a DMA copy it
 * runs on the caller's compute queue, so the kernels that follow it start
 * without a cross-engine hand-off. Errors: PA_ERR_INVALID_ARG (including a
 * source that is not pinned host memory), PA_ERR_HIP. */
pa_status pa_stage_copy(void* dst, const void* host_src, int64_t bytes, pa_stream stream);

/* Read and clear the device error word of `pool` (PA_DEV_* bits set by the
 * kernels of calls on that pool since it was last read; NULL: the word of calls
 * tied to no pool). A one-thread kernel on `stream` swaps the word with 0
 * after the stream's earlier work, so a flag set at any moment is reported
 * exactly once; the call then synchronises the stream. Flags set by kernels
 * still running on other streams are reported by a later call. Pools do not
 * share words: checking one leaves the others' flags in place. Mixed pages
 * (pa_demote_blocks, pa_decode_mixed) flag the cold pool's word.
 * *device_error may be NULL to only clear. Concurrent calls are serialised.
 * Errors: PA_ERR_INVALID_ARG (pool on another device than the current one),
 * PA_ERR_HIP. */
pa_status pa_check_errors(const pa_pool* pool, pa_stream stream, int32_t* device_error);

/* ----------------------------------------------------------------------------
 * Measurement helpers (not part of the method).
 *
 * pa_decode_contiguous runs the same decode arithmetic over a contiguous cache
 * k[num_seqs][num_heads][max_tokens][head_dim] (same for v), with no block
 * table, so that the cost of the table indirection can be measured on equal
 * terms ("PagedAttention — 把 KV cache 当虚拟内存页来管理", 踩过的坑 states an
 * attention-kernel slowdown from the indirection). Float KV only; seq_order
 * as in pa_decode_ordered (may be NULL).
 * pa_stream_copy copies bytes (a multiple of 16, 16-byte aligned pointers)
 * with a plain streaming kernel: a bandwidth probe and a counter calibration
 * (a copy of known size for the HBM byte counters).
 * ------------------------------------------------------------------------- */
pa_status pa_decode_contiguous(const void* k, const void* v, pa_dtype kv_dtype, int32_t num_heads,
                               int32_t head_dim, int32_t max_tokens, const void* q,
                               pa_dtype q_dtype, void* out, const int32_t* context_lens,
                               const int32_t* seq_order, int32_t num_seqs, float sm_scale,
                               int32_t partition_tokens, void* workspace, int64_t workspace_bytes,
                               pa_stream stream);

pa_status pa_stream_copy(void* dst, const void* src, int64_t bytes, pa_stream stream);

/* *device_view = the address at which kernels reach the pinned host memory
 * at host (hipHostMalloc, or a pinned tensor). Device calls accept such
 * addresses wherever they read small step data (tables, contexts, order,
 * slots, pairs): the kernels then read host memory in place over the host
 * link. Errors: PA_ERR_INVALID_ARG (NULL, or memory that is not pinned). */
pa_status pa_host_view(void* host, void** device_view);

/* Reads bytes (a multiple of 16, 16-byte aligned) with a plain streaming
 * kernel (non-temporal loads, the policy of the decode kernel's K/V reads)
 * and folds them into a checksum: the achievable read bandwidth. sink is
 * device memory of at least 4096 bytes that may receive a word. */
pa_status pa_stream_read(const void* src, int64_t bytes, void* sink, pa_stream stream);

/* ----------------------------------------------------------------------------
 * Host block manager.
 *
 * Free list, per-block reference counts, copy-on-write on append and a
 * sliding-window ring:
 *  - blocks are handed out on demand from the shared free list; any free block
 *    serves ("KV Cache与长上下文管理", the section on fragmentation);
 *  - a sequence appending into a block whose count is above one gets a copy:
 *    the shared count drops by one and the copy starts at one ("PagedAttention
 *    — 把 KV cache 当虚拟内存页来管理", 实践案例 / 案例 3);
 *  - with window_blocks > 0 a sequence keeps at most that many live blocks;
 *    the oldest is invalidated and its physical block reused for new tokens,
 *    editing only the table ("KV Cache与长上下文管理", the section on the second
 *    problem paging solves; "PagedAttention的终极用途", part 三).
 * Policy details: the free list is FIFO, initialised in free_order (NULL =
 * ascending ids); allocation pops the head; blocks whose count drops to zero
 * go to the tail in logical order. Copy-on-write is triggered only by an
 * append at offset > 0 into a shared last block. A ring eviction of a block
 * still shared by another sequence drops its count and takes a fresh block.
 * Every call is atomic: on error the state is unchanged. Not thread-safe: the
 * caller serialises calls on one manager.
 * ------------------------------------------------------------------------- */
typedef struct pa_bm pa_bm;

/* block_size: 16, 32 or 64 (the pool's). free_order: NULL or a permutation
 * of [0, num_blocks) (host int32).
 * Errors: PA_ERR_INVALID_ARG (sizes, not a permutation), PA_ERR_UNSUPPORTED
 * (block size). */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                       int32_t window_blocks, pa_bm** out);
pa_status pa_bm_destroy(pa_bm* bm);

/* Register seq with prefill_tokens tokens; slots_out (host int64
 * [prefill_tokens], may be NULL when prefill_tokens == 0) receives their
 * slots. Errors: PA_ERR_STATE (seq exists), PA_ERR_INVALID_ARG (negative, or
 * more blocks than the window), PA_ERR_OUT_OF_BLOCKS. */
pa_status pa_bm_add_seq(pa_bm* bm, int64_t seq, int32_t prefill_tokens, int64_t* slots_out);

/* Prefix caching: register seq from its n token ids (host int32), sharing
 * cached blocks. A system prompt or a common prefix is stored once and reused
 * ("KV Cache与长上下文管理", section 二 item 2). Each leading full block is looked
 * up under the key (previous physical block of the sequence or -1, the
 * block's block_size token ids); a live block under that key is shared (count
 * + 1). From the first miss on, blocks are fresh; fresh full blocks enter the
 * index. A key names the whole prefix, since it includes the block before.
 * The partly filled last block is never shared. A block leaves the index when
 * its count reaches zero. slots_out [n] receives each token's slot, -1 for
 * tokens of shared blocks (pa_write_kv skips them); *shared_blocks the number
 * of shared blocks. Errors: PA_ERR_STATE (seq exists), PA_ERR_UNSUPPORTED
 * (manager with a ring), PA_ERR_OUT_OF_BLOCKS (nothing changes),
 * PA_ERR_INVALID_ARG. */
pa_status pa_bm_add_seq_prefix(pa_bm* bm, int64_t seq, const int32_t* tokens, int32_t n,
                               int64_t* slots_out, int32_t* shared_blocks);

/* child shares every block of parent; each count rises by one.
 * Errors: PA_ERR_STATE (unknown or swapped-out parent, existing child). */
pa_status pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child);

/* Make room for one token of seq. *slot_out receives its slot; *copy_src /
 * *copy_dst receive the block pair to copy first, or -1 / -1.
 * Errors: PA_ERR_STATE (unknown or swapped-out seq), PA_ERR_OUT_OF_BLOCKS. */
pa_status pa_bm_append(pa_bm* bm, int64_t seq, int64_t* slot_out, int32_t* copy_src,
                       int32_t* copy_dst);

/* pa_bm_append for seqs[0..n) in order, atomically as a whole. slots_out
 * [n]; pairs_out [n][2] receives the copy pairs compacted in order, and
 * *n_pairs their number. Errors: as pa_bm_append (state unchanged). */
pa_status pa_bm_append_batch(pa_bm* bm, const int64_t* seqs, int32_t n, int64_t* slots_out,
                             int32_t* pairs_out, int32_t* n_pairs);

/* Release seq; blocks whose count reaches zero return to the free list (a
 * swapped-out seq returns its host blocks to the host free list).
 * Errors: PA_ERR_STATE. */
pa_status pa_bm_free_seq(pa_bm* bm, int64_t seq);

/* Table row (logical order) and live context length of seq. row may be NULL
 * to query sizes only. While seq is swapped out the row holds its host-pool
 * block ids. Errors: PA_ERR_STATE, PA_ERR_OUT_OF_RANGE (cap too small). */
pa_status pa_bm_table(const pa_bm* bm, int64_t seq, int32_t* row, int32_t cap,
                      int32_t* n_blocks, int32_t* ctx_len);

/* Rows of seqs[0..n) into tables [n][cap] (unused entries -1) and their live
 * context lengths into ctx_out [n]. Errors: PA_ERR_STATE (unknown or
 * swapped-out seq), PA_ERR_OUT_OF_RANGE. */
pa_status pa_bm_export(const pa_bm* bm, const int64_t* seqs, int32_t n, int32_t* tables,
                       int32_t cap, int32_t* ctx_out);

pa_status pa_bm_ref_count(const pa_bm* bm, int32_t block, int32_t* out);
pa_status pa_bm_num_free(const pa_bm* bm, int32_t* out);
/* The free list in order (head first) into out [cap]; *n receives its length. */
pa_status pa_bm_free_list(const pa_bm* bm, int32_t* out, int32_t cap, int32_t* n);

/* *out = 1 if some block held by a resident sequence of seqs[0..n) has a
 * count above one (shared with a fork or a prefix), else 0: the hint for
 * choosing PA_SCHED_SHARED. Errors: PA_ERR_STATE (unknown sequence). */
pa_status pa_bm_batch_shares(const pa_bm* bm, const int64_t* seqs, int32_t n, int32_t* out);

/* ----------------------------------------------------------------------------
 * Swapping whole sequences between the device pool and a host pool.
 *
 * Only a paged cache can swap page by page: cold pages go to host memory and
 * come back on demand, instead of moving a whole contiguous cache ("KV Cache与
 * 长上下文管理", the fourth point on what paging makes possible). The unit here
 * is one sequence's live blocks.
 *
 * pa_bm_set_host_pool gives the manager a host pool of num_host_blocks blocks
 * (once; host_free_order NULL = ascending ids, else a permutation; the host
 * free list is FIFO like the device one).
 * pa_bm_swap_out: every live block of seq, in logical order, takes the head
 * of the host free list; pairs_out [cap][2] receives the (device, host) pairs
 * to copy (pa_swap_blocks, PA_SWAP_OUT) and *n_pairs their number. A device
 * block whose count reaches zero returns to the device free list (tail, in
 * logical order); a block still held by other sequences only loses a count.
 * pa_bm_swap_in: every host block of seq takes the head of the device free
 * list (count one); pairs_out receives the (host, device) pairs (PA_SWAP_IN)
 * and the host blocks return to the tail of the host free list. Blocks that
 * were shared before the swap-out come back as private copies.
 * Copy the pairs before the freed blocks are reused (same stream order).
 * Errors: PA_ERR_STATE (unknown seq, wrong state, no host pool, host pool set
 * twice), PA_ERR_OUT_OF_BLOCKS (not enough free blocks on the receiving
 * side; nothing changes), PA_ERR_OUT_OF_RANGE (cap too small),
 * PA_ERR_INVALID_ARG. */
pa_status pa_bm_set_host_pool(pa_bm* bm, int32_t num_host_blocks, const int32_t* host_free_order);
pa_status pa_bm_swap_out(pa_bm* bm, int64_t seq, int32_t* pairs_out, int32_t cap, int32_t* n_pairs);
pa_status pa_bm_swap_in(pa_bm* bm, int64_t seq, int32_t* pairs_out, int32_t cap, int32_t* n_pairs);
/* *out = 1 if seq is swapped out, else 0. Errors: PA_ERR_STATE (unknown seq). */
pa_status pa_bm_is_swapped(const pa_bm* bm, int64_t seq, int32_t* out);
/* The host free list in order (head first) into out [cap]; *n its length. */
pa_status pa_bm_host_free_list(const pa_bm* bm, int32_t* out, int32_t cap, int32_t* n);

/* ----------------------------------------------------------------------------
 * Mixed-precision pages: an fp16 hot block per sequence, int8 (or int4) cold
 * blocks.
 *
 * Pages used often stay in FP16 and pages used rarely are stored as INT8
 * ("PagedAttention 的技术溯源与演进脉络", §4.1 item 2, mixed-precision page
 * management; FP16 -> INT8 halves the KV bytes, "KV Cache与长上下文管理",
 * section 二.3). Here the hot page of a sequence is its newest block, the one
 * each decode step writes. Two pools with block_size 16 and the same heads and
 * head_dim: a PA_F16 "hot" pool (one block per sequence for its whole life)
 * and a PA_I8 or PA_I4 "cold" pool (with its scales; INT4 is the next step
 * of the same page's compression list). A sequence of ctx tokens holds
 * n_cold = max(0, ceil(ctx / 16) - 1) cold blocks (tokens [0, 16 n_cold)) and
 * its hot block (tokens [16 n_cold, ctx)).
 *
 * The manager (pa_mbm_*, host only, FIFO free lists in caller-given orders,
 * freed blocks to the tail, every call atomic):
 *  - pa_mbm_add_seq: prefill of n tokens; cold_slots_out / hot_slots_out [n]
 *    give each token's slot in the cold or the hot pool (-1 in the other):
 *    write them with pa_write_kv on each pool (a whole cold block in one call
 *    is quantised as one group: the demotion rule below).
 *  - pa_mbm_append_batch: one token per sequence; hot_slots_out [n] is its
 *    slot in the hot pool; when a sequence's hot block is full (a multiple of
 *    16 tokens, > 0) the block is demoted first: a fresh cold block is taken
 *    and the (hot, cold) pair reported in demote_pairs_out [n][2] (*n_pairs of
 *    them), and the token goes to offset 0 of the same hot block.
 *  - pa_mbm_fork: child shares the parent's cold blocks (counts + 1) and takes
 *    a fresh hot block; *copy_src / *copy_dst is the hot pair to copy
 *    (pa_copy_blocks on the hot pool).
 *  - pa_mbm_export: cold tables [n][cap] (-1 padded), hot blocks [n], context
 *    lengths [n].
 * Errors: PA_ERR_STATE (unknown / existing sequence), PA_ERR_OUT_OF_BLOCKS,
 * PA_ERR_OUT_OF_RANGE (cap), PA_ERR_INVALID_ARG. */
typedef struct pa_mbm pa_mbm;
pa_status pa_mbm_create(int32_t num_cold, int32_t num_hot, const int32_t* cold_order,
                        const int32_t* hot_order, pa_mbm** out);
pa_status pa_mbm_destroy(pa_mbm* m);
pa_status pa_mbm_add_seq(pa_mbm* m, int64_t seq, int32_t prefill_tokens, int64_t* cold_slots_out,
                         int64_t* hot_slots_out);
pa_status pa_mbm_append_batch(pa_mbm* m, const int64_t* seqs, int32_t n, int64_t* hot_slots_out,
                              int32_t* demote_pairs_out, int32_t* n_pairs);
pa_status pa_mbm_fork(pa_mbm* m, int64_t parent, int64_t child, int32_t* copy_src, int32_t* copy_dst);
pa_status pa_mbm_free_seq(pa_mbm* m, int64_t seq);
pa_status pa_mbm_export(const pa_mbm* m, const int64_t* seqs, int32_t n, int32_t* cold_tables,
                        int32_t cap, int32_t* hot_out, int32_t* ctx_out);
pa_status pa_mbm_ref_count(const pa_mbm* m, int32_t cold_block, int32_t* out);
/* As pa_bm_batch_shares, over the cold blocks. */
pa_status pa_mbm_batch_shares(const pa_mbm* m, const int64_t* seqs, int32_t n, int32_t* out);
/* Free lists in order (head first); either output may be NULL to query sizes. */
pa_status pa_mbm_free_lists(const pa_mbm* m, int32_t* cold_out, int32_t cold_cap, int32_t* n_cold,
                            int32_t* hot_out, int32_t hot_cap, int32_t* n_hot);

/* Demote hot blocks: for every (hot, cold) pair ([n][2] device int32) and
 * head, the hot block's 16 fp16 rows of K (and of V) are quantised as one
 * group into the cold block: s = fp16(max|x| / 127) (IEEE fp32 divide, RNE),
 * codes clamp(rne(x / s), -127, 127) (0 if s == 0) — the pa_write_kv int8
 * rule for a whole block written at once; for an int4 cold pool 7 in place of
 * 127 (codes stored as in the PA_I4 layout). Ids outside their pools flag
 * PA_DEV_BAD_PAIR and are skipped. Errors: PA_ERR_INVALID_ARG (pool kinds or
 * geometry do not match), PA_ERR_HIP. */
pa_status pa_demote_blocks(pa_pool* hot_pool, pa_pool* cold_pool, const int32_t* pairs, int32_t n,
                           pa_stream stream);

/* Paged decode over mixed-precision pages: as pa_decode_ordered, where token t
 * of sequence s is cold row K[cold_tables[s][t / 16]][h][t % 16] * scale for
 * t < 16 n_cold, and hot row Khot[hot_blocks[s]][h][t - 16 n_cold] otherwise.
 * partition_tokens: 0 or a multiple of 16; workspace, seq_order and schedule
 * as pa_decode_ordered. A hot block
 * id outside the hot pool flags PA_DEV_BAD_TABLE_ENTRY and its rows are
 * masked. Errors: as pa_decode, plus PA_ERR_INVALID_ARG when the pools are not
 * an int8 or int4 cold pool and an fp16 hot pool of block size 16 with equal
 * heads and head_dim. */
pa_status pa_decode_mixed(pa_pool* cold_pool, pa_pool* hot_pool, const void* q, pa_dtype q_dtype, void* out,
                          const int32_t* cold_tables, int32_t max_blocks, const int32_t* hot_blocks,
                          const int32_t* context_lens, const int32_t* seq_order, int32_t schedule,
                          int32_t num_seqs,
                          int32_t max_context_len, float sm_scale, int32_t partition_tokens,
                          void* workspace, int64_t workspace_bytes, pa_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H_ */
