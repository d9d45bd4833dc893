/*
 * pagedkv.h — C ABI of the MI355X (gfx950) paged KV-cache decode library.
 *
 * The library implements the data-parallel hot path of PagedAttention:
 *
 *   - decode attention that reads every sequence's keys and values through a block
 *     table of fixed-size, non-contiguous physical blocks and combines them with a
 *     running softmax, so that the result is that of attention over a contiguous
 *     layout ("PagedAttention: Optimizing KV Cache in vLLM", grasp.study, §3 "Making it
 *     Work: The PagedAttention Kernel");
 *   - the KV-cache write that stores new tokens' K/V into their slots ("What is
 *     PagedAttention?", qubittool glossary, "How It Works: Map Logical to Physical
 *     Blocks": decode appends into the partly filled last block);
 *   - the block copy behind copy-on-write (same lesson, §4 "Advanced Benefit: Zero-Cost
 *     Sharing with Copy-on-Write");
 *   - a host-side block allocator (free list, reference counts, copy-on-write
 *     decisions) that only produces block tables, slot mappings and copy lists
 *     (glossary, "How It Works: Share Without Mutating State").
 *
 * Conventions for every entry point
 *   - All pointers to tensors are device pointers unless the parameter says "host".
 *     The caller owns every buffer, including the attention workspace; the library
 *     never allocates or frees device memory and never synchronises a stream -- except
 *     the virtual-memory pool object (pkv_vmm_*), whose purpose is to map and unmap
 *     device memory, and only in its own calls.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.  All
 *     kernels of one call are enqueued on that stream in order.
 *   - Every function returns a pkv_status.  Argument checks happen on the host before
 *     anything is enqueued; on any non-OK status nothing was enqueued and no state
 *     changed.  pkv_last_error() returns a thread-local message for the last failure.
 *     Launch errors are reported as PKV_HIP_ERROR; faults during execution surface at
 *     the caller's next synchronisation, as for any asynchronous HIP work.
 *   - No function aborts or throws across the ABI.
 *   - Tensor pointers (q, out, k_new, v_new, the pools, the workspace) must be 16-byte
 *     aligned; a misaligned one is rejected with PKV_INVALID_ARG.
 *
 * Physical KV pool layout (one K pool and one V pool, same shape)
 *   - Element type: float32, bfloat16 or fp8 e4m3fn (OCP E4M3: bias 7, max 448, no
 *     infinities), b = 4, 2 or 1 bytes; x = 16 / b elements per 16-byte chunk.
 *   - num_blocks x Hkv regions, row-major over (block, kv head); each region holds the
 *     block_size (bs) token slots of one kv head: bs * D elements, contiguous.
 *   - A region is bs/16 sub-tiles of 16 tokens (tokens 16u..16u+15 in sub-tile u), each
 *     16*D elements, in order.  Inside a sub-tile, for token t (0..15) and dim d:
 *         K element index  ((d / x) * 16 + t) * x + d % x
 *         V element index  (((d / (4x)) * 4 + t / 4) * 16 + d % 16) * x
 *                          + ((d / 16) % (x/4)) * 4 + t % 4
 *     i.e. a K chunk holds x consecutive dims of one token, and a V chunk holds four
 *     consecutive tokens for each of x/4 dims spaced 16 apart.  One wavefront load of
 *     64 consecutive chunks then delivers exactly the operands of the gfx950 matrix
 *     instructions the decode kernel issues, with no shuffles.
 *   - A slot is  block * bs + offset  (offset < bs).
 *   - Supported shapes: D in {64, 128}; bs in {16, 32}; D a multiple of 4x.
 *
 * Query / output layout: q and out are [num_seqs, Hq, D] row-major.  Query head h reads
 * kv head h / G with G = Hq / Hkv (contiguous groups; G = 1 is multi-head attention).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 2

typedef enum {
  PKV_OK = 0,
  PKV_INVALID_ARG = 1,   /* a pointer, size or shape is invalid */
  PKV_UNSUPPORTED = 2,   /* valid but not implemented (dtype combination, D, bs, G) */
  PKV_OUT_OF_BLOCKS = 3, /* the allocator cannot meet the request; state unchanged */
  PKV_UNKNOWN_SEQ = 4,   /* the allocator has no sequence with that id */
  PKV_HIP_ERROR = 5      /* the HIP runtime reported an error */
} pkv_status;

typedef enum {
  PKV_F32 = 0,
  PKV_BF16 = 1,
  PKV_FP8_E4M3FN = 2
} pkv_dtype;

/* ABI version (PKV_ABI_VERSION of the built library). */
int pkv_abi_version(void);

/* Thread-local message describing the last non-OK status on this thread ("" if none). */
const char* pkv_last_error(void);

/* ------------------------------------------------------------------------------------
 * Decode attention
 *
 * One query token per sequence: for sequence s, query head h (kv head g = h / G),
 *     out[s,h,:] = sum_t w_t V_s[t,g,:] / sum_t w_t,
 *     w_t = exp(scale * k_scale * <q[s,h,:], Kcode_s[t,g,:]> - max),  t < context_lens[s]
 * where K_s / V_s are the sequence's tokens in logical order: token t sits in slot
 * block_tables[s][t / bs] * bs + t % bs.  V values are v_scale * Vcode.  For f32 and
 * bf16 caches pass k_scale = v_scale = 1.  A sequence with context_lens[s] = 0 gets a
 * zero output.  ("PagedAttention: Optimizing KV Cache in vLLM", grasp.study, §3: the
 * block-aware kernel walks the blocks in logical order with a running softmax and
 * equals contiguous attention.)
 *
 * Arguments
 *   out             [num_seqs, Hq, D] of q_dtype (written).
 *   q               [num_seqs, Hq, D] of q_dtype.
 *   k_cache, v_cache  pools as laid out above, num_blocks blocks of kv_dtype.
 *   block_tables    int32 [num_seqs, max_blocks_per_seq]; row s lists the physical
 *                   blocks of sequence s in logical order; entries past
 *                   ceil(context_lens[s] / bs) are never read (pad with -1).
 *   context_lens    int32 [num_seqs], 0 <= context_lens[s] <= max_blocks_per_seq * bs
 *                   (larger values are clamped to that bound; negative ones read as 0).
 *   q_dtype/kv_dtype  supported: (F32, F32), (BF16, BF16), (BF16, FP8_E4M3FN).
 *   num_splits      wavefronts the work is spread over; 0 = pkv_paged_attention_default_splits
 *                   (the same with or without shared_prefix_blocks).
 *                   The kv heads are grouped c = 4, 2 or 1 at a time (the largest that
 *                   divides Hkv and is at most num_splits), and the (sequence, head group,
 *                   block) list is cut into num_splits / c equal shares, each walked by c
 *                   waves side by side, one kv head each.  Results depend only on the
 *                   split count and Hkv, not on the physical block numbering.
 *   workspace       device scratch of at least pkv_paged_attention_workspace_size()
 *                   bytes, owned by the caller, no initial contents required.  It starts
 *                   with a header of round_up(4 * (num_seqs + 4), 256) bytes: every sequence's
 *                   offset in the work list and the split pass's own record of its share
 *                   count and head grouping.  The partial (max, sum, accumulator) of every
 *                   sequence head whose work spans more than one share follows.  The split
 *                   pass writes all of it; the reduce pass reads it.
 *   shared_prefix_blocks  device int32 [num_seqs] or NULL, a load-policy hint; the output
 *                   bits do not depend on it.  Sequences may share physical blocks (forks
 *                   and common prefixes, counted by reference: "What is PagedAttention?",
 *                   glossary, "Share Without Mutating State"), and those are always leading
 *                   blocks.  Entry s is how many leading logical blocks of sequence s other
 *                   sequences of the call also read (pkv_alloc_shared_prefix_blocks).  K/V
 *                   of those blocks go through ordinary cached loads, so that the sequences
 *                   reading a shared block at about the same time can find it in L2 or the
 *                   MALL.  Every other block, and every block when the pointer is NULL, is
 *                   streamed with the non-temporal hint, the faster way on MI355X to read
 *                   bytes used once.  Any value is safe: <= 0 means none, and a value past
 *                   the sequence's blocks means all.  Must be 4-byte aligned.  (The decode
 *                   step over an f32 cache with head_dim 128 always streams.)
 * Preconditions (not checked on the device): block table entries of used blocks lie in
 * [0, num_blocks) — an entry outside that range is read as a block of zeros, never out
 * of bounds; out does not alias any input.
 * ------------------------------------------------------------------------------------ */
pkv_status pkv_paged_attention_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                              int head_dim, int block_size, pkv_dtype q_dtype,
                                              pkv_dtype kv_dtype, int num_splits,
                                              size_t* bytes /* host, out */);

/* The split count used when num_splits = 0: one share per wave of 2 workgroups (of 4 waves)
 * per CU for f32 / bf16 caches and 4 for fp8 caches (the fastest counts measured on MI355X),
 * capped by what the current device keeps resident of the plain and the appending split
 * kernels (queried once per device and cached). */
pkv_status pkv_paged_attention_default_splits(int head_dim, int block_size, pkv_dtype q_dtype,
                                              pkv_dtype kv_dtype, int* splits /* host, out */);

/* Enqueues both phases below (split pass, then reduce) on `stream`. */
pkv_status pkv_paged_attention_decode(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int num_seqs,
                                      int num_q_heads, int num_kv_heads, int head_dim,
                                      int block_size, int num_blocks, int max_blocks_per_seq,
                                      float scale, float k_scale, float v_scale,
                                      pkv_dtype q_dtype, pkv_dtype kv_dtype, int num_splits,
                                      void* workspace, size_t workspace_bytes,
                                      const int32_t* shared_prefix_blocks, void* stream);

/* Phase 1 alone: every wavefront streams its share of blocks with a running softmax;
 * sequence heads that fit in one share are written to `out` finished, the others leave
 * partials in `workspace`.  Same arguments as pkv_paged_attention_decode. */
pkv_status pkv_paged_attention_split(void* out, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_tables,
                                     const int32_t* context_lens, int num_seqs,
                                     int num_q_heads, int num_kv_heads, int head_dim,
                                     int block_size, int num_blocks, int max_blocks_per_seq,
                                     float scale, float k_scale, float v_scale,
                                     pkv_dtype q_dtype, pkv_dtype kv_dtype, int num_splits,
                                     void* workspace, size_t workspace_bytes,
                                     const int32_t* shared_prefix_blocks, void* stream);

/* Phase 2 alone: merges the partials of split sequence heads (rescaling each by
 * exp(m_p - max m)) into `out` and writes zeros for empty sequences.  Must follow phase 1
 * over the same sequences (out, q, tables, lengths, shapes) on the same stream and
 * workspace.  It takes the share count and head grouping from the record phase 1 left in
 * the workspace header, so whatever its own num_splits and shared_prefix_blocks, it merges
 * exactly the partials phase 1 wrote, and it needs only the header to lie inside
 * workspace_bytes.  Its num_splits only picks between two merge kernels that fold the
 * partials in different orders: with phase 1's num_splits the bits equal those of
 * pkv_paged_attention_decode, otherwise they may differ by rounding.  A header that no
 * phase 1 over num_seqs sequences wrote, or one whose partials would lie outside
 * workspace_bytes, is not followed: the heads this pass would merge are set to NaN, and
 * nothing outside the workspace is read. */
pkv_status pkv_paged_attention_reduce(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int num_seqs,
                                      int num_q_heads, int num_kv_heads, int head_dim,
                                      int block_size, int num_blocks, int max_blocks_per_seq,
                                      float scale, float k_scale, float v_scale,
                                      pkv_dtype q_dtype, pkv_dtype kv_dtype, int num_splits,
                                      void* workspace, size_t workspace_bytes,
                                      const int32_t* shared_prefix_blocks, void* stream);

/* ------------------------------------------------------------------------------------
 * Decode attention that allocates nothing, for callers that cannot allocate device memory or
 * pass a workspace: code under HIP graph capture, tight serving loops, and harnesses that
 * forbid allocation.  Same arguments and result as pkv_paged_attention_decode (both passes)
 * minus the workspace: the library's own scratch stands in for it, a 48 MiB device array
 * (PKV_NOALLOC_SCRATCH_BYTES) that every device the library runs on holds until the process
 * ends.  A call whose workspace (pkv_paged_attention_workspace_size at its split count)
 * exceeds that is rejected with PKV_INVALID_ARG before anything is enqueued; pass a smaller
 * num_splits then.  No call allocates or frees memory; the first call on a device looks the
 * array up once (hipGetSymbolAddress).  The scratch needs no initial contents and keeps the
 * last call's; all calls on one device share it, so calls that can overlap on one device (on
 * different streams without ordering between them) race and must be serialised by the
 * caller.  Uses the current device; `stream` must belong to it.
 * ------------------------------------------------------------------------------------ */
#define PKV_NOALLOC_SCRATCH_BYTES (48u << 20)
pkv_status pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                              const int32_t* block_tables, const int32_t* context_lens,
                                              int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                              int block_size, int num_blocks, int max_blocks_per_seq,
                                              float scale, float k_scale, float v_scale, pkv_dtype q_dtype,
                                              pkv_dtype kv_dtype, int num_splits,
                                              const int32_t* shared_prefix_blocks, void* stream);

/* ------------------------------------------------------------------------------------
 * Decode attention over a contiguous per-sequence placement: the alternative to paging that
 * keeps each sequence's K/V at consecutive addresses of a virtual range and maps physical
 * pages as it grows ("What is PagedAttention?", glossary, "Frequently Asked Questions" and
 * "Common Use Cases"; the pkv_vmm_* pool below provides such ranges).  The result is the
 * attention of pkv_paged_attention_decode; only the addressing differs: logical block j of
 * sequence s is pool block seq_first_block[s] + j of the pools at k_base / v_base (the pool
 * layout above), so no block table is read.
 *
 *   seq_first_block  int32 [num_seqs] (device): each sequence's first pool block.  Blocks
 *                    seq_first_block[s] .. + ceil(context_lens[s] / bs) - 1 must be mapped
 *                    and inside [0, num_blocks); a block outside that range reads as zeros.
 *   max_blocks_per_seq  blocks each sequence may span (its slice); lengths are clamped to
 *                    max_blocks_per_seq * bs.
 *   Every other argument as for pkv_paged_attention_decode (no shared-prefix counts); both
 *   passes are enqueued, on the same workspace layout.
 * ------------------------------------------------------------------------------------ */
pkv_status pkv_contiguous_attention_decode(void* out, const void* q, const void* k_base, const void* v_base,
                                           const int32_t* seq_first_block, const int32_t* context_lens,
                                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                           int block_size, int num_blocks, int max_blocks_per_seq, float scale,
                                           float k_scale, float v_scale, pkv_dtype q_dtype, pkv_dtype kv_dtype,
                                           int num_splits, void* workspace, size_t workspace_bytes,
                                           void* stream);

/* ------------------------------------------------------------------------------------
 * Decode step with append: the KV-cache write of each sequence's new token fused into the
 * attention pass ("What is PagedAttention?", glossary, "How It Works: Map Logical to
 * Physical Blocks": a decode step appends one token into the sequence's last block; then
 * attention over all its tokens follows, as for pkv_paged_attention_decode).
 *
 * For every sequence s with L = context_lens[s] >= 1: the token at position L-1, in slot
 * block_tables[s][(L-1)/bs] * bs + (L-1) % bs, receives k_new[s] and v_new[s] (stored
 * exactly as pkv_kv_cache_write stores them: bit copies for f32 / bf16, the same
 * quantisation for fp8), and out[s] is attention over tokens 0..L-1 including it.  The
 * result equals pkv_kv_cache_write of those slots followed by pkv_paged_attention_decode.
 *
 *   k_new, v_new   [num_seqs, Hkv, D] of q_dtype (bf16 inputs for an fp8 cache); rows of
 *                  sequences with L = 0 are ignored.
 *   k_cache, v_cache  written (the appended slots only) and read.
 *   Every other argument as for pkv_paged_attention_decode; the workspace is shared with
 *   it and the default split count is the same.
 * Precondition: the block receiving a sequence's token is referenced by no other sequence
 * in the batch (the allocator's copy-on-write guarantees this); an appended slot in a
 * block outside [0, num_blocks) is neither written nor read.
 * ------------------------------------------------------------------------------------ */
pkv_status pkv_paged_decode_step(void* out, const void* q, const void* k_new, const void* v_new,
                                 void* k_cache, void* v_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, int num_seqs, int num_q_heads,
                                 int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                 int max_blocks_per_seq, float scale, float k_scale, float v_scale,
                                 pkv_dtype q_dtype, pkv_dtype kv_dtype, int num_splits,
                                 void* workspace, size_t workspace_bytes,
                                 const int32_t* shared_prefix_blocks, void* stream);

/* Phase 1 of the decode step alone (append + split pass); phase 2 is
 * pkv_paged_attention_reduce with the same arguments and workspace. */
pkv_status pkv_paged_decode_step_split(void* out, const void* q, const void* k_new,
                                       const void* v_new, void* k_cache, void* v_cache,
                                       const int32_t* block_tables, const int32_t* context_lens,
                                       int num_seqs, int num_q_heads, int num_kv_heads,
                                       int head_dim, int block_size, int num_blocks,
                                       int max_blocks_per_seq, float scale, float k_scale,
                                       float v_scale, pkv_dtype q_dtype, pkv_dtype kv_dtype,
                                       int num_splits, void* workspace, size_t workspace_bytes,
                                       const int32_t* shared_prefix_blocks, void* stream);

/* ------------------------------------------------------------------------------------
 * Decode with prefix groups: blocks that several sequences share are read once for all of
 * them.  Sharers' block tables point at the same physical blocks ("PagedAttention: Optimizing
 * KV Cache in vLLM", §4 "Copy-on-Write"; "What is PagedAttention?", glossary, "Share Without
 * Mutating State"); the pages keep attention per sequence, and reading a shared block once
 * per group is this library's own use of that layout.  The result is that of
 * pkv_paged_attention_decode / pkv_paged_decode_step over the same tables.
 *
 * The sequences come in column chunks of consecutive sequences (pkv_alloc_prefix_groups):
 *   chunk_first   int32 [num_seqs] (device): index of the first sequence of s's chunk; a chunk
 *                 holds at most 32 / G sequences (G = Hq / Hkv), so that its (sequence, query
 *                 head) pairs are at most 32 columns.
 *   chunk_src     int32 [num_seqs] (device), read at each chunk's first sequence: the chunk
 *                 sequence whose table row holds the shared blocks.
 *   group_blocks  int32 [num_seqs] (device): leading blocks of s read for it in the group
 *                 pass; at the source, the most of any chunk sequence.
 * Precondition (not checked on the device): for every s, its first group_blocks[s] table
 * entries equal its chunk source's.  The kernel takes group_blocks[s] only up to the full
 * blocks of s's cached tokens (with append, the block receiving the new token is never among
 * them) and up to the source's own count; a chunk that is not well formed (first or source
 * outside the chunk's 32 / G sequences) reads no group blocks, so its sequences are walked on
 * their own.  One split pass walks every chunk's shared blocks once, for all its sequences'
 * query heads at once, and every sequence's remaining blocks; the merge pass combines the two
 * parts.  Both passes are enqueued.
 *
 *   workspace      pkv_paged_attention_grouped_workspace_size bytes (it depends on num_splits
 *                  and max_blocks_per_seq), no initial contents needed.
 *   Every other argument as for pkv_paged_attention_decode / pkv_paged_decode_step (no
 *   shared_prefix_blocks: shared blocks are read once anyway).  num_splits >= 2 is used (at
 *   least one share of each kind).
 * ------------------------------------------------------------------------------------ */
pkv_status pkv_paged_attention_grouped_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                                      int block_size, pkv_dtype q_dtype, pkv_dtype kv_dtype,
                                                      int num_splits, int max_blocks_per_seq,
                                                      size_t* bytes /* host, out */);
pkv_status pkv_paged_attention_decode_grouped(void* out, const void* q, const void* k_cache, const void* v_cache,
                                              const int32_t* block_tables, const int32_t* context_lens,
                                              const int32_t* chunk_first, const int32_t* chunk_src,
                                              const int32_t* group_blocks, int num_seqs, int num_q_heads,
                                              int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                              int max_blocks_per_seq, float scale, float k_scale, float v_scale,
                                              pkv_dtype q_dtype, pkv_dtype kv_dtype, int num_splits, void* workspace,
                                              size_t workspace_bytes, void* stream);
pkv_status pkv_paged_decode_step_grouped(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                                         void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                         const int32_t* chunk_first, const int32_t* chunk_src,
                                         const int32_t* group_blocks, int num_seqs, int num_q_heads, int num_kv_heads,
                                         int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                                         float scale, float k_scale, float v_scale, pkv_dtype q_dtype,
                                         pkv_dtype kv_dtype, int num_splits, void* workspace, size_t workspace_bytes,
                                         void* stream);

/* Measurement aid: the next split pass launched on the calling thread (by any decode or
 * decode-step entry point), or the next multi-query attention kernel
 * (pkv_paged_attention_prefill), records start_event when its kernel begins and stop_event
 * when it ends, as part of its own dispatch (hipExtLaunchKernel), so that the events time the
 * kernel alone; the setting then clears.  start_event / stop_event are hipEvent_t handles
 * created with timing enabled (either may be NULL).  Always returns PKV_OK. */
pkv_status pkv_set_launch_events(void* start_event, void* stop_event);

/* ------------------------------------------------------------------------------------
 * Multi-query attention with a causal mask over the same pool: a prefill, a chunk of a
 * prefill, or the check of drafted tokens in speculative decoding.  "What is
 * PagedAttention?" (glossary), "How It Works: Map Logical to Physical Blocks": a prefill
 * allocates blocks for the whole input; "PagedAttention: Optimizing KV Cache in vLLM", §3:
 * walking the blocks in logical order gives attention over contiguous K/V, and
 * "Conclusion": speculative decoding checks drafted tokens against the cache.  The pages do
 * not write out this attention; it is read as causal attention:
 *
 *   Sequence s has n_s = query_start[s+1] - query_start[s] query tokens, the last n_s of its
 *   L_s = context_lens[s] tokens; query i (0 <= i < n_s) sits at position
 *   P = L_s - n_s + i and attends to tokens 0..P.  All L_s tokens, the queries' own included,
 *   must already be in the pool (pkv_kv_cache_write first).  A query with P < 0 gets zeros.
 *
 *   out, q         [num_q_tokens, Hq, D] of q_dtype, row-major; sequence s's queries are
 *                  rows query_start[s] .. query_start[s+1]-1 in position order.
 *   query_start    int32 [num_seqs + 1] (device), non-decreasing, from 0 to num_q_tokens;
 *                  entries are clamped to [0, num_q_tokens].
 *   max_query_len  host bound on every n_s: query rows past it in a sequence are neither
 *                  computed nor written.  It also picks the kernel: with max_query_len * G
 *                  <= 32 (a few drafted tokens, short chunks) the work is cut like decode's
 *                  (kv heads in groups of 4, 2 or 1, num_splits / group equal shares of the
 *                  (sequence, head group, block) list, one wave per head of a group) with a
 *                  merge pass, which needs the workspace; otherwise query tiles of 256
 *                  (query, head) columns (128 with f32) each stream their sequence's K/V
 *                  through LDS.
 *   num_splits     shares for the few-query path (0 = a default like decode's); ignored
 *                  otherwise.
 *   shared_prefix_blocks  as for pkv_paged_attention_decode, on the few-query path; the
 *                  tile path always reads through the caches (its query tiles re-read K/V).
 *   workspace      device scratch of pkv_paged_attention_prefill_workspace_size bytes; no
 *                  initial contents needed.  The few-query path needs it.  On the tile path it
 *                  is optional: with it, a plan pass first writes the launch order of the
 *                  query tiles (each XCD's (sequence, kv head) units longest first, a unit's
 *                  tiles together), one 32-byte record per workgroup slot; with NULL the
 *                  tiles run in a fixed default order.  The output bytes are the same either
 *                  way.  There is no plan (size 0) when num_seqs * num_kv_heads > 16384.
 *   Every other argument as for pkv_paged_attention_decode.  out is written once per
 *   query row and head.
 * Limits: on the tile path max_blocks_per_seq <= 16376 and num_blocks * Hkv < 2^31 (the
 * sequence's table entries are staged on chip, as phys * Hkv); num_q_tokens * Hq < 2^31.
 * ------------------------------------------------------------------------------------ */
pkv_status pkv_paged_attention_prefill_workspace_size(int num_seqs, int num_q_heads,
                                                      int num_kv_heads, int head_dim,
                                                      int block_size, pkv_dtype q_dtype,
                                                      pkv_dtype kv_dtype, int max_query_len,
                                                      int num_splits, size_t* bytes /* host, out */);
pkv_status pkv_paged_attention_prefill(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, const int32_t* query_start,
                                       int num_seqs, int num_q_tokens, int num_q_heads,
                                       int num_kv_heads, int head_dim, int block_size,
                                       int num_blocks, int max_blocks_per_seq, int max_query_len,
                                       float scale, float k_scale, float v_scale,
                                       pkv_dtype q_dtype, pkv_dtype kv_dtype, int num_splits,
                                       void* workspace, size_t workspace_bytes,
                                       const int32_t* shared_prefix_blocks, void* stream);

/* ------------------------------------------------------------------------------------
 * KV-cache write: stores T new tokens into their slots ("What is PagedAttention?",
 * glossary, "How It Works: Map Logical to Physical Blocks": a decode step appends into
 * the sequence's partly filled last block).
 *
 *   k_new, v_new   [T, Hkv, D] of in_dtype, row-major.
 *   slot_mapping   int64 [T]; token n goes to slot slot_mapping[n]; a negative slot skips
 *                  the token; a slot >= num_blocks * bs is skipped as well (never written
 *                  out of bounds).
 *   in_dtype/kv_dtype  (F32, F32) and (BF16, BF16) copy bits; (F32 or BF16, FP8_E4M3FN)
 *                  quantise: code = round-to-nearest-even(clamp(x * (1/k_scale), +-448))
 *                  with 1/k_scale rounded to float32 once on the host and one float32
 *                  multiply per element (v_scale for V).  The result is bit-exact.
 * Precondition: slots are distinct within one call (duplicates race).
 * ------------------------------------------------------------------------------------ */
pkv_status pkv_kv_cache_write(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                              int head_dim, int block_size, int num_blocks, pkv_dtype in_dtype,
                              pkv_dtype kv_dtype, float k_scale, float v_scale, void* stream);

/* ------------------------------------------------------------------------------------
 * Block copy for copy-on-write ("PagedAttention: Optimizing KV Cache in vLLM", §4: the
 * writer gets a private block holding the shared block's contents).
 *
 *   block_mapping  int32 [num_pairs][2] (device) of (src, dst) block ids; for each pair
 *                  the whole block (all kv heads, all bs slots) of K and of V is copied.
 *                  Pairs with an id outside [0, num_blocks) are skipped.
 * Preconditions: dst blocks are distinct and no dst is also a src in the same call.  Enqueue
 * before the pkv_kv_cache_write that writes into the copies (same stream).
 * ------------------------------------------------------------------------------------ */
pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping,
                           int num_pairs, int num_kv_heads, int head_dim, int block_size,
                           int num_blocks, pkv_dtype kv_dtype, void* stream);

/* ------------------------------------------------------------------------------------
 * Block copy between two pools of the same layout, for swap ("What is PagedAttention?",
 * glossary, "How It Works: Map Logical to Physical Blocks": swap is one of the explicit
 * responses to an allocation that cannot be met).
 *
 *   dst_k, dst_v / src_k, src_v  K and V pools of dst_num_blocks / src_num_blocks blocks,
 *                  each device memory or pinned host memory the device can access
 *                  (hipHostMalloc); one side is typically the device pool and the other a
 *                  host pool.
 *   block_mapping  int32 [num_pairs][2] of (src, dst) block ids, device-accessible; the
 *                  whole block (all kv heads, all bs slots) of K and of V is copied.  Pairs
 *                  with an id outside its pool are skipped.  pkv_seq_swap produces them.
 * Preconditions: dst blocks distinct; the pools do not overlap.  Other arguments as for
 * pkv_copy_blocks.
 * ------------------------------------------------------------------------------------ */
pkv_status pkv_swap_blocks(void* dst_k, void* dst_v, int dst_num_blocks, const void* src_k,
                           const void* src_v, int src_num_blocks, const int32_t* block_mapping,
                           int num_pairs, int num_kv_heads, int head_dim, int block_size,
                           pkv_dtype kv_dtype, void* stream);

/* ------------------------------------------------------------------------------------
 * Device-side mirror of a decode step's table update ("What is PagedAttention?", glossary,
 * "How It Works: Map Logical to Physical Blocks": a decode step appends one token into the
 * sequence's last block and takes a new block only when that one is full).
 *
 * After pkv_seq_append gave each of num_seqs sequences one token (slot_mapping[s], the slots
 * it returned, copied to the device), this applies the same change to device copies of the
 * block tables and lengths, so that only the slots cross to the device each step: for every
 * s with 0 <= slot < num_blocks * bs, position p = context_lens[s] gets
 * block_tables[s][p / bs] = slot / bs (a new block, a copy-on-write copy or the unchanged
 * tail) and context_lens[s] becomes p + 1.
 *
 *   block_tables   int32 [num_seqs, max_blocks_per_seq] (device, updated in place); row s
 *                  belongs to the s-th sequence passed to pkv_seq_append.
 *   context_lens   int32 [num_seqs] (device, updated in place).
 *   slot_mapping   int64 [num_seqs], in device memory or in pinned host memory (read by the
 *                  kernel over the host link, so a step needs no upload; the caller must not
 *                  rewrite it before the kernel has run); a negative slot leaves row s
 *                  unchanged.  Any other pointer: PKV_INVALID_ARG.
 * Rows whose slot does not match their length (slot % bs != p % bs) or whose new position
 * lies past max_blocks_per_seq blocks are left unchanged (a caller error, never a fault).
 * ------------------------------------------------------------------------------------ */
pkv_status pkv_apply_append(int32_t* block_tables, int32_t* context_lens, const int64_t* slot_mapping,
                            int num_seqs, int max_blocks_per_seq, int block_size, int num_blocks,
                            void* stream);

/* ------------------------------------------------------------------------------------
 * Host block allocator (host memory only; not thread-safe — callers serialise).
 *
 * Hands out physical block ids from a free list, counts references per block, shares
 * blocks between sequences and decides copy-on-write ("What is PagedAttention?",
 * glossary, "How It Works: Map Logical to Physical Blocks" and "Share Without Mutating
 * State"; "PagedAttention: Optimizing KV Cache in vLLM", §4).  Every call that can fail
 * is all-or-nothing: on any non-OK status the allocator state is exactly as before.
 * Slots follow the pool convention slot = block * bs + offset.
 * ------------------------------------------------------------------------------------ */
typedef struct pkv_alloc pkv_alloc;

/* Creates an allocator over blocks 0..num_blocks-1.  free_order (host, nullable, a
 * permutation of 0..num_blocks-1) fixes the order in which free blocks are first handed
 * out; NULL means ascending.  Returns NULL on invalid arguments (see pkv_last_error). */
pkv_alloc* pkv_alloc_create(int num_blocks, int block_size, const int32_t* free_order);
void pkv_alloc_destroy(pkv_alloc* a);

/* Prefill: a new sequence with `length` tokens takes ceil(length / bs) blocks.
 * slots_out (host, nullable) receives the `length` slots in token order. */
pkv_status pkv_seq_create(pkv_alloc* a, int64_t seq_id, int64_t length, int64_t* slots_out);

/* Sharing: `child` (new id) gets the parent's first ceil(prefix_len / bs) blocks, each
 * block's reference count is incremented, nothing is copied; child length = prefix_len. */
pkv_status pkv_seq_fork(pkv_alloc* a, int64_t parent, int64_t child, int64_t prefix_len);

/* Appends n tokens to one sequence.  slots_out (host, [n], nullable) gets their slots.
 * If the sequence's last block is partly filled and shared (count > 1) a private copy is
 * taken first: its (src, dst) pair goes to cow_out (host, [1][2], nullable) and
 * *n_cow_out (nullable) is 1, else 0. */
pkv_status pkv_seq_extend(pkv_alloc* a, int64_t seq_id, int64_t n, int64_t* slots_out,
                          int32_t* cow_out, int* n_cow_out);

/* Decode step: appends one token to each of n distinct sequences.  slots_out (host,
 * [n]) gets one slot per sequence; every copy-on-write taken is written to cow_out
 * (host, [n][2], (src, dst)) and counted in *n_cow_out.  Run pkv_copy_blocks on those
 * pairs before pkv_kv_cache_write on the slots. */
pkv_status pkv_seq_append(pkv_alloc* a, const int64_t* seq_ids, int n, int64_t* slots_out,
                          int32_t* cow_out, int* n_cow_out);

/* Releases a sequence; blocks whose reference count drops to zero return to the pool. */
pkv_status pkv_seq_free(pkv_alloc* a, int64_t seq_id);

/* Swap (the pages' named response to an allocation that cannot be met: "What is
 * PagedAttention?", glossary, "How It Works: Map Logical to Physical Blocks").  Moves
 * sequence seq_id from allocator `from` to allocator `to` -- typically the device pool's
 * and a pinned host pool's, in either direction -- all-or-nothing:
 *   - `to` takes one fresh block per logical block of the sequence (PKV_OUT_OF_BLOCKS if
 *     it has too few free; nothing changes then); sharing does not survive a swap;
 *   - pairs_out[2j], pairs_out[2j+1] = (block in `from`, block in `to`) of logical block j,
 *     for j < *n_pairs_out (the sequence's block count, pkv_seq_info); host memory;
 *   - the sequence leaves `from`: its blocks' reference counts drop, and blocks no other
 *     sequence holds return to `from`'s free list.
 * The caller copies the pairs with pkv_swap_blocks before anything writes the blocks freed
 * in `from` (enqueue the copy first on the stream that later writes them).  Both
 * allocators need the same block size; seq_id must not exist in `to`. */
pkv_status pkv_seq_swap(pkv_alloc* from, pkv_alloc* to, int64_t seq_id, int32_t* pairs_out,
                        int* n_pairs_out);

/* For each listed sequence, how many of its leading blocks have a reference count above 1,
 * i.e. are also read by another sequence (a prefix shared by forking: "What is
 * PagedAttention?", glossary, "Share Without Mutating State"), into host int32 out[n].  The
 * attention calls take these counts as their shared_prefix_blocks hint.  UNKNOWN_SEQ if a
 * sequence does not exist (nothing written). */
pkv_status pkv_alloc_shared_prefix_blocks(const pkv_alloc* a, const int64_t* seq_ids, int n,
                                          int32_t* out);

/* Column chunks for the decode with prefix groups (host arrays [n], for the listed sequences
 * in order).  A group is a run of listed sequences whose first block is the same shared
 * physical block (reference count > 1; a sequence whose first block is not shared is a group
 * of its own); each group is cut into chunks of at most max_chunk consecutive sequences
 * (max_chunk = 32 / G for the attention calls).  chunk_first[i] = index of the first sequence
 * of i's chunk; chunk_src[i] = the chunk sequence with the most shared leading blocks (its
 * table row is read); group_blocks[i] = leading blocks i shares with the source (equal table
 * entries), and at the source the most of any other chunk sequence (0 for a chunk of one).
 * UNKNOWN_SEQ if a sequence does not exist (nothing written). */
pkv_status pkv_alloc_prefix_groups(const pkv_alloc* a, const int64_t* seq_ids, int n, int max_chunk,
                                   int32_t* chunk_first, int32_t* chunk_src, int32_t* group_blocks);

/* Writes block tables (host int32 [n][max_blocks], padded with -1) and lengths (host
 * int32 [n], nullable) for the listed sequences. */
pkv_status pkv_alloc_block_tables(const pkv_alloc* a, const int64_t* seq_ids, int n,
                                  int max_blocks, int32_t* tables_out, int32_t* lens_out);

/* Occupancy of an allocator's pool, for waste accounting ("PagedAttention: Optimizing KV
 * Cache in vLLM", §2 "The Solution": paging leaves at most the last block of a sequence
 * partly empty; §4: shared blocks are stored once).  All counts are over the current state:
 *   used_blocks     physical blocks with a reference count > 0 (free_blocks the rest);
 *   shared_blocks   physical blocks with a reference count > 1;
 *   logical_blocks  sum over sequences of their block-table lengths;
 *   tokens          sum over sequences of their lengths (a shared token once per holder);
 *   stored_tokens   slots of used blocks that hold a token of at least one holder, so
 *                   used_blocks * block_size - stored_tokens is the unused space in held
 *                   blocks. */
typedef struct pkv_alloc_stats {
  int64_t num_blocks, free_blocks, used_blocks, shared_blocks;
  int64_t logical_blocks, tokens, stored_tokens, num_seqs;
} pkv_alloc_stats;
pkv_status pkv_alloc_stats_get(const pkv_alloc* a, pkv_alloc_stats* out);

/* Queries (host). */
int pkv_alloc_num_free(const pkv_alloc* a);
int pkv_alloc_num_blocks(const pkv_alloc* a);
int pkv_alloc_block_size(const pkv_alloc* a);
int pkv_alloc_refcount(const pkv_alloc* a, int block); /* -1 if out of range */
int pkv_alloc_num_seqs(const pkv_alloc* a);
pkv_status pkv_seq_info(const pkv_alloc* a, int64_t seq_id, int64_t* length_out,
                        int* num_blocks_out);
/* Copies the first `cap` free block ids (host) into ids_out and returns how many exist. */
int pkv_alloc_free_list(const pkv_alloc* a, int32_t* ids_out, int cap);

/* Slot mapping for whole sequences (host): for s in order and t < lens[s], writes
 * tables[s][t / bs] * bs + t % bs to slots_out (host, [sum lens]).  Used to place the
 * tokens of prefilled sequences whose tables were built elsewhere. */
pkv_status pkv_build_slot_mapping(const int32_t* tables, const int32_t* lens, int num_seqs,
                                  int max_blocks, int block_size, int64_t* slots_out);

/* ------------------------------------------------------------------------------------
 * KV pool in contiguous virtual memory, backed on demand (the alternative the pages set
 * against paging: "What is PagedAttention?", glossary, "Frequently Asked Questions" and
 * "Common Use Cases": contiguous virtual memory whose physical pages are mapped as a
 * sequence grows, versus paged blocks).  For comparing placements; the attention kernels
 * read it unchanged.
 *
 * pkv_vmm_create reserves, for K and for V, a virtual range of the pool layout with one
 * contiguous slice of max_blocks_per_seq blocks per sequence after a first page that stays
 * mapped, zeroed, for the pool's lifetime (block 0 lives there; the kernels read block 0 in
 * place of a table entry outside the pool).  Physical memory is mapped in pages: a page
 * holds whole blocks and whole device granules, and is the smallest such size at least
 * page_bytes (0: the runtime's recommended granule).  Each slice starts on a page.
 * block_bytes is one block of one pool (Hkv * bs * D * element bytes).  Returns NULL on
 * failure (see pkv_last_error; PKV_UNSUPPORTED where the device has no virtual memory
 * management).
 *
 * pkv_vmm_reserve maps physical memory (page by page, K and V) so that blocks
 * [0, num_blocks) of seq's slice are backed; all-or-nothing.  pkv_vmm_release unmaps and
 * frees all of seq's pages, and pkv_vmm_destroy everything; both first wait for all work on
 * the pool's device (hipDeviceSynchronize), so that no kernel still in flight reads an
 * unmapped page (pkv_vmm_release returns PKV_HIP_ERROR, with nothing unmapped, if that wait
 * fails).  No kernel may read a slice beyond its mapped blocks.
 *
 * Sequence seq's logical block j is pool block pkv_vmm_seq_first_block(seq) + j of the
 * pools at pkv_vmm_k_base / pkv_vmm_v_base, which hold pkv_vmm_num_blocks blocks (most of
 * them unmapped).  pkv_vmm_mapped_bytes counts the physical bytes mapped, both pools and the
 * base pages included; pkv_vmm_page_bytes is the page size.
 * ------------------------------------------------------------------------------------ */
typedef struct pkv_vmm pkv_vmm;
pkv_vmm* pkv_vmm_create(int device, int max_seqs, int max_blocks_per_seq, size_t block_bytes,
                        size_t page_bytes);
void pkv_vmm_destroy(pkv_vmm* v);
pkv_status pkv_vmm_reserve(pkv_vmm* v, int seq, int num_blocks);
pkv_status pkv_vmm_release(pkv_vmm* v, int seq);
void* pkv_vmm_k_base(const pkv_vmm* v);
void* pkv_vmm_v_base(const pkv_vmm* v);
int pkv_vmm_num_blocks(const pkv_vmm* v);
int pkv_vmm_seq_first_block(const pkv_vmm* v, int seq);
int pkv_vmm_mapped_blocks(const pkv_vmm* v, int seq);
size_t pkv_vmm_mapped_bytes(const pkv_vmm* v);
size_t pkv_vmm_page_bytes(const pkv_vmm* v);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
