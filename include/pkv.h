/*
 * pkv.h — paged KV-cache attention for one continuous-batching step, on one
 * AMD Instinct MI355X (gfx950).
 *
 * The problem (pages by title and section):
 *   - Each sequence's keys/values live in fixed-size blocks of a shared pool;
 *     a per-sequence block table maps logical block j to a physical block;
 *     only a sequence's last block may be partly filled.
 *     ("LLM 7 - Efficient LLM Serving", 3. KV Cache and PagedAttention,
 *     "Paging the Cache"; "The Serving Playbook", "Paged KV cache".)
 *   - Each step appends the new tokens' K/V into slots assigned by a slot
 *     mapping, then attends ("LLM 7", 3., "What the Cache Stores"; "The
 *     Serving Playbook", "CUDA graphs and the CPU you forgot about").
 *   - Context lengths are read from a device buffer, not passed as launch
 *     arguments, so launches are identical from step to step ("Inference
 *     Engineering, Part 2: What Actually Runs the Model", "What a kernel is,
 *     and three meanings of the word").
 *   - Query heads share KV heads in contiguous groups (grouped-query
 *     attention: "Inference Engineering, Part 2", "The KV cache").
 *   - A decode row is split along the KV axis into partitions whose partial
 *     softmax summaries a second pass rescales into the answer ("The Serving
 *     Playbook", "The block table lives in the hottest kernel in the system";
 *     "Kernel fusion, briefly"); the partial summaries combine by the online
 *     softmax rule ("LLM 7", 2. FlashAttention, "Online Softmax Makes Tiling
 *     Possible").
 *   - A prefill chunk attends causally to the cached prefix and to itself
 *     ("The Serving Playbook", "Chunked prefill"; "Prefill and decode want
 *     different machines").
 *
 * Conventions for every entry point
 *   - All tensors are device memory owned by the caller; the library never
 *     allocates or frees device memory and never synchronizes the host.
 *     Every call only enqueues kernels on `stream` (a hipStream_t; NULL = the
 *     null stream), so calls may be captured into a HIP graph.
 *   - Element type: the pool's dtype (PKV_F32 or PKV_BF16) for query, key,
 *     value and out; bf16 for all four with a PKV_FP8_E4M3 pool. Integer
 *     tensors are int32 except slot_mapping (int64).
 *   - Every pointer must be 16-byte aligned; tensors are dense row-major.
 *   - scale (the softmax scale of the attention calls, 1/sqrt(head_dim) in the
 *     usual case) must be finite and positive, and so must its product with
 *     log2(e) and an e4m3 layer's K scale; otherwise PKV_ERR_INVALID_ARG.
 *   - Errors: a non-zero pkv_status is returned and nothing is enqueued;
 *     pkv_last_error() gives a message (thread-local). Values *inside*
 *     device buffers (block ids, lengths, slots) cannot be checked without a
 *     synchronization and are the caller's contract: block ids in
 *     [0, num_blocks), 0 <= context_lens[b] <= max_blocks_per_seq*block_size,
 *     slots < num_blocks*block_size, no two tokens of one call with the same
 *     slot (they would race).
 *   - Supported geometry: block_size 16, or 32 for bf16 and e4m3 pools (the
 *     pages give 16 as the usual choice and favour 32 for traffic made mostly
 *     of long generations: "The Serving Playbook", "The block table lives in
 *     the hottest kernel in the system"); head_dim
 *     64 or 128; query heads per KV head (num_q_heads / num_kv_heads) from 1
 *     to 8.
 *
 * Pool layout in HBM, per layer (this is the "reshape" of reshape_and_cache:
 * the head dimension is cut into 16-byte vectors so that loads stay wide
 * despite the block-table indirection):
 *   K: [num_blocks][num_kv_heads][head_dim/x][block_size][x], x = 16/elem_bytes
 *      (16 for e4m3, 8 for bf16, 4 for fp32): for a fixed 16-byte slice of
 *      the head dimension, the 16 tokens of a block are consecutive 16-byte
 *      vectors.
 *   V: [num_blocks][num_kv_heads][block_size][head_dim]: each token's value
 *      row is contiguous.
 *   One (block, kv head) tile of K or V is block_size*head_dim*elem_bytes
 *   contiguous bytes (4 KiB for bf16 at head_dim 128).
 *
 * Eight-bit pools (PKV_FP8_E4M3). The pages note that an eight-bit KV cache
 * costs little in quality and halves the bytes decode streams ("The Serving
 * Playbook", "Quantized serving"); they fix neither the code nor the scale
 * granularity. This library stores OCP FP8 E4M3 codes (1 sign, 4 exponent
 * bits with bias 7, 3 mantissa bits; S.1111.111 is NaN; no infinity; largest
 * magnitude 448) with one fp32 scale per layer for K and one for V (set with
 * kv_pool_set_fp8_scales; 1.0 by default). A code c stands for
 * value(c) * scale. reshape_and_cache quantizes each bf16 input x as: y =
 * fp32(x) * fp32(1/scale) rounded in fp32; y clamped to [-448, 448] (NaN
 * stays NaN); rounded to the nearest code, ties to even. Attention treats the
 * pool as holding value(c) * scale exactly (codes widen to bf16 without
 * rounding; the K scale multiplies the softmax scale, the V scale the
 * output).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKV_OK = 0,
    PKV_ERR_INVALID_ARG = -1,   /* bad pointer, size, alignment or index */
    PKV_ERR_UNSUPPORTED = -2,   /* valid but not implemented (geometry, dtype) */
    PKV_ERR_HIP = -3,           /* the HIP runtime reported an error */
    PKV_ERR_WORKSPACE = -4      /* workspace missing or too small */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 } pkv_dtype;

/* Opaque handle: geometry plus per-layer K/V pool pointers (host memory only). */
typedef struct pkv_pool pkv_pool;

/* Text of the last non-OK status returned on this thread ("" if none). */
const char* pkv_last_error(void);

/* Bytes of one layer's K pool and V pool for the given geometry (each is
 * num_blocks*num_kv_heads*block_size*head_dim*elem_bytes). */
pkv_status kv_pool_bytes(int num_blocks, int block_size, int num_kv_heads, int head_dim,
                         pkv_dtype dtype, size_t* k_bytes_per_layer,
                         size_t* v_bytes_per_layer);

/* Wrap caller-allocated per-layer pools (device pointers, each at least
 * kv_pool_bytes() long, 16-byte aligned) in a handle. The handle copies the
 * two pointer arrays; it does not own the device memory. */
pkv_status kv_pool_create(pkv_pool** out, int num_layers, int num_blocks, int block_size,
                          int num_kv_heads, int head_dim, pkv_dtype dtype,
                          void* const* k_layers, void* const* v_layers);

/* Per-layer dequantization scales of an e4m3 pool: k_scales and v_scales
 * are host arrays of num_layers floats (num_layers must equal the pool's),
 * copied into the handle; later calls with this handle use them. Each scale
 * must be positive and finite with a finite, nonzero fp32 inverse; otherwise
 * PKV_ERR_INVALID_ARG and the handle is unchanged. Changing a scale does not
 * rewrite codes already stored. PKV_ERR_INVALID_ARG for a pool of another
 * dtype. Not thread-safe against concurrent calls on the same handle. */
pkv_status kv_pool_set_fp8_scales(pkv_pool* pool, int num_layers, const float* k_scales,
                                  const float* v_scales);

/* Free the handle (never the device memory). NULL is accepted. */
pkv_status kv_pool_destroy(pkv_pool* pool);

/* Append: for t < num_tokens with slot s = slot_mapping[t] >= 0, write
 * key[t][h][:] and value[t][h][:] (all KV heads h) into block s / block_size,
 * offset s % block_size of `layer`'s pools, in the layout above. Negative
 * slots are skipped. Values are copied bit for bit (e4m3 pools: quantized
 * with the layer's scales by the rule above).
 *   key, value: [num_tokens][num_kv_heads][head_dim], pool dtype (bf16 for
 *     an e4m3 pool).
 *   slot_mapping: int64 [num_tokens].
 * num_tokens == 0 is a no-op. */
pkv_status reshape_and_cache(const pkv_pool* pool, int layer, const void* key,
                             const void* value, const int64_t* slot_mapping,
                             int num_tokens, void* stream);

/* Copy-on-write: when sequences that share a block diverge, the shared block
 * is duplicated into a private one ("LLM 7 - Efficient LLM Serving", 3. KV
 * Cache and PagedAttention, "Sharing and Preemption"; "The Serving
 * Playbook", "Sharing is a reference count"). For every pair p <
 * num_pairs, block block_pairs[2p+1] of every layer's K and V pool becomes a
 * bit-for-bit copy of block block_pairs[2p] (all KV heads, all 16 slots).
 *   block_pairs: int32 [num_pairs][2] (source, destination), device memory.
 * Block ids must lie in [0, num_blocks); no destination may appear twice or
 * also be a source in the same call (the copies would race). num_pairs == 0
 * is a no-op. Any pool dtype. */
pkv_status copy_blocks(const pkv_pool* pool, const int32_t* block_pairs, int num_pairs, void* stream);

/* Workspace bytes paged_attention_decode needs for these arguments (0 when no
 * sequence can be split). Depends only on host-side sizes. */
pkv_status paged_attention_decode_workspace_bytes(const pkv_pool* pool, int num_seqs,
                                                  int num_q_heads, int max_blocks_per_seq,
                                                  int partition_size, size_t* bytes);

/* Decode attention: sequence b's single query row attends to the first
 * context_lens[b] tokens of its cache (the token appended this step included):
 *   out[b][i] = sum_t softmax_t(scale * <query[b][i], K_b[t][i/G]>) V_b[t][i/G]
 * with G = num_q_heads / num_kv_heads and K_b/V_b read through
 * block_tables[b][t / block_size]. context_lens[b] == 0 gives a zero row.
 *   out, query: [num_seqs][num_q_heads][head_dim], pool dtype (bf16 for an
 *     e4m3 pool; out is rounded to nearest even from fp32 accumulators).
 *   block_tables: int32 [num_seqs][max_blocks_per_seq]; entries past a
 *     sequence's last block are never read.
 *   context_lens: int32 [num_seqs].
 *   partition_size: how the KV axis is split over wavefronts.
 *     0 (recommended): balanced split. The 64-token windows of all
 *       (sequence, KV head) rows are shared equally by one wavefront per
 *       resident wave slot of the GPU; a row cut between wavefronts leaves
 *       partial (max, sum, output) summaries, and the wavefront that
 *       finishes the row's last piece combines them in the same launch (a
 *       completion counter per row, in the workspace). The split is derived
 *       on the device from context_lens. Used for up to 4096 sequences;
 *       larger batches fall back to 512-token partitions.
 *     > 0: fixed partitions of that many tokens (a multiple of 64); a
 *       sequence longer than one partition is combined by a second kernel.
 *     < 0: never split (one wavefront per (sequence, KV head)).
 *   workspace: device memory of at least
 *     paged_attention_decode_workspace_bytes(...) bytes (may be NULL when
 *     that is 0), 16-byte aligned. Its first 16 KiB hold completion
 *     counters (one int32 per balanced-split wavefront): they must be zero
 *     before the workspace's first use (allocate it zero-filled), and every
 *     call that completes leaves them zero again, so one workspace serves any
 *     sequence of decode calls of any variant (plain, _append, _multi,
 *     _shared) and sizes up to its length. The rest of the workspace is
 *     scratch whose contents on entry are ignored. Calls that share a
 *     workspace must be ordered (same stream). */
pkv_status paged_attention_decode(const pkv_pool* pool, int layer, void* out,
                                  const void* query, const int32_t* block_tables,
                                  const int32_t* context_lens, int num_seqs,
                                  int num_q_heads, int max_blocks_per_seq, float scale,
                                  int partition_size, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the same
 * computation as paged_attention_decode (same arguments minus the workspace,
 * same kernels, same results), with the workspace in a library-owned device
 * array of 36 MiB (each GPU the library runs on holds one until the process
 * ends). It allocates nothing and calls no allocating routine. Calls whose
 * workspace (paged_attention_decode_workspace_bytes) exceeds 36 MiB return
 * PKV_ERR_WORKSPACE; the balanced split (partition_size 0) of up to 4096
 * sequences with up to 8 query heads per KV head at head_dim 128 needs at
 * most ~33 MiB. Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (different streams, or host threads enqueueing
 * without ordering) race and give undefined results; calls ordered on one
 * stream are safe. */
pkv_status paged_attention_decode_noalloc(const pkv_pool* pool, int layer, void* out, const void* query,
                                          const int32_t* block_tables, const int32_t* context_lens,
                                          int num_seqs, int num_q_heads, int max_blocks_per_seq, float scale,
                                          int partition_size, void* stream);

/* Append and decode in one call, for latency-bound steps: the same result as
 * reshape_and_cache of each sequence's new token at position
 * context_lens[b] - 1 (slot block_tables[b][(ctx-1) / block_size] *
 * block_size + (ctx-1) % block_size) followed by paged_attention_decode,
 * with one kernel launch fewer. The wavefront whose segment ends a
 * sequence's row writes that row's new K/V into the slot, in the form the
 * pool stores (bf16 bits, or e4m3 codes quantized exactly as
 * reshape_and_cache does), and waits for the stores before it reads the
 * slot; outputs and pool contents are bit-identical to the two calls. The
 * pages append the new token's K/V and then attend ("LLM 7", 3., "What the
 * Cache Stores"), and note that at small batch the launches, not the work,
 * set the step time ("The Serving Playbook", "CUDA graphs and the CPU you
 * forgot about"). With partition_size < 0 a short-context step is one kernel.
 * At large batch the two calls are faster: the extra work sits on the
 * row-ending wave's critical path.
 *   key, value: [num_seqs][num_kv_heads][head_dim], bf16, 16-byte aligned;
 *     row b is written only when context_lens[b] >= 1.
 *   Everything else: as for paged_attention_decode (same workspace size).
 * bf16 and e4m3 pools; an fp32 pool gives PKV_ERR_UNSUPPORTED. */
pkv_status paged_attention_decode_append(const pkv_pool* pool, int layer, void* out, const void* query,
                                         const void* key, const void* value, const int32_t* block_tables,
                                         const int32_t* context_lens, int num_seqs, int num_q_heads,
                                         int max_blocks_per_seq, float scale, int partition_size,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* Decode with several query rows per sequence (speculative verification of
 * queries_per_seq - 1 draft tokens plus one, or a short chunk): sequence b's
 * queries_per_seq = T new tokens are already appended, so its cache holds
 * ctx = context_lens[b] >= T tokens, and query row j sits at position
 * ctx - T + j and attends causally to keys 0 .. ctx - T + j. This is the
 * prefill-chunk computation with equal chunk lengths (the pages treat decode
 * and chunked prefill as one rule over a query length: "Inference
 * Engineering, Part 2", "Prefill, decode, and the KV cache"; "The Serving
 * Playbook", "Chunked prefill"), run with the decode kernels' KV-axis split.
 *   out, query: [num_seqs][queries_per_seq][num_q_heads][head_dim], bf16
 *     (the rows of one sequence are consecutive tokens).
 *   block_tables, context_lens, partition_size, workspace: as for
 *     paged_attention_decode; the workspace size comes from
 *     paged_attention_decode_multi_workspace_bytes. context_lens[b] == 0 gives
 *     zero rows; 0 < context_lens[b] < queries_per_seq is a caller error.
 * bf16 and e4m3 pools. While queries_per_seq x (num_q_heads / num_kv_heads)
 * <= 16 the rows of one KV head share one matrix-core tile of the decode
 * kernels. Beyond that each sequence's rows run as an equal-length chunk on
 * the prefill-chunk kernel (no KV-axis split): the workspace size is then 0
 * and workspace may be NULL. queries_per_seq == 1 is paged_attention_decode. */
pkv_status paged_attention_decode_multi_workspace_bytes(const pkv_pool* pool, int num_seqs,
                                                        int queries_per_seq, int num_q_heads,
                                                        int max_blocks_per_seq, int partition_size,
                                                        size_t* bytes);
pkv_status paged_attention_decode_multi(const pkv_pool* pool, int layer, void* out, const void* query,
                                        int queries_per_seq, const int32_t* block_tables,
                                        const int32_t* context_lens, int num_seqs, int num_q_heads,
                                        int max_blocks_per_seq, float scale, int partition_size,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* Decode over shared prefixes. Sequences that share their leading tokens
 * point their block tables at the same physical blocks ("The Serving
 * Playbook", "Paged KV cache" and "Sharing is a reference count": parallel
 * sampling, beam search and a common system prompt are all several block
 * tables over one set of blocks). When such sequences decode in one batch,
 * their common blocks can be streamed from HBM a single time for the whole
 * group ("The Serving Playbook", "RadixAttention", "The tree changes what
 * the scheduler should do"). The result is that of paged_attention_decode on
 * the same arguments (within rounding); only the work is organised
 * differently. A group's shared region is its prefix rounded down to whole
 * 64-token windows; it is cut into pieces of partition_size tokens (the last
 * one shorter), each read once and multiplied against all members' query
 * heads together on the matrix cores. Every member's tokens after the shared
 * region are then read on their own with the balanced split of
 * paged_attention_decode, and the pieces are merged by the online-softmax
 * combine.
 *   out, query, block_tables, context_lens, scale: as for
 *     paged_attention_decode (one query row per sequence).
 *   group_starts: int32 [num_groups + 1], device memory. Group k is
 *     sequences group_starts[k] .. group_starts[k+1]-1; group_starts[0] == 0,
 *     non-decreasing, group_starts[num_groups] == num_seqs (so every sequence
 *     is in exactly one group; a sequence that shares nothing is a group of
 *     one with prefix 0). No group may have more than max_group_size members.
 *   prefix_lens: int32 [num_groups], device memory: group k's first
 *     prefix_lens[k] tokens sit in the same physical blocks, with the same
 *     block-table entries, for every member (caller contract). The blocks are
 *     read through the group's first sequence's table, so the shared region
 *     never extends past that sequence's context; a member whose context ends
 *     inside the region uses only the pieces wholly before its context end.
 *   partition_size: piece size, > 0 and a multiple of 64, or 0 for 512.
 *   workspace: at least paged_attention_decode_shared_workspace_bytes(...)
 *     bytes, 16-byte aligned, with the zero counters at its start that
 *     paged_attention_decode describes (this call leaves them untouched).
 * bf16 and e4m3 pools (the shared products run on bf16 MFMA) and at most 4096
 * sequences; otherwise PKV_ERR_UNSUPPORTED. */
pkv_status paged_attention_decode_shared_workspace_bytes(const pkv_pool* pool, int num_seqs,
                                                         int num_q_heads, int max_blocks_per_seq,
                                                         int partition_size, size_t* bytes);
pkv_status paged_attention_decode_shared(const pkv_pool* pool, int layer, void* out, const void* query,
                                         const int32_t* block_tables, const int32_t* context_lens,
                                         const int32_t* group_starts, const int32_t* prefix_lens,
                                         int num_seqs, int num_groups, int max_group_size,
                                         int num_q_heads, int max_blocks_per_seq, float scale,
                                         int partition_size, void* workspace, size_t workspace_bytes,
                                         void* stream);

/* Prefill-chunk attention: sequence s owns query rows
 * cu_q_lens[s] .. cu_q_lens[s+1]-1 (T_s = its chunk length, T_s <= max_q_len).
 * The chunk's own K/V must already be appended, so the cache holds
 * ctx_s = context_lens[s] >= T_s tokens; chunk row r is at absolute position
 * ctx_s - T_s + r and attends causally to positions 0 .. ctx_s - T_s + r.
 *   out, query: [total_q_tokens][num_q_heads][head_dim], bf16.
 *   cu_q_lens: int32 [num_seqs + 1], cu_q_lens[0] == 0, non-decreasing,
 *     cu_q_lens[num_seqs] == total_q_tokens.
 *   block_tables: int32 [num_seqs][max_blocks_per_seq]; context_lens: int32
 *     [num_seqs]. The contraction runs on bf16 MFMA: PKV_BF16 and
 *     PKV_FP8_E4M3 pools (e4m3 codes widen to bf16 exactly); an fp32 pool
 *     gives PKV_ERR_UNSUPPORTED. */
pkv_status paged_attention_prefill_chunk(const pkv_pool* pool, int layer, void* out,
                                         const void* query, const int32_t* cu_q_lens,
                                         const int32_t* block_tables,
                                         const int32_t* context_lens, int num_seqs,
                                         int total_q_tokens, int max_q_len, int num_q_heads,
                                         int max_blocks_per_seq, float scale, void* stream);

/* ---- gather ceiling (measurement support, not part of the attention path) ----
 * Decode at serving batch sizes is bound by streaming the KV cache through the
 * block table ("The Serving Playbook", "The block table lives in the hottest
 * kernel in the system"; "Inference Engineering, Part 2", "The KV cache").
 * This call reads exactly the K/V words paged_attention_decode reads for the
 * same arguments -- tokens 0 .. context_lens[b]-1 of every (sequence, KV head)
 * row, through block_tables, with the decode kernels' 16-byte streaming loads
 * and the balanced split's work order -- and does no attention arithmetic: it
 * folds them into
 *   checksum[b][h] = XOR of every 32-bit word of K_b[t][h] and V_b[t][h],
 *                    t < context_lens[b]  (0 for an empty sequence),
 * the words taken as the pool stores them. Its kernel time (timing kind
 * PKV_KERNEL_GATHER) is the rate a gather of these tiles sustains on the
 * device, against which the decode kernel's time can be set.
 *   checksum: uint32 [num_seqs][num_kv_heads], device memory, overwritten.
 *   block_tables, context_lens, max_blocks_per_seq: as for
 *     paged_attention_decode.
 *   workspace: at least (num_seqs + 1) * 4 bytes of device memory (contents
 *     on entry ignored).
 *   1 <= num_seqs <= 8192 (0 is a no-op); any pool dtype and geometry.
 * Two kernels are enqueued on `stream` (a one-workgroup plan kernel, then the
 * gather). */
pkv_status paged_kv_gather_checksum(const pkv_pool* pool, int layer, uint32_t* checksum,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    int num_seqs, int max_blocks_per_seq, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* ---- kernel timing (measurement support, not part of the attention path) ----
 * While enabled, every kernel of the kinds selected by kind_mask (bit k for
 * pkv_kernel_kind k; 0 selects all) that the library enqueues is launched
 * with a pair of HIP events that the launch itself stamps at the kernel's
 * start and end (hipExtLaunchKernelGGL; the events are created by
 * pkv_timing_enable, never inside the calls), so a pair times the kernel
 * alone. Timed launches cost a little host time, so measure only the kinds
 * needed. pkv_timing_read waits for the
 * recorded events and returns, for one kernel kind, the number of launches
 * recorded and their summed duration in milliseconds. Recording stops
 * silently once max_launches launches have been recorded. Not for use under
 * graph capture. */
typedef enum {
    PKV_KERNEL_APPEND = 0,
    PKV_KERNEL_DECODE_PARTITION = 1,
    PKV_KERNEL_DECODE_REDUCE = 2,
    PKV_KERNEL_PREFILL = 3,
    PKV_KERNEL_DECODE_PREFIX = 4,   /* shared-prefix partitions of paged_attention_decode_shared */
    PKV_KERNEL_GATHER = 5,          /* the gather kernel of paged_kv_gather_checksum */
    PKV_KERNEL_KINDS = 6
} pkv_kernel_kind;

pkv_status pkv_timing_enable(int max_launches, unsigned int kind_mask);
pkv_status pkv_timing_disable(void);
pkv_status pkv_timing_read(pkv_kernel_kind kind, int* launches, double* total_ms);

/* The recorded launches of one kernel kind one by one: writes the duration in
 * milliseconds of the first min(capacity, recorded) launches, in launch
 * order, to ms[] (a host array of `capacity` floats) and their count to
 * *launches. Waits for the events like pkv_timing_read. */
pkv_status pkv_timing_read_launches(pkv_kernel_kind kind, float* ms, int capacity, int* launches);

/* Device-value checks. Values inside device buffers (block ids, context
 * lengths, slots, chunk bounds) are the caller's contract and are not checked
 * by the release library, libpkv.so: checking them on the host would need a
 * synchronization, and a wrong block id becomes a wild read in the hottest
 * kernel ("The Serving Playbook", "The block table lives in the hottest
 * kernel in the system"). The debug library, libpkv_debug.so (the same
 * sources built with PKV_DEBUG=1, same entry points), tests each such value
 * in the kernels before forming any address from it:
 *   PKV_DEBUG_SLOT    a slot >= num_blocks * block_size: that write is skipped;
 *   PKV_DEBUG_BLOCK   a block id outside [0, num_blocks) in a block table or
 *                     a copy pair: block 0 is read instead / the copy skipped;
 *   PKV_DEBUG_CONTEXT a context length outside [0, max_blocks_per_seq *
 *                     block_size]: clamped into that range;
 *   PKV_DEBUG_CHUNK   prefill chunk bounds from cu_q_lens that leave the
 *                     query tensor, exceed max_q_len or the context: the
 *                     sequence is skipped.
 * The affected outputs are then defined (finite, no out-of-range access) but
 * not meaningful. pkv_debug_read_errors waits for the device
 * (hipDeviceSynchronize), returns the bits set since the last clear in
 * *flags, and clears them if `clear` is non-zero. The release library returns
 * PKV_ERR_UNSUPPORTED with *flags = 0. Not for use under graph capture. */
enum {
    PKV_DEBUG_SLOT = 1,
    PKV_DEBUG_BLOCK = 2,
    PKV_DEBUG_CONTEXT = 4,
    PKV_DEBUG_CHUNK = 8
};
pkv_status pkv_debug_read_errors(unsigned int* flags, int clear);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
