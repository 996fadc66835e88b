/*
 * pagedkv.h - C ABI of libpagedkv.so: the paged KV-cache decode path on
 * AMD Instinct MI355X (gfx950).
 *
 * The operations, each one or two hand-written HIP kernels:
 *
 *   pkv_paged_attention_decode  single-query attention of every sequence in
 *                               a batch over its KV cache, which lives in
 *                               fixed-size physical blocks reached through a
 *                               per-sequence block table;
 *   pkv_reshape_and_cache       write new tokens' key/value rows into the
 *                               cache slots the block manager assigned;
 *   pkv_copy_blocks             copy whole physical blocks (the copy step of
 *                               copy-on-write);
 *   pkv_swap_blocks             move whole blocks between the device cache and
 *                               a pool in pinned host memory;
 *   pkv_reshape_and_cache_fp8,  the same write and attention over an 8-bit
 *   pkv_paged_attention_decode_fp8  (E4M3) cache;
 *   pkv_paged_attention_prefill causal attention of many query tokens per
 *                               sequence over the same paged cache (and
 *                               _prefill_fp8 over the 8-bit cache);
 *   pkv_paged_attention_decode_grouped  decode of sequences that share blocks
 *                               (forks of one prompt), each shared tile read
 *                               once for all of them (and _grouped_fp8 over
 *                               the 8-bit cache); pkv_group_tiles builds its
 *                               tile lists from the block tables.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every array argument is a DEVICE pointer (memory the caller allocated
 *   on the current HIP device, e.g. a torch tensor's data_ptr()); the pools
 *   of pkv_swap_blocks may also be pinned host memory.  The
 *   library never allocates device memory, never frees caller memory and
 *   keeps no pointer after the call's work has been enqueued.
 * - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *   asynchronous on that stream; calls on one stream run in order, so
 *   copy_blocks -> reshape_and_cache -> paged_attention_decode performs
 *   "copy, redirect, then write, then attend".
 * - All arrays are dense, row-major (C order), with no padding.
 * - KV cache layout, for both k_cache and v_cache:
 *       [num_blocks][num_kv_heads][block_size][head_dim]
 *   so one (block, kv head) tile is block_size*head_dim contiguous elements
 *   and one physical block is num_kv_heads*block_size*head_dim contiguous
 *   elements.
 * - Slot numbering: slot = physical_block * block_size + offset.
 * - Element type is given by `dtype`; q, out, k, v and both caches share it
 *   (except in the _fp8 calls, whose caches hold 8-bit codes).
 *   Attention accumulates in fp32 and rounds the result to nearest even.
 * - Return value: PKV_OK (0) or a negative pkv_status.  Argument errors are
 *   detected on the host before anything is enqueued.  PKV_EHIP reports a
 *   failed launch; pkv_last_error() gives the HIP error text.
 * - Calls are thread-safe for distinct streams and buffers.
 * - Content preconditions (table entries inside the pool, lengths within the
 *   table, distinct slots, copy destinations distinct and not sources) are
 *   not checked on the hot path; the kernels only stay in bounds.  With
 *   PKV_DEBUG=1 in the environment every call synchronises its stream,
 *   checks them on the host and returns PKV_EINVAL (first offending index in
 *   pkv_last_error()) before enqueuing anything.
 *
 * Sources: the three web pages on PagedAttention ("Memory Optimization in
 * LLM Serving with PagedAttention"; "vLLM and PagedAttention: How Ideas
 * from Operating Systems Accelerated LLM Inference"; "Scaling LLM
 * Inference: Memory Management with PagedAttention and vLLM").
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_F32 = 0,   /* IEEE binary32 */
  PKV_F16 = 1,   /* IEEE binary16 */
  PKV_BF16 = 2,  /* bfloat16 */
  PKV_E4M3 = 3   /* 8-bit OCP E4M3 cache codes (copy and swap calls, which move bytes) */
} pkv_dtype;

/* OR-ed into the dtype argument of pkv_supported, pkv_paged_attention_plan
 * and pkv_paged_attention_workspace_bytes: the caches hold E4M3 codes (the
 * 8-bit cache of pkv_paged_attention_decode_fp8); the low bits stay the
 * type of q and out. */
#define PKV_KV_E4M3 0x100

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,        /* null pointer, negative size, Hq % Hkv != 0, ... */
  PKV_EUNSUPPORTED = -2,  /* head_dim / block_size / dtype not compiled in */
  PKV_EWORKSPACE = -3,    /* workspace missing or smaller than required */
  PKV_EHIP = -4           /* a HIP launch failed; see pkv_last_error() */
} pkv_status;

/* Decode kernel variants for pkv_paged_attention_decode_ex. */
typedef enum {
  PKV_PATH_AUTO = 0,       /* MFMA when 2 <= Hq/Hkv <= 16 and 16-bit, else VALU */
  PKV_PATH_VALU = 1,       /* one query head per workgroup, vector ALU dot products */
  PKV_PATH_MFMA = 2,       /* one KV head per workgroup, all its query heads on MFMA */
  PKV_PATH_CONTIGUOUS = 3  /* control: ignore block_tables; sequence s's logical
                              block j is physical block s*max_blocks_per_seq + j */
} pkv_decode_path;

/* OR-ed into the path argument (decode, plan and workspace calls): sequences
 * of the batch share physical blocks (forks of one prompt, beams, cached
 * prompts; "Memory Optimization in LLM Serving with PagedAttention", section
 * "Advanced Capabilities: Memory Sharing with Copy-on-Write").  Without it
 * the kernels read K/V with streaming (nontemporal) loads, which suit a
 * batch whose blocks are each read once per call (the lines are not kept for
 * reuse; a random gather of 4 KiB tiles measured 6.2-6.5 TB/s with them
 * against 5.6-5.8 TB/s without).  With it the K/V loads keep the cache's
 * default policy, so a block read by several sequences of the call is served
 * from the cache after its first read.  The result is the same either way;
 * only the speed differs. */
#define PKV_PATH_SHARED_BLOCKS 0x100

/* Library version, e.g. "pagedkv 0.1.0 gfx950". Static string. */
const char* pkv_version(void);

/* Static text of a status code. */
const char* pkv_status_string(int status);

/* Text of the last HIP error seen by this thread ("" if none). */
const char* pkv_last_error(void);

/* Supported shapes: nonzero if (dtype, head_dim, block_size) is compiled in.
 * head_dim in {64, 128, 256}; block_size in {8, 16, 32}; with PKV_KV_E4M3,
 * all but head_dim 64 with block_size 8. */
int pkv_supported(pkv_dtype dtype, int head_dim, int block_size);

/* How a decode call divides its work (the grid argument; pkv_plan.grid
 * reports DIRECT or PLANNED). */
typedef enum {
  PKV_GRID_AUTO = 0,     /* the library chooses (see pkv_paged_attention_plan) */
  PKV_GRID_DIRECT = 1,   /* one workgroup per (head unit, partition, sequence) in index order */
  PKV_GRID_PLANNED = 2   /* a planning kernel lists the partitions, largest first */
} pkv_grid;

/* The plan of a decode call (filled by pkv_paged_attention_plan). */
typedef struct {
  int path;              /* PKV_PATH_VALU or PKV_PATH_MFMA */
  int grid;              /* pkv_grid */
  int partition_tokens;  /* P: tokens per partition at most */
  int max_parts;         /* ceil(min(max_context_len, table capacity) / P) */
  int longest_first;     /* 1 if workgroups start longest sequence / partition first */
  size_t workspace_bytes;
} pkv_plan;

/*
 * How a decode call with these sizes would run.
 *
 * Kernel: grouped query heads (2 <= Hq/Hkv <= 16, fp16/bf16, head_dim 64 or
 * 128, block_size 16 or 32) run on the MFMA kernel, which reads each KV tile
 * once for the whole group; everything else on the vector-ALU kernel.
 *
 * Partitions: a context of L tokens is cut into n = ceil(L / P) partitions
 * of equal size (rounded up to a multiple of max(32, block_size) tokens, the
 * last one shorter), one workgroup per partition and head unit (a KV head
 * for MFMA, a query head for VALU), merged by a second kernel when n > 1.
 * partition_tokens == 0 lets the library choose P: when the (sequence, head)
 * units are too few to give every compute unit about two workgroups, the
 * contexts are cut to do so (never below 512 tokens); otherwise contexts
 * longer than half the length bound are cut in two (never below 2048
 * tokens), so that no single long context ends the launch alone; at most
 * 256 units of the kernel (4096 tokens for 16-bit types with head_dim 128).
 * An explicit P must be a multiple of 32 and of block_size and at most 2^20.
 *
 * Grid DIRECT: workgroups in (head unit, partition, sequence) order.  When
 * the grid holds more than one round of resident workgroups and the batch
 * at most 1024 sequences, each workgroup ranks the lengths itself and
 * sequence row z is the z-th longest (half-octave bins, stable), so the
 * longest sequences start first.  Grid PLANNED (PKV_GRID_AUTO picks it for
 * such grids with more than 1024 sequences; at most 65535 partitions per
 * sequence and 2^31 - 1 workgroups): a one-workgroup kernel first lists
 * the (sequence, partition) items largest partition first (half-octave
 * size bins, stable, a sequence's partitions together) in the workspace,
 * and the decode grid follows the list, skipping the empty partitions of
 * the direct grid.  In both the head unit is the fastest index.
 *
 * The plan only changes the order of floating-point operations inside one
 * output row, never which tokens contribute.  Writes the plan to *out (if
 * not NULL).  Returns PKV_OK or the status pkv_paged_attention_decode_ex
 * would return for these sizes.  Host only; queries the current device's
 * compute-unit count and kernel occupancy (once, then cached).
 */
int pkv_paged_attention_plan(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                             int block_size, int max_blocks_per_seq, int max_context_len,
                             pkv_dtype dtype, int partition_tokens, int path, int grid,
                             pkv_plan* out);

/*
 * Workspace bytes pkv_paged_attention_decode(_ex) needs for these sizes (the
 * plan's workspace_bytes): with max_parts > 1 the partial states (head_dim
 * + 2 fp32 per sequence, query head and partition), and with the planned
 * grid its work list (16 bytes per sequence and partition, plus 8 bytes per
 * sequence), each part rounded to 16 bytes; 0 for a direct grid with one
 * partition per sequence.  Returns (size_t)-1 for invalid sizes.  Host only.
 */
size_t pkv_paged_attention_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                           int head_dim, int block_size, int max_blocks_per_seq,
                                           int max_context_len, pkv_dtype dtype,
                                           int partition_tokens, int path, int grid);

/*
 * paged_attention_decode: out[s][h][:] = softmax(scale * K_s q[s][h]) V_s
 *
 * For each sequence s and query head h, with L = context_lens[s] and
 * kv head g = h / (num_q_heads / num_kv_heads), token t < L of the sequence
 * is read from physical block block_tables[s][t / block_size] at offset
 * t % block_size.  The keys of its L tokens are scored against q[s][h],
 * scaled by `scale`, passed through a softmax over the L scores, and the
 * value rows are summed with those weights.
 *
 * Passages: the kernel gathers a sequence's scattered KV blocks through its
 * block table to compute the attention ("Memory Optimization in LLM Serving
 * with PagedAttention", section "How PagedAttention Works"; "vLLM and
 * PagedAttention ...", paragraph on the engine's custom kernels).  Only the
 * last block of a sequence is partly filled (same section, bullet on
 * fragmentation), so the kernel reads ceil(L / block_size) table entries and
 * masks the tail by index.  The attention formula and the grouping of query
 * heads onto KV heads are standard readings; the pages do not print them.
 *
 * Arguments (sizes are element counts unless noted):
 *   out           [num_seqs][num_q_heads][head_dim]       written
 *   q             [num_seqs][num_q_heads][head_dim]       read
 *   k_cache,
 *   v_cache       [num_blocks][num_kv_heads][block_size][head_dim]   read
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]    read; entries at
 *                 index >= ceil(L / block_size) are never read
 *   context_lens  int32 [num_seqs]                        read
 *   scale         softmax scale (usually 1/sqrt(head_dim))
 *   max_context_len  host-side upper bound of context_lens (sizes the grid;
 *                 no device-to-host read happens)
 *   workspace     device scratch of at least
 *                 pkv_paged_attention_workspace_bytes(...) bytes, 16-byte
 *                 aligned (may be NULL when that is 0); contents need not be
 *                 initialised.  Calls that share a workspace must be ordered
 *                 (for example, on one stream).
 *
 * Result for L == 0: a zero row.  Preconditions that are not checked on the
 * device: 0 <= context_lens[s] <= min(max_context_len,
 * max_blocks_per_seq*block_size) and table entries in [0, num_blocks).
 * Violations never cause out-of-bounds accesses: a length is clamped to
 * those bounds, and a table entry outside [0, num_blocks) makes that
 * (sequence, head) output NaN.  `out` must not alias any input.
 */
int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               float scale, int num_seqs, int num_q_heads, int num_kv_heads,
                               int head_dim, int block_size, int num_blocks,
                               int max_blocks_per_seq, int max_context_len, pkv_dtype dtype,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device scratch pkv_paged_attention_decode_noalloc holds per GPU. */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * paged_attention_decode_noalloc: pkv_paged_attention_decode (same
 * arguments without the workspace, the library's own plan) for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It calls no hipMalloc, hipFree or
 * other allocating routine; its workspace is a scratch array of
 * PKV_NOALLOC_SCRATCH_BYTES in device memory that the library holds on every
 * GPU it runs on until the process ends (looked up on its first call on a
 * device).  Results are those of pkv_paged_attention_decode with a workspace
 * of its own (the same kernels and plan).
 *
 * A call whose plan needs more workspace than that
 * (pkv_paged_attention_workspace_bytes(..., 0, PKV_PATH_AUTO, PKV_GRID_AUTO)
 * above PKV_NOALLOC_SCRATCH_BYTES) returns PKV_EWORKSPACE before touching the
 * device, with the sizes in pkv_last_error(); argument errors as
 * pkv_paged_attention_decode.  Every call on one GPU uses that GPU's one
 * array, which keeps the last call's contents (nothing in it needs to start
 * at zero): calls that overlap on one GPU (on different streams, or from
 * different threads without ordering) race and give wrong results; order
 * them, for example on one stream.
 */
int pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, float scale, int num_seqs,
                                       int num_q_heads, int num_kv_heads, int head_dim,
                                       int block_size, int num_blocks, int max_blocks_per_seq,
                                       int max_context_len, pkv_dtype dtype, void* stream);

/* Same as pkv_paged_attention_decode with an explicit partition size
 * (0 = library choice; see pkv_paged_attention_plan for the rules), kernel
 * variant (pkv_decode_path) and grid (pkv_grid).  Used for tuning sweeps,
 * tests of every grid and the contiguous-layout control. */
int pkv_paged_attention_decode_ex(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, float scale, int num_seqs,
                                  int num_q_heads, int num_kv_heads, int head_dim,
                                  int block_size, int num_blocks, int max_blocks_per_seq,
                                  int max_context_len, pkv_dtype dtype, void* workspace,
                                  size_t workspace_bytes, int partition_tokens, int path,
                                  int grid, void* stream);

/* Same as pkv_paged_attention_decode_ex, and records begin_event on `stream`
 * right before the attention kernel is launched and end_event right after
 * it (before the partition merge and after the planning kernel), so that
 * hipEventElapsedTime gives the attention kernel's own duration.  The events
 * are hipEvent_t handles the caller created; either may be NULL.  For
 * measurement; the result is the same as pkv_paged_attention_decode_ex's. */
int pkv_paged_attention_decode_timed(void* out, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_tables,
                                     const int32_t* context_lens, float scale, int num_seqs,
                                     int num_q_heads, int num_kv_heads, int head_dim,
                                     int block_size, int num_blocks, int max_blocks_per_seq,
                                     int max_context_len, pkv_dtype dtype, void* workspace,
                                     size_t workspace_bytes, int partition_tokens, int path,
                                     int grid, void* begin_event, void* end_event, void* stream);

/*
 * reshape_and_cache: for every token j with slot = slot_mapping[j] >= 0,
 *   k_cache[slot / block_size][g][slot % block_size][:] = k[j][g][:]
 *   v_cache[slot / block_size][g][slot % block_size][:] = v[j][g][:]
 * for every kv head g.  A byte-exact copy; no arithmetic on the values.
 *
 * Passage: blocks are filled as generation proceeds, each new token going
 * into the slot its sequence's block table provides ("Memory Optimization
 * in LLM Serving with PagedAttention", section "How PagedAttention Works",
 * on-demand allocation; "vLLM and PagedAttention ...", paragraph on the
 * solution); after a copy-on-write the write goes to the new copy (section
 * "Advanced Capabilities: Memory Sharing with Copy-on-Write").
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim]    read
 *   slot_mapping  int64 [num_tokens]; negative = skip     read
 *   k_cache, v_cache  as above                            written at the slots
 *
 * Slots must be distinct (else which write wins is unspecified).  A slot
 * >= num_blocks*block_size is skipped (never written out of bounds).
 * num_tokens == 0 is a no-op.
 */
int pkv_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                          const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                          int head_dim, int block_size, int num_blocks, pkv_dtype dtype,
                          void* stream);

/*
 * copy_blocks: for every pair i, k_cache[dst_i] = k_cache[src_i] and
 * v_cache[dst_i] = v_cache[src_i], whole physical blocks
 * (num_kv_heads*block_size*head_dim elements each), byte for byte.
 *
 * Passage: copy-on-write allocates a new block and copies the content of
 * the shared block into it before the table is redirected and the token is
 * written ("Memory Optimization in LLM Serving with PagedAttention", section
 * "Advanced Capabilities: Memory Sharing with Copy-on-Write"); one block is
 * copied, not the whole cache ("vLLM and PagedAttention ...", paragraph on
 * sharing).
 *
 *   src_dst_pairs  int64 [num_pairs][2] = {src, dst}      read
 *
 * Destinations must be distinct and must not be the source of any pair in
 * the same call (copy-on-write always copies into a fresh block).  A pair
 * with an index outside [0, num_blocks) is skipped.  num_pairs == 0 is a
 * no-op.
 */
int pkv_copy_blocks(void* k_cache, void* v_cache, const int64_t* src_dst_pairs, int num_pairs,
                    int num_kv_heads, int head_dim, int block_size, int num_blocks,
                    pkv_dtype dtype, void* stream);

/*
 * swap_blocks: for every pair i, dst_k[dst_i] = src_k[src_i] and
 * dst_v[dst_i] = src_v[src_i], whole blocks as in copy_blocks, byte for
 * byte, between two block pools of the same block shape: the device cache
 * and a pool in pinned host memory (swap out), or back (swap in).
 *
 * Passage: when memory runs short the engine evicts whole sequences, by
 * swapping their blocks to CPU memory or by recomputation ("vLLM and
 * PagedAttention: How Ideas from Operating Systems Accelerated LLM
 * Inference", paragraph on the engine).  Which blocks move, and where, is
 * the block manager's decision (paged_kv_cache_389_amd/block_manager.py).
 *
 *   dst_k, dst_v   [num_dst_blocks][num_kv_heads][block_size][head_dim]   written
 *   src_k, src_v   [num_src_blocks][...]                                 read
 *   src_dst_pairs  int64 [num_pairs][2] = {src, dst}                     read
 *
 * Every pointer must be device-accessible: device memory, or host memory
 * from hipHostMalloc (PyTorch's pinned memory), which the kernel reads or
 * writes directly over the host link.  Destinations must be distinct; the
 * source and destination pools must not overlap.  A pair with an index
 * outside its pool is skipped.  num_pairs == 0 is a no-op.  Asynchronous
 * on `stream` like every call: the host may read a swapped-out pool only
 * after synchronising with it.
 */
int pkv_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                    const int64_t* src_dst_pairs, int num_pairs, int num_kv_heads, int head_dim,
                    int block_size, int num_src_blocks, int num_dst_blocks, pkv_dtype dtype,
                    void* stream);

/*
 * An 8-bit KV cache (E4M3 codes with one scale per cache).
 *
 * Passage: quantising the KV cache to INT8/FP8 is named among the memory
 * features of serving libraries ("Memory Optimization in LLM Serving with
 * PagedAttention", section "Broader Context").  The pages fix nothing more;
 * the readings: OCP E4M3 codes (sign, 4-bit exponent with bias 7, 3-bit
 * fraction; largest finite 448, NaN 0x7F, no infinity), one float scale for
 * the K cache and one for the V cache, and a stored code c meaning
 * value(c) * scale.
 *
 * reshape_and_cache_fp8: as pkv_reshape_and_cache, but the caches are uint8
 * [num_blocks][num_kv_heads][block_size][head_dim] and each element x of k
 * (v) is stored as the code of the float32 quotient x / k_scale (v_scale):
 * NaN -> 0x7F, magnitudes above 448 (infinity included) saturate to +-448,
 * everything else rounds to the nearest code, ties to the even one; zero
 * keeps its sign.  k and v are of type `dtype` (PKV_F32, PKV_F16 or
 * PKV_BF16), [num_tokens][num_kv_heads][head_dim]; head_dim must be a
 * multiple of 16.  Slots behave as in pkv_reshape_and_cache.  Scales must
 * be finite and nonzero (else PKV_EINVAL).
 */
int pkv_reshape_and_cache_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                              const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                              int head_dim, int block_size, int num_blocks, pkv_dtype dtype,
                              float k_scale, float v_scale, void* stream);

/*
 * paged_attention_decode_fp8: pkv_paged_attention_decode_timed over E4M3
 * caches: the keys and values of the attention are value(code) * k_scale
 * and value(code) * v_scale.  q and out are of type `dtype` (PKV_F32,
 * PKV_F16 or PKV_BF16); k_cache and v_cache are uint8 codes in the cache
 * layout.  The scales multiply outside the dot products (scores by
 * scale * k_scale, the output by v_scale), which is exact up to rounding
 * order.  The workspace size is pkv_paged_attention_workspace_bytes with
 * dtype | PKV_KV_E4M3.  Kernels as for 16-bit caches: AUTO takes the MFMA
 * kernel for 16-bit queries with 2 <= Hq/Hkv <= 16 (head_dim 64 or 128,
 * block_size 16 or 32) and the vector-ALU kernel otherwise; the
 * CONTIGUOUS control returns PKV_EUNSUPPORTED.  Everything else, events
 * included, as pkv_paged_attention_decode_timed.
 */
int pkv_paged_attention_decode_fp8(void* out, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, float scale, float k_scale,
                                   float v_scale, int num_seqs, int num_q_heads, int num_kv_heads,
                                   int head_dim, int block_size, int num_blocks,
                                   int max_blocks_per_seq, int max_context_len, pkv_dtype dtype,
                                   void* workspace, size_t workspace_bytes, int partition_tokens,
                                   int path, int grid, void* begin_event, void* end_event,
                                   void* stream);

/*
 * paged_attention_prefill: causal attention of many query tokens per
 * sequence over the paged cache (prefill, or the recomputation of an
 * evicted sequence).
 *
 * Sequence s has L = context_lens[s] tokens in the cache (its new tokens
 * included: write them with reshape_and_cache first) and n = query_start[s+1]
 * - query_start[s] query rows q[query_start[s] .. query_start[s+1]), which
 * are its last n positions: query i sits at position p = L - n + i and
 *   out[query_start[s] + i][h][:] = softmax(scale * K_{0..p} q) V_{0..p}
 * over tokens 0 .. p, each read through block_tables[s] as in decode; a
 * query with p < 0 gives a zero row.
 *
 * Passage: the engine evicts whole sequences when memory runs short and
 * brings them back by swapping or by recomputation ("vLLM and PagedAttention:
 * How Ideas from Operating Systems Accelerated LLM Inference", paragraph on
 * the engine); recomputation attends many tokens at once over the paged
 * cache.  The causal reading is not printed on the pages.
 *
 *   out, q        [total_q][num_q_heads][head_dim]   (q read, out written)
 *   query_start   int32 [num_seqs + 1], non-decreasing, query_start[0] = 0,
 *                 query_start[num_seqs] = total_q  (read; values are clamped
 *                 to [0, total_q])
 *   max_q_len     host-side bound of every n (sizes the grid; query rows past
 *                 it may be left unwritten)
 *   k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
 *   max_blocks_per_seq, num_blocks: as in pkv_paged_attention_decode.
 *   begin_event, end_event: optional hipEvent_t recorded around the kernel.
 *
 * dtype PKV_F16 or PKV_BF16; head_dim 64 or 128; block_size 16 or 32;
 * num_q_heads / num_kv_heads must divide 16 (else PKV_EUNSUPPORTED).  No
 * workspace.  A table entry outside [0, num_blocks) makes the rows that read
 * it NaN; nothing is read or written out of bounds.  `out` must not alias
 * an input.  num_seqs, total_q or max_q_len == 0 is a no-op.
 */
int pkv_paged_attention_prefill(void* out, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* query_start,
                                float scale, int num_seqs, int total_q, int max_q_len,
                                int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                int num_blocks, int max_blocks_per_seq, int max_context_len,
                                pkv_dtype dtype, void* begin_event, void* end_event,
                                void* stream);

/* paged_attention_prefill_fp8: pkv_paged_attention_prefill over E4M3 caches
 * (uint8 codes in the cache layout, written by pkv_reshape_and_cache_fp8):
 * keys and values are value(code) * k_scale and value(code) * v_scale, the
 * scales applied outside the products as in pkv_paged_attention_decode_fp8.
 * Scales must be finite and nonzero (else PKV_EINVAL); everything else as
 * pkv_paged_attention_prefill. */
int pkv_paged_attention_prefill_fp8(void* out, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* block_tables,
                                    const int32_t* context_lens, const int32_t* query_start,
                                    float scale, float k_scale, float v_scale, int num_seqs,
                                    int total_q, int max_q_len, int num_q_heads,
                                    int num_kv_heads, int head_dim, int block_size,
                                    int num_blocks, int max_blocks_per_seq, int max_context_len,
                                    pkv_dtype dtype, void* begin_event, void* end_event,
                                    void* stream);

/*
 * paged_attention_decode_grouped: decode attention of sequences that share
 * KV blocks, reading each shared tile once for all of them.
 *
 * The output is that of pkv_paged_attention_decode for every sequence named
 * in a group:
 *   out[s][h][:] = softmax(scale * K_s q[s][h]) V_s   over the L = context_lens[s]
 * tokens of s, with fp32 accumulation; only the order in which its tiles
 * are summed differs.  Rows of sequences in no group are not written.
 *
 * Passage: sequences forked from one prompt (parallel sampling, beam search)
 * map their shared prefix to the same physical blocks through their block
 * tables, with reference counts and copy-on-write on the last partly filled
 * block ("Memory Optimization in LLM Serving with PagedAttention", section
 * "Advanced Capabilities: Memory Sharing with Copy-on-Write"; "vLLM and
 * PagedAttention: How Ideas from Operating Systems Accelerated LLM
 * Inference", paragraph on sharing).  Reading a shared block once for all
 * its sequences is this library's addition.
 *
 * Instead of block tables the call takes, per group, the list of distinct
 * 16-token tiles its members reach, built from the tables on the device by
 * pkv_group_tiles (pass its group_tile_start and group_tile_end) or on the
 * host by paged_kv_cache_389_amd.block_manager.group_tiles (a prefix
 * group_tile_start, group_tile_end NULL):
 *   group_members     int32 [num_groups][max_members]: sequence indices, -1 for
 *                     an empty place; a sequence in at most one group
 *   group_tile_start  int32 [num_groups + 1]: group j's entries are
 *                     group_tiles[group_tile_start[j] .. group_tile_start[j+1]),
 *                     group_tile_start[0] = 0, non-decreasing, at most
 *                     num_tiles (the kernel clamps the offsets to [0, num_tiles])
 *   group_tile_end    NULL, or int32 [num_groups]: group j's rows are then
 *                     group_tiles[group_tile_start[j] .. group_tile_end[j])
 *                     (group_tile_start needs num_groups entries; groups may
 *                     leave unused rows between them, as pkv_group_tiles does)
 *   group_tiles       int32 [num_tiles][4], 16-byte aligned: (physical block b,
 *                     tile index t, member mask, unused).  Entry (b, t, mask)
 *                     says that for every member m with bit m of mask set,
 *                     tokens 16t .. 16t+15 of the member live in block b at
 *                     offsets (16t mod block_size) .. +15, i.e.
 *                     block_tables[s_m][16t / block_size] == b.  Every member
 *                     must have exactly one entry for each of its tiles
 *                     0 .. ceil(L/16) - 1 and none past them.
 *   out, q            [num_seqs][num_q_heads][head_dim]
 *   k_cache, v_cache  [num_blocks][num_kv_heads][block_size][head_dim]
 *   context_lens      int32 [num_seqs]; clamped to [0, max_context_len]
 *   part_tiles        0: one workgroup per (group, KV head) walks the whole
 *                     list; > 0: the list is cut into parts of part_tiles rows,
 *                     one workgroup each, whose (max, sum, output) states a
 *                     second kernel merges (more workgroups for few groups)
 *   max_group_tiles   host-side bound of every group's row count (sizes the
 *                     grid; rows of a group past it are not read)
 *   workspace         device memory of at least
 *                     pkv_paged_attention_grouped_workspace_bytes(...) bytes,
 *                     16-byte aligned, caller-owned, contents need no
 *                     initialisation (null when that size is 0)
 *   begin_event, end_event: optional hipEvent_t recorded around the first
 *                     kernel (the merge, when there is one, runs after it).
 * All arrays are device memory, read only except out.
 *
 * dtype PKV_F16 or PKV_BF16; head_dim 64 or 128; block_size 16 or 32;
 * max_members * (num_q_heads / num_kv_heads) <= 16; num_groups and
 * num_kv_heads <= 65535, at most 65535 parts per group (else
 * PKV_EUNSUPPORTED).  group_tiles not 16-byte aligned, a null pointer or a
 * bad size returns PKV_EINVAL; a missing or short workspace PKV_EWORKSPACE.
 * A block outside [0, num_blocks) makes the rows of its group NaN; nothing
 * is read or written out of bounds whatever the list holds.  A missing or
 * repeated tile gives a wrong row, not a fault; PKV_DEBUG=1 checks the list
 * (coverage, pool, membership) on the host first.  `out` must not alias an
 * input.  num_groups or num_seqs == 0 is a no-op.
 */
int pkv_paged_attention_decode_grouped(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* context_lens,
                                       const int32_t* group_members, const int32_t* group_tiles,
                                       const int32_t* group_tile_start,
                                       const int32_t* group_tile_end, int num_tiles,
                                       float scale, int num_seqs, int num_groups, int max_members,
                                       int num_q_heads, int num_kv_heads, int head_dim,
                                       int block_size, int num_blocks, int max_context_len,
                                       pkv_dtype dtype, int part_tiles, int max_group_tiles,
                                       void* workspace, size_t workspace_bytes,
                                       void* begin_event, void* end_event, void* stream);

/* paged_attention_decode_grouped_fp8: pkv_paged_attention_decode_grouped over
 * E4M3 caches (uint8 codes in the cache layout, written by
 * pkv_reshape_and_cache_fp8): keys and values are value(code) * k_scale and
 * value(code) * v_scale, the scales applied outside the products as in
 * pkv_paged_attention_decode_fp8.  Scales must be finite and nonzero (else
 * PKV_EINVAL); dtype is the type of q and out; everything else as
 * pkv_paged_attention_decode_grouped. */
int pkv_paged_attention_decode_grouped_fp8(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* context_lens, const int32_t* group_members, const int32_t* group_tiles,
    const int32_t* group_tile_start, const int32_t* group_tile_end, int num_tiles, float scale,
    float k_scale, float v_scale,
    int num_seqs, int num_groups, int max_members, int num_q_heads, int num_kv_heads,
    int head_dim, int block_size, int num_blocks, int max_context_len, pkv_dtype dtype,
    int part_tiles, int max_group_tiles, void* workspace, size_t workspace_bytes,
    void* begin_event, void* end_event, void* stream);

/*
 * group_tiles: the tile lists of pkv_paged_attention_decode_grouped, built on
 * the device from the block tables (for each group, the same rows in the same
 * order as the host builder paged_kv_cache_389_amd.block_manager.group_tiles).
 *
 * For group j (members group_members[j][0 .. max_members), -1 = none), every
 * distinct (physical block b, 16-token tile index t) that a member reaches
 * (t < ceil(L / 16), L = context_lens[s] clamped to [0, len_cap], len_cap =
 * min(max_context_len, max_blocks_per_seq * block_size), b =
 * block_tables[s][16 t / block_size]) becomes one row (b, t, mask, 0), mask
 * bit m set for every member m that maps t to b; rows in t order, then b
 * ascending.  Group j's rows are written from row j * stride, stride =
 * max_members * ceil(len_cap / 16) (always enough), and
 * group_tile_start[j] = j * stride, group_tile_end[j] = one past its last row:
 * pass both to the grouped decode.
 *
 * Passage: block tables map a sequence's logical blocks to physical ones
 * ("Memory Optimization in LLM Serving with PagedAttention", section "How
 * PagedAttention Works"); forks of one prompt share its blocks (section
 * "Advanced Capabilities: Memory Sharing with Copy-on-Write").
 *
 *   block_tables      int32 [num_seqs][max_blocks_per_seq]  (read)
 *   context_lens      int32 [num_seqs]                      (read)
 *   group_members     int32 [num_groups][max_members]       (read)
 *   group_tiles       int32 [tiles_capacity][4], 16-byte aligned (written), at
 *                     least pkv_group_tiles_capacity(...) rows
 *   group_tile_start, group_tile_end  int32 [num_groups]    (written)
 * Device memory; one kernel, one workgroup per group, on `stream`.
 * max_members at most 16 and block_size a multiple of 16 (else
 * PKV_EUNSUPPORTED); a short capacity returns PKV_EWORKSPACE; null pointers,
 * negative sizes or a misaligned group_tiles PKV_EINVAL.  Members outside
 * [0, num_seqs) are ignored; table entries are copied as they are (the decode
 * turns an out-of-pool block into NaN rows).  num_groups == 0 is a no-op.
 */
int pkv_group_tiles(const int32_t* block_tables, const int32_t* context_lens,
                    const int32_t* group_members, int num_seqs, int max_blocks_per_seq,
                    int num_groups, int max_members, int block_size, int max_context_len,
                    int32_t* group_tiles, int tiles_capacity, int32_t* group_tile_start,
                    int32_t* group_tile_end, void* stream);

/* Rows of group_tiles pkv_group_tiles needs:
 * num_groups * max_members * ceil(len_cap / 16); (size_t)-1 for a bad size. */
size_t pkv_group_tiles_capacity(int num_groups, int max_members, int block_size,
                                int max_blocks_per_seq, int max_context_len);

/* Bytes of workspace pkv_paged_attention_decode_grouped needs for these
 * arguments (0 when every group is one part); (size_t)-1 for a negative
 * argument. */
size_t pkv_paged_attention_grouped_workspace_bytes(int num_groups, int num_kv_heads,
                                                   int head_dim, int part_tiles,
                                                   int max_group_tiles);

/*
 * Reference reads (measurement only; not part of the attention path).  They
 * give the practical ceiling a paged read is judged against beside the HBM3E
 * peak: the pages locate the cost of serving in memory traffic ("Scaling LLM
 * Inference: Memory Management with PagedAttention and vLLM", section "The KV
 * Cache Bottleneck"), so the read rate the memory system sustains bounds
 * every kernel here.  Each folds what it reads into one XOR per wave,
 * combined with an atomic XOR into *sink (one uint32 the caller clears); the
 * value carries no meaning beyond keeping every load live.
 *
 * ceiling_stream_read: reads `bytes` contiguous bytes at `src` (16-byte
 * aligned, bytes a positive multiple of 16) with `workgroups` workgroups of
 * 256 threads, 16-byte loads, eight in flight per lane.
 *
 * ceiling_gather_read: reads chunks[i] (int32 [num_chunks], device) of
 * `chunk_bytes` (2048, 4096 or 8192) bytes each, chunk c at pool + c *
 * chunk_bytes, and at pool2 + c * chunk_bytes as well when pool2 is not NULL
 * (the K and V tiles of one block); `pool_bytes` bounds each pool, and an
 * index outside it reads nothing (no fault).  Waves take contiguous runs of
 * the list (64 indices per vector load) and keep about 16 KiB of chunk loads
 * in flight, the way the decode kernels read tiles through a block table.
 * cached = 0: streaming (nontemporal) loads, as the decode kernels' K/V
 * loads; 1: loads with the cache's default policy (other values PKV_EINVAL).
 *
 * Both are asynchronous on `stream`; a null pointer or a bad size returns
 * PKV_EINVAL, a failed launch PKV_EHIP.
 */
int pkv_ceiling_stream_read(const void* src, size_t bytes, int workgroups, uint32_t* sink,
                            void* stream);
int pkv_ceiling_gather_read(const void* pool, const void* pool2, size_t pool_bytes,
                            const int32_t* chunks, int num_chunks, int chunk_bytes, int cached,
                            int workgroups, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
