// Host/device interface of the paged decode kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"
#include "order.h"

namespace pkv {

// Everything a decode launch needs.  Passed by value as the kernel argument.
//
// Grid.  Direct: (units * max_parts, 1, B), workgroup (x, z) computes
// partition x / units of head unit x % units of sequence z, or of the z-th
// longest sequence when `sorted` (each workgroup ranks the lengths itself,
// as the hardware starts workgroups in index order).  Planned: a
// small kernel first lists the (sequence, partition) work items, largest
// partition first, and workgroup x computes unit x % units of item
// x / units (units * items the grid's x; the items past the count exit at
// once).  In both the head unit is the fastest index: workgroup b runs on
// XCD b % 8, so every XCD gets the same share of each item.
struct DecodeArgs {
  void* out;                  // [B][Hq][HD] element type
  const void* q;              // [B][Hq][HD]
  const void* k_cache;        // [NB][Hkv][BS][HD] element type, or 8-bit codes
  const void* v_cache;
  const int32_t* block_tables;  // [B][max_blocks]
  const int32_t* context_lens;  // [B]
  const int32_t* items;       // planned grid: [item capacity][4] (s, part << 16 | n, t0, t1)
  const int32_t* item_count;  // planned grid: number of listed items
  // partial softmax states of split contexts, [B][Hq][max_parts]: o has HD
  // floats per state, ml 2 (max in log2 units, sum)
  float* part_o;
  float* part_ml;
  float scale_log2e;          // scale * log2(e) (* K scale for 8-bit codes): scores in log2 units
  float v_scale;              // 8-bit caches: the V scale (1 otherwise)
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;                  // Hq / Hkv
  int num_blocks;
  int max_blocks;             // row stride of block_tables
  int len_cap;                // lengths are clamped to this (<= max_blocks*BS)
  int part_tokens;            // P: tokens per partition at most
  int part_align;             // partition sizes are multiples of this
  int max_parts;              // ceil(len_cap / P): partitions per sequence at most
  int contiguous;             // 1: ignore tables; block j of seq s is s*max_blocks + j
  int planned;                // 0: direct grid; 1: planned, each workgroup finds its item
                              // (B <= 1024); 2: planned, items listed by the planning kernel
  int cached_kv;              // 1: K/V loads keep the cache's default policy (blocks shared
                              // across the batch are served from the cache after their first
                              // read); 0: streaming (nontemporal) loads, each block read once
};

enum class Elem { F32 = 0, F16 = 1, BF16 = 2 };

// Arguments of the grouped decode kernel (attn_grouped.hip).  Grid
// (num_kv_heads, num_groups).  Group j lists its member sequences in
// members[j][0 .. max_members) (-1: none) and its tiles in
// tiles[tile_start[j] .. tile_start[j+1]): (physical block, 16-token tile
// index within the sequences, member bit mask, unused).
struct GroupedArgs {
  void* out;                    // [B][Hq][HD]
  const void* q;                // [B][Hq][HD]
  const void* k_cache;          // [NB][Hkv][BS][HD]
  const void* v_cache;
  const int32_t* context_lens;  // [B]
  const int32_t* members;       // [num_groups][max_members]
  const int32_t* tiles;         // [total][4], 16-byte aligned
  const int32_t* tile_start;    // [num_groups + 1]; clamped to [0, num_tiles]
  // optional [num_groups]: group j's rows end here (then tile_start needs only
  // num_groups entries and groups may leave gaps); null: at tile_start[j + 1]
  const int32_t* tile_end = nullptr;
  int num_tiles;                // rows of tiles
  float scale_log2e;            // scale * log2(e) (* K scale for 8-bit codes)
  float v_scale = 1.f;          // 8-bit caches: the V scale
  int num_seqs;
  int num_groups;
  int max_members;              // max_members * group <= 16
  int num_q_heads;
  int num_kv_heads;
  int group;                    // Hq / Hkv
  int num_blocks;
  int len_cap;                  // lengths are clamped to this
  // Parts: with part_tiles > 0 group j's list is cut into ceil(n_j / part_tiles)
  // parts of part_tiles rows (grid z, at most max_parts); a group of several
  // parts leaves one (max, sum, output) state per part and column in
  // part_ml / part_o, [num_groups][max_parts][Hkv][16] (x2 / x HD floats),
  // which the merge kernel combines.
  int part_tiles = 0;
  int max_parts = 1;
  float* part_o = nullptr;
  float* part_ml = nullptr;
};

// Arguments of the prefill kernel (attn_prefill.hip): causal attention of
// the last n = query_start[s+1] - query_start[s] positions of each sequence.
// Grid (num_kv_heads * chunks, 1, num_seqs); a workgroup's 4 waves take
// consecutive query tokens (16/G per column group of 16).
struct PrefillArgs {
  void* out;                    // [total_q][Hq][HD]
  const void* q;                // [total_q][Hq][HD]
  const void* k_cache;          // [NB][Hkv][BS][HD]
  const void* v_cache;
  const int32_t* block_tables;  // [B][max_blocks]
  const int32_t* context_lens;  // [B]
  const int32_t* query_start;   // [B + 1]
  float scale_log2e;            // scale * log2(e) (* K scale for 8-bit codes)
  float v_scale;                // 8-bit caches: the V scale (1 otherwise)
  int num_seqs;
  int total_q;                  // rows of q / out (query_start is clamped to it)
  int num_q_heads;
  int num_kv_heads;
  int group;                    // Hq / Hkv, a divisor of 16
  int num_blocks;
  int max_blocks;
  int len_cap;                  // lengths are clamped to this (<= max_blocks*BS)
  int chunks;                   // ceil(max_q_len / query tokens per workgroup)
};

// The work of one decode workgroup: tokens [t0, t1) (partition `part` of
// n) of head unit `unit` of sequence s, or nothing (valid false: an item
// slot past the list, or a partition past the context).  t1 == 0 only for
// an empty context, whose single partition writes the zero row.
struct WorkItem {
  int s, part, n, t0, t1, unit;
  bool valid;
};

__device__ inline WorkItem work_item(const DecodeArgs& a, int units, PlanScratch& sm) {
  WorkItem w;
  w.unit = blockIdx.x % units;
  const int k = blockIdx.x / units;
  if (a.planned == 2) {
    // scalar reads: the count and the item are fetched together
    const int cnt = load_uniform(a.item_count);
    const i32x4 it = load_uniform4(a.items + 4 * (size_t)k);
    w.s = it[0];
    w.part = it[1] >> 16;
    w.n = it[1] & 0xffff;
    w.t0 = it[2];
    w.t1 = it[3];
    w.valid = k < cnt;
  } else if (a.planned == 1) {
    // every thread takes this branch or none: the planning has barriers
    int item[5];
    w.valid = plan_item(a.context_lens, a.num_seqs, a.len_cap, a.part_tokens, a.part_align, k, sm,
                        item);
    w.s = uniform(item[0]);
    w.part = uniform(item[1]);
    w.n = uniform(item[2]);
    w.t0 = uniform(item[3]);
    w.t1 = uniform(item[4]);
  } else {
    w.s = blockIdx.z;
    w.part = k;
    int L = load_uniform(a.context_lens + w.s);
    L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
    w.n = num_parts(L, a.part_tokens);
    const int ps = part_size(L, w.n, a.part_align);
    w.t0 = k * ps;
    w.t1 = min(L, w.t0 + ps);
    w.valid = k < w.n;
  }
  return w;
}

// Launchers (one translation unit each).  Return hipSuccess or the launch error.
// kv_fp8: the caches hold E4M3 codes (q and out keep the element type e).
hipError_t launch_decode_valu(Elem e, bool kv_fp8, int head_dim, int block_size,
                              const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_mfma(Elem e, bool kv_fp8, int head_dim, int block_size,
                              const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_reduce(Elem e, int head_dim, const DecodeArgs& a, hipStream_t stream);
bool decode_valu_supported(Elem e, bool kv_fp8, int head_dim, int block_size);
// Tokens per unit of work of the vector-ALU kernel (a wave handles at most
// 64 units per pass); the MFMA kernel's unit is 16 tokens.
int valu_unit_tokens(Elem e, bool kv_fp8, int head_dim, int block_size);
bool decode_mfma_supported(Elem e, int head_dim, int block_size);
bool prefill_supported(Elem e, int head_dim, int block_size, int group);
bool grouped_supported(Elem e, int head_dim, int block_size);
// kv_fp8: the caches hold E4M3 codes (v_scale applies; the K scale is in
// scale_log2e).
hipError_t launch_decode_grouped(Elem e, bool kv_fp8, int head_dim, int block_size,
                                 const GroupedArgs& a, hipStream_t stream);
hipError_t launch_grouped_merge(Elem e, int head_dim, const GroupedArgs& a, hipStream_t stream);
// The grouped decode's tile lists from the block tables (group_tiles.hip).
// Group j's rows go to tiles[j * stride ..] with tile_start[j] = j * stride
// and tile_end[j] after its last row; one workgroup per group.
hipError_t launch_build_group_tiles(const int32_t* block_tables, const int32_t* context_lens,
                                    const int32_t* members, int num_seqs, int max_blocks,
                                    int num_groups, int max_members, int block_size, int len_cap,
                                    int32_t* tiles, int stride, int32_t* tile_start,
                                    int32_t* tile_end, hipStream_t stream);
// Query tokens one prefill workgroup covers (its grid is ceil(max_q_len / this)
// chunks per KV head and sequence).
int prefill_tokens_per_workgroup(int group);
// kv_fp8: the caches hold E4M3 codes (v_scale applies; the K scale is in
// scale_log2e).
hipError_t launch_prefill(Elem e, bool kv_fp8, int head_dim, int block_size, const PrefillArgs& a,
                          hipStream_t stream);
// Decode workgroups resident per compute unit (0 if the runtime cannot say).
int decode_valu_occupancy(Elem e, bool kv_fp8, int head_dim, int block_size);
int decode_mfma_occupancy(Elem e, bool kv_fp8, int head_dim, int block_size, int group);

// Writes the work items of a planned grid (see DecodeArgs): items[4k ..
// 4k+3] = (s, part << 16 | n, t0, t1) for k < *count, largest partition
// first (half-octave size bins; stable, and a sequence's partitions
// together), using scratch[2 * num_seqs].
hipError_t launch_plan_items(const int32_t* lens, int num_seqs, int len_cap, int part_tokens,
                             int part_align, int32_t* scratch, int32_t* items, int32_t* count,
                             hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                    int row_bytes, int block_size, int num_blocks,
                                    hipStream_t stream);
// The quantising write: rows of element type e become E4M3 codes of
// x / k_scale (K) and x / v_scale (V).
hipError_t launch_reshape_and_cache_fp8(Elem e, const void* k, const void* v, void* k_cache,
                                        void* v_cache, const int64_t* slot_mapping,
                                        int num_tokens, int num_kv_heads, int head_dim,
                                        int block_size, int num_blocks, float k_scale,
                                        float v_scale, hipStream_t stream);
// dst pools[pairs[i][1]] = src pools[pairs[i][0]] for K and V (pools may be
// the same, for copy-on-write).
hipError_t launch_copy_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                              const int64_t* pairs, int num_pairs, size_t block_bytes, int num_src,
                              int num_dst, hipStream_t stream);

}  // namespace pkv
