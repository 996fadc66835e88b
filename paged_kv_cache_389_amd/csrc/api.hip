// C ABI of libpagedkv.so: argument validation, the split heuristic and
// kernel dispatch.  See include/pagedkv.h for the contract of every call.
#include <stdint.h>
#include <stdlib.h>

#include <string>

#include "decode.h"
#include "order.h"
#include "pagedkv.h"

using namespace pkv;

namespace {

thread_local std::string g_last_error;

constexpr int kPartAlign = 32;          // tokens; partitions are whole 32-token spans
constexpr int kMinAutoPartition = 512;  // the library never splits finer than this
constexpr int kWgPerCu = 4;             // split until about this many workgroups per CU
constexpr int kMaxGridYZ = 65535;
constexpr int kMaxDevices = 64;
constexpr int kBalancedRequest = -1;    // partition_tokens value that asks for the balanced grid

int elem_size(pkv_dtype d) { return d == PKV_F32 ? 4 : 2; }
bool dtype_ok(int d) { return d == PKV_F32 || d == PKV_F16 || d == PKV_BF16; }
Elem to_elem(pkv_dtype d) {
  return d == PKV_F32 ? Elem::F32 : (d == PKV_F16 ? Elem::F16 : Elem::BF16);
}

int fail_hip(hipError_t e) {
  g_last_error = hipGetErrorString(e);
  return PKV_EHIP;
}

int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Compute units of the current device (cached per device; 256 if unknown).
int compute_units() {
  static int cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  __atomic_store_n(&cached[dev], n, __ATOMIC_RELAXED);
  return n;
}

// The kernel a decode call runs and how its grid divides the work.
struct Plan {
  bool mfma = false;
  int grid_mode = kGridPartitions;
  int part_tokens = 0;   // partitions grid: tokens per partition
  int max_parts = 1;     // partitions grid: partitions the grid covers per sequence
  int ranges = 0;        // balanced grid: waves (4 per workgroup), one range each
  int unit_group = 1;    // balanced grid: query heads per work unit
  int len_cap = 0;       // context lengths are clamped to this
  bool sort = false;     // partitions grid: visit sequences longest first
  bool sort_kernel = false;  // ... through the order kernel (large batches)
  int status = PKV_OK;
};

// Workgroups of the balanced kernel resident on the whole device (cached
// per device and kernel; a fallback when the runtime cannot say).
int resident_workgroups(bool mfma, Elem e, int head_dim, int block_size, int group) {
  constexpr int kKeys = 2 * 3 * 3 * 3 * 3;   // kernel x dtype x head_dim x block_size x GMAX
  static int cached[kMaxDevices][kKeys];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  const int gmax = group <= 4 ? 0 : (group <= 8 ? 1 : 2);
  const int hdk = head_dim == 64 ? 0 : (head_dim == 128 ? 1 : 2);
  const int bsk = block_size == 8 ? 0 : (block_size == 16 ? 1 : 2);
  const int key = (((((mfma ? 1 : 0) * 3 + (int)e) * 3 + hdk) * 3 + bsk) * 3 + gmax);
  int per_cu = dev >= 0 ? __atomic_load_n(&cached[dev][key], __ATOMIC_RELAXED) : 0;
  if (per_cu <= 0) {
    per_cu = mfma ? decode_mfma_occupancy(e, head_dim, block_size, group)
                  : decode_valu_occupancy(e, head_dim, block_size);
    if (per_cu <= 0) per_cu = mfma ? 3 : 4;
    if (dev >= 0) __atomic_store_n(&cached[dev][key], per_cu, __ATOMIC_RELAXED);
  }
  return per_cu * compute_units();
}

Plan make_plan(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
               int max_blocks_per_seq, int max_context_len, pkv_dtype dtype, int requested,
               int path) {
  Plan pl;
  const Elem e = to_elem(dtype);
  if (!decode_valu_supported(e, head_dim, block_size)) {
    pl.status = PKV_EUNSUPPORTED;
    return pl;
  }
  const int group = num_q_heads / num_kv_heads;
  const bool mfma_ok = group >= 2 && group <= 16 && decode_mfma_supported(e, head_dim, block_size);
  if (path == PKV_PATH_MFMA && !mfma_ok) {
    pl.status = PKV_EUNSUPPORTED;
    return pl;
  }
  pl.mfma = path == PKV_PATH_MFMA || ((path == PKV_PATH_AUTO || path == PKV_PATH_CONTIGUOUS) && mfma_ok);

  const int64_t table_cap = (int64_t)max_blocks_per_seq * block_size;
  pl.len_cap = (int)(table_cap < max_context_len ? table_cap : max_context_len);
  const int unit = pl.mfma ? 16 : valu_unit_tokens(e, head_dim, block_size);
  const int units_per_seq = pl.mfma ? num_kv_heads : num_q_heads;

  // Balanced grid on request (partition_tokens == -1): equal shares of all
  // tiles, one workgroup per resident slot, so every workgroup starts at
  // once and ends at about the same time whatever the length mix.  It needs
  // the tile prefix of the batch in LDS (at most kBalancedMaxSeqs
  // sequences, an int total).
  const int64_t seq_tiles = (pl.len_cap + unit - 1) / unit;
  if (requested == kBalancedRequest) {
    if (num_seqs > kBalancedMaxSeqs || (int64_t)num_seqs * seq_tiles >= (1ll << 31) - 1) {
      pl.status = PKV_EUNSUPPORTED;
      return pl;
    }
    pl.grid_mode = kGridBalanced;
    pl.unit_group = pl.mfma ? group : 1;
    // one range per resident wave, at most one per 4 tiles of the largest
    // possible batch, a multiple of 32 (8 XCDs x 4 waves)
    const int64_t waves = 4 * (int64_t)resident_workgroups(pl.mfma, e, head_dim, block_size, group);
    const int64_t tiles_upper = (int64_t)num_seqs * units_per_seq * seq_tiles;
    int64_t r = waves < tiles_upper / 4 ? waves : tiles_upper / 4;
    r = r / 32 * 32;
    pl.ranges = (int)(r < 32 ? 32 : r);
    return pl;
  }

  // a wave handles at most 64 units of a partition
  const int p_max = 256 * unit / kPartAlign * kPartAlign;
  int p;
  if (requested > 0) {
    if (requested % kPartAlign || requested % block_size || requested > p_max) {
      pl.status = PKV_EINVAL;
      return pl;
    }
    p = requested;
  } else {
    // one partition per (sequence, head) unit unless those units are too
    // few to give every compute unit several workgroups
    const int64_t units = (int64_t)num_seqs * units_per_seq;
    const int64_t target = (int64_t)kWgPerCu * compute_units();
    const int64_t parts = units >= target ? 1 : (target + units - 1) / units;
    const int len = pl.len_cap > 0 ? pl.len_cap : 1;
    p = round_up((int)((len + parts - 1) / parts), kPartAlign);
    if (p < kMinAutoPartition) p = round_up(len < kMinAutoPartition ? len : kMinAutoPartition, kPartAlign);
    if (p > p_max) p = p_max;
  }
  pl.part_tokens = p;
  pl.max_parts = pl.len_cap > 0 ? (pl.len_cap + p - 1) / p : 1;
  // Longest first pays off once the grid is more than about two rounds of
  // resident workgroups (the VALU kernel keeps 4 per compute unit, the MFMA
  // kernel 3); with fewer, nearly every workgroup starts at once anyway.
  const int64_t wgs = (int64_t)pl.max_parts * units_per_seq * num_seqs;
  const int64_t resident = (int64_t)(pl.mfma ? 3 : 4) * compute_units();
  pl.sort = num_seqs > 1 && wgs > 2 * resident;
  pl.sort_kernel = pl.sort && num_seqs > kFusedOrderMax;
  return pl;
}

// Workspace layout, each part 16-byte aligned:
//  partitions grid: partial outputs [B][Hq][max_parts][HD] fp32 and partial
//    (max, sum) [B][Hq][max_parts][2] fp32 (only with several partitions),
//    then the sequence order [B] int32 (only with the order kernel);
//  balanced grid: partial outputs [2*ranges][unit_group][HD] fp32, partial
//    (max, sum) [2*ranges][unit_group][2] fp32, the tile prefix [B+1] int32.
struct Layout {
  size_t part_o = 0, part_ml = 0, extra = 0, total = 0;   // byte offsets, size
};

size_t align16(size_t x) { return (x + 15) / 16 * 16; }

Layout workspace_layout(int num_seqs, int num_q_heads, int head_dim, const Plan& pl) {
  Layout lo;
  size_t states = 0;
  if (pl.grid_mode == kGridBalanced)
    states = (size_t)2 * pl.ranges * pl.unit_group;
  else if (pl.max_parts > 1)
    states = (size_t)num_seqs * num_q_heads * pl.max_parts;
  lo.part_o = 0;
  lo.part_ml = align16(states * head_dim * sizeof(float));
  lo.extra = lo.part_ml + align16(states * 2 * sizeof(float));
  size_t extra_bytes = 0;
  if (pl.grid_mode == kGridBalanced)
    extra_bytes = (size_t)(num_seqs + 1) * sizeof(int32_t);
  else if (pl.sort_kernel)
    extra_bytes = (size_t)num_seqs * sizeof(int32_t);
  lo.total = extra_bytes ? lo.extra + align16(extra_bytes) : (states ? lo.extra : 0);
  return lo;
}

size_t workspace_for(int num_seqs, int num_q_heads, int head_dim, const Plan& pl) {
  return workspace_layout(num_seqs, num_q_heads, head_dim, pl).total;
}

}  // namespace

extern "C" {

const char* pkv_version(void) { return "pagedkv 0.1.0 gfx950"; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_EUNSUPPORTED: return "unsupported shape or dtype";
    case PKV_EWORKSPACE: return "workspace missing or too small";
    case PKV_EHIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* pkv_last_error(void) { return g_last_error.c_str(); }

int pkv_supported(pkv_dtype dtype, int head_dim, int block_size) {
  if (!dtype_ok(dtype)) return 0;
  return decode_valu_supported(to_elem(dtype), head_dim, block_size) ? 1 : 0;
}

size_t pkv_paged_attention_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                           int head_dim, int block_size, int max_blocks_per_seq,
                                           int max_context_len, pkv_dtype dtype,
                                           int partition_tokens, int path) {
  if (!dtype_ok(dtype) || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 ||
      partition_tokens < kBalancedRequest || path < PKV_PATH_AUTO || path > PKV_PATH_CONTIGUOUS ||
      num_q_heads % num_kv_heads)
    return (size_t)-1;
  const Plan pl = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                            max_blocks_per_seq, max_context_len, dtype, partition_tokens, path);
  if (pl.status != PKV_OK) return (size_t)-1;
  return workspace_for(num_seqs, num_q_heads, head_dim, pl);
}

int pkv_paged_attention_plan(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                             int block_size, int max_blocks_per_seq, int max_context_len,
                             pkv_dtype dtype, int partition_tokens, int path, pkv_plan* out) {
  if (!dtype_ok(dtype) || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 ||
      partition_tokens < kBalancedRequest || path < PKV_PATH_AUTO || path > PKV_PATH_CONTIGUOUS ||
      num_q_heads % num_kv_heads)
    return PKV_EINVAL;
  const Plan pl = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                            max_blocks_per_seq, max_context_len, dtype, partition_tokens, path);
  if (pl.status != PKV_OK) return pl.status;
  if (out) {
    out->path = pl.mfma ? PKV_PATH_MFMA : PKV_PATH_VALU;
    out->grid = pl.grid_mode == kGridBalanced ? PKV_GRID_BALANCED : PKV_GRID_PARTITIONS;
    out->partition_tokens = pl.grid_mode == kGridBalanced ? 0 : pl.part_tokens;
    out->max_parts = pl.grid_mode == kGridBalanced ? 0 : pl.max_parts;
    out->ranges = pl.ranges;
    out->longest_first = pl.sort ? 1 : 0;
    out->workspace_bytes = workspace_for(num_seqs, num_q_heads, head_dim, pl);
  }
  return PKV_OK;
}

int pkv_paged_attention_decode_ex(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, float scale, int num_seqs,
                                  int num_q_heads, int num_kv_heads, int head_dim,
                                  int block_size, int num_blocks, int max_blocks_per_seq,
                                  int max_context_len, pkv_dtype dtype, void* workspace,
                                  size_t workspace_bytes, int partition, int path,
                                  void* stream) {
  if (!dtype_ok(dtype) || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      max_context_len < 0 || partition < kBalancedRequest || path < PKV_PATH_AUTO ||
      path > PKV_PATH_CONTIGUOUS)
    return PKV_EINVAL;
  if (num_q_heads % num_kv_heads) return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  const bool contiguous = path == PKV_PATH_CONTIGUOUS;
  if (!out || !q || !k_cache || !v_cache || !context_lens || (!block_tables && !contiguous))
    return PKV_EINVAL;
  if (num_seqs > kMaxGridYZ || num_q_heads > kMaxGridYZ) return PKV_EUNSUPPORTED;
  if (max_blocks_per_seq > (1 << 30) / block_size) return PKV_EUNSUPPORTED;
  if (contiguous && (int64_t)num_seqs * max_blocks_per_seq > num_blocks) return PKV_EINVAL;

  const Elem e = to_elem(dtype);
  const Plan pl = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                            max_blocks_per_seq, max_context_len, dtype, partition, path);
  if (pl.status != PKV_OK) return pl.status;
  const Layout lo = workspace_layout(num_seqs, num_q_heads, head_dim, pl);
  const size_t need = lo.total;
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_EWORKSPACE;
  if (need > 0 && reinterpret_cast<uintptr_t>(workspace) % 16) return PKV_EINVAL;
  const bool use_mfma = pl.mfma;

  DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  char* ws = static_cast<char*>(workspace);
  a.part_o = need ? reinterpret_cast<float*>(ws + lo.part_o) : nullptr;
  a.part_ml = need ? reinterpret_cast<float*>(ws + lo.part_ml) : nullptr;
  a.seq_order = pl.sort_kernel ? reinterpret_cast<const int32_t*>(ws + lo.extra) : nullptr;
  a.tile_start = pl.grid_mode == kGridBalanced ? reinterpret_cast<int32_t*>(ws + lo.extra) : nullptr;
  a.order_mode = pl.sort_kernel ? 1 : (pl.sort ? 2 : 0);
  a.grid_mode = pl.grid_mode;
  a.ranges = pl.ranges;
  a.unit_group = pl.unit_group;
  a.scale_log2e = (float)((double)scale * 1.4426950408889634);
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.len_cap = pl.len_cap;
  a.part_tokens = pl.part_tokens;
  a.max_parts = pl.max_parts;
  a.contiguous = contiguous ? 1 : 0;

  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (pl.sort_kernel) {
    err = launch_seq_order(context_lens, num_seqs, pl.len_cap,
                           const_cast<int32_t*>(a.seq_order), st);
    if (err != hipSuccess) return fail_hip(err);
  }
  err = use_mfma ? launch_decode_mfma(e, head_dim, block_size, a, st)
                 : launch_decode_valu(e, head_dim, block_size, a, st);
  if (err != hipSuccess) return fail_hip(err);
  if (pl.grid_mode == kGridBalanced || pl.max_parts > 1) {
    err = launch_decode_reduce(e, head_dim, a, st);
    if (err != hipSuccess) return fail_hip(err);
  }
  return PKV_OK;
}

int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               float scale, int num_seqs, int num_q_heads, int num_kv_heads,
                               int head_dim, int block_size, int num_blocks,
                               int max_blocks_per_seq, int max_context_len, pkv_dtype dtype,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return pkv_paged_attention_decode_ex(out, q, k_cache, v_cache, block_tables, context_lens,
                                       scale, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                       block_size, num_blocks, max_blocks_per_seq,
                                       max_context_len, dtype, workspace, workspace_bytes, 0,
                                       PKV_PATH_AUTO, stream);
}

int pkv_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                          const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                          int head_dim, int block_size, int num_blocks, pkv_dtype dtype,
                          void* stream) {
  if (!dtype_ok(dtype) || num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_blocks <= 0)
    return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PKV_EINVAL;
  const int row_bytes = head_dim * elem_size(dtype);
  if (row_bytes % 16) return PKV_EUNSUPPORTED;
  hipError_t err = launch_reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, num_tokens,
                                            num_kv_heads, row_bytes, block_size, num_blocks,
                                            static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PKV_OK : fail_hip(err);
}

int pkv_copy_blocks(void* k_cache, void* v_cache, const int64_t* src_dst_pairs, int num_pairs,
                    int num_kv_heads, int head_dim, int block_size, int num_blocks,
                    pkv_dtype dtype, void* stream) {
  if (!dtype_ok(dtype) || num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_blocks <= 0)
    return PKV_EINVAL;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src_dst_pairs) return PKV_EINVAL;
  const size_t block_bytes = (size_t)num_kv_heads * block_size * head_dim * elem_size(dtype);
  if (block_bytes % 16) return PKV_EUNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int first = 0; first < num_pairs; first += kMaxGridYZ) {
    const int n = num_pairs - first < kMaxGridYZ ? num_pairs - first : kMaxGridYZ;
    hipError_t err = launch_copy_blocks(k_cache, v_cache, src_dst_pairs + 2 * (size_t)first, n,
                                        block_bytes, num_blocks, st);
    if (err != hipSuccess) return fail_hip(err);
  }
  return PKV_OK;
}

}  // extern "C"
