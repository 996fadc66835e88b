// C ABI of libpagedkv.so: argument validation, the split heuristic and
// kernel dispatch.  See include/pagedkv.h for the contract of every call.
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <string>
#include <vector>

#include "decode.h"
#include "order.h"
#include "pagedkv.h"

using namespace pkv;

namespace {

thread_local std::string g_last_error;

constexpr int kPartAlign = 32;          // tokens; partitions are whole 32-token spans
constexpr int kMinAutoPartition = 512;  // the library never splits finer than this
constexpr int kWgPerCu = 2;             // split until about this many workgroups per CU
constexpr int kSplitFloor = 2048;       // tokens; many-unit batches split no finer
constexpr int kMaxGridYZ = 65535;
constexpr int kMaxDevices = 64;
constexpr int kMaxItemParts = 65535;    // a work item packs (part, n) into 16 bits each
constexpr int kMaxPartition = 1 << 20;  // tokens; explicit partition sizes up to this

int elem_size(int d) { return d == PKV_F32 ? 4 : (d == PKV_E4M3 ? 1 : 2); }
// types of q, out and unquantised caches
bool dtype_ok(int d) { return d == PKV_F32 || d == PKV_F16 || d == PKV_BF16; }
// cache element types the byte-moving calls accept
bool cache_dtype_ok(int d) { return dtype_ok(d) || d == PKV_E4M3; }
// plan / workspace / supported: a q type, optionally with PKV_KV_E4M3
bool plan_dtype_ok(int d) {
  return dtype_ok(d & 0xFF) && ((d & ~0xFF) == 0 || (d & ~0xFF) == PKV_KV_E4M3);
}
bool finite_nonzero(float x) { return x == x && x != 0.f && x - x == 0.f; }
Elem to_elem(int d) {
  d &= 0xFF;
  return d == PKV_F32 ? Elem::F32 : (d == PKV_F16 ? Elem::F16 : Elem::BF16);
}

int fail_hip(hipError_t e) {
  g_last_error = hipGetErrorString(e);
  return PKV_EHIP;
}

int round_up(int x, int m) { return (x + m - 1) / m * m; }

// The path argument of the decode calls: a pkv_decode_path, optionally
// OR-ed with PKV_PATH_SHARED_BLOCKS (K/V loads that keep blocks in the cache
// for the other sequences of the batch that share them).
bool split_path(int path, int* kernel, bool* shared) {
  *shared = (path & PKV_PATH_SHARED_BLOCKS) != 0;
  *kernel = path & ~PKV_PATH_SHARED_BLOCKS;
  return *kernel >= PKV_PATH_AUTO && *kernel <= PKV_PATH_CONTIGUOUS;
}

// ------------------------------------------------------------ debug checks
//
// With PKV_DEBUG=1 in the environment every call synchronises its stream,
// copies its index arrays to the host and checks the content preconditions
// the kernels do not check (they only stay in bounds): lengths within the
// table, table entries inside the pool, slots in range and distinct,
// copy destinations distinct and never a source of the same call.  A
// violation returns PKV_EINVAL before anything is enqueued, with the first
// offending index in pkv_last_error().

bool debug_checks() {
  const char* e = getenv("PKV_DEBUG");
  return e && e[0] == '1';
}

int debug_fail(const std::string& what) {
  g_last_error = "PKV_DEBUG: " + what;
  return PKV_EINVAL;
}

// Copy n elements of a device (or pinned host) array after the stream's
// earlier work; false (with the HIP error recorded) on failure.
template <typename T>
bool fetch(std::vector<T>& dst, const T* src, size_t n, hipStream_t st) {
  dst.resize(n);
  if (n == 0) return true;
  hipError_t err = hipStreamSynchronize(st);
  if (err == hipSuccess) err = hipMemcpy(dst.data(), src, n * sizeof(T), hipMemcpyDefault);
  if (err != hipSuccess) {
    g_last_error = hipGetErrorString(err);
    return false;
  }
  return true;
}

// lengths in [0, len_cap] and the first ceil(L / bs) table entries in the pool
int debug_check_tables(const int32_t* context_lens, const int32_t* block_tables, int num_seqs,
                       int max_blocks, int block_size, int num_blocks, int64_t len_cap,
                       hipStream_t st) {
  std::vector<int32_t> lens, tables;
  if (!fetch(lens, context_lens, num_seqs, st)) return PKV_EHIP;
  if (block_tables && !fetch(tables, block_tables, (size_t)num_seqs * max_blocks, st))
    return PKV_EHIP;
  for (int s = 0; s < num_seqs; ++s) {
    if (lens[s] < 0 || lens[s] > len_cap)
      return debug_fail("context_lens[" + std::to_string(s) + "] = " + std::to_string(lens[s]) +
                        " outside [0, " + std::to_string(len_cap) + "]");
    if (!block_tables) continue;
    const int nb = (lens[s] + block_size - 1) / block_size;
    for (int j = 0; j < nb; ++j) {
      const int32_t b = tables[(size_t)s * max_blocks + j];
      if (b < 0 || b >= num_blocks)
        return debug_fail("block_tables[" + std::to_string(s) + "][" + std::to_string(j) +
                          "] = " + std::to_string(b) + " outside the pool");
    }
  }
  return PKV_OK;
}

int debug_check_slots(const int64_t* slot_mapping, int num_tokens, int64_t num_slots,
                      hipStream_t st) {
  std::vector<int64_t> slots;
  if (!fetch(slots, slot_mapping, num_tokens, st)) return PKV_EHIP;
  std::vector<int64_t> seen;
  for (int j = 0; j < num_tokens; ++j) {
    if (slots[j] >= num_slots)
      return debug_fail("slot_mapping[" + std::to_string(j) + "] = " + std::to_string(slots[j]) +
                        " outside the pool");
    if (slots[j] >= 0) seen.push_back(slots[j]);
  }
  std::sort(seen.begin(), seen.end());
  for (size_t i = 1; i < seen.size(); ++i)
    if (seen[i] == seen[i - 1]) return debug_fail("slot " + std::to_string(seen[i]) + " repeated");
  return PKV_OK;
}

// same_pool: destinations must also differ from every source (copy-on-write)
int debug_check_pairs(const int64_t* pairs, int num_pairs, int num_src, int num_dst,
                      bool same_pool, hipStream_t st) {
  std::vector<int64_t> p;
  if (!fetch(p, pairs, (size_t)num_pairs * 2, st)) return PKV_EHIP;
  std::vector<int64_t> src, dst;
  for (int i = 0; i < num_pairs; ++i) {
    if (p[2 * i] < 0 || p[2 * i] >= num_src || p[2 * i + 1] < 0 || p[2 * i + 1] >= num_dst)
      return debug_fail("pair " + std::to_string(i) + " = (" + std::to_string(p[2 * i]) + ", " +
                        std::to_string(p[2 * i + 1]) + ") outside the pools");
    src.push_back(p[2 * i]);
    dst.push_back(p[2 * i + 1]);
  }
  std::sort(dst.begin(), dst.end());
  for (size_t i = 1; i < dst.size(); ++i)
    if (dst[i] == dst[i - 1])
      return debug_fail("destination block " + std::to_string(dst[i]) + " repeated");
  if (same_pool) {
    std::sort(src.begin(), src.end());
    for (int64_t d : dst)
      if (std::binary_search(src.begin(), src.end(), d))
        return debug_fail("block " + std::to_string(d) + " is both a source and a destination");
  }
  return PKV_OK;
}

// Grouped decode: members in [0, num_seqs) and in at most one group; tile
// list offsets non-decreasing from 0; every entry's block in the pool; and
// for every member exactly one entry with its bit for each of its tiles
// 0 .. ceil(L / 16) - 1 and none past them.
int debug_check_groups(const int32_t* context_lens, const int32_t* members, const int32_t* tiles,
                       const int32_t* tile_start, const int32_t* tile_end, int num_tiles,
                       int num_seqs, int num_groups, int max_members, int num_blocks,
                       int64_t len_cap, int max_group_tiles, hipStream_t st) {
  std::vector<int32_t> lens, mem, start, end, ent;
  if (!fetch(lens, context_lens, num_seqs, st) ||
      !fetch(mem, members, (size_t)num_groups * max_members, st) ||
      !fetch(start, tile_start, (size_t)num_groups + (tile_end ? 0 : 1), st) ||
      (tile_end && !fetch(end, tile_end, (size_t)num_groups, st)))
    return PKV_EHIP;
  if (!tile_end) {   // a prefix: group j ends where group j + 1 starts
    if (start[0] != 0) return debug_fail("group_tile_start[0] != 0");
    end.assign(start.begin() + 1, start.end());
    start.pop_back();
  }
  for (int j = 0; j < num_groups; ++j) {
    if (start[j] < 0 || end[j] < start[j] || end[j] > num_tiles)
      return debug_fail("group " + std::to_string(j) + " rows [" + std::to_string(start[j]) +
                        ", " + std::to_string(end[j]) + ") outside the " +
                        std::to_string(num_tiles) + " rows of group_tiles");
    if (max_group_tiles >= 0 && end[j] - start[j] > max_group_tiles)
      return debug_fail("group " + std::to_string(j) + " lists more than max_group_tiles rows");
  }
  if (!fetch(ent, tiles, (size_t)num_tiles * 4, st)) return PKV_EHIP;
  std::vector<char> seen(num_seqs, 0);
  for (int j = 0; j < num_groups; ++j) {
    std::vector<std::vector<int>> count(max_members);
    for (int m = 0; m < max_members; ++m) {
      const int s = mem[(size_t)j * max_members + m];
      if (s < 0) continue;
      if (s >= num_seqs || seen[s])
        return debug_fail("group_members[" + std::to_string(j) + "][" + std::to_string(m) +
                          "] = " + std::to_string(s) + " outside the batch or in two groups");
      seen[s] = 1;
      if (lens[s] < 0 || lens[s] > len_cap)
        return debug_fail("context_lens[" + std::to_string(s) + "] outside [0, len_cap]");
      count[m].assign((lens[s] + 15) / 16, 0);
    }
    for (int i = start[j]; i < end[j]; ++i) {
      const int32_t b = ent[4 * (size_t)i], t = ent[4 * (size_t)i + 1], mask = ent[4 * (size_t)i + 2];
      if (b < 0 || b >= num_blocks)
        return debug_fail("group_tiles[" + std::to_string(i) + "] block outside the pool");
      for (int m = 0; m < max_members; ++m) {
        if (!((mask >> m) & 1)) continue;
        if (mem[(size_t)j * max_members + m] < 0 || t < 0 || t >= (int)count[m].size() ||
            count[m][t]++)
          return debug_fail("group_tiles[" + std::to_string(i) + "]: tile " + std::to_string(t) +
                            " of member " + std::to_string(m) + " absent, past its length or twice");
      }
    }
    for (int m = 0; m < max_members; ++m)
      for (size_t t = 0; t < count[m].size(); ++t)
        if (!count[m][t])
          return debug_fail("group " + std::to_string(j) + " member " + std::to_string(m) +
                            " has no entry for tile " + std::to_string(t));
  }
  return PKV_OK;
}

int debug_check_query_start(const int32_t* query_start, int num_seqs, int total_q, int max_q_len,
                            hipStream_t st) {
  std::vector<int32_t> qs;
  if (!fetch(qs, query_start, (size_t)num_seqs + 1, st)) return PKV_EHIP;
  if (qs[0] != 0 || qs[num_seqs] != total_q)
    return debug_fail("query_start must run from 0 to total_q");
  for (int s = 0; s < num_seqs; ++s)
    if (qs[s + 1] < qs[s] || qs[s + 1] - qs[s] > max_q_len)
      return debug_fail("query_start[" + std::to_string(s + 1) + "]: " +
                        std::to_string(qs[s + 1] - qs[s]) + " queries (max_q_len " +
                        std::to_string(max_q_len) + ")");
  return PKV_OK;
}

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
  int part_tokens = 0;   // P: tokens per partition at most
  int part_align = 32;   // partition sizes are multiples of this
  int max_parts = 1;     // partitions per sequence at most
  int len_cap = 0;       // context lengths are clamped to this
  int planned = 0;       // 0 direct; 1 planned, found in each workgroup; 2 planned, listed
                         // by the planning kernel
  int status = PKV_OK;
};

// Decode workgroups resident on the whole device (cached per device and
// kernel; a fallback when the runtime cannot say).
int resident_workgroups(bool mfma, Elem e, bool kv_fp8, int head_dim, int block_size,
                        int group) {
  constexpr int kKeys = 2 * 3 * 2 * 3 * 3 * 3;   // kernel x dtype x cache x hd x bs x GMAX
  static int cached[kMaxDevices][kKeys];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  const int gmax = group <= 4 ? 0 : (group <= 8 ? 1 : 2);
  const int hdk = head_dim == 64 ? 0 : (head_dim == 128 ? 1 : 2);
  const int bsk = block_size == 8 ? 0 : (block_size == 16 ? 1 : 2);
  const int key =
      ((((((mfma ? 1 : 0) * 3 + (int)e) * 2 + (kv_fp8 ? 1 : 0)) * 3 + hdk) * 3 + bsk) * 3 + gmax);
  int per_cu = dev >= 0 ? __atomic_load_n(&cached[dev][key], __ATOMIC_RELAXED) : 0;
  if (per_cu <= 0) {
    per_cu = mfma ? decode_mfma_occupancy(e, kv_fp8, head_dim, block_size, group)
                  : decode_valu_occupancy(e, kv_fp8, head_dim, block_size);
    if (per_cu <= 0) per_cu = mfma ? 3 : 4;
    if (dev >= 0) __atomic_store_n(&cached[dev][key], per_cu, __ATOMIC_RELAXED);
  }
  return per_cu * compute_units();
}

// dtype: the type of q and out, with PKV_KV_E4M3 for an 8-bit cache (no
// contiguous control).
Plan make_plan(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
               int max_blocks_per_seq, int max_context_len, int dtype, int requested,
               int path, int grid) {
  Plan pl;
  const Elem e = to_elem(dtype);
  const bool kv_fp8 = (dtype & PKV_KV_E4M3) != 0;
  if (!decode_valu_supported(e, kv_fp8, head_dim, block_size) ||
      (kv_fp8 && path == PKV_PATH_CONTIGUOUS)) {
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
  const int unit = pl.mfma ? 16 : valu_unit_tokens(e, kv_fp8, head_dim, block_size);
  const int units_per_seq = pl.mfma ? num_kv_heads : num_q_heads;
  pl.part_align = block_size > kPartAlign ? block_size : kPartAlign;

  // the library's partitions give each of the 4 waves at most 64 units (one
  // vector of table entries); an explicit size may take several passes
  const int p_max = 256 * unit / pl.part_align * pl.part_align;
  int p;
  if (requested > 0) {
    if (requested % pl.part_align || requested > kMaxPartition) {
      pl.status = PKV_EINVAL;
      return pl;
    }
    p = requested;
  } else {
    // Few (sequence, head) units: cut the contexts so that every compute
    // unit gets about kWgPerCu workgroups.  Many units: the grid is full
    // anyway, but a context much longer than the others would be one long
    // workgroup that ends last, so contexts longer than half the bound are
    // cut in two (never below kSplitFloor tokens per partition; twice that
    // over 8-bit codes, the same bytes per partition).
    const int64_t units = (int64_t)num_seqs * units_per_seq;
    const int64_t target = (int64_t)kWgPerCu * compute_units();
    const int len = pl.len_cap > 0 ? pl.len_cap : 1;
    if (units >= target) {
      const int floor_tokens = kv_fp8 ? 2 * kSplitFloor : kSplitFloor;
      p = round_up((len + 1) / 2, pl.part_align);
      if (p < floor_tokens) p = floor_tokens;
      if (p >= len) p = round_up(len, pl.part_align);
    } else {
      const int64_t parts = (target + units - 1) / units;
      p = round_up((int)((len + parts - 1) / parts), pl.part_align);
      if (p < kMinAutoPartition)
        p = round_up(len < kMinAutoPartition ? len : kMinAutoPartition, pl.part_align);
    }
    if (p > p_max) p = p_max;
  }
  pl.part_tokens = p;
  pl.max_parts = pl.len_cap > 0 ? (pl.len_cap + p - 1) / p : 1;
  const int64_t direct_x = (int64_t)pl.max_parts * units_per_seq;
  if (direct_x > INT32_MAX) {   // the direct grid's x is units * parts
    pl.status = PKV_EUNSUPPORTED;
    return pl;
  }
  // Largest first pays off once the grid holds more than one round of
  // resident workgroups; with fewer, every workgroup starts at once anyway.
  // Each workgroup finds its own item for up to kFusedOrderMax sequences (no
  // extra launch); larger batches are listed by the planning kernel.
  const int64_t wgs = direct_x * num_seqs;
  const bool plannable = wgs <= INT32_MAX && pl.max_parts <= kMaxItemParts;
  const int64_t resident = resident_workgroups(pl.mfma, e, kv_fp8, head_dim, block_size, group);
  const bool want = grid == PKV_GRID_PLANNED ||
                    (grid == PKV_GRID_AUTO && num_seqs > 1 && wgs > resident);
  if (want) {
    if (!plannable) {
      if (grid == PKV_GRID_PLANNED) {
        pl.status = PKV_EUNSUPPORTED;
        return pl;
      }
    } else {
      pl.planned = num_seqs <= kFusedOrderMax ? 1 : 2;
    }
  }
  return pl;
}

// Workspace layout, each part 16-byte aligned: with several partitions the
// partial outputs [B][Hq][max_parts][HD] fp32 and the partial (max, sum)
// [B][Hq][max_parts][2] fp32; then for the planned grid the planner's
// scratch [2B] int32, the items [B * max_parts][4] int32 and their count.
struct Layout {
  size_t part_o = 0, part_ml = 0, scratch = 0, items = 0, count = 0, total = 0;
};

size_t align16(size_t x) { return (x + 15) / 16 * 16; }

Layout workspace_layout(int num_seqs, int num_q_heads, int head_dim, const Plan& pl) {
  Layout lo;
  const size_t states = pl.max_parts > 1 ? (size_t)num_seqs * num_q_heads * pl.max_parts : 0;
  lo.part_o = 0;
  lo.part_ml = align16(states * head_dim * sizeof(float));
  lo.scratch = lo.part_ml + align16(states * 2 * sizeof(float));
  if (pl.planned != 2) {
    lo.total = lo.scratch;
    return lo;
  }
  lo.items = lo.scratch + align16((size_t)2 * num_seqs * sizeof(int32_t));
  lo.count = lo.items + (size_t)num_seqs * pl.max_parts * 4 * sizeof(int32_t);
  lo.total = lo.count + 16;
  return lo;
}

// Grouped decode with parts: the part states [num_groups][max_parts][Hkv][16]
// of HD floats (outputs) and 2 floats (max, sum), each part 16-byte aligned;
// nothing when every group is one part.
struct GroupedLayout {
  int max_parts = 1;
  size_t part_o = 0, part_ml = 0, total = 0;
};

GroupedLayout grouped_layout(int num_groups, int num_kv_heads, int head_dim, int part_tiles,
                             int max_group_tiles) {
  GroupedLayout lo;
  if (part_tiles > 0 && max_group_tiles > part_tiles)
    lo.max_parts = (int)(((int64_t)max_group_tiles + part_tiles - 1) / part_tiles);
  if (lo.max_parts <= 1) return lo;
  const size_t states = (size_t)num_groups * lo.max_parts * num_kv_heads * 16;
  lo.part_ml = align16(states * head_dim * sizeof(float));
  lo.total = lo.part_ml + align16(states * 2 * sizeof(float));
  return lo;
}

size_t workspace_for(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                     const Plan& pl) {
  return workspace_layout(num_seqs, num_q_heads, head_dim, pl).total;
}

// ------------------------------------------------ allocation-free decode
//
// The workspace of pkv_paged_attention_decode_noalloc: one array in device
// memory per GPU the library runs on, held until the process ends.  In host
// code `scratch` names a host-side stand-in, not a device address: the
// device address is taken once per device with hipGetSymbolAddress (with
// that device current) and only that address is passed to the kernels.
// Calls on one GPU share its array; nothing in it needs to start at zero
// (the decode writes every partial state and list entry it reads).
constexpr size_t kNoAllocScratchBytes = (size_t)PKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// The current device's address of `scratch` (looked up on the first call on
// that device, then cached).
int noalloc_scratch(void** out) {
  static void* cached[kMaxDevices];
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return fail_hip(err);
  if (dev < 0 || dev >= kMaxDevices) {
    g_last_error = "device index beyond the library's table";
    return PKV_EUNSUPPORTED;
  }
  void* p = __atomic_load_n(&cached[dev], __ATOMIC_ACQUIRE);
  if (!p) {
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return fail_hip(err);
    if (!p) {
      g_last_error = "hipGetSymbolAddress returned no address for the scratch array";
      return PKV_EHIP;
    }
    __atomic_store_n(&cached[dev], p, __ATOMIC_RELEASE);
  }
  *out = p;
  return PKV_OK;
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
  if (!plan_dtype_ok(dtype)) return 0;
  return decode_valu_supported(to_elem(dtype), (dtype & PKV_KV_E4M3) != 0, head_dim, block_size)
             ? 1
             : 0;
}

size_t pkv_paged_attention_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                           int head_dim, int block_size, int max_blocks_per_seq,
                                           int max_context_len, pkv_dtype dtype,
                                           int partition_tokens, int path, int grid) {
  bool shared = false;
  if (!plan_dtype_ok(dtype) || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 ||
      partition_tokens < 0 || !split_path(path, &path, &shared) ||
      grid < PKV_GRID_AUTO || grid > PKV_GRID_PLANNED || num_q_heads % num_kv_heads)
    return (size_t)-1;
  const Plan pl = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                            max_blocks_per_seq, max_context_len, dtype, partition_tokens, path, grid);
  if (pl.status != PKV_OK) return (size_t)-1;
  return workspace_for(num_seqs, num_q_heads, num_kv_heads, head_dim, pl);
}

int pkv_paged_attention_plan(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                             int block_size, int max_blocks_per_seq, int max_context_len,
                             pkv_dtype dtype, int partition_tokens, int path, int grid,
                             pkv_plan* out) {
  bool shared = false;
  if (!plan_dtype_ok(dtype) || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 ||
      partition_tokens < 0 || !split_path(path, &path, &shared) ||
      grid < PKV_GRID_AUTO || grid > PKV_GRID_PLANNED || num_q_heads % num_kv_heads)
    return PKV_EINVAL;
  const Plan pl = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                            max_blocks_per_seq, max_context_len, dtype, partition_tokens, path, grid);
  if (pl.status != PKV_OK) return pl.status;
  if (out) {
    out->path = pl.mfma ? PKV_PATH_MFMA : PKV_PATH_VALU;
    out->grid = pl.planned ? PKV_GRID_PLANNED : PKV_GRID_DIRECT;
    out->partition_tokens = pl.part_tokens;
    out->max_parts = pl.max_parts;
    out->longest_first = pl.planned ? 1 : 0;
    out->workspace_bytes = workspace_for(num_seqs, num_q_heads, num_kv_heads, head_dim, pl);
  }
  return PKV_OK;
}

}  // extern "C"

namespace {

// Every decode entry point: kv_fp8 says the caches hold E4M3 codes with the
// given scales (ignored otherwise).
int decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* context_lens, float scale,
                bool kv_fp8, float k_scale, float v_scale, int num_seqs, int num_q_heads,
                int num_kv_heads, int head_dim, int block_size, int num_blocks,
                int max_blocks_per_seq, int max_context_len, int dtype, void* workspace,
                size_t workspace_bytes, int partition, int path, int grid, void* begin_event,
                void* end_event, void* stream) {
  bool shared_blocks = false;
  if (!dtype_ok(dtype) || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      max_context_len < 0 || partition < 0 || !split_path(path, &path, &shared_blocks) ||
      grid < PKV_GRID_AUTO || grid > PKV_GRID_PLANNED)
    return PKV_EINVAL;
  if (num_q_heads % num_kv_heads) return PKV_EINVAL;
  if (kv_fp8 && (!finite_nonzero(k_scale) || !finite_nonzero(v_scale))) return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  const bool contiguous = path == PKV_PATH_CONTIGUOUS;
  if (!out || !q || !k_cache || !v_cache || !context_lens || (!block_tables && !contiguous))
    return PKV_EINVAL;
  if (num_seqs > kMaxGridYZ || num_q_heads > kMaxGridYZ) return PKV_EUNSUPPORTED;
  if (max_blocks_per_seq > (1 << 30) / block_size) return PKV_EUNSUPPORTED;
  if (contiguous && (int64_t)num_seqs * max_blocks_per_seq > num_blocks) return PKV_EINVAL;

  const Elem e = to_elem(dtype);
  const Plan pl = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                            max_blocks_per_seq, max_context_len,
                            kv_fp8 ? (dtype | PKV_KV_E4M3) : dtype, partition, path, grid);
  if (pl.status != PKV_OK) return pl.status;
  const Layout lo = workspace_layout(num_seqs, num_q_heads, head_dim, pl);
  const size_t need = lo.total;
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_EWORKSPACE;
  if (need > 0 && reinterpret_cast<uintptr_t>(workspace) % 16) return PKV_EINVAL;
  if (debug_checks()) {
    const int rc = debug_check_tables(context_lens, contiguous ? nullptr : block_tables, num_seqs,
                                      max_blocks_per_seq, block_size, num_blocks, pl.len_cap,
                                      static_cast<hipStream_t>(stream));
    if (rc != PKV_OK) return rc;
  }
  const bool use_mfma = pl.mfma;

  DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  char* ws = static_cast<char*>(workspace);
  a.part_o = pl.max_parts > 1 ? reinterpret_cast<float*>(ws + lo.part_o) : nullptr;
  a.part_ml = pl.max_parts > 1 ? reinterpret_cast<float*>(ws + lo.part_ml) : nullptr;
  a.items = pl.planned == 2 ? reinterpret_cast<const int32_t*>(ws + lo.items) : nullptr;
  a.item_count = pl.planned == 2 ? reinterpret_cast<const int32_t*>(ws + lo.count) : nullptr;
  a.planned = pl.planned;
  a.scale_log2e = (float)((double)scale * (kv_fp8 ? (double)k_scale : 1.0) * 1.4426950408889634);
  a.v_scale = kv_fp8 ? v_scale : 1.f;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.len_cap = pl.len_cap;
  a.part_tokens = pl.part_tokens;
  a.part_align = pl.part_align;
  a.max_parts = pl.max_parts;
  a.contiguous = contiguous ? 1 : 0;
  a.cached_kv = shared_blocks ? 1 : 0;

  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (pl.planned == 2) {
    err = launch_plan_items(context_lens, num_seqs, pl.len_cap, pl.part_tokens, pl.part_align,
                            reinterpret_cast<int32_t*>(ws + lo.scratch),
                            reinterpret_cast<int32_t*>(ws + lo.items),
                            reinterpret_cast<int32_t*>(ws + lo.count), st);
    if (err != hipSuccess) return fail_hip(err);
  }
  if (begin_event && (err = hipEventRecord(static_cast<hipEvent_t>(begin_event), st)) != hipSuccess)
    return fail_hip(err);
  err = use_mfma ? launch_decode_mfma(e, kv_fp8, head_dim, block_size, a, st)
                 : launch_decode_valu(e, kv_fp8, head_dim, block_size, a, st);
  if (err != hipSuccess) return fail_hip(err);
  if (end_event && (err = hipEventRecord(static_cast<hipEvent_t>(end_event), st)) != hipSuccess)
    return fail_hip(err);
  if (pl.max_parts > 1) {
    err = launch_decode_reduce(e, head_dim, a, st);
    if (err != hipSuccess) return fail_hip(err);
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_paged_attention_decode_timed(void* out, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_tables,
                                     const int32_t* context_lens, float scale, int num_seqs,
                                     int num_q_heads, int num_kv_heads, int head_dim,
                                     int block_size, int num_blocks, int max_blocks_per_seq,
                                     int max_context_len, pkv_dtype dtype, void* workspace,
                                     size_t workspace_bytes, int partition, int path, int grid,
                                     void* begin_event, void* end_event, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, false, 1.f, 1.f,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, dtype, workspace, workspace_bytes,
                     partition, path, grid, begin_event, end_event, stream);
}

int pkv_paged_attention_decode_fp8(void* out, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, float scale, float k_scale,
                                   float v_scale, int num_seqs, int num_q_heads, int num_kv_heads,
                                   int head_dim, int block_size, int num_blocks,
                                   int max_blocks_per_seq, int max_context_len, pkv_dtype dtype,
                                   void* workspace, size_t workspace_bytes, int partition,
                                   int path, int grid, void* begin_event, void* end_event,
                                   void* stream) {
  if ((path & ~PKV_PATH_SHARED_BLOCKS) == PKV_PATH_CONTIGUOUS) return PKV_EUNSUPPORTED;
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, true, k_scale,
                     v_scale, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_blocks_per_seq, max_context_len, dtype, workspace,
                     workspace_bytes, partition, path, grid, begin_event, end_event, stream);
}

int pkv_paged_attention_decode_ex(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, float scale, int num_seqs,
                                  int num_q_heads, int num_kv_heads, int head_dim,
                                  int block_size, int num_blocks, int max_blocks_per_seq,
                                  int max_context_len, pkv_dtype dtype, void* workspace,
                                  size_t workspace_bytes, int partition, int path, int grid,
                                  void* stream) {
  return pkv_paged_attention_decode_timed(out, q, k_cache, v_cache, block_tables, context_lens,
                                          scale, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                          block_size, num_blocks, max_blocks_per_seq,
                                          max_context_len, dtype, workspace, workspace_bytes,
                                          partition, path, grid, nullptr, nullptr, stream);
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
                                       PKV_PATH_AUTO, PKV_GRID_AUTO, stream);
}

int pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, float scale, int num_seqs,
                                       int num_q_heads, int num_kv_heads, int head_dim,
                                       int block_size, int num_blocks, int max_blocks_per_seq,
                                       int max_context_len, pkv_dtype dtype, void* stream) {
  // the workspace this call would need, before anything touches the device
  const size_t need = pkv_paged_attention_workspace_bytes(
      num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
      max_context_len, dtype, 0, PKV_PATH_AUTO, PKV_GRID_AUTO);
  if (need == (size_t)-1) {
    // the argument error pkv_paged_attention_decode reports for these sizes
    return pkv_paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                      num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                      num_blocks, max_blocks_per_seq, max_context_len, dtype,
                                      nullptr, 0, stream);
  }
  if (need > kNoAllocScratchBytes) {
    g_last_error = "the call needs " + std::to_string(need) +
                   " bytes of workspace, more than the " +
                   std::to_string(kNoAllocScratchBytes) +
                   " bytes of scratch the allocation-free entry point holds";
    return PKV_EWORKSPACE;
  }
  void* ws = nullptr;
  if (need > 0) {
    const int rc = noalloc_scratch(&ws);
    if (rc != PKV_OK) return rc;
  }
  return pkv_paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                    num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                    num_blocks, max_blocks_per_seq, max_context_len, dtype, ws,
                                    ws ? kNoAllocScratchBytes : 0, stream);
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
  if (debug_checks()) {
    const int rc = debug_check_slots(slot_mapping, num_tokens, (int64_t)num_blocks * block_size,
                                     static_cast<hipStream_t>(stream));
    if (rc != PKV_OK) return rc;
  }
  hipError_t err = launch_reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, num_tokens,
                                            num_kv_heads, row_bytes, block_size, num_blocks,
                                            static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PKV_OK : fail_hip(err);
}

}  // extern "C"

namespace {

// Both prefill entry points: kv_fp8 says the caches hold E4M3 codes with the
// given scales (ignored otherwise).
int prefill_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* context_lens,
                 const int32_t* query_start, float scale, bool kv_fp8, float k_scale,
                 float v_scale, int num_seqs, int total_q, int max_q_len, int num_q_heads,
                 int num_kv_heads, int head_dim, int block_size, int num_blocks,
                 int max_blocks_per_seq, int max_context_len, int dtype, void* begin_event,
                 void* end_event, void* stream) {
  if (kv_fp8 && (!finite_nonzero(k_scale) || !finite_nonzero(v_scale))) return PKV_EINVAL;
  if (!dtype_ok(dtype) || num_seqs < 0 || total_q < 0 || max_q_len < 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_context_len < 0 || num_q_heads % num_kv_heads)
    return PKV_EINVAL;
  const int group = num_q_heads / num_kv_heads;
  if (!prefill_supported(to_elem(dtype), head_dim, block_size, group)) return PKV_EUNSUPPORTED;
  if (num_seqs == 0 || total_q == 0 || max_q_len == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return PKV_EINVAL;
  if (num_seqs > kMaxGridYZ) return PKV_EUNSUPPORTED;
  if (max_blocks_per_seq > (1 << 30) / block_size) return PKV_EUNSUPPORTED;
  const int per_wg = prefill_tokens_per_workgroup(group);
  const int64_t chunks = ((int64_t)max_q_len + per_wg - 1) / per_wg;
  if (chunks * num_kv_heads > INT32_MAX) return PKV_EUNSUPPORTED;
  const int64_t table_cap = (int64_t)max_blocks_per_seq * block_size;
  if (debug_checks()) {
    hipStream_t dst = static_cast<hipStream_t>(stream);
    int rc = debug_check_query_start(query_start, num_seqs, total_q, max_q_len, dst);
    if (rc == PKV_OK)
      rc = debug_check_tables(context_lens, block_tables, num_seqs, max_blocks_per_seq,
                              block_size, num_blocks,
                              table_cap < max_context_len ? table_cap : max_context_len, dst);
    if (rc != PKV_OK) return rc;
  }
  PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.scale_log2e = (float)((double)scale * (kv_fp8 ? (double)k_scale : 1.0) * 1.4426950408889634);
  a.v_scale = kv_fp8 ? v_scale : 1.f;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.len_cap = (int)(table_cap < max_context_len ? table_cap : max_context_len);
  a.chunks = (int)chunks;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (begin_event && (err = hipEventRecord(static_cast<hipEvent_t>(begin_event), st)) != hipSuccess)
    return fail_hip(err);
  err = launch_prefill(to_elem(dtype), kv_fp8, head_dim, block_size, a, st);
  if (err != hipSuccess) return fail_hip(err);
  if (end_event && (err = hipEventRecord(static_cast<hipEvent_t>(end_event), st)) != hipSuccess)
    return fail_hip(err);
  return PKV_OK;
}

// Both grouped decode entry points: kv_fp8 says the caches hold E4M3 codes
// with the given scales (ignored otherwise).
int grouped_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* context_lens, const int32_t* group_members,
                 const int32_t* group_tiles, const int32_t* group_tile_start,
                 const int32_t* group_tile_end, int num_tiles,
                 float scale, int num_seqs, int num_groups, int max_members, int num_q_heads,
                 int num_kv_heads, int head_dim, int block_size, int num_blocks,
                 int max_context_len, int dtype, bool kv_fp8, float k_scale, float v_scale,
                 int part_tiles, int max_group_tiles, void* workspace, size_t workspace_bytes,
                 void* begin_event, void* end_event, void* stream) {
  if (!dtype_ok(dtype) || num_seqs < 0 || num_groups < 0 || max_members <= 0 || num_tiles < 0 ||
      num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0 || max_context_len < 0 || num_q_heads % num_kv_heads || part_tiles < 0 ||
      max_group_tiles < 0)
    return PKV_EINVAL;
  if (kv_fp8 && (!finite_nonzero(k_scale) || !finite_nonzero(v_scale))) return PKV_EINVAL;
  if (num_groups == 0 || num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !context_lens || !group_members || !group_tiles ||
      !group_tile_start)
    return PKV_EINVAL;
  if (reinterpret_cast<uintptr_t>(group_tiles) % 16) return PKV_EINVAL;
  const Elem e = to_elem(dtype);
  const int group = num_q_heads / num_kv_heads;
  if (!grouped_supported(e, head_dim, block_size) || max_members > 16 ||
      (int64_t)max_members * group > 16 ||
      num_groups > kMaxGridYZ || num_kv_heads > kMaxGridYZ)
    return PKV_EUNSUPPORTED;
  const GroupedLayout lo = grouped_layout(num_groups, num_kv_heads, head_dim, part_tiles,
                                          max_group_tiles);
  if (lo.max_parts > kMaxGridYZ) return PKV_EUNSUPPORTED;
  if (lo.total > 0 && (!workspace || workspace_bytes < lo.total)) return PKV_EWORKSPACE;
  if (lo.total > 0 && reinterpret_cast<uintptr_t>(workspace) % 16) return PKV_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_checks()) {
    const int rc = debug_check_groups(context_lens, group_members, group_tiles, group_tile_start,
                                      group_tile_end, num_tiles, num_seqs, num_groups,
                                      max_members, num_blocks,
                                      max_context_len, part_tiles > 0 ? max_group_tiles : -1,
                                      st);
    if (rc != PKV_OK) return rc;
  }
  GroupedArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.context_lens = context_lens;
  a.members = group_members;
  a.tiles = group_tiles;
  a.tile_start = group_tile_start;
  a.tile_end = group_tile_end;
  a.num_tiles = num_tiles;
  a.scale_log2e = (float)((double)scale * (kv_fp8 ? (double)k_scale : 1.0) * 1.4426950408889634);
  a.v_scale = kv_fp8 ? v_scale : 1.f;
  a.num_seqs = num_seqs;
  a.num_groups = num_groups;
  a.max_members = max_members;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.num_blocks = num_blocks;
  a.len_cap = max_context_len;
  a.part_tiles = lo.max_parts > 1 ? part_tiles : 0;
  a.max_parts = lo.max_parts;
  char* ws = static_cast<char*>(workspace);
  a.part_o = lo.total ? reinterpret_cast<float*>(ws + lo.part_o) : nullptr;
  a.part_ml = lo.total ? reinterpret_cast<float*>(ws + lo.part_ml) : nullptr;
  hipError_t err;
  if (begin_event && (err = hipEventRecord(static_cast<hipEvent_t>(begin_event), st)) != hipSuccess)
    return fail_hip(err);
  err = launch_decode_grouped(e, kv_fp8, head_dim, block_size, a, st);
  if (err != hipSuccess) return fail_hip(err);
  if (end_event && (err = hipEventRecord(static_cast<hipEvent_t>(end_event), st)) != hipSuccess)
    return fail_hip(err);
  if (lo.max_parts > 1 && (err = launch_grouped_merge(e, head_dim, a, st)) != hipSuccess)
    return fail_hip(err);
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_paged_attention_prefill(void* out, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* query_start,
                                float scale, int num_seqs, int total_q, int max_q_len,
                                int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                int num_blocks, int max_blocks_per_seq, int max_context_len,
                                pkv_dtype dtype, void* begin_event, void* end_event,
                                void* stream) {
  return prefill_impl(out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                      false, 1.f, 1.f, num_seqs, total_q, max_q_len, num_q_heads, num_kv_heads,
                      head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                      dtype, begin_event, end_event, stream);
}

int pkv_paged_attention_prefill_fp8(void* out, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* block_tables,
                                    const int32_t* context_lens, const int32_t* query_start,
                                    float scale, float k_scale, float v_scale, int num_seqs,
                                    int total_q, int max_q_len, int num_q_heads,
                                    int num_kv_heads, int head_dim, int block_size,
                                    int num_blocks, int max_blocks_per_seq, int max_context_len,
                                    pkv_dtype dtype, void* begin_event, void* end_event,
                                    void* stream) {
  return prefill_impl(out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                      true, k_scale, v_scale, num_seqs, total_q, max_q_len, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                      max_context_len, dtype, begin_event, end_event, stream);
}

size_t pkv_group_tiles_capacity(int num_groups, int max_members, int block_size,
                                int max_blocks_per_seq, int max_context_len) {
  if (num_groups < 0 || max_members <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 ||
      max_context_len < 0)
    return (size_t)-1;
  const int64_t table_cap = (int64_t)max_blocks_per_seq * block_size;
  const int64_t len_cap = table_cap < max_context_len ? table_cap : max_context_len;
  return (size_t)num_groups * (size_t)max_members * (size_t)((len_cap + 15) / 16);
}

int pkv_group_tiles(const int32_t* block_tables, const int32_t* context_lens,
                    const int32_t* group_members, int num_seqs, int max_blocks_per_seq,
                    int num_groups, int max_members, int block_size, int max_context_len,
                    int32_t* group_tiles, int tiles_capacity, int32_t* group_tile_start,
                    int32_t* group_tile_end, void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_groups < 0 || max_members <= 0 ||
      block_size <= 0 || max_context_len < 0 || tiles_capacity < 0)
    return PKV_EINVAL;
  if (max_members > 16 || block_size % 16) return PKV_EUNSUPPORTED;
  if (num_groups == 0) return PKV_OK;
  if (!group_tile_start || !group_tile_end || !group_members || !block_tables || !context_lens ||
      !group_tiles)
    return PKV_EINVAL;
  if (reinterpret_cast<uintptr_t>(group_tiles) % 16) return PKV_EINVAL;
  const size_t need = pkv_group_tiles_capacity(num_groups, max_members, block_size,
                                               max_blocks_per_seq, max_context_len);
  if (need > (size_t)INT32_MAX) return PKV_EUNSUPPORTED;   // row offsets are int32
  if ((size_t)tiles_capacity < need) return PKV_EWORKSPACE;
  const int64_t table_cap = (int64_t)max_blocks_per_seq * block_size;
  const int len_cap = (int)(table_cap < max_context_len ? table_cap : max_context_len);
  const int stride = max_members * ((len_cap + 15) / 16);
  hipError_t err = launch_build_group_tiles(block_tables, context_lens, group_members, num_seqs,
                                            max_blocks_per_seq, num_groups, max_members,
                                            block_size, len_cap, group_tiles, stride,
                                            group_tile_start, group_tile_end,
                                            static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PKV_OK : fail_hip(err);
}

size_t pkv_paged_attention_grouped_workspace_bytes(int num_groups, int num_kv_heads,
                                                   int head_dim, int part_tiles,
                                                   int max_group_tiles) {
  if (num_groups < 0 || num_kv_heads <= 0 || head_dim <= 0 || part_tiles < 0 ||
      max_group_tiles < 0)
    return (size_t)-1;
  const GroupedLayout lo = grouped_layout(num_groups, num_kv_heads, head_dim, part_tiles,
                                          max_group_tiles);
  return lo.total;
}

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
                                       void* begin_event, void* end_event, void* stream) {
  return grouped_impl(out, q, k_cache, v_cache, context_lens, group_members, group_tiles,
                      group_tile_start, group_tile_end, num_tiles, scale, num_seqs, num_groups,
                      max_members, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_context_len, dtype, false, 1.f, 1.f, part_tiles, max_group_tiles,
                      workspace, workspace_bytes, begin_event, end_event, stream);
}

int pkv_paged_attention_decode_grouped_fp8(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* context_lens, const int32_t* group_members, const int32_t* group_tiles,
    const int32_t* group_tile_start, const int32_t* group_tile_end, int num_tiles, float scale,
    float k_scale, float v_scale,
    int num_seqs, int num_groups, int max_members, int num_q_heads, int num_kv_heads,
    int head_dim, int block_size, int num_blocks, int max_context_len, pkv_dtype dtype,
    int part_tiles, int max_group_tiles, void* workspace, size_t workspace_bytes,
    void* begin_event, void* end_event, void* stream) {
  return grouped_impl(out, q, k_cache, v_cache, context_lens, group_members, group_tiles,
                      group_tile_start, group_tile_end, num_tiles, scale, num_seqs, num_groups,
                      max_members, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_context_len, dtype, true, k_scale, v_scale, part_tiles,
                      max_group_tiles, workspace, workspace_bytes, begin_event, end_event,
                      stream);
}

int pkv_reshape_and_cache_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                              const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                              int head_dim, int block_size, int num_blocks, pkv_dtype dtype,
                              float k_scale, float v_scale, void* stream) {
  if (!dtype_ok(dtype) || num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_blocks <= 0 || !finite_nonzero(k_scale) || !finite_nonzero(v_scale))
    return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PKV_EINVAL;
  if (head_dim % 16) return PKV_EUNSUPPORTED;
  if (debug_checks()) {
    const int rc = debug_check_slots(slot_mapping, num_tokens, (int64_t)num_blocks * block_size,
                                     static_cast<hipStream_t>(stream));
    if (rc != PKV_OK) return rc;
  }
  hipError_t err = launch_reshape_and_cache_fp8(to_elem(dtype), k, v, k_cache, v_cache,
                                                slot_mapping, num_tokens, num_kv_heads, head_dim,
                                                block_size, num_blocks, k_scale, v_scale,
                                                static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PKV_OK : fail_hip(err);
}

int pkv_copy_blocks(void* k_cache, void* v_cache, const int64_t* src_dst_pairs, int num_pairs,
                    int num_kv_heads, int head_dim, int block_size, int num_blocks,
                    pkv_dtype dtype, void* stream) {
  if (!cache_dtype_ok(dtype) || num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_blocks <= 0)
    return PKV_EINVAL;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src_dst_pairs) return PKV_EINVAL;
  const size_t block_bytes = (size_t)num_kv_heads * block_size * head_dim * elem_size(dtype);
  if (block_bytes % 16) return PKV_EUNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_checks()) {
    const int rc = debug_check_pairs(src_dst_pairs, num_pairs, num_blocks, num_blocks, true, st);
    if (rc != PKV_OK) return rc;
  }
  for (int first = 0; first < num_pairs; first += kMaxGridYZ) {
    const int n = num_pairs - first < kMaxGridYZ ? num_pairs - first : kMaxGridYZ;
    hipError_t err = launch_copy_blocks(k_cache, v_cache, k_cache, v_cache,
                                        src_dst_pairs + 2 * (size_t)first, n, block_bytes,
                                        num_blocks, num_blocks, st);
    if (err != hipSuccess) return fail_hip(err);
  }
  return PKV_OK;
}

int pkv_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                    const int64_t* src_dst_pairs, int num_pairs, int num_kv_heads, int head_dim,
                    int block_size, int num_src_blocks, int num_dst_blocks, pkv_dtype dtype,
                    void* stream) {
  if (!cache_dtype_ok(dtype) || num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_src_blocks <= 0 || num_dst_blocks <= 0)
    return PKV_EINVAL;
  if (num_pairs == 0) return PKV_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !src_dst_pairs) return PKV_EINVAL;
  const size_t block_bytes = (size_t)num_kv_heads * block_size * head_dim * elem_size(dtype);
  if (block_bytes % 16) return PKV_EUNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_checks()) {
    const int rc = debug_check_pairs(src_dst_pairs, num_pairs, num_src_blocks, num_dst_blocks,
                                     false, st);
    if (rc != PKV_OK) return rc;
  }
  for (int first = 0; first < num_pairs; first += kMaxGridYZ) {
    const int n = num_pairs - first < kMaxGridYZ ? num_pairs - first : kMaxGridYZ;
    hipError_t err = launch_copy_blocks(dst_k, dst_v, src_k, src_v,
                                        src_dst_pairs + 2 * (size_t)first, n, block_bytes,
                                        num_src_blocks, num_dst_blocks, st);
    if (err != hipSuccess) return fail_hip(err);
  }
  return PKV_OK;
}

}  // extern "C"
