// Tile lists of the grouped decode, built on the device from the block
// tables.
//
// Group j's rows name every distinct (physical block, 16-token tile index)
// that its members reach, with the mask of the members that reach it
// (block tables map a sequence's logical blocks to physical ones; forks of
// one prompt hold the prompt's blocks in common: "Memory Optimization in LLM
// Serving with PagedAttention", sections "How PagedAttention Works" and
// "Advanced Capabilities: Memory Sharing with Copy-on-Write").  Rows are in
// group order, then tile index, then block ascending, and
// tile_start[j] .. tile_start[j+1] are group j's.
//
// One workgroup does the whole batch.  Phase 1 gives every group its tile
// count T_j (the longest member's) and a prefix over the groups in LDS.
// Phase 2 walks the (group, tile) items in chunks of one per thread: each
// thread reads its members' table entries at that tile, keeps the first
// member holding each distinct block, ranks the distinct blocks and ORs the
// masks; a block-wide scan of the per-item row counts places the rows.
#include "common.h"
#include "decode.h"

namespace pkv {

namespace {

constexpr int kBuildThreads = 1024;
constexpr int kMaxMembers = 16;

// Exclusive scan of v over the workgroup (kBuildThreads threads); the total
// goes to *total.  Uses wave_sums[kBuildThreads / 64].
__device__ inline int block_scan(int v, int* wave_sums, int* total) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int up = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += up;
  }
  if (lane == kWave - 1) wave_sums[wave] = incl;
  __syncthreads();
  if (tid < kWave) {
    const int w = tid < kBuildThreads / kWave ? wave_sums[tid] : 0;
    int wincl = w;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int up = __shfl_up(wincl, off, kWave);
      if (tid >= off) wincl += up;
    }
    if (tid < kBuildThreads / kWave) wave_sums[tid] = wincl - w;
    if (tid == kBuildThreads / kWave - 1) *total = wincl;
  }
  __syncthreads();
  const int r = incl - v + wave_sums[wave];
  __syncthreads();   // wave_sums and *total may be reused by the caller
  return r;
}

struct BuildArgs {
  const int32_t* block_tables;   // [B][max_blocks]
  const int32_t* context_lens;   // [B]
  const int32_t* members;        // [G][M]
  int32_t* tiles;                // [cap][4]
  int32_t* tile_start;           // [G + 1]
  int num_seqs, max_blocks, num_groups, max_members, block_size, len_cap, cap;
};

__device__ inline int member_seq(const BuildArgs& a, int j, int m) {
  const int s = a.members[(size_t)j * a.max_members + m];
  return (s >= 0 && s < a.num_seqs) ? s : -1;
}

__device__ inline int member_tiles(const BuildArgs& a, int s) {
  if (s < 0) return 0;
  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  return (L + 15) / 16;
}

constexpr int kCacheSlots = 4096;   // (group, member) places cached in LDS

template <int GMAX>
__global__ __launch_bounds__(kBuildThreads) void build_group_tiles_kernel(BuildArgs a) {
  __shared__ int item_start[GMAX + 1];   // prefix of the groups' tile counts
  __shared__ int wave_sums[kBuildThreads / kWave];
  __shared__ int total;
  // when every (group, member) place fits: its sequence and tile count, so
  // that phase 2 reads only table entries from global memory
  __shared__ int cache_seq[kCacheSlots], cache_tiles[kCacheSlots];
  const int tid = threadIdx.x;
  const int G = a.num_groups, M = a.max_members;
  const int tpb = a.block_size / 16;
  const bool cached = (int64_t)G * M <= kCacheSlots;
  if (cached)
    for (int k = tid; k < G * M; k += kBuildThreads) {
      const int s = member_seq(a, k / M, k % M);
      cache_seq[k] = s;
      cache_tiles[k] = member_tiles(a, s);
    }
  __syncthreads();

  // phase 1: T_j, scanned over the groups in chunks of one per thread
  int run = 0;
  for (int j0 = 0; j0 < G; j0 += kBuildThreads) {
    const int j = j0 + tid;
    int T = 0;
    if (j < G)
      for (int m = 0; m < M; ++m)
        T = max(T, cached ? cache_tiles[j * M + m] : member_tiles(a, member_seq(a, j, m)));
    const int ex = block_scan(T, wave_sums, &total);
    if (j < G) item_start[j] = run + ex;
    run += total;   // every thread reads the same total
  }
  if (tid == 0) item_start[G] = run;
  __syncthreads();
  const int items = run;

  // phase 2: one (group, tile) item per thread per chunk
  int rows_before = 0;
  for (int i0 = 0; i0 < items; i0 += kBuildThreads) {
    const int i = i0 + tid;
    int j = -1, t = 0, count = 0;
    int blk[kMaxMembers];
    bool on[kMaxMembers], keep[kMaxMembers];
    if (i < items) {
      // the last group whose first item is at most i (empty groups share
      // their start with the next one and are skipped)
      int lo = 0, hi = G - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (item_start[mid] <= i) lo = mid; else hi = mid - 1;
      }
      j = lo;
      t = i - item_start[j];
    }
#pragma unroll
    for (int m = 0; m < kMaxMembers; ++m) {
      blk[m] = 0;
      on[m] = false;
      if (j >= 0 && m < M) {
        const int s = cached ? cache_seq[j * M + m] : member_seq(a, j, m);
        if (t < (cached ? cache_tiles[j * M + m] : member_tiles(a, s))) {
          on[m] = true;
          blk[m] = a.block_tables[(size_t)s * a.max_blocks + min(t / tpb, a.max_blocks - 1)];
        }
      }
    }
    // the first member holding each distinct block keeps a row for it
#pragma unroll
    for (int m = 0; m < kMaxMembers; ++m) {
      bool first = on[m];
#pragma unroll
      for (int p = 0; p < m; ++p) first = first && !(on[p] && blk[p] == blk[m]);
      keep[m] = first;
      count += first ? 1 : 0;
    }
    const int ex = block_scan(count, wave_sums, &total);
    const int base = rows_before + ex;
    if (j >= 0 && t == 0) {
      // this group's start, and that of every empty group just before it
      for (int jj = j; jj >= 0 && item_start[jj] == i; --jj) a.tile_start[jj] = base;
    }
#pragma unroll
    for (int m = 0; m < kMaxMembers; ++m) {
      if (!keep[m]) continue;
      int rank = 0, mask = 0;
#pragma unroll
      for (int p = 0; p < kMaxMembers; ++p) {
        if (!on[p]) continue;
        if (blk[p] == blk[m]) mask |= 1 << p;
        else if (keep[p] && blk[p] < blk[m]) ++rank;
      }
      const int row = base + rank;
      if (row < a.cap)
        *reinterpret_cast<i32x4*>(a.tiles + 4 * (size_t)row) = i32x4{blk[m], t, mask, 0};
    }
    rows_before += total;
  }
  // the trailing empty groups and the end of the list
  if (tid == 0)
    for (int jj = G; jj >= 0 && item_start[jj] == items; --jj) a.tile_start[jj] = rows_before;
}

}  // namespace

int group_tiles_max_groups() { return 4096; }

hipError_t launch_build_group_tiles(const int32_t* block_tables, const int32_t* context_lens,
                                    const int32_t* members, int num_seqs, int max_blocks,
                                    int num_groups, int max_members, int block_size, int len_cap,
                                    int32_t* tiles, int cap, int32_t* tile_start,
                                    hipStream_t stream) {
  BuildArgs a{block_tables, context_lens, members, tiles, tile_start, num_seqs, max_blocks,
              num_groups, max_members, block_size, len_cap, cap};
  hipLaunchKernelGGL(build_group_tiles_kernel<4096>, dim3(1), dim3(kBuildThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
