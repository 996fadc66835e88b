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
// One workgroup per group, all in parallel: group j's rows go to a region
// of `stride` rows of its own (tile_start[j] = j * stride, tile_end[j] after
// its last row), so no group waits for another's count.  The workgroup walks
// the group's tile indices one per thread: each thread reads its members'
// table entries at that tile, keeps the first member holding each distinct
// block, ranks the distinct blocks and ORs the masks; a block-wide scan of
// the per-tile row counts places the rows.
#include "common.h"
#include "decode.h"

namespace pkv {

namespace {

constexpr int kBuildThreads = 256;
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
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kBuildThreads / kWave; ++w) {
    before += w < wave ? wave_sums[w] : 0;
    all += wave_sums[w];
  }
  if (tid == 0) *total = all;
  __syncthreads();   // wave_sums may be reused by the caller
  return incl - v + before;
}

struct BuildArgs {
  const int32_t* block_tables;   // [B][max_blocks]
  const int32_t* context_lens;   // [B]
  const int32_t* members;        // [G][M]
  int32_t* tiles;                // [G * stride][4]
  int32_t* tile_start;           // [G]
  int32_t* tile_end;             // [G]
  int num_seqs, max_blocks, num_groups, max_members, block_size, len_cap, stride;
};

__global__ __launch_bounds__(kBuildThreads) void build_group_tiles_kernel(BuildArgs a) {
  __shared__ int seq[kMaxMembers], ntiles[kMaxMembers];
  __shared__ int wave_sums[kBuildThreads / kWave];
  __shared__ int total;
  const int j = blockIdx.x, tid = threadIdx.x;
  const int M = a.max_members, tpb = a.block_size / 16;
  if (tid < kMaxMembers) {
    int s = -1, n = 0;
    if (tid < M) {
      s = a.members[(size_t)j * M + tid];
      if (s < 0 || s >= a.num_seqs) s = -1;
      if (s >= 0) {
        int L = a.context_lens[s];
        L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
        n = (L + 15) / 16;
      }
    }
    seq[tid] = s;
    ntiles[tid] = n;
  }
  __syncthreads();
  int T = 0;
#pragma unroll
  for (int m = 0; m < kMaxMembers; ++m) T = max(T, ntiles[m]);
  const size_t base0 = (size_t)j * a.stride;
  int rows = 0;
  for (int t0 = 0; t0 < T; t0 += kBuildThreads) {
    const int t = t0 + tid;
    int blk[kMaxMembers];
    bool on[kMaxMembers], keep[kMaxMembers];
    int count = 0;
#pragma unroll
    for (int m = 0; m < kMaxMembers; ++m) {
      on[m] = t < ntiles[m];
      blk[m] = on[m] ? a.block_tables[(size_t)seq[m] * a.max_blocks +
                                      min(t / tpb, a.max_blocks - 1)]
                     : 0;
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
      const int row = rows + ex + rank;
      if (row < a.stride)
        *reinterpret_cast<i32x4*>(a.tiles + 4 * (base0 + row)) = i32x4{blk[m], t, mask, 0};
    }
    rows += total;
  }
  if (tid == 0) {
    a.tile_start[j] = (int)base0;
    a.tile_end[j] = (int)(base0 + min(rows, a.stride));
  }
}

}  // namespace

hipError_t launch_build_group_tiles(const int32_t* block_tables, const int32_t* context_lens,
                                    const int32_t* members, int num_seqs, int max_blocks,
                                    int num_groups, int max_members, int block_size, int len_cap,
                                    int32_t* tiles, int stride, int32_t* tile_start,
                                    int32_t* tile_end, hipStream_t stream) {
  BuildArgs a{block_tables, context_lens, members, tiles, tile_start, tile_end, num_seqs,
              max_blocks, num_groups, max_members, block_size, len_cap, stride};
  hipLaunchKernelGGL(build_group_tiles_kernel, dim3(num_groups), dim3(kBuildThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
