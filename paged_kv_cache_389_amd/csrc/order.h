// Largest-first work lists: sizes are binned by half octaves below a bound
// (bin b holds sizes in (cap * 2^-(b+1)/2, cap * 2^-b/2], 32 bins; bin 0 is
// the largest), and a list takes bin 0 first and, inside a bin, increasing
// sequence index.  The decode kernels compute their own item of such a
// list for batches of at most kFusedOrderMax sequences (plan_item); the
// planning kernel writes the list for larger ones.
#pragma once

#include "common.h"

namespace pkv {

// Partitions.  A context of L > 0 tokens is cut into n = ceil(L / P)
// partitions of equal size, rounded up to `align` tokens (the last one
// shorter), so no partition is a small remainder; P (part_tokens) is a
// multiple of align, hence every partition holds at most P tokens and the
// last one at least one.  A context of L <= 0 tokens has one (empty)
// partition, which writes the zero row.
__host__ __device__ inline int num_parts(int L, int P) { return L <= 0 ? 1 : (L + P - 1) / P; }
__host__ __device__ inline int part_size(int L, int n, int align) {
  const int ps = (L + n - 1) / n;
  return (ps + align - 1) / align * align;
}

constexpr int kBins = 32;
constexpr int kFusedOrderMax = 1024;   // 4 sequences per thread of a 256-thread workgroup

// Half-octave bin of a length below `cap`: 0 for lengths in (cap/sqrt2, cap],
// then one bin per factor sqrt(2); lengths <= 0 and the shortest go last.
__device__ inline int length_bin(int L, int cap) {
  if (L <= 0) return kBins - 1;
  if (L >= cap) return 0;
  // b = floor(2 * log2(cap / L)), from the hardware log2 (exact enough for a bin)
  const float r = __builtin_amdgcn_logf((float)cap) - __builtin_amdgcn_logf((float)L);
  const int b = (int)(2.f * r);
  return b < kBins - 1 ? b : kBins - 1;
}

// LDS of plan_item().
struct PlanScratch {
  int weight[kBins];   // partitions per bin, then their exclusive prefix
  int wave_total[4];
  int total;
  int found[5];        // s, part, n, t0, t1 of the item
};

// Item k of the batch's work list, computed by the whole 256-thread
// workgroup (every thread must call it; num_seqs <= kFusedOrderMax).  The
// list holds, for every sequence, its n = num_parts(L, P) partitions of
// part_size(L, n, align) tokens (one empty item for L == 0), ordered by the
// half-octave bin of the partition size, largest first, then by sequence
// index, a sequence's partitions together.  Thread t holds sequences
// 4t .. 4t+3; LDS atomics weight the bins, a 32-lane scan places them, and
// one block scan over the sequences of item k's bin finds the item.  Five
// barriers.  Returns false when k is past the list (for every thread).
__device__ inline bool plan_item(const int32_t* __restrict__ lens, int num_seqs, int len_cap,
                                 int P, int align, int k, PlanScratch& sm, int* item) {
  constexpr int kPer = kFusedOrderMax / 256;
  const int tid = threadIdx.x, wave = uniform(tid / kWave), lane = tid % kWave;
  if (tid < kBins) sm.weight[tid] = 0;
  if (tid == 0) sm.found[0] = -1;
  int Lv[kPer], nv[kPer], bv[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = kPer * tid + e;
    int L = i < num_seqs ? lens[i] : 0;
    L = L < 0 ? 0 : (L > len_cap ? len_cap : L);
    Lv[e] = L;
    nv[e] = i < num_seqs ? num_parts(L, P) : 0;
    bv[e] = L <= 0 ? kBins - 1 : length_bin(part_size(L, nv[e], align), P);
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kPer; ++e)
    if (nv[e]) atomicAdd(&sm.weight[bv[e]], nv[e]);
  __syncthreads();
  if (wave == 0) {
    const int w = lane < kBins ? sm.weight[lane] : 0;
    int incl = w;
#pragma unroll
    for (int off = 1; off < kBins; off <<= 1) {
      const int up = __shfl_up(incl, off, 64);
      if (lane >= off) incl += up;
    }
    if (lane < kBins) sm.weight[lane] = incl - w;
    if (lane == kBins - 1) sm.total = incl;
  }
  __syncthreads();
  if (k >= sm.total) return false;
  // the bin holding item k: the last bin whose first item is at most k
  int b = 0;
  for (int j = 1; j < kBins; ++j)
    if (sm.weight[j] <= k) b = j;
  const int kk = k - sm.weight[b];
  int c[kPer], sum = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    c[e] = bv[e] == b ? nv[e] : 0;
    sum += c[e];
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int up = __shfl_up(incl, off, 64);
    if (lane >= off) incl += up;
  }
  if (lane == kWave - 1) sm.wave_total[wave] = incl;
  __syncthreads();
  int excl = incl - sum;
  for (int w = 0; w < wave; ++w) excl += sm.wave_total[w];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    if (c[e] && excl <= kk && kk < excl + c[e]) {
      const int part = kk - excl, n = nv[e], L = Lv[e];
      const int ps = part_size(L, n, align);
      sm.found[0] = kPer * tid + e;
      sm.found[1] = part;
      sm.found[2] = n;
      sm.found[3] = part * ps;
      sm.found[4] = min(L, part * ps + ps);
    }
    excl += c[e];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 5; ++j) item[j] = sm.found[j];
  return item[0] >= 0;
}

}  // namespace pkv
