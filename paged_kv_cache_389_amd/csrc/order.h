// Longest-first orders: lengths are binned by half octaves below a bound
// (bin b holds lengths in (cap * 2^-(b+1)/2, cap * 2^-b/2], 32 bins; bin 0
// is the longest), and an order lists bin 0 first and, inside a bin,
// increasing index.  The work planner bins partition sizes this way; the
// decode kernels of the direct grid rank sequences by length themselves
// for batches of at most kFusedOrderMax sequences (sorted_sequence).
#pragma once

#include "common.h"

namespace pkv {

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

// LDS a 256-thread workgroup needs for sorted_sequence().
struct OrderScratch {
  int cnt[kFusedOrderMax / 256][4][kBins];   // per (chunk, wave) bin counts, then their prefix
  int base[kBins];                           // first position of each bin
  int result;
};

// The sequence at position z of the longest-first order, computed by the
// whole workgroup (blockDim.x == 256, num_seqs <= kFusedOrderMax; every
// thread must call it).  Each thread bins the lengths of sequences tid,
// tid + 256, ...; ballots rank every sequence inside its bin within its
// wave; the per-(chunk, wave) bin counts give every sequence its position,
// and the thread holding position z publishes its index.  Three barriers.
__device__ inline int sorted_sequence(const int32_t* __restrict__ lens, int num_seqs, int len_cap,
                                      int z, OrderScratch& sm) {
  constexpr int KMAX = kFusedOrderMax / 256;
  const int tid = threadIdx.x, wave = uniform(tid / kWave), lane = tid % kWave;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int cap = len_cap > 0 ? len_cap : 1;
  const int nk = (num_seqs + 255) / 256;
  int bins[KMAX], rank[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int i = k * 256 + tid;
    bins[k] = (k < nk && i < num_seqs) ? length_bin(min(lens[i], cap), cap) : -1;
    rank[k] = 0;
  }
  if (tid == 0) sm.result = z;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (k < nk) {
      int cnt = 0;
#pragma unroll
      for (int b = 0; b < kBins; ++b) {
        const uint64_t mask = __ballot(bins[k] == b);
        if (bins[k] == b) rank[k] = __popcll(mask & below);
        if (lane == b) cnt = __popcll(mask);
      }
      if (lane < kBins) sm.cnt[k][wave][lane] = cnt;
    }
  }
  __syncthreads();
  if (wave == 0) {
    // lane b: exclusive prefix of bin b over (chunk, wave) in order, the
    // bin's total, then the exclusive prefix of the totals across bins
    int run = 0;
    if (lane < kBins) {
      for (int k = 0; k < nk; ++k)
        for (int w = 0; w < 4; ++w) {
          const int c = sm.cnt[k][w][lane];
          sm.cnt[k][w][lane] = run;
          run += c;
        }
    }
    int incl = run;
#pragma unroll
    for (int off = 1; off < kBins; off <<= 1) {
      const int up = __shfl_up(incl, off, 64);
      if (lane >= off) incl += up;
    }
    if (lane < kBins) sm.base[lane] = incl - run;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (bins[k] >= 0 && sm.base[bins[k]] + sm.cnt[k][wave][bins[k]] + rank[k] == z)
      sm.result = k * 256 + tid;
  }
  __syncthreads();
  return sm.result;
}

}  // namespace pkv
