// Work list of the planned decode grid.
//
// The decode grid gives each (sequence, partition, head unit) its own
// workgroup, and the hardware starts workgroups in index order, handing a
// compute unit the next one whenever one ends.  This kernel lists the
// (sequence, partition) items so that the largest partitions come first
// and the smallest last (list scheduling, longest job first): the grid then
// ends with short workgroups instead of a long one that started late.
// Items of a sequence stay together, and sequences whose partitions are of
// similar size keep their original order (stable within half-octave bins),
// so neighbours that share cached blocks stay neighbours.
//
// One workgroup of 1024 threads handles any batch size in chunks of 1024:
//  1. snapshot the clamped lengths and count the sequences of each bin of
//     partition size (ballots);
//  2. rank every sequence inside its bin (ballot of the lanes below it plus
//     the counts of the waves and chunks before it) and write the sequence
//     order;
//  3. scan the partition counts along that order and write each sequence's
//     items at its offset.
#include "common.h"
#include "decode.h"
#include "order.h"

namespace pkv {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kPlanLdsSeqs = 4096;   // batches up to this size keep the order in LDS

// The order and the clamped lengths live in LDS (kLds, at most
// kPlanLdsSeqs sequences) or in scratch ([0, B) the order, [B, 2B) the
// lengths).  Item k is (s, part << 16 | n, t0, t1): tokens [t0, t1) of
// sequence s, partition `part` of its n.
template <bool kLds>
__global__ __launch_bounds__(kPlanThreads) void plan_items_kernel(
    const int32_t* __restrict__ lens, int num_seqs, int len_cap, int P, int align,
    int32_t* __restrict__ scratch, int32_t* __restrict__ items, int32_t* __restrict__ count) {
  __shared__ int s_cnt[kPlanWaves][kBins];
  __shared__ int s_base[kBins];
  __shared__ int s_wsum[kPlanWaves];
  __shared__ int s_carry;
  __shared__ int s_arrays[kLds ? 2 * kPlanLdsSeqs : 1];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t* order = kLds ? s_arrays : scratch;
  int32_t* snap = kLds ? s_arrays + kPlanLdsSeqs : scratch + num_seqs;

  // bin 0 holds the largest partitions (sizes in (P/sqrt2, P]); empty
  // sequences (one item that writes a zero row) go last
  auto bin_of = [&](int L) {
    if (L <= 0) return kBins - 1;
    return length_bin(part_size(L, num_parts(L, P), align), P);
  };

  // pass 1: snapshot the lengths; lane b of each wave counts bin b
  int mine = 0;
  for (int c0 = 0; c0 < num_seqs; c0 += kPlanThreads) {
    const int i = c0 + tid;
    int bin = -1;
    if (i < num_seqs) {
      int L = lens[i];
      L = L < 0 ? 0 : (L > len_cap ? len_cap : L);
      snap[i] = L;
      bin = bin_of(L);
    }
#pragma unroll
    for (int b = 0; b < kBins; ++b) {
      const int n = __popcll(__ballot(bin == b));
      if (lane == b) mine += n;
    }
  }
  if (lane < kBins) s_cnt[wave][lane] = mine;
  __syncthreads();
  if (wave == 0) {
    // bin totals, then their exclusive prefix across lanes (bin 0 first)
    int total = 0;
    if (lane < kBins)
      for (int w = 0; w < kPlanWaves; ++w) total += s_cnt[w][lane];
    int incl = total;
#pragma unroll
    for (int off = 1; off < kBins; off <<= 1) {
      const int up = __shfl_up(incl, off, 64);
      if (lane >= off) incl += up;
    }
    if (lane < kBins) s_base[lane] = incl - total;
  }
  __syncthreads();

  // pass 2: the order, chunk by chunk
  for (int c0 = 0; c0 < num_seqs; c0 += kPlanThreads) {
    const int i = c0 + tid;
    const bool valid = i < num_seqs;
    const int bin = valid ? bin_of(snap[i]) : -1;
    int rank = 0, cnt = 0;
#pragma unroll
    for (int b = 0; b < kBins; ++b) {
      const uint64_t mask = __ballot(bin == b);
      if (bin == b) rank = __popcll(mask & below);
      if (lane == b) cnt = __popcll(mask);
    }
    if (lane < kBins) s_cnt[wave][lane] = cnt;
    __syncthreads();
    if (valid) {
      int pos = s_base[bin] + rank;
      for (int w = 0; w < wave; ++w) pos += s_cnt[w][bin];
      order[pos] = i;
    }
    __syncthreads();
    if (wave == 0 && lane < kBins) {
      int add = 0;
      for (int w = 0; w < kPlanWaves; ++w) add += s_cnt[w][lane];
      s_base[lane] += add;
    }
    __syncthreads();
  }

  // pass 3: items, in order; an exclusive scan of the partition counts
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int c0 = 0; c0 < num_seqs; c0 += kPlanThreads) {
    const int r = c0 + tid;
    const int s = r < num_seqs ? order[r] : -1;
    const int n = s >= 0 ? num_parts(snap[s], P) : 0;
    int incl = n;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int up = __shfl_up(incl, off, 64);
      if (lane >= off) incl += up;
    }
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    int start = s_carry + incl - n;
    for (int w = 0; w < wave; ++w) start += s_wsum[w];
    if (n > 0) {
      const int L = snap[s];
      const int ps = part_size(L, n, align);
      for (int j = 0; j < n; ++j) {
        const int t0 = j * ps;
        *reinterpret_cast<i32x4*>(items + 4 * (size_t)(start + j)) =
            i32x4{s, (j << 16) | n, t0, min(L, t0 + ps)};
      }
    }
    __syncthreads();
    if (tid == 0) {
      int add = 0;
      for (int w = 0; w < kPlanWaves; ++w) add += s_wsum[w];
      s_carry += add;
    }
    __syncthreads();
  }
  if (tid == 0) *count = s_carry;
}

hipError_t launch_plan_items(const int32_t* lens, int num_seqs, int len_cap, int part_tokens,
                             int part_align, int32_t* scratch, int32_t* items, int32_t* count,
                             hipStream_t st) {
  if (num_seqs <= kPlanLdsSeqs)
    hipLaunchKernelGGL(plan_items_kernel<true>, dim3(1), dim3(kPlanThreads), 0, st, lens,
                       num_seqs, len_cap, part_tokens, part_align, scratch, items, count);
  else
    hipLaunchKernelGGL(plan_items_kernel<false>, dim3(1), dim3(kPlanThreads), 0, st, lens,
                       num_seqs, len_cap, part_tokens, part_align, scratch, items, count);
  return hipGetLastError();
}

}  // namespace pkv
