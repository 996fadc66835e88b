// Longest-first order of the sequences of a decode batch.
//
// The decode grid gives each (sequence, head, partition) its own workgroup,
// and the hardware starts workgroups in index order.  With context lengths
// that vary a lot, a long sequence that happens to have a high index starts
// late and finishes alone.  This kernel writes a permutation of the
// sequence indices, longest first, that the decode kernels read their
// sequence index through (list scheduling, longest job first).
//
// Lengths are binned by half octaves below the batch's length bound
// (bin b holds lengths in (cap * 2^-(b+1)/2, cap * 2^-b/2], 32 bins), and
// the sort is stable within a bin, so sequences of similar length keep
// their original order and neighbours that share cached blocks stay
// neighbours.  One workgroup of 1024 threads handles any batch size in
// chunks of 1024 with two passes: the first counts each bin with ballots,
// the second ranks every lane inside its bin (ballot of the lanes below it
// plus the counts of the waves before it) and turns the rank into a
// position.
#include "common.h"
#include "decode.h"
#include "order.h"

namespace pkv {

constexpr int kOrderThreads = 1024;
constexpr int kOrderWaves = kOrderThreads / kWave;

__global__ __launch_bounds__(kOrderThreads) void seq_order_kernel(const int32_t* __restrict__ lens,
                                                                  int num_seqs, int len_cap,
                                                                  int32_t* __restrict__ order) {
  __shared__ int s_cnt[kOrderWaves][kBins];
  __shared__ int s_base[kBins];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int cap = len_cap > 0 ? len_cap : 1;

  // pass 1: lane b of each wave counts bin b over every chunk
  int mine = 0;
  for (int c0 = 0; c0 < num_seqs; c0 += kOrderThreads) {
    const int i = c0 + tid;
    const int bin = i < num_seqs ? length_bin(min(lens[i], cap), cap) : -1;
#pragma unroll
    for (int b = 0; b < kBins; ++b) {
      const int n = __popcll(__ballot(bin == b));
      if (lane == b) mine += n;
    }
  }
  if (lane < kBins) s_cnt[wave][lane] = mine;
  __syncthreads();
  if (wave == 0) {
    // bin totals, then their exclusive prefix sum across lanes (bin 0 first)
    int total = 0;
    if (lane < kBins)
      for (int w = 0; w < kOrderWaves; ++w) total += s_cnt[w][lane];
    int incl = total;
#pragma unroll
    for (int off = 1; off < kBins; off <<= 1) {
      const int up = __shfl_up(incl, off, 64);
      if (lane >= off) incl += up;
    }
    if (lane < kBins) s_base[lane] = incl - total;
  }
  __syncthreads();

  // pass 2: positions, chunk by chunk
  for (int c0 = 0; c0 < num_seqs; c0 += kOrderThreads) {
    const int i = c0 + tid;
    const bool valid = i < num_seqs;
    const int bin = valid ? length_bin(min(lens[i], cap), cap) : -1;
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
      // lengths changed between the two passes (a racing writer) could push a
      // position out of range; never write outside the array
      if (pos < num_seqs) order[pos] = i;
    }
    __syncthreads();
    if (wave == 0 && lane < kBins) {
      int add = 0;
      for (int w = 0; w < kOrderWaves; ++w) add += s_cnt[w][lane];
      s_base[lane] += add;
    }
    __syncthreads();
  }
}

hipError_t launch_seq_order(const int32_t* lens, int num_seqs, int len_cap, int32_t* order,
                            hipStream_t st) {
  hipLaunchKernelGGL(seq_order_kernel, dim3(1), dim3(kOrderThreads), 0, st, lens, num_seqs,
                     len_cap, order);
  return hipGetLastError();
}

}  // namespace pkv
