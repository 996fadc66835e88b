// Balanced-mode prologue shared by the decode kernels: the tile prefix over
// the batch's sequences, computed in LDS by every workgroup.
#pragma once

#include "common.h"
#include "decode.h"

namespace pkv {

struct TilePrefix {
  int start[kBalancedMaxSeqs + 1];
  int wave_total[4];
};

// start[s] = sum over s' < s of ceil(L_s' / tt) (L clamped to [0, len_cap]),
// for s = 0 .. B, by a 256-thread workgroup (4 sequences per thread, a wave
// scan, then the wave totals).  Workgroup 0 also stores it to a.tile_start
// for the reduce.  The host guarantees B <= kBalancedMaxSeqs and that the
// total fits an int.
__device__ inline void tile_prefix(const DecodeArgs& a, int tt, TilePrefix& sm) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int B = a.num_seqs;
  int v[4], sum = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = tid * 4 + k;
    int L = i < B ? a.context_lens[i] : 0;
    L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
    v[k] = (L + tt - 1) / tt;
    sum += v[k];
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int up = __shfl_up(incl, off, 64);
    if (lane >= off) incl += up;
  }
  if (lane == kWave - 1) sm.wave_total[wave] = incl;
  __syncthreads();
  int run = incl - sum;
  for (int w = 0; w < wave; ++w) run += sm.wave_total[w];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = tid * 4 + k;
    if (i < B) sm.start[i] = run;
    run += v[k];
  }
  if (tid == 0) sm.start[B] = sm.wave_total[0] + sm.wave_total[1] + sm.wave_total[2] +
                              sm.wave_total[3];
  __syncthreads();
  if (blockIdx.x == 0)
    for (int i = tid; i <= B; i += 256) a.tile_start[i] = sm.start[i];
}

// The sequence owning tile `off` of a head unit (0 <= off < start[B]): the
// last s with start[s] <= off, which has at least one tile.
__device__ inline int seq_of_tile(const TilePrefix& sm, int B, int off) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (sm.start[mid] <= off)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// One piece of a range: tiles [ta, tb) of head unit hu of sequence s; the
// piece is the whole unit when whole is set, else it is written to `slot`.
struct Piece {
  int s, hu, ta, tb;
  bool whole;
  int slot;
};

// Walks the pieces of range w (tiles [r0, r1)) of the sequence-major
// layout with U head units per sequence; call next() until it returns false.
struct RangeWalk {
  int64_t r, r1, r0;
  int U, B, w;
  __device__ inline bool next(const TilePrefix& sm, Piece& p) {
    if (r >= r1) return false;
    const int s = seq_of_tile(sm, B, (int)(r / U));
    const int nt = sm.start[s + 1] - sm.start[s];
    const int64_t base = (int64_t)U * sm.start[s];
    const int hu = (int)((r - base) / nt);
    const int64_t S = base + (int64_t)hu * nt;
    const int64_t E = S + nt;
    const int64_t e = E < r1 ? E : r1;
    p.s = s;
    p.hu = hu;
    p.ta = (int)(r - S);
    p.tb = (int)(e - S);
    p.whole = (r == S) && (e == E);
    p.slot = 2 * w + (r == r0 ? 0 : 1);
    r = e;
    return true;
  }
};

}  // namespace pkv
