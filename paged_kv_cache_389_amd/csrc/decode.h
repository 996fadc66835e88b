// Host/device interface of the paged decode kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// How the decode grid divides the work.
//  kGridPartitions: one workgroup per (partition, head unit, sequence); a
//    partition is part_tokens tokens; several partitions per sequence are
//    merged by the partition reduce.
//  kGridBalanced: a fixed number of workgroups (about the resident count),
//    each streaming an equal share of all tiles of all (head unit, sequence)
//    pairs laid end to end; a unit cut by a share boundary leaves partial
//    states in its workgroups' slots, merged by the balanced reduce.
enum GridMode { kGridPartitions = 0, kGridBalanced = 1 };

constexpr int kBalancedMaxSeqs = 1024;   // the in-kernel tile prefix holds 4 per thread

// Everything a decode launch needs.  Passed by value as the kernel argument.
struct DecodeArgs {
  void* out;                  // [B][Hq][HD] element type
  const void* q;              // [B][Hq][HD]
  const void* k_cache;        // [NB][Hkv][BS][HD]
  const void* v_cache;
  const int32_t* block_tables;  // [B][max_blocks]
  const int32_t* context_lens;  // [B]
  const int32_t* seq_order;   // [B] sequence of grid row z (longest first), or null
  int order_mode;             // 0: row z is sequence z; 1: read seq_order;
                              // 2: compute the longest-first order in the kernel
  // partial softmax states: partitions mode [B][Hq][max_parts], balanced mode
  // [2 * ranges][group]; o has HD floats per state, ml 2 (max in log2 units, sum)
  float* part_o;
  float* part_ml;
  int32_t* tile_start;        // balanced mode: [B + 1] tile prefix over sequences
  float scale_log2e;          // scale * log2(e): scores are kept in log2 units
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;                  // Hq / Hkv
  int num_blocks;
  int max_blocks;             // row stride of block_tables
  int len_cap;                // lengths are clamped to this (<= max_blocks*BS)
  int part_tokens;            // partitions mode: tokens per partition
  int max_parts;              // partitions mode: partitions the grid covers per sequence
  int contiguous;             // 1: ignore tables; block j of seq s is s*max_blocks + j
  int grid_mode;              // GridMode
  int ranges;                 // balanced mode: waves (a multiple of 32), one range each
  int unit_group;             // balanced mode: query heads per work unit (1 or group)
};

enum class Elem { F32 = 0, F16 = 1, BF16 = 2 };

// Sequence handled by grid row z when the order comes from memory (mode 1;
// an out-of-range entry falls back to z itself) or is the identity.
__device__ inline int sequence_of(const DecodeArgs& a, int z) {
  if (a.order_mode != 1) return z;
  const int s = a.seq_order[z];
  return (unsigned)s < (unsigned)a.num_seqs ? s : z;
}

// ---------------------------------------------------------- balanced mode
//
// Tiles of all work units laid end to end, sequence major: with U head units
// per sequence and nt_s = ceil(L_s / tile_tokens) tiles per unit, unit
// (s, hu) covers tiles [U*start[s] + hu*nt_s, U*start[s] + (hu+1)*nt_s) of
// T = U*Ts, where start[] is the prefix of nt over sequences and Ts =
// start[B].  Sequence-major keeps the heads of a sequence, and neighbouring
// sequences (which may share prompt blocks), in neighbouring ranges.  With R = min(ranges, T) ranges (so none is empty), range
// w covers [T*w/R, T*(w+1)/R).  A range leaves a partial state for its
// first unit when that unit began before the range (slot 2w) and for its
// last unit when that unit ends after it (slot 2w+1); a range that lies
// inside one unit leaves one state, in slot 2w.

__device__ inline int effective_ranges(int64_t T, int ranges) {
  return T < ranges ? (int)T : ranges;
}

__device__ inline int64_t range_begin(int64_t T, int w, int R) { return T * w / R; }

// The range holding tile r (0 <= r < T).
__device__ inline int range_of(int64_t r, int64_t T, int R) {
  return (int)(((r + 1) * R - 1) / T);
}

// Range handled by wave `wave` (of 4) of workgroup b (-1: none).  The
// dispatcher places workgroup b on XCD b % 8, so with all ranges in use
// (`ranges`, a multiple of 32) XCD x gets the contiguous ranges
// x*R/8 .. (x+1)*R/8 - 1 and neighbouring units (sequences that share
// blocks) share its L2.
__device__ inline int range_of_wave(int b, int wave, int R, int ranges) {
  if (R == ranges) {
    const int wgs = ranges / 4;
    return ((b % 8) * (wgs / 8) + b / 8) * 4 + wave;
  }
  const int w = b * 4 + wave;
  return w < R ? w : -1;
}

// Launchers (one translation unit each).  Return hipSuccess or the launch error.
hipError_t launch_decode_valu(Elem e, int head_dim, int block_size, const DecodeArgs& a,
                              hipStream_t stream);
hipError_t launch_decode_mfma(Elem e, int head_dim, int block_size, const DecodeArgs& a,
                              hipStream_t stream);
hipError_t launch_decode_reduce(Elem e, int head_dim, const DecodeArgs& a, hipStream_t stream);
bool decode_valu_supported(Elem e, int head_dim, int block_size);
// Tokens per unit of work of the vector-ALU kernel (a wave handles at most
// 64 units per pass); the MFMA kernel's unit is 16 tokens.
int valu_unit_tokens(Elem e, int head_dim, int block_size);
bool decode_mfma_supported(Elem e, int head_dim, int block_size);
// Workgroups of the balanced-mode kernel resident per compute unit (0 if
// the runtime cannot say).
int decode_valu_occupancy(Elem e, int head_dim, int block_size);
int decode_mfma_occupancy(Elem e, int head_dim, int block_size, int group);

// Writes order[0..num_seqs) = the sequence indices, longest context first
// (stable within half-octave length bins).
hipError_t launch_seq_order(const int32_t* lens, int num_seqs, int len_cap, int32_t* order,
                            hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                    int row_bytes, int block_size, int num_blocks,
                                    hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int num_pairs,
                              size_t block_bytes, int num_blocks, hipStream_t stream);

}  // namespace pkv
