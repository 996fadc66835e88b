// Host/device interface of the paged decode kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

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
  float* part_o;              // [B][Hq][max_parts][HD] unnormalised partial outputs
  float* part_ml;             // [B][Hq][max_parts][2]  (running max in log2 units, sum)
  float scale_log2e;          // scale * log2(e): scores are kept in log2 units
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;                  // Hq / Hkv
  int num_blocks;
  int max_blocks;             // row stride of block_tables
  int len_cap;                // lengths are clamped to this (<= max_blocks*BS, <= grid cover)
  int part_tokens;            // partition size in tokens (multiple of 32, at most
                              // 256 of the kernel's units)
  int max_parts;              // partitions per sequence the grid covers
  int contiguous;             // 1: ignore tables; block j of seq s is s*max_blocks + j
};

enum class Elem { F32 = 0, F16 = 1, BF16 = 2 };

// Sequence handled by grid row z when the order comes from memory (mode 1;
// an out-of-range entry falls back to z itself) or is the identity.
__device__ inline int sequence_of(const DecodeArgs& a, int z) {
  if (a.order_mode != 1) return z;
  const int s = a.seq_order[z];
  return (unsigned)s < (unsigned)a.num_seqs ? s : z;
}

// Launchers (one translation unit each).  Return hipSuccess or the launch error.
hipError_t launch_decode_valu(Elem e, int head_dim, int block_size, const DecodeArgs& a,
                              hipStream_t stream);
hipError_t launch_decode_mfma(Elem e, int head_dim, int block_size, const DecodeArgs& a,
                              hipStream_t stream);
hipError_t launch_decode_reduce(Elem e, int head_dim, const DecodeArgs& a, hipStream_t stream);
bool decode_valu_supported(Elem e, int head_dim, int block_size);
// Tokens per unit of work of the vector-ALU kernel (a wave handles at most
// 64 units per partition); the MFMA kernel's unit is 16 tokens.
int valu_unit_tokens(Elem e, int head_dim, int block_size);
bool decode_mfma_supported(Elem e, int head_dim, int block_size);

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
