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
  float* part_ml;             // [B][Hq][max_parts][2]  (running max in log2 units, sum)
  float* part_o;              // [B][Hq][max_parts][HD] unnormalised partial outputs
  float scale_log2e;          // scale * log2(e): scores are kept in log2 units
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;                  // Hq / Hkv
  int num_blocks;
  int max_blocks;             // row stride of block_tables
  int len_cap;                // lengths are clamped to this (<= max_blocks*BS, <= grid cover)
  int part_tokens;            // partition size in tokens (multiple of 32)
  int max_parts;              // partitions per sequence the grid covers
  int contiguous;             // 1: ignore tables; block j of seq s is s*max_blocks + j
};

enum class Elem { F32 = 0, F16 = 1, BF16 = 2 };

// Launchers (one translation unit each).  Return hipSuccess or the launch error.
hipError_t launch_decode_valu(Elem e, int head_dim, int block_size, const DecodeArgs& a,
                              hipStream_t stream);
hipError_t launch_decode_mfma(Elem e, int head_dim, int block_size, const DecodeArgs& a,
                              hipStream_t stream);
hipError_t launch_decode_reduce(Elem e, int head_dim, const DecodeArgs& a, hipStream_t stream);
bool decode_valu_supported(Elem e, int head_dim, int block_size);
bool decode_mfma_supported(Elem e, int head_dim, int block_size);

hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                    int row_bytes, int block_size, int num_blocks,
                                    hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int num_pairs,
                              size_t block_bytes, int num_blocks, hipStream_t stream);

}  // namespace pkv
