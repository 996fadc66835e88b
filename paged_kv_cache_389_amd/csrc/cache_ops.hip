// Cache writers: the slot scatter of new tokens and the whole-block copy of
// copy-on-write.  Both move bytes only, with 16-byte vector loads/stores.
#include "common.h"
#include "decode.h"

namespace pkv {

// One workgroup per new token.  Its K and V rows ([Hkv][HD] each) go to
// offset slot % BS of physical block slot / BS, for every KV head.  A
// negative slot is skipped (padding); a slot past the pool is skipped so a
// bad slot can never write out of bounds.
//
// Passage: new tokens fill the slots their blocks provide as generation
// proceeds ("Memory Optimization in LLM Serving with PagedAttention", section
// "How PagedAttention Works"); after copy-on-write they land in the copy
// (section "Advanced Capabilities: Memory Sharing with Copy-on-Write").
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v, u32x4* __restrict__ k_cache,
    u32x4* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, int num_kv_heads,
    int row_vecs, int block_size, int64_t num_slots) {
  const int token = blockIdx.x;
  const int64_t slot = slot_mapping[token];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / block_size;
  const int off = (int)(slot % block_size);
  const int per_token = num_kv_heads * row_vecs;
  const u32x4* ks = k + (size_t)token * per_token;
  const u32x4* vs = v + (size_t)token * per_token;
  for (int i = threadIdx.x; i < per_token; i += blockDim.x) {
    const int g = i / row_vecs, c = i % row_vecs;
    const size_t dst = (((size_t)blk * num_kv_heads + g) * block_size + off) * row_vecs + c;
    k_cache[dst] = ks[i];
    v_cache[dst] = vs[i];
  }
}

// The quantising variant for an 8-bit cache: one workgroup per new token;
// each thread turns 16 source elements (type E) of the token's K or V rows
// into 16 E4M3 codes of x / scale (E4M3::encode4: float32 quotient,
// saturated, nearest even) and stores them with one 16-byte store.  Slots
// are handled as above.  Quantising the cache is named among the memory
// features of serving libraries ("Memory Optimization ...", section "Broader
// Context"); the format, the per-cache scales and the rounding are readings.
template <typename E>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const typename E::storage* __restrict__ k, const typename E::storage* __restrict__ v,
    u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache,
    const int64_t* __restrict__ slot_mapping, int num_kv_heads, int row_vecs, int block_size,
    int64_t num_slots, float k_scale, float v_scale) {
  using T = typename E::storage;
  const int token = blockIdx.x;
  const int64_t slot = slot_mapping[token];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / block_size;
  const int off = (int)(slot % block_size);
  const int per_token = num_kv_heads * row_vecs;   // 16-code vectors per token and cache
  for (int i = threadIdx.x; i < 2 * per_token; i += blockDim.x) {
    const bool is_v = i >= per_token;
    const int j = is_v ? i - per_token : i;
    const int g = j / row_vecs, c = j % row_vecs;
    const T* src = (is_v ? v : k) + ((size_t)token * per_token + j) * 16;
    const float scale = is_v ? v_scale : k_scale;
    float x[16];
    if constexpr (sizeof(T) == 4) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32x4 r = ld16(src + 4 * w);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * w + e] = __uint_as_float(r[e]);
      }
    } else {
#pragma unroll
      for (int w = 0; w < 2; ++w) E::unpack16(ld16(src + 8 * w), x + 8 * w);
    }
    u32x4 codes;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      codes[w] = E4M3::encode4(x[4 * w], x[4 * w + 1], x[4 * w + 2], x[4 * w + 3], scale);
    const size_t dst = (((size_t)blk * num_kv_heads + g) * block_size + off) * row_vecs + c;
    (is_v ? v_cache : k_cache)[dst] = codes;
  }
}

// Grid (chunks, 2, pairs): y selects the K or the V pool; each workgroup
// copies one chunk of 256 threads x 4 vectors (16 KiB) of one block from
// block src of the source pools to block dst of the destination pools.
// Pairs naming a block outside its pool are skipped.
//
// Passages: copy-on-write copies the shared block's content into a new block
// ("Memory Optimization ...", section "Advanced Capabilities: Memory Sharing
// with Copy-on-Write"); one block is copied, not the whole cache ("vLLM and
// PagedAttention ...", paragraph on sharing).  The engine evicts whole
// sequences by swapping their blocks to CPU memory (same page, paragraph on
// the engine): the same copy between a device pool and a pool in pinned
// host memory, which the kernel reads or writes directly over the host link.
constexpr int kCopyUnroll = 4;
__global__ __launch_bounds__(256) void copy_blocks_kernel(u32x4* dst_k, u32x4* dst_v,
                                                          const u32x4* src_k, const u32x4* src_v,
                                                          const int64_t* __restrict__ pairs,
                                                          int64_t block_vecs, int num_src,
                                                          int num_dst) {
  const int64_t src = pairs[2 * (size_t)blockIdx.z];
  const int64_t dst = pairs[2 * (size_t)blockIdx.z + 1];
  if (src < 0 || src >= num_src || dst < 0 || dst >= num_dst) return;
  const u32x4* from = (blockIdx.y == 0 ? src_k : src_v) + src * block_vecs;
  u32x4* to = (blockIdx.y == 0 ? dst_k : dst_v) + dst * block_vecs;
  const int64_t base = (int64_t)blockIdx.x * 256 * kCopyUnroll + threadIdx.x;
  u32x4 buf[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * 256;
    if (i < block_vecs) buf[u] = from[i];
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * 256;
    if (i < block_vecs) to[i] = buf[u];
  }
}

hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                    int row_bytes, int block_size, int num_blocks,
                                    hipStream_t st) {
  const int row_vecs = row_bytes / 16;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(num_tokens), dim3(256), 0, st,
                     static_cast<const u32x4*>(k), static_cast<const u32x4*>(v),
                     static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache), slot_mapping,
                     num_kv_heads, row_vecs, block_size, (int64_t)num_blocks * block_size);
  return hipGetLastError();
}

template <typename E>
static hipError_t launch_rc_fp8_t(const void* k, const void* v, void* k_cache, void* v_cache,
                                  const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                  int head_dim, int block_size, int num_blocks, float k_scale,
                                  float v_scale, hipStream_t st) {
  using T = typename E::storage;
  hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<E>, dim3(num_tokens), dim3(256), 0, st,
                     static_cast<const T*>(k), static_cast<const T*>(v),
                     static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache), slot_mapping,
                     num_kv_heads, head_dim / 16, block_size, (int64_t)num_blocks * block_size,
                     k_scale, v_scale);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache_fp8(Elem e, const void* k, const void* v, void* k_cache,
                                        void* v_cache, const int64_t* slot_mapping,
                                        int num_tokens, int num_kv_heads, int head_dim,
                                        int block_size, int num_blocks, float k_scale,
                                        float v_scale, hipStream_t st) {
  switch (e) {
    case Elem::F32:
      return launch_rc_fp8_t<F32>(k, v, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads,
                                  head_dim, block_size, num_blocks, k_scale, v_scale, st);
    case Elem::F16:
      return launch_rc_fp8_t<F16>(k, v, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads,
                                  head_dim, block_size, num_blocks, k_scale, v_scale, st);
    case Elem::BF16:
      return launch_rc_fp8_t<BF16>(k, v, k_cache, v_cache, slot_mapping, num_tokens,
                                   num_kv_heads, head_dim, block_size, num_blocks, k_scale,
                                   v_scale, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_copy_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                              const int64_t* pairs, int num_pairs, size_t block_bytes, int num_src,
                              int num_dst, hipStream_t st) {
  const int64_t block_vecs = (int64_t)(block_bytes / 16);
  const int64_t per_wg = 256 * kCopyUnroll;
  dim3 grid((unsigned)((block_vecs + per_wg - 1) / per_wg), 2, (unsigned)num_pairs);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, st, static_cast<u32x4*>(dst_k),
                     static_cast<u32x4*>(dst_v), static_cast<const u32x4*>(src_k),
                     static_cast<const u32x4*>(src_v), pairs, block_vecs, num_src, num_dst);
  return hipGetLastError();
}

}  // namespace pkv
