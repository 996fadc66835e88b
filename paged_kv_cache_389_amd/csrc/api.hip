// C ABI of libpagedkv.so: argument validation, the split heuristic and
// kernel dispatch.  See include/pagedkv.h for the contract of every call.
#include <stdlib.h>

#include <string>

#include "decode.h"
#include "pagedkv.h"

using namespace pkv;

namespace {

thread_local std::string g_last_error;

constexpr int kMinPartition = 32;       // tokens; keeps partitions tile aligned
constexpr int kDefaultPartition = 512;  // tokens per workgroup on long contexts
constexpr int kMaxGridYZ = 65535;

int elem_size(pkv_dtype d) { return d == PKV_F32 ? 4 : 2; }
bool dtype_ok(int d) { return d == PKV_F32 || d == PKV_F16 || d == PKV_BF16; }
Elem to_elem(pkv_dtype d) {
  return d == PKV_F32 ? Elem::F32 : (d == PKV_F16 ? Elem::F16 : Elem::BF16);
}

int fail_hip(hipError_t e) {
  g_last_error = hipGetErrorString(e);
  return PKV_EHIP;
}

int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Tokens per partition.  Short contexts run as one partition (no reduce);
// longer ones are cut into fixed-size pieces so that very uneven lengths
// still spread evenly over the 256 compute units.
int partition_tokens(int max_context_len, int block_size, int requested) {
  const int unit = block_size > kMinPartition ? block_size : kMinPartition;
  if (requested > 0) return requested;
  if (max_context_len <= kDefaultPartition) return round_up(max_context_len > 0 ? max_context_len : 1, unit);
  return round_up(kDefaultPartition, unit);
}

bool partition_ok(int p, int block_size) {
  return p >= kMinPartition && p % kMinPartition == 0 && p % block_size == 0;
}

size_t workspace_for(int num_seqs, int num_q_heads, int head_dim, int max_parts) {
  if (max_parts <= 1) return 0;
  return (size_t)num_seqs * num_q_heads * max_parts * (size_t)(head_dim + 2) * sizeof(float);
}

}  // namespace

extern "C" {

const char* pkv_version(void) { return "pagedkv 0.1.0 gfx950"; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_EUNSUPPORTED: return "unsupported shape or dtype";
    case PKV_EWORKSPACE: return "workspace missing or too small";
    case PKV_EHIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* pkv_last_error(void) { return g_last_error.c_str(); }

int pkv_supported(pkv_dtype dtype, int head_dim, int block_size) {
  if (!dtype_ok(dtype)) return 0;
  return decode_valu_supported(to_elem(dtype), head_dim, block_size) ? 1 : 0;
}

size_t pkv_paged_attention_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                           int head_dim, int block_size, int max_context_len,
                                           int partition) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_context_len < 0 || partition < 0)
    return (size_t)-1;
  const int p = partition_tokens(max_context_len, block_size, partition);
  if (!partition_ok(p, block_size)) return (size_t)-1;
  const int max_parts = (max_context_len + p - 1) / p;
  return workspace_for(num_seqs, num_q_heads, head_dim, max_parts);
}

int pkv_paged_attention_decode_ex(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, float scale, int num_seqs,
                                  int num_q_heads, int num_kv_heads, int head_dim,
                                  int block_size, int num_blocks, int max_blocks_per_seq,
                                  int max_context_len, pkv_dtype dtype, void* workspace,
                                  size_t workspace_bytes, int partition, int path,
                                  void* stream) {
  if (!dtype_ok(dtype) || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      max_context_len < 0 || partition < 0 || path < PKV_PATH_AUTO || path > PKV_PATH_CONTIGUOUS)
    return PKV_EINVAL;
  if (num_q_heads % num_kv_heads) return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  const bool contiguous = path == PKV_PATH_CONTIGUOUS;
  if (!out || !q || !k_cache || !v_cache || !context_lens || (!block_tables && !contiguous))
    return PKV_EINVAL;
  if (num_seqs > kMaxGridYZ || num_q_heads > kMaxGridYZ) return PKV_EUNSUPPORTED;
  if (contiguous && (int64_t)num_seqs * max_blocks_per_seq > num_blocks) return PKV_EINVAL;

  const Elem e = to_elem(dtype);
  const int group = num_q_heads / num_kv_heads;
  const bool mfma_ok = group >= 2 && group <= 16 && decode_mfma_supported(e, head_dim, block_size);
  bool use_mfma;
  if (path == PKV_PATH_MFMA) {
    if (!mfma_ok) return PKV_EUNSUPPORTED;
    use_mfma = true;
  } else if (path == PKV_PATH_VALU) {
    use_mfma = false;
  } else {
    use_mfma = mfma_ok;
  }
  if (!decode_valu_supported(e, head_dim, block_size)) return PKV_EUNSUPPORTED;

  const int p = partition_tokens(max_context_len, block_size, partition);
  if (!partition_ok(p, block_size)) return PKV_EINVAL;
  const int64_t table_cap = (int64_t)max_blocks_per_seq * block_size;
  const int len_cap = (int)(table_cap < max_context_len ? table_cap : max_context_len);
  const int max_parts = len_cap > 0 ? (len_cap + p - 1) / p : 1;
  const size_t need = workspace_for(num_seqs, num_q_heads, head_dim, max_parts);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_EWORKSPACE;

  DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.part_ml = static_cast<float*>(workspace);
  a.part_o = need ? static_cast<float*>(workspace) + (size_t)num_seqs * num_q_heads * max_parts * 2
                  : nullptr;
  a.scale_log2e = (float)((double)scale * 1.4426950408889634);
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.len_cap = len_cap;
  a.part_tokens = p;
  a.max_parts = max_parts;
  a.contiguous = contiguous ? 1 : 0;

  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err = use_mfma ? launch_decode_mfma(e, head_dim, block_size, a, st)
                            : launch_decode_valu(e, head_dim, block_size, a, st);
  if (err != hipSuccess) return fail_hip(err);
  if (max_parts > 1) {
    err = launch_decode_reduce(e, head_dim, a, st);
    if (err != hipSuccess) return fail_hip(err);
  }
  return PKV_OK;
}

int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               float scale, int num_seqs, int num_q_heads, int num_kv_heads,
                               int head_dim, int block_size, int num_blocks,
                               int max_blocks_per_seq, int max_context_len, pkv_dtype dtype,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return pkv_paged_attention_decode_ex(out, q, k_cache, v_cache, block_tables, context_lens,
                                       scale, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                       block_size, num_blocks, max_blocks_per_seq,
                                       max_context_len, dtype, workspace, workspace_bytes, 0,
                                       PKV_PATH_AUTO, stream);
}

int pkv_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                          const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                          int head_dim, int block_size, int num_blocks, pkv_dtype dtype,
                          void* stream) {
  if (!dtype_ok(dtype) || num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_blocks <= 0)
    return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PKV_EINVAL;
  const int row_bytes = head_dim * elem_size(dtype);
  if (row_bytes % 16) return PKV_EUNSUPPORTED;
  hipError_t err = launch_reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, num_tokens,
                                            num_kv_heads, row_bytes, block_size, num_blocks,
                                            static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PKV_OK : fail_hip(err);
}

int pkv_copy_blocks(void* k_cache, void* v_cache, const int64_t* src_dst_pairs, int num_pairs,
                    int num_kv_heads, int head_dim, int block_size, int num_blocks,
                    pkv_dtype dtype, void* stream) {
  if (!dtype_ok(dtype) || num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_blocks <= 0)
    return PKV_EINVAL;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src_dst_pairs) return PKV_EINVAL;
  const size_t block_bytes = (size_t)num_kv_heads * block_size * head_dim * elem_size(dtype);
  if (block_bytes % 16) return PKV_EUNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int first = 0; first < num_pairs; first += kMaxGridYZ) {
    const int n = num_pairs - first < kMaxGridYZ ? num_pairs - first : kMaxGridYZ;
    hipError_t err = launch_copy_blocks(k_cache, v_cache, src_dst_pairs + 2 * (size_t)first, n,
                                        block_bytes, num_blocks, st);
    if (err != hipSuccess) return fail_hip(err);
  }
  return PKV_OK;
}

}  // extern "C"
