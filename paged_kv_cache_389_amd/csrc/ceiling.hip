// Reference read kernels: what a plain read reaches on this part, reported
// beside the HBM3E peak so that the paged kernels can be judged against the
// memory system's practical limit as well as against the data sheet.
//
// * stream_read: one contiguous range, 16-byte loads, eight in flight per
//   lane, grid-stride over the range.
// * gather_read: chunks of 2, 4 or 8 KiB (the size of one 16-token K or V
//   tile of a paged cache) at the positions a list of chunk indices names,
//   read the way the decode kernels read tiles: each wave takes a contiguous
//   run of the list, fetches 64 indices with one vector load, and keeps
//   about 16 KiB of chunk loads in flight in a rolling register pipeline,
//   each chunk through a buffer descriptor built in scalar registers; the
//   chunk may be read in a second pool too (K and V tiles of one block), and
//   the loads may stream (nontemporal, as the decode kernels' K/V loads) or
//   keep the cache's default policy.
//
// Both fold what they read into one XOR per wave (an atomic on `sink`), so
// no load can be dropped.  Neither belongs to the attention path.
#include "common.h"
#include "pagedkv.h"

namespace pkv {
namespace {

__device__ inline uint32_t fold(u32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

__device__ inline void flush_sink(uint32_t acc, uint32_t* sink) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if (threadIdx.x % kWave == 0) atomicXor(sink, acc);
}

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src,
                                                          size_t n16, uint32_t* sink) {
  constexpr int U = 8;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= fold(v[u]);
  }
  for (; i < n16; i += stride) acc ^= fold(src[i]);
  flush_sink(acc, sink);
}

// Wave w reads list entries [w * per_wave, min(n, (w + 1) * per_wave)),
// U chunks in flight: the loads of chunk i + U - 1 are issued before chunk i
// is folded (chunks past the run get an empty descriptor and read zeros).
// With TWO the chunk's index is read in both pools (the K and V tiles of one
// block); POL is the loads' cache policy (kStream or 0).
template <int CB, int U, bool TWO, int POL>
__global__ __launch_bounds__(256) void gather_read_kernel(const char* __restrict__ pool,
                                                          const char* __restrict__ pool2,
                                                          int pool_chunks,
                                                          const int32_t* __restrict__ chunks,
                                                          int num_chunks, int per_wave,
                                                          uint32_t* sink) {
  constexpr int L = CB / 1024;   // 16-byte loads per lane per chunk and pool
  constexpr int NP = TWO ? 2 : 1;
  const int lane = threadIdx.x % kWave;
  const int wave = uniform((int)(blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave));
  const int64_t first = (int64_t)wave * per_wave;
  const int64_t last = first + per_wave < num_chunks ? first + per_wave : num_chunks;
  uint32_t acc = 0;
  for (int64_t pass = first; pass < last; pass += kWave) {
    const int mine = (int)(last - pass < kWave ? last - pass : kWave);
    const int idx_v = lane < mine ? chunks[pass + lane] : 0;
    auto issue = [&](int i, u32x4* v) {
      int c = lane_value(idx_v, i < kWave ? i : kWave - 1);
      const bool live = i < mine && (unsigned)c < (unsigned)pool_chunks;
      if (!live) c = 0;
      const rsrc_t r = make_rsrc(pool + (size_t)c * CB, live ? CB : 0u);
#pragma unroll
      for (int j = 0; j < L; ++j) v[j] = bld16<POL>(r, lane * 16u, j * 1024u);
      if constexpr (TWO) {
        const rsrc_t r2 = make_rsrc(pool2 + (size_t)c * CB, live ? CB : 0u);
#pragma unroll
        for (int j = 0; j < L; ++j) v[L + j] = bld16<POL>(r2, lane * 16u, j * 1024u);
      }
    };
    u32x4 v[U][NP * L];
#pragma unroll
    for (int j = 0; j < U - 1; ++j) issue(j, v[j]);
    for (int i0 = 0; i0 < mine; i0 += U) {
#pragma unroll
      for (int j = 0; j < U; ++j) {
        issue(i0 + j + U - 1, v[(j + U - 1) % U]);
#pragma unroll
        for (int k = 0; k < NP * L; ++k) acc ^= fold(v[j][k]);
      }
    }
  }
  flush_sink(acc, sink);
}

template <int CB, int U>
void launch_gather(bool two, bool cached, int wgs, hipStream_t st, const char* p, const char* p2,
                   int pc, const int32_t* chunks, int n, int per_wave, uint32_t* sink) {
  if (two && cached)
    hipLaunchKernelGGL((gather_read_kernel<CB, U, true, 0>), dim3(wgs), dim3(256), 0, st, p, p2,
                       pc, chunks, n, per_wave, sink);
  else if (two)
    hipLaunchKernelGGL((gather_read_kernel<CB, U, true, kStream>), dim3(wgs), dim3(256), 0, st, p,
                       p2, pc, chunks, n, per_wave, sink);
  else if (cached)
    hipLaunchKernelGGL((gather_read_kernel<CB, U, false, 0>), dim3(wgs), dim3(256), 0, st, p, p2,
                       pc, chunks, n, per_wave, sink);
  else
    hipLaunchKernelGGL((gather_read_kernel<CB, U, false, kStream>), dim3(wgs), dim3(256), 0, st, p,
                       p2, pc, chunks, n, per_wave, sink);
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" {

int pkv_ceiling_stream_read(const void* src, size_t bytes, int workgroups, uint32_t* sink,
                            void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 || workgroups <= 0 ||
      reinterpret_cast<uintptr_t>(src) % 16)
    return PKV_EINVAL;
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), bytes / 16,
                     sink);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

int pkv_ceiling_gather_read(const void* pool, const void* pool2, size_t pool_bytes,
                            const int32_t* chunks, int num_chunks, int chunk_bytes, int cached,
                            int workgroups, uint32_t* sink, void* stream) {
  if (!pool || !chunks || !sink || num_chunks <= 0 || workgroups <= 0 ||
      (chunk_bytes != 2048 && chunk_bytes != 4096 && chunk_bytes != 8192) ||
      pool_bytes < (size_t)chunk_bytes || (cached != 0 && cached != 1))
    return PKV_EINVAL;
  const size_t pc = pool_bytes / (size_t)chunk_bytes;
  const int pool_chunks = pc > (size_t)INT32_MAX ? INT32_MAX : (int)pc;
  const int64_t waves = (int64_t)workgroups * 4;
  const int per_wave = (int)((num_chunks + waves - 1) / waves);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const char* p = static_cast<const char*>(pool);
  const char* p2 = static_cast<const char*>(pool2);
  const bool two = pool2 != nullptr;
  switch (chunk_bytes) {
    case 2048:
      launch_gather<2048, 9>(two, cached, workgroups, st, p, p2, pool_chunks, chunks, num_chunks,
                             per_wave, sink);
      break;
    case 4096:
      launch_gather<4096, 5>(two, cached, workgroups, st, p, p2, pool_chunks, chunks, num_chunks,
                             per_wave, sink);
      break;
    default:
      launch_gather<8192, 3>(two, cached, workgroups, st, p, p2, pool_chunks, chunks, num_chunks,
                             per_wave, sink);
      break;
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

}  // extern "C"
