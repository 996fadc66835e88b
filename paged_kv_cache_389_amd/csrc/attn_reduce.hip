// Merge of the partial softmax states of a split context.
//
// A partition p of one (sequence, query head) left its running max m_p (in
// log2 units), its running sum l_p and its unnormalised output o_p[HD], all
// fp32.  With M = max_p m_p and w_p = 2^(m_p - M) the result is
//   out = (sum_p w_p o_p) / (sum_p w_p l_p),
// the same value a single pass over the whole context gives (log-sum-exp
// merge).  The pages do not describe this step; it is the split-context
// reduce of a paged decode kernel for long contexts.
//
// A second kernel merges them: the states of one launch are visible to the
// next launch on the stream without any fence inside the decode kernel (a
// device-wide fence per partition costs far more than the launch).
//
// One wave per (sequence, query head), four per workgroup.  Lane j owns the
// weight of state c0 + j of the current chunk of 64 states.  The partial
// outputs are read as float4: one load instruction covers 64 / (HD/4)
// states side by side, so all of a chunk's loads are issued back to back,
// and the states held by different lane groups are summed with shuffles at
// the end.
#include "common.h"
#include "decode.h"

namespace pkv {

// Merge `n` partial states of one query head into out[HD]; state(j) gives
// the index of the j-th state in part_o / part_ml.  One wave.
template <typename E, int HD, typename StateOf>
__device__ inline void merge_states(const DecodeArgs& a, int n, StateOf state,
                                    typename E::storage* out) {
  constexpr int F4 = HD / 4;            // float4 per partial row
  constexpr int PPL = kWave / F4;       // states per load instruction (1, 2 or 4)
  static_assert(PPL >= 1 && PPL * F4 == kWave, "unsupported head_dim");
  const int lane = threadIdx.x % kWave;

  float M = -INFINITY;
  for (int p = lane; p < n; p += kWave) M = fmaxf(M, a.part_ml[2 * state(p)]);
  M = wave_max(M);

  const int d4 = lane % F4, psub = lane / F4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float Ls = 0.f;
  for (int c0 = 0; c0 < n; c0 += kWave) {
    const int nc = min(kWave, n - c0);
    float w = 0.f;
    if (lane < nc) {
      const f32x2 mlp = *reinterpret_cast<const f32x2*>(a.part_ml + 2 * state(c0 + lane));
      w = fast_exp2(mlp[0] - M);
      Ls = __builtin_fmaf(w, mlp[1], Ls);
    }
    constexpr int U = 8;   // load instructions in flight per step
    for (int j0 = 0; j0 < nc; j0 += U * PPL) {
      f32x4 v[U];
      float wv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * PPL + psub;
        wv[u] = __shfl(w, j < nc ? j : 0, 64);
        v[u] = j < nc ? *reinterpret_cast<const f32x4*>(a.part_o + state(c0 + j) * HD + 4 * d4)
                      : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * PPL + psub;
        if (j < nc) acc += wv[u] * v[u];
      }
    }
  }
  Ls = wave_sum(Ls);
#pragma unroll
  for (int off = F4; off < kWave; off <<= 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], off, 64);
  }
  if (psub == 0) {
    const float inv = 1.f / Ls;
    float r[4] = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    store_rounded<E, 4>(out + 4 * d4, r);
  }
}

// One wave per (sequence, query head), four per workgroup; contexts of one
// partition were written by the decode kernel.
template <typename E, int HD>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
  using T = typename E::storage;
  const int tid = threadIdx.x, wave = tid / kWave;
  const int h = blockIdx.x * 4 + wave, s = blockIdx.y;
  if (h >= a.num_q_heads) return;
  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int nparts = num_parts(L, a.part_tokens);
  if (nparts <= 1) return;
  const size_t base = ((size_t)s * a.num_q_heads + h) * a.max_parts;
  T* out = static_cast<T*>(a.out) + ((size_t)s * a.num_q_heads + h) * HD;
  merge_states<E, HD>(a, nparts, [&](int j) { return base + j; }, out);
}

template <typename E, int HD>
static hipError_t launch_reduce_t(const DecodeArgs& a, hipStream_t st) {
  dim3 grid((a.num_q_heads + 3) / 4, a.num_seqs);
  hipLaunchKernelGGL((decode_reduce_kernel<E, HD>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename E>
static hipError_t launch_reduce_e(int hd, const DecodeArgs& a, hipStream_t st) {
  switch (hd) {
    case 64: return launch_reduce_t<E, 64>(a, st);
    case 128: return launch_reduce_t<E, 128>(a, st);
    case 256: return launch_reduce_t<E, 256>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_reduce(Elem e, int hd, const DecodeArgs& a, hipStream_t st) {
  switch (e) {
    case Elem::F32: return launch_reduce_e<F32>(hd, a, st);
    case Elem::F16: return launch_reduce_e<F16>(hd, a, st);
    case Elem::BF16: return launch_reduce_e<BF16>(hd, a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
