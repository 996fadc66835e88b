// Paged decode attention, vector-ALU variant, and the partition reduce.
//
// One workgroup (4 waves) computes one query head of one sequence over one
// partition of its context.  The sequence's KV lives in fixed-size physical
// blocks reached through its block table ("Memory Optimization in LLM
// Serving with PagedAttention", section "How PagedAttention Works"); only the
// last block is partly filled, and its tail is masked by token index.
//
// Data movement: a (block, kv head) tile is block_size rows of head_dim
// contiguous elements.  A wave reads it with 16-byte loads, LPR lanes per row
// and 64/LPR rows per load instruction, so every load instruction covers
// whole rows and is fully coalesced.  Each lane keeps the 16 bytes of the
// query that match its columns; a row's dot product is LPR partial dot
// products (v_dot2 for 16-bit types) summed across the row with DPP.
//
// Softmax: every row group of a wave keeps its own online state (running
// max m in log2 units, running sum l, unnormalised output o) over the tokens
// it sees; the 4*RPI states of the workgroup are merged in LDS at the end.
// When the context is split into several partitions, each partition stores
// (m, l, o) in fp32 and a second kernel merges them (log-sum-exp rule).
#include "common.h"
#include "decode.h"

namespace pkv {

template <typename E, int HD, int BS>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
  using T = typename E::storage;
  constexpr int VEC = E::kVec;           // elements per 16-byte load
  constexpr int LPR = HD / VEC;          // lanes per token row
  constexpr int RPI = kWave / LPR;       // token rows per load instruction
  constexpr int TPL = BS / RPI;          // loads per block per lane (K, and again V)
  constexpr int CH = TPL < 8 ? TPL : 8;  // loads issued together (bounds registers)
  constexpr int NWAVES = 4;
  constexpr int NROWS = NWAVES * RPI;    // online-softmax states per workgroup
  static_assert(RPI * LPR == kWave && BS % RPI == 0 && TPL % CH == 0, "unsupported shape");

  const int part = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int row = lane / LPR, col = lane % LPR;

  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int P = a.part_tokens;
  const int tok_begin = part * P;
  T* out = static_cast<T*>(a.out) + ((size_t)s * a.num_q_heads + h) * HD;
  if (L == 0) {
    if (part == 0)
      for (int d = tid; d < HD; d += 256) out[d] = E::round(0.f);
    return;
  }
  if (tok_begin >= L) return;
  const int tok_end = min(L, tok_begin + P);
  const int nparts = (L + P - 1) / P;
  const int g = h / a.group;

  const T* qrow = static_cast<const T*>(a.q) + ((size_t)s * a.num_q_heads + h) * HD;
  const u32x4 qv = ld16(qrow + col * VEC);
  const T* kbase = static_cast<const T*>(a.k_cache) + (size_t)g * BS * HD + row * HD + col * VEC;
  const T* vbase = static_cast<const T*>(a.v_cache) + (size_t)g * BS * HD + row * HD + col * VEC;
  const size_t block_stride = (size_t)a.num_kv_heads * BS * HD;
  const int32_t* table = a.block_tables + (size_t)s * a.max_blocks;

  float m = -INFINITY, l = 0.f, o[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) o[e] = 0.f;
  int bad = 0;

  const int blk_end = (tok_end + BS - 1) / BS;
  for (int jb = tok_begin / BS + wave; jb < blk_end; jb += NWAVES) {
    const int phys = uniform(a.contiguous ? s * a.max_blocks + jb : table[jb]);
    if (phys < 0 || phys >= a.num_blocks) {
      bad = 1;
      continue;
    }
    const T* kt = kbase + (size_t)phys * block_stride;
    const T* vt = vbase + (size_t)phys * block_stride;
    const bool whole = (jb + 1) * BS <= tok_end;
#pragma unroll
    for (int c0 = 0; c0 < TPL; c0 += CH) {
      u32x4 kr[CH], vr[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) kr[i] = ld16(kt + (c0 + i) * RPI * HD);
#pragma unroll
      for (int i = 0; i < CH; ++i) vr[i] = ld16(vt + (c0 + i) * RPI * HD);
      float sc[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i)
        sc[i] = group_sum<LPR>(E::dot16(kr[i], qv, 0.f)) * a.scale_log2e;

      if (whole) {
        // every token of the block is inside the context
        float mb = sc[0];
#pragma unroll
        for (int i = 1; i < CH; ++i) mb = fmaxf(mb, sc[i]);
        const float mn = fmaxf(m, mb);
        const float corr = fast_exp2(m - mn);
        m = mn;
        l *= corr;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] *= corr;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          const float p = fast_exp2(sc[i] - mn);
          l += p;
          float vf[VEC];
          E::unpack16(vr[i], vf);
#pragma unroll
          for (int e = 0; e < VEC; ++e) o[e] = __builtin_fmaf(p, vf[e], o[e]);
        }
      } else {
        // last block: tokens at or past tok_end are masked by index, never
        // by arithmetic, so whatever those slots hold cannot reach the result
        const int t0 = jb * BS + c0 * RPI + row;
        float mb = -INFINITY;
#pragma unroll
        for (int i = 0; i < CH; ++i)
          if (t0 + i * RPI < tok_end) mb = fmaxf(mb, sc[i]);
        const float mn = fmaxf(m, mb);
        const float mu = (mn == -INFINITY) ? 0.f : mn;
        const float corr = fast_exp2(m - mu);
        m = mn;
        l *= corr;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] *= corr;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          if (t0 + i * RPI < tok_end) {
            const float p = fast_exp2(sc[i] - mu);
            l += p;
            float vf[VEC];
            E::unpack16(vr[i], vf);
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] = __builtin_fmaf(p, vf[e], o[e]);
          }
        }
      }
    }
  }

  // merge the workgroup's NROWS partial states
  __shared__ float sm_m[NROWS], sm_l[NROWS];
  __shared__ float sm_o[NROWS][HD];
  __shared__ int sm_bad[NWAVES];
  const int r = wave * RPI + row;
  if (col == 0) {
    sm_m[r] = m;
    sm_l[r] = l;
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) sm_o[r][col * VEC + e] = o[e];
  if (lane == 0) sm_bad[wave] = bad;
  __syncthreads();

  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < NROWS; ++i) M = fmaxf(M, sm_m[i]);
  int any_bad = 0;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) any_bad |= sm_bad[w];
  const size_t pidx = ((size_t)s * a.num_q_heads + h) * a.max_parts + part;
  for (int d = tid; d < HD; d += 256) {
    float Ls = 0.f, O = 0.f;
#pragma unroll
    for (int i = 0; i < NROWS; ++i) {
      const float w = fast_exp2(sm_m[i] - M);
      Ls = __builtin_fmaf(w, sm_l[i], Ls);
      O = __builtin_fmaf(w, sm_o[i][d], O);
    }
    if (any_bad) O = __builtin_nanf("");
    if (nparts == 1) {
      out[d] = E::round(O / Ls);
    } else {
      a.part_o[pidx * HD + d] = O;
      if (d == 0) {
        a.part_ml[2 * pidx] = M;
        a.part_ml[2 * pidx + 1] = Ls;
      }
    }
  }
}

// Merge the partitions of one (sequence, query head): with per-partition
// running max m_p (log2 units), sum l_p and unnormalised output o_p,
//   M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
template <typename E, int HD>
__global__ __launch_bounds__(HD) void decode_reduce_kernel(DecodeArgs a) {
  using T = typename E::storage;
  const int h = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;
  const size_t base = ((size_t)s * a.num_q_heads + h) * a.max_parts;
  const float* ml = a.part_ml + 2 * base;
  const float* po = a.part_o + base * HD + d;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ml[2 * p]);
  float Ls = 0.f, O = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float w = fast_exp2(ml[2 * p] - M);
    Ls = __builtin_fmaf(w, ml[2 * p + 1], Ls);
    O = __builtin_fmaf(w, po[(size_t)p * HD], O);
  }
  T* out = static_cast<T*>(a.out) + ((size_t)s * a.num_q_heads + h) * HD;
  out[d] = E::round(O / Ls);
}

// ------------------------------------------------------------------ dispatch

template <typename E, int HD, int BS>
static hipError_t launch_valu_t(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.max_parts, a.num_q_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_valu_kernel<E, HD, BS>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename E, int HD>
static hipError_t launch_valu_hd(int bs, const DecodeArgs& a, hipStream_t st) {
  switch (bs) {
    case 8: return launch_valu_t<E, HD, 8>(a, st);
    case 16: return launch_valu_t<E, HD, 16>(a, st);
    case 32: return launch_valu_t<E, HD, 32>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename E>
static hipError_t launch_valu_e(int hd, int bs, const DecodeArgs& a, hipStream_t st) {
  switch (hd) {
    case 64: return launch_valu_hd<E, 64>(bs, a, st);
    case 128: return launch_valu_hd<E, 128>(bs, a, st);
    case 256: return launch_valu_hd<E, 256>(bs, a, st);
  }
  return hipErrorInvalidValue;
}

bool decode_valu_supported(Elem e, int hd, int bs) {
  (void)e;
  return (hd == 64 || hd == 128 || hd == 256) && (bs == 8 || bs == 16 || bs == 32);
}

hipError_t launch_decode_valu(Elem e, int hd, int bs, const DecodeArgs& a, hipStream_t st) {
  switch (e) {
    case Elem::F32: return launch_valu_e<F32>(hd, bs, a, st);
    case Elem::F16: return launch_valu_e<F16>(hd, bs, a, st);
    case Elem::BF16: return launch_valu_e<BF16>(hd, bs, a, st);
  }
  return hipErrorInvalidValue;
}

template <typename E, int HD>
static hipError_t launch_reduce_t(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.num_q_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_reduce_kernel<E, HD>), grid, dim3(HD), 0, st, a);
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
