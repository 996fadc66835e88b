// Paged prefill attention: many query tokens per sequence, causal, on the
// matrix cores.
//
// Sequence s has L cached tokens (its new ones included, written by
// reshape_and_cache beforehand) and n query tokens, its last n positions:
// query i sits at position L - n + i and attends to positions 0 .. L - n + i,
// read through the sequence's block table.  This is the attention a
// recomputation of evicted sequences runs ("vLLM and PagedAttention: How
// Ideas from Operating Systems Accelerated LLM Inference", paragraph on the
// engine: eviction by swapping or recomputation); the pages print no
// formula, and the causal reading above is the plainest one.
//
// A wave owns kPrefillGroups groups of 16 query columns, each 16/G query
// tokens times the G query heads of one KV head; every K/V tile it loads
// serves all its groups.  Against a 16-token tile of keys a group forms the same
// contraction as grouped decode (S^T = K Q^T, 16x16x32 MFMAs; O^T += V^T P^T,
// 16x16x16), so the operand layouts are those of the decode MFMA kernel; the
// only new element is a causal bound per column: column c sees tokens below
// limit_c, masked by index in the tiles that reach past the wave's smallest
// bound.  Each wave streams its own tiles 0 .. ceil(max limit / 16) with the
// table entries of 64 tiles fetched by one vector load and the next tile's
// loads in flight while the current one is computed; the four waves of a
// workgroup take consecutive query tokens of one (sequence, KV head), so
// their tiles overlap and mostly hit in the caches.  No cross-wave merge is
// needed: a wave owns its columns' whole context.
#include "common.h"
#include "decode.h"
#include "mfma_ops.h"

namespace pkv {

constexpr int kPrefillStages = 2;
// Probabilities enter the PV product rounded to the input type once (no
// bf16 head + remainder split as in decode, which doubles the PV work of
// this compute-heavy kernel).
constexpr bool kPrefillSplitP = false;
// How far (log2 units) a tile's maximum may pass the reference maximum
// before the accumulators are rescaled: probabilities stay below 2^8.
constexpr float kPrefillSlack = 8.f;

// Column groups of 16 per wave: each K/V tile a wave loads serves CG groups.
constexpr int kPrefillGroups = 4;

template <int HD, int CG>
struct PrefillShared {
  u32x4 q[4][CG][HD / 32][kWave];   // per wave and column group: Q^T in the B layout
};

// C is the cache element: E itself, or E4M3 codes, loaded at half the width
// (16 codes of a K row per load, feeding two k-steps; V rows at half width)
// and widened to E right before the products, as in the decode MFMA kernel;
// the K scale is folded into scale_log2e and the V scale multiplies the output.
template <typename E, typename C, int HD, int BS, int CG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_mfma_kernel(
    PrefillArgs a) {
  using TQ = typename E::storage;   // query and output
  using T = typename C::storage;    // cache element
  using Ops = MfmaOps<E>;
  constexpr bool k8 = sizeof(T) == 1;
  constexpr int KSTEPS = HD / 32;
  constexpr int DPL = HD / 16;
  constexpr int VW = DPL / 2;
  constexpr int KL = k8 ? KSTEPS / 2 : KSTEPS;   // 16-byte K loads per tile
  constexpr int VL = k8 ? VW / 2 : VW;           // dwords of V loaded per lane and token
  constexpr int TPB = BS / 16;
  constexpr int NS = kPrefillStages;
  static_assert(HD % 32 == 0 && BS % 16 == 0 && (VW == 2 || VW == 4), "unsupported shape");
  __shared__ PrefillShared<HD, CG> sm;

  const int g = blockIdx.x % a.num_kv_heads;
  // heaviest query chunks (latest positions) first
  const int chunk = a.chunks - 1 - (int)(blockIdx.x / a.num_kv_heads);
  const int s = blockIdx.z;
  const int lane = threadIdx.x % kWave, wave = uniform(threadIdx.x / kWave);
  const int n = lane & 15, g4 = lane >> 4;
  const int G = a.group, tpg = 16 / G, tpw = CG * tpg;   // query tokens per group / wave

  int q0 = load_uniform(a.query_start + s), q1 = load_uniform(a.query_start + s + 1);
  q0 = min(max(q0, 0), a.total_q);
  q1 = min(max(q1, q0), a.total_q);
  const int nq = q1 - q0;
  int L = load_uniform(a.context_lens + s);
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int first = (chunk * 4 + wave) * tpw;   // the wave's first query token
  if (first >= nq) return;                      // no barrier follows: waves leave freely

  // this lane's column in group c: query token i[c] (row q0 + i[c]), head h
  const int h = g * G + n % G;
  int i[CG], limit[CG];
  bool valid[CG];
  int lim_max = 0, lim_min = INT32_MAX;
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    i[c] = first + c * tpg + n / G;
    valid[c] = i[c] < nq;
    const int pos = L - nq + i[c];
    limit[c] = (valid[c] && pos >= 0) ? pos + 1 : 0;   // tokens [0, limit) are visible
    lim_max = max(lim_max, limit[c]);
    if (valid[c]) lim_min = min(lim_min, limit[c]);
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
    lim_max = max(lim_max, __shfl_xor(lim_max, off, 64));
    lim_min = min(lim_min, __shfl_xor(lim_min, off, 64));
  }
  lim_max = uniform(lim_max);
  lim_min = uniform(lim_min);

  // Q^T of the wave's columns into its LDS slots (B layout)
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    const TQ* qrow = static_cast<const TQ*>(a.q) +
                     ((size_t)(q0 + (valid[c] ? i[c] : 0)) * a.num_q_heads + h) * HD;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      sm.q[wave][c][kk][lane] =
          valid[c] ? ld16(qrow + mfma_dim0<C>(kk, g4)) : u32x4{0, 0, 0, 0};
  }

  const size_t block_bytes = (size_t)a.num_kv_heads * BS * HD * sizeof(T);
  const char* kbase = static_cast<const char*>(a.k_cache) + (size_t)g * BS * HD * sizeof(T);
  const char* vbase = static_cast<const char*>(a.v_cache) + (size_t)g * BS * HD * sizeof(T);
  const uint32_t koff = (uint32_t)((n * HD + mfma_dim0<C>(0, g4)) * sizeof(T));
  const uint32_t voff = (uint32_t)(((4 * g4) * HD + n * DPL) * sizeof(T));
  const int32_t* table = a.block_tables + (size_t)s * a.max_blocks;

  f32x4 acc[CG][DPL];
  float m[CG], l[CG];
#pragma unroll
  for (int c = 0; c < CG; ++c) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[c][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[c] = -INFINITY;
    l[c] = 0.f;
  }
  int bad = 0;
  const int ntiles = (lim_max + 15) / 16;

  for (int pass = 0; pass < ntiles; pass += kWave) {
    const int mine = min(kWave, ntiles - pass);
    const int tbl = table[min((pass + lane) / TPB, a.max_blocks - 1)];

    auto load_tile = [&](int t, u32x4* ka, uint32_t (*vv)[VL]) {
      const bool live = t < mine;
      const int u = pass + t;
      int phys = lane_value(tbl, t < kWave ? t : kWave - 1);
      if (live && (unsigned)phys >= (unsigned)a.num_blocks) bad = 1;
      if (!live || (unsigned)phys >= (unsigned)a.num_blocks) phys = 0;
      const size_t toff = (size_t)phys * block_bytes + (size_t)(u % TPB) * 16 * HD * sizeof(T);
      const uint32_t nbytes = live ? (uint32_t)(16 * HD * sizeof(T)) : 0u;
      const rsrc_t kt = make_rsrc(kbase + toff, nbytes);
      const rsrc_t vt = make_rsrc(vbase + toff, nbytes);
#pragma unroll
      for (int kk = 0; kk < KL; ++kk) ka[kk] = bld16(kt, koff, kk * (k8 ? 64 : 32) * sizeof(T));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (VL == 1) {
          vv[r][0] = bld4(vt, voff, r * HD * sizeof(T));
        } else if constexpr (VL == 2) {
          const u32x2 x = bld8(vt, voff, r * HD * sizeof(T));
          vv[r][0] = x[0];
          vv[r][1] = x[1];
        } else {
          const u32x4 x = bld16(vt, voff, r * HD * sizeof(T));
          vv[r][0] = x[0];
          vv[r][1] = x[1];
          vv[r][2] = x[2];
          vv[r][3] = x[3];
        }
      }
    };

    auto compute_tile = [&](int t, const u32x4* kl, uint32_t (*vl)[VL]) {
      const int u = pass + t;
      // the tile's operands in E's 16-bit values (8-bit codes widened here,
      // after their loads have landed)
      u32x4 ka[KSTEPS];
      uint32_t vv[4][VW];
      if constexpr (k8) {
#pragma unroll
        for (int kk = 0; kk < KL; ++kk) {
          ka[2 * kk] = u32x4{codes_to_pair<E, false>(kl[kk][0]), codes_to_pair<E, true>(kl[kk][0]),
                             codes_to_pair<E, false>(kl[kk][1]), codes_to_pair<E, true>(kl[kk][1])};
          ka[2 * kk + 1] =
              u32x4{codes_to_pair<E, false>(kl[kk][2]), codes_to_pair<E, true>(kl[kk][2]),
                    codes_to_pair<E, false>(kl[kk][3]), codes_to_pair<E, true>(kl[kk][3])};
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int w = 0; w < VL; ++w) {
            vv[r][2 * w] = codes_to_pair<E, false>(vl[r][w]);
            vv[r][2 * w + 1] = codes_to_pair<E, true>(vl[r][w]);
          }
      } else {
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) ka[kk] = kl[kk];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int w = 0; w < VW; ++w) vv[r][w] = vl[r][w];
      }
      const bool edge = u * 16 + 16 > lim_min;   // some column's bound or the context ends here
      const int t0 = u * 16 + 4 * g4;
      if (edge) {
        // value rows past the context are zeroed so that whatever those
        // slots hold cannot reach the product
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t0 + r >= L) {
#pragma unroll
            for (int w = 0; w < VW; ++w) vv[r][w] = 0u;
          }
      }
      u32x2 pb[CG], pr[CG];
#pragma unroll
      for (int c = 0; c < CG; ++c) {
        __asm__ volatile("" ::: "memory");
        u32x4 qb[KSTEPS];
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) qb[kk] = sm.q[wave][c][kk][lane];
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) sacc = Ops::qk(ka[kk], qb[kk], sacc);
        float sr[4];   // scores in log2 units
#pragma unroll
        for (int r = 0; r < 4; ++r) sr[r] = sacc[r] * a.scale_log2e;
        if (edge) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (t0 + r >= limit[c]) sr[r] = -INFINITY;   // the column's causal bound
        }
        // Lazy rescaling: m is a reference maximum (log2 units) that moves
        // only when a tile's maximum passes it by more than kPrefillSlack, so
        // the probabilities stay below 2^kPrefillSlack and the accumulators
        // are rescaled a few times per context instead of at most tiles.
        // The normalised result is the same; only the reference differs.
        // each lane checks its own four scores; the column maximum (a
        // reduction across the four token groups) is needed only to rescale
        const float lmax = fmaxf(fmaxf(sr[0], sr[1]), fmaxf(sr[2], sr[3]));
        if (__any(lmax > m[c] + kPrefillSlack)) {
          const float mn = fmaxf(m[c], rows_max(lmax));
          const float corr = (mn == -INFINITY) ? 1.f : fast_exp2(m[c] - mn);
          m[c] = mn;
          l[c] *= corr;
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[c][e] *= corr;
        }
        const float mu = (m[c] == -INFINITY) ? 0.f : m[c];
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = fast_exp2(sr[r] - mu);   // exp2(-inf) == 0
        l[c] += (p[0] + p[1]) + (p[2] + p[3]);
        pb[c] = u32x2{Ops::pack2(p[0], p[1]), Ops::pack2(p[2], p[3])};
        pr[c] = u32x2{0u, 0u};
        if constexpr (kPrefillSplitP) {
          pr[c][0] = Ops::pack2(p[0] - Ops::widen_lo(pb[c][0]), p[1] - Ops::widen_hi(pb[c][0]));
          pr[c][1] = Ops::pack2(p[2] - Ops::widen_lo(pb[c][1]), p[3] - Ops::widen_hi(pb[c][1]));
        }
      }
      // one V^T operand per lane-dim e serves every column group
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const u32x2 va = {pair_of(e, vv[0], vv[1]), pair_of(e, vv[2], vv[3])};
#pragma unroll
        for (int c = 0; c < CG; ++c) {
          acc[c][e] = Ops::pv(va, pb[c], acc[c][e]);
          if constexpr (kPrefillSplitP) acc[c][e] = Ops::pv(va, pr[c], acc[c][e]);
        }
      }
    };

    u32x4 kb[NS][KL];
    uint32_t vb[NS][4][VL];
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) load_tile(j, kb[j], vb[j]);
    for (int i0 = 0; i0 < mine; i0 += NS) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        load_tile(i0 + j + NS - 1, kb[(j + NS - 1) % NS], vb[(j + NS - 1) % NS]);
        if (i0 + j < mine) compute_tile(i0 + j, kb[j], vb[j]);
      }
    }
  }

  const bool any_bad = __any(bad);
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    // the four token groups of a column hold partial sums of l
    const float lsum = rows_sum(l[c]);
    if (!valid[c]) continue;
    TQ* orow = static_cast<TQ*>(a.out) + ((size_t)(q0 + i[c]) * a.num_q_heads + h) * HD;
    // no visible token: zero row; 8-bit V: code units -> values
    const float inv = lsum > 0.f ? (k8 ? a.v_scale : 1.f) / lsum : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float o[DPL];
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = any_bad ? __builtin_nanf("") : acc[c][e][r] * inv;
      store_rounded<E, DPL>(orow + (4 * g4 + r) * DPL, o);
    }
  }
}

template <typename E, typename C, int HD, int BS>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((prefill_mfma_kernel<E, C, HD, BS, kPrefillGroups>),
                     dim3(a.num_kv_heads * a.chunks, 1, a.num_seqs), dim3(256), 0, st, a);
  return hipGetLastError();
}

int prefill_tokens_per_workgroup(int group) { return 4 * kPrefillGroups * (16 / group); }

template <typename E, typename C, int HD>
static hipError_t launch_prefill_hd(int bs, const PrefillArgs& a, hipStream_t st) {
  switch (bs) {
    case 16: return launch_prefill_t<E, C, HD, 16>(a, st);
    case 32: return launch_prefill_t<E, C, HD, 32>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename E, typename C>
static hipError_t launch_prefill_e(int hd, int bs, const PrefillArgs& a, hipStream_t st) {
  switch (hd) {
    case 64: return launch_prefill_hd<E, C, 64>(bs, a, st);
    case 128: return launch_prefill_hd<E, C, 128>(bs, a, st);
  }
  return hipErrorInvalidValue;
}

bool prefill_supported(Elem e, int hd, int bs, int group) {
  return (e == Elem::F16 || e == Elem::BF16) && (hd == 64 || hd == 128) &&
         (bs == 16 || bs == 32) && group >= 1 && group <= 16 && 16 % group == 0;
}

hipError_t launch_prefill(Elem e, bool kv_fp8, int hd, int bs, const PrefillArgs& a,
                          hipStream_t st) {
  switch (e) {
    case Elem::F16:
      return kv_fp8 ? launch_prefill_e<F16, E4M3>(hd, bs, a, st)
                    : launch_prefill_e<F16, F16>(hd, bs, a, st);
    case Elem::BF16:
      return kv_fp8 ? launch_prefill_e<BF16, E4M3>(hd, bs, a, st)
                    : launch_prefill_e<BF16, BF16>(hd, bs, a, st);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
