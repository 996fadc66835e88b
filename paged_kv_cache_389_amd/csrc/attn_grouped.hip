// Grouped paged decode: sequences that share KV blocks read each shared
// tile once for all of them.
//
// Sequences forked from one prompt (parallel sampling, beam search) hold the
// prompt's blocks in common through their block tables ("Memory
// Optimization in LLM Serving with PagedAttention", section "Advanced
// Capabilities: Memory Sharing with Copy-on-Write"; "vLLM and
// PagedAttention", the paragraph on sharing).  Decode attention of each
// sequence on its own reads a shared block once per sequence.  Here one
// workgroup takes a group of up to 16 / G such sequences and one KV head g:
// its 16 matrix-core columns are (member m, query head g*G + j), and it walks
// the group's tile list, which names every distinct (physical block, 16-token
// tile index) that some member reaches, with the mask of the members that
// reach it.  A shared tile is loaded once and feeds every member's column;
// a tile of one member alone is loaded once with the other columns masked.
// The arithmetic per column is that of the grouped-query decode kernel
// (same operand layouts, online softmax in log2 units, bf16 probabilities
// split into a head and a remainder), so each output row is the plain
// decode attention of its sequence; only the order in which a column's
// tiles are folded in differs.
//
// Per column: tokens at or past the member's length, and tiles outside its
// mask, get probability zero.  Value rows that no member of the tile reaches
// are zeroed before the product, so unwritten slots cannot reach a result.
// The waves (four, or eight over 8-bit codes) take tiles round-robin and
// merge in LDS.  A group's list
// may be cut into parts (grid z) whose (max, sum, output) states a second
// kernel merges; the cache may hold E4M3 codes.
#include "common.h"
#include "decode.h"
#include "mfma_ops.h"

namespace pkv {

namespace {

constexpr int kCols = 16;

// Rows [t_begin, t_begin + ntile) of the list that part `part` of group grp
// covers, offsets clamped to the list; returns the group's part count (at
// least one: an empty group is one empty part).
__device__ inline int group_range(const GroupedArgs& a, int grp, int part, int& t_begin,
                                  int& ntile) {
  const int t0 = min(max(load_uniform(a.tile_start + grp), 0), a.num_tiles);
  const int t1 = min(max(load_uniform(a.tile_end ? a.tile_end + grp : a.tile_start + grp + 1), t0),
                     a.num_tiles);
  if (a.part_tiles <= 0) {
    t_begin = t0;
    ntile = t1 - t0;
    return 1;
  }
  const int nparts = max(1, (t1 - t0 + a.part_tiles - 1) / a.part_tiles);
  t_begin = min(t0 + part * a.part_tiles, t1);
  ntile = min(a.part_tiles, t1 - t_begin);
  return nparts;
}

template <int HD, int NW>
struct GroupShared {
  static constexpr int OS = HD + 4;   // padded row stride of the output tiles
  u32x4 q[HD / 32][kWave];
  float m[NW][kCols], l[NW][kCols];
  __attribute__((aligned(16))) float o[NW][kCols][OS];
  int seq[kCols];   // sequence of each column, -1 for none
  int bad[NW];
};

// Largest value of v over the 16 lanes of each 16-lane row.
__device__ inline int row16_max(int v) {
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppXor1, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppXor2, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppRowHalfMirror, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppRowMirror, 0xF, 0xF, true));
  return v;
}

// C is the cache element: E itself, or E4M3 codes (loaded at half width and
// widened to E's 16-bit values right before the products; the K scale is in
// scale_log2e, the V scale multiplies the merged output).
template <typename E, typename C, int HD, int BS, int NW = 4>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(3))) void
decode_grouped_kernel(GroupedArgs a) {
  using T = typename C::storage;       // cache element
  using Q = typename E::storage;       // query / output element
  using Ops = MfmaOps<E>;
  constexpr bool k8 = sizeof(T) == 1;
  constexpr int KSTEPS = HD / 32;      // QK MFMAs per tile
  constexpr int DPL = HD / 16;         // V dims per lane per token == PV MFMAs per tile
  constexpr int VW = DPL / 2;          // dwords of 16-bit V per lane per token
  constexpr int KL = k8 ? KSTEPS / 2 : KSTEPS;   // 16-byte K loads per tile
  constexpr int VL = k8 ? VW / 2 : VW;           // dwords of V loaded per lane per token
  constexpr int TPB = BS / 16;         // tiles per block
  static_assert(!k8 || KSTEPS % 2 == 0, "8-bit K loads cover two k-steps");
  constexpr int NS = 2;                // register stages of the tile pipeline
  static_assert(HD % 32 == 0 && BS % 16 == 0 && (VW == 2 || VW == 4), "unsupported shape");
  __shared__ GroupShared<HD, NW> sm;

  const int g = blockIdx.x, grp = blockIdx.y, part = blockIdx.z;
  // the group's rows of the list, clamped to the list (any offsets stay in
  // bounds), and this workgroup's part of them
  int t_begin, ntile;
  const int nparts = group_range(a, grp, part, t_begin, ntile);
  if (part >= nparts) return;
  const int tid = threadIdx.x, wave = uniform(tid / kWave), lane = tid % kWave;
  const int n = lane & 15, g4 = lane >> 4;
  const int G = a.group;

  // column n: member n / G of the group, query head g*G + n % G
  const int mem = n / G;
  int s_n = -1;
  if (mem < a.max_members) s_n = a.members[(size_t)grp * a.max_members + mem];
  if (s_n >= a.num_seqs) s_n = -1;
  int len_n = s_n >= 0 ? a.context_lens[s_n] : 0;
  len_n = len_n < 0 ? 0 : (len_n > a.len_cap ? a.len_cap : len_n);
  const int bit_n = s_n >= 0 ? (1 << mem) : 0;

  // the query rows of the columns (B layout), zero for empty columns
  if (wave == 0) {
    const Q* qh = static_cast<const Q*>(a.q) +
                  ((size_t)(s_n >= 0 ? s_n : 0) * a.num_q_heads + (size_t)g * G + n % G) * HD;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      sm.q[kk][lane] = s_n >= 0 ? ld16(qh + mfma_dim0<C>(kk, g4)) : u32x4{0, 0, 0, 0};
    if (g4 == 0) sm.seq[n] = s_n;
  }

  const size_t block_bytes = (size_t)a.num_kv_heads * BS * HD * sizeof(T);
  const char* kbase = static_cast<const char*>(a.k_cache) + (size_t)g * BS * HD * sizeof(T);
  const char* vbase = static_cast<const char*>(a.v_cache) + (size_t)g * BS * HD * sizeof(T);
  const uint32_t koff = (uint32_t)((n * HD + mfma_dim0<C>(0, g4)) * sizeof(T));
  const uint32_t voff = (uint32_t)(((4 * g4) * HD + n * DPL) * sizeof(T));

  f32x4 acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  int bad = 0;

  // passes of at most 64 of the wave's tiles (wave, wave + 4, ...): lane i
  // holds the list entry (block, tile index, member mask) of the i-th
  bool waited = false;
  for (int pass = wave; pass < ntile; pass += kWave * NW) {
    const int mine = min(kWave, (ntile - pass + NW - 1) / NW);
    i32x4 ent = {0, 0, 0, 0};
    if (lane < mine)
      ent = *reinterpret_cast<const i32x4*>(a.tiles + 4 * ((size_t)t_begin + pass + NW * lane));
    const int blk_v = ent[0], tix_v = ent[1], msk_v = ent[2];

    // loads of the wave's i-th tile of the pass (an empty descriptor past
    // `mine`: those loads return zeros without a memory access)
    auto load_tile = [&](int i, u32x4* ka, uint32_t (*vv)[VL]) {
      const bool live = i < mine;
      const int ii = i < kWave ? i : kWave - 1;
      int phys = lane_value(blk_v, ii);
      const int tix = lane_value(tix_v, ii);
      if (live && (unsigned)phys >= (unsigned)a.num_blocks) bad = 1;
      if (!live || (unsigned)phys >= (unsigned)a.num_blocks) phys = 0;
      const size_t toff =
          (size_t)phys * block_bytes + (size_t)((unsigned)tix % TPB) * 16 * HD * sizeof(T);
      constexpr uint32_t kTileBytes = 16 * HD * sizeof(T);
      const uint32_t nbytes = live ? kTileBytes : 0u;
      const rsrc_t kt = make_rsrc(kbase + toff, nbytes);
      const rsrc_t vt = make_rsrc(vbase + toff, nbytes);
#pragma unroll
      for (int kk = 0; kk < KL; ++kk) ka[kk] = bld16<kStream>(kt, koff, kk * (k8 ? 64 : 32) * sizeof(T));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (VL == 1) {
          vv[r][0] = bld4<kStream>(vt, voff, r * HD * sizeof(T));
        } else if constexpr (VL == 2) {
          const u32x2 x = bld8<kStream>(vt, voff, r * HD * sizeof(T));
          vv[r][0] = x[0];
          vv[r][1] = x[1];
        } else {
          const u32x4 x = bld16<kStream>(vt, voff, r * HD * sizeof(T));
          vv[r][0] = x[0];
          vv[r][1] = x[1];
          vv[r][2] = x[2];
          vv[r][3] = x[3];
        }
      }
    };

    auto compute_tile = [&](int i, const u32x4* kl, uint32_t (*vl)[VL]) {
      const int tix = lane_value(tix_v, i);
      const int msk = lane_value(msk_v, i);
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
      __asm__ volatile("" ::: "memory");   // Q^T is read from LDS per tile
      u32x4 qb[KSTEPS];
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) qb[kk] = sm.q[kk][lane];
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) sacc = Ops::qk(ka[kk], qb[kk], sacc);
      // tokens 16*tix + 4*g4 + r of column n
      const int tok0 = tix * 16 + 4 * g4;
      const bool col_on = (msk & bit_n) != 0;
      float sc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sc[r] = (col_on && tok0 + r < len_n) ? sacc[r] * a.scale_log2e : -INFINITY;
      // value rows past every member's length in this tile are zeroed
      const int reach = row16_max(col_on ? len_n : 0);
      if (tix * 16 + 16 > reach) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tok0 + r >= reach) {
#pragma unroll
            for (int w = 0; w < VW; ++w) vv[r][w] = 0u;
          }
      }
      const float mb = rows_max(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
      const float mn = fmaxf(m, mb);
      const float mu = (mn == -INFINITY) ? 0.f : mn;
      const float corr = fast_exp2(m - mu);
      m = mn;
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = fast_exp2(sc[r] - mu);   // exp2(-inf) == 0
      l = __builtin_fmaf(l, corr, (p[0] + p[1]) + (p[2] + p[3]));
      if (__any(corr != 1.f)) {
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] *= corr;
      }
      const u32x2 pb = {Ops::pack2(p[0], p[1]), Ops::pack2(p[2], p[3])};
      u32x2 pr = {0u, 0u};
      if constexpr (Ops::kSplit) {
        pr[0] = Ops::pack2(p[0] - Ops::widen_lo(pb[0]), p[1] - Ops::widen_hi(pb[0]));
        pr[1] = Ops::pack2(p[2] - Ops::widen_lo(pb[1]), p[3] - Ops::widen_hi(pb[1]));
      }
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const u32x2 va = {pair_of(e, vv[0], vv[1]), pair_of(e, vv[2], vv[3])};
        acc[e] = Ops::pv(va, pb, acc[e]);
        if constexpr (Ops::kSplit) acc[e] = Ops::pv(va, pr, acc[e]);
      }
    };

    u32x4 kb[NS][KL];
    uint32_t vb[NS][4][VL];
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) load_tile(j, kb[j], vb[j]);
    if (!waited) {   // Q^T is in LDS (the first tile loads overlap its write)
      __syncthreads();
      waited = true;
    }
    for (int i0 = 0; i0 < mine; i0 += NS) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        load_tile(i0 + j + NS - 1, kb[(j + NS - 1) % NS], vb[(j + NS - 1) % NS]);
        if (i0 + j < mine) compute_tile(i0 + j, kb[j], vb[j]);
      }
    }
  }
  if (!waited) __syncthreads();   // a wave with no tiles still meets the Q barrier

  // merge the four waves in LDS; every column's row is normalised and stored,
  // or, when the group has several parts, its unnormalised state
  const float lsum = rows_sum(l);
  if (g4 == 0) {
    sm.m[wave][n] = m;
    sm.l[wave][n] = lsum;
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.o[wave][n][(4 * g4 + r) * DPL + e] = acc[e][r];
  const int any_bad = __any(bad);
  if (lane == 0) sm.bad[wave] = any_bad;
  __syncthreads();

  int all_bad = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) all_bad |= sm.bad[w];
  for (int idx = tid; idx < kCols * (HD / 4); idx += NW * kWave) {
    const int col = idx / (HD / 4), d = (idx % (HD / 4)) * 4;
    const int s = sm.seq[col];
    if (s < 0) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.m[w][col]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float Ls = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = fast_exp2(sm.m[w][col] - Mu);
      Ls = __builtin_fmaf(wt, sm.l[w][col], Ls);
      O += wt * *reinterpret_cast<const f32x4*>(&sm.o[w][col][d]);
    }
    if constexpr (k8) O *= a.v_scale;   // 8-bit V: code units -> values (commutes with merges)
    if (nparts > 1) {
      const size_t st = (((size_t)grp * a.max_parts + part) * a.num_kv_heads + g) * kCols + col;
      if (all_bad) O = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
      *reinterpret_cast<f32x4*>(a.part_o + st * HD + d) = O;
      if (d == 0) *reinterpret_cast<f32x2*>(a.part_ml + 2 * st) = f32x2{M, Ls};
      continue;
    }
    float r[4];
    if (all_bad) {
      r[0] = r[1] = r[2] = r[3] = __builtin_nanf("");
    } else if (Ls > 0.f) {
      const float inv = 1.f / Ls;
      r[0] = O[0] * inv;
      r[1] = O[1] * inv;
      r[2] = O[2] * inv;
      r[3] = O[3] * inv;
    } else {   // an empty context: the zero row
      r[0] = r[1] = r[2] = r[3] = 0.f;
    }
    Q* out = static_cast<Q*>(a.out) + ((size_t)s * a.num_q_heads + (size_t)g * G + col % G) * HD;
    store_rounded<E, 4>(out + d, r);
  }
}

// Merge of a group's part states, one workgroup per (KV head, group): for
// every column with a sequence, the log-sum-exp combination of its parts'
// (max, sum, output) states, normalised and rounded into its row.
template <typename E, int HD>
__global__ __launch_bounds__(256) void grouped_merge_kernel(GroupedArgs a) {
  using T = typename E::storage;
  const int g = blockIdx.x, grp = blockIdx.y;
  int t_begin, ntile;
  const int nparts = min(group_range(a, grp, 0, t_begin, ntile), a.max_parts);
  if (nparts <= 1) return;
  const int G = a.group;
  for (int idx = threadIdx.x; idx < kCols * (HD / 4); idx += 256) {
    const int col = idx / (HD / 4), d = (idx % (HD / 4)) * 4;
    const int mem = col / G;
    if (mem >= a.max_members) continue;
    const int s = a.members[(size_t)grp * a.max_members + mem];
    if (s < 0 || s >= a.num_seqs) continue;
    const size_t st0 = (((size_t)grp * a.max_parts) * a.num_kv_heads + g) * kCols + col;
    const size_t pstride = (size_t)a.num_kv_heads * kCols;
    float M = -INFINITY;
    for (int p = 0; p < nparts; ++p) M = fmaxf(M, a.part_ml[2 * (st0 + p * pstride)]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float Ls = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < nparts; ++p) {
      const size_t st = st0 + p * pstride;
      const f32x2 ml = *reinterpret_cast<const f32x2*>(a.part_ml + 2 * st);
      const float wt = fast_exp2(ml[0] - Mu);
      Ls = __builtin_fmaf(wt, ml[1], Ls);
      O += wt * *reinterpret_cast<const f32x4*>(a.part_o + st * HD + d);
    }
    float r[4];
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;   // no token at all: the zero row
    r[0] = O[0] * inv;
    r[1] = O[1] * inv;
    r[2] = O[2] * inv;
    r[3] = O[3] * inv;
    T* out = static_cast<T*>(a.out) + ((size_t)s * a.num_q_heads + (size_t)g * G + col % G) * HD;
    store_rounded<E, 4>(out + d, r);
  }
}

// Eight waves per workgroup over 8-bit codes (half the bytes per tile: twice
// the waves keep as many bytes in flight per item), four otherwise.
template <typename E, typename C, int HD>
hipError_t launch_hd(int bs, const GroupedArgs& a, hipStream_t st) {
  constexpr int NW = sizeof(typename C::storage) == 1 ? 8 : 4;
  const dim3 grid(a.num_kv_heads, a.num_groups, a.max_parts);
  switch (bs) {
    case 16: hipLaunchKernelGGL((decode_grouped_kernel<E, C, HD, 16, NW>), grid, dim3(NW * 64), 0, st, a); break;
    case 32: hipLaunchKernelGGL((decode_grouped_kernel<E, C, HD, 32, NW>), grid, dim3(NW * 64), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename E, int HD>
hipError_t launch_merge_hd(const GroupedArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((grouped_merge_kernel<E, HD>), dim3(a.num_kv_heads, a.num_groups), dim3(256),
                     0, st, a);
  return hipGetLastError();
}

template <typename E, typename C>
hipError_t launch_e(int hd, int bs, const GroupedArgs& a, hipStream_t st) {
  switch (hd) {
    case 64: return launch_hd<E, C, 64>(bs, a, st);
    case 128: return launch_hd<E, C, 128>(bs, a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool grouped_supported(Elem e, int head_dim, int block_size) {
  return (e == Elem::F16 || e == Elem::BF16) && (head_dim == 64 || head_dim == 128) &&
         (block_size == 16 || block_size == 32);
}

hipError_t launch_decode_grouped(Elem e, bool kv_fp8, int head_dim, int block_size,
                                 const GroupedArgs& a, hipStream_t stream) {
  switch (e) {
    case Elem::F16:
      return kv_fp8 ? launch_e<F16, E4M3>(head_dim, block_size, a, stream)
                    : launch_e<F16, F16>(head_dim, block_size, a, stream);
    case Elem::BF16:
      return kv_fp8 ? launch_e<BF16, E4M3>(head_dim, block_size, a, stream)
                    : launch_e<BF16, BF16>(head_dim, block_size, a, stream);
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_grouped_merge(Elem e, int head_dim, const GroupedArgs& a, hipStream_t stream) {
  const bool f16 = e == Elem::F16;
  if (e != Elem::F16 && e != Elem::BF16) return hipErrorInvalidValue;
  switch (head_dim) {
    case 64: return f16 ? launch_merge_hd<F16, 64>(a, stream) : launch_merge_hd<BF16, 64>(a, stream);
    case 128: return f16 ? launch_merge_hd<F16, 128>(a, stream) : launch_merge_hd<BF16, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
