// Paged decode attention for grouped query heads, on the matrix cores.
//
// One workgroup (4 waves) computes all G query heads that share one KV head
// of one sequence, over one partition of the context.  Against a tile of 16
// tokens the G query rows form a small dense contraction, so both products
// run as gfx950 MFMA instructions with fp32 accumulation:
//
//   S^T[16 tok][16 head] = K[16 tok][HD] * Q^T[HD][16 head]   (16x16x32, HD/32 steps)
//   O^T[HD][16 head]    += V^T[HD][16 tok] * P^T[16 tok][16 head]   (16x16x16, HD/16 tiles)
//
// Lane l of a wave owns head column n = l % 16 and token/dim group
// g4 = l / 16.  Operand layouts line up without any data exchange:
// * K is read in the matrix-core A layout: lane l loads 16 bytes of token
//   row n at dims 32*kk + 8*g4 .. +8 (each load instruction covers 64
//   contiguous bytes of all 16 rows).  Q^T is held in the matching B layout.
// * The S result gives lane l the scores of tokens 4*g4 + i (i < 4) for its
//   head n, which is exactly the B layout P^T needs for the second product.
// * V is read row-wise: lane l loads tokens 4*g4 + i, dims n*HD/16 .. +HD/16.
//   Regrouping those registers gives, for each e < HD/16, the A operand of
//   V^T restricted to the dims n*HD/16 + e (a byte permute per register
//   pair, no LDS); output tile e then holds dims (4*g4 + i)*HD/16 + e.
// The softmax state (running max in log2 units, running sum) is per head,
// so it lives in lane column n; the max over a tile's 16 tokens needs two
// cross-group shuffles.  With bf16 the probabilities are split into a bf16
// high part and a bf16 remainder and both are multiplied in, which keeps
// them at about 16 significant bits.
//
// Latency hiding, as in the vector-ALU kernel: wave w takes tiles w, w+4,
// ... of the partition; the physical blocks of all its tiles are fetched up
// front with one vector load (lane i holds the entry of the wave's i-th
// tile), and the loads of tile i+1 are issued before tile i is computed.
// The four waves' states are merged in LDS, sized for at most GMAX heads.
//
// Passages: a sequence's KV blocks are gathered through its block table
// ("Memory Optimization in LLM Serving with PagedAttention", section "How
// PagedAttention Works"); only the last block is partly filled (same
// section).  Grouped query heads are not on the pages: query head h reads
// KV head h / G.
#include "common.h"
#include "decode.h"
#include "mfma_ops.h"

namespace pkv {

// Register stages of the tile pipeline (see mfma_accumulate).
constexpr int kMfmaStages = 2;

// LDS of one workgroup: Q^T (B layout, indexed by lane) and the four
// waves' softmax states for up to GMAX heads.
template <int HD, int GMAX>
struct MfmaShared {
  static constexpr int OS = HD + 4;   // padded row stride of the output tiles
  u32x4 q[HD / 32][kWave];
  float m[4][GMAX], l[4][GMAX];
  __attribute__((aligned(16))) float o[4][GMAX][OS];
  int bad[4];
};

// One wave's state for the 16 head columns: acc[e] holds O^T rows
// (4*g4 + r)*DPL + e (r < 4) of head column n = lane % 16; m and l are the
// column's running max (log2 units) and, per token group g4, partial sum.
template <int DPL>
struct MfmaState {
  f32x4 acc[DPL];
  float m, l;
  int bad;
};

// Write Q^T of the G query heads of KV head g of sequence s into q (B
// layout: lane (n, g4) holds head n, the dims mfma_dim0 gives; zero past G).
template <typename E, typename C, int HD>
__device__ inline void mfma_load_q(const DecodeArgs& a, int s, int g, u32x4 (*q)[kWave]) {
  using T = typename E::storage;
  const int lane = threadIdx.x % kWave, n = lane & 15, g4 = lane >> 4;
  const int G = a.group;
  const int hn = n < G ? n : G - 1;
  const T* qh = static_cast<const T*>(a.q) + ((size_t)s * a.num_q_heads + (size_t)g * G + hn) * HD;
#pragma unroll
  for (int kk = 0; kk < HD / 32; ++kk)
    q[kk][lane] = (n < G) ? ld16(qh + mfma_dim0<C>(kk, g4)) : u32x4{0, 0, 0, 0};
}

// Fold tiles ta + first, ta + first + stride, ... (< tb) of KV head g of
// sequence s (tile = 16 tokens; tokens at or past L > 0 are masked) into
// the calling wave's state, with Q^T read from q (LDS).
// The physical blocks of the first pass of tiles ta + first + stride * i
// (lane i), read along with the query: the index is clamped to the table
// row, so the load is in bounds whatever the length.
template <int BS>
__device__ inline int mfma_first_blocks(const DecodeArgs& a, int s, int ta, int first,
                                        int stride) {
  const int lane = threadIdx.x % kWave;
  const int blk = min((ta + first + stride * lane) / (BS / 16), a.max_blocks - 1);
  return a.contiguous ? s * a.max_blocks + blk : a.block_tables[(size_t)s * a.max_blocks + blk];
}

//
// With kWaitQ the workgroup's Q^T is still being written to LDS: every wave
// passes one barrier, right after issuing the loads of its first tiles
// (or at once if it has none), so those loads overlap the query's.
//
// C is the cache element: E itself, or E4M3 codes, which are loaded at half
// the width and turned into E's 16-bit values right before the products
// (the scales are applied outside: K's in scale_log2e, V's on the output).
//
// POL is the cache policy of the K/V loads: kStream (each block is read once
// per launch) or 0 (blocks shared across the batch, served from the cache
// after their first read; DecodeArgs::cached_kv).
template <typename E, typename C, int HD, int BS, bool kWaitQ = false, int NS = kMfmaStages,
          int POL = kStream>
__device__ inline void mfma_accumulate(const DecodeArgs& a, int s, int g, int L, int ta, int tb,
                                       int first, int stride, int tbl0, const u32x4 (*q)[kWave],
                                       MfmaState<HD / 16>& st) {
  using T = typename C::storage;       // cache element
  using Ops = MfmaOps<E>;
  constexpr bool k8 = sizeof(T) == 1;
  constexpr int KSTEPS = HD / 32;      // QK MFMAs per tile
  constexpr int DPL = HD / 16;         // V dims per lane per token == PV MFMAs per tile
  constexpr int VW = DPL / 2;          // dwords of 16-bit V per lane per token
  constexpr int KL = k8 ? KSTEPS / 2 : KSTEPS;   // 16-byte K loads per tile
  constexpr int VL = k8 ? VW / 2 : VW;           // dwords of V loaded per lane per token
  constexpr int TPB = BS / 16;         // tiles per block
  static_assert(HD % 32 == 0 && BS % 16 == 0 && (VW == 2 || VW == 4), "unsupported shape");
  static_assert(!k8 || KSTEPS % 2 == 0, "8-bit K loads cover two k-steps");

  const int lane = threadIdx.x % kWave;
  const int n = lane & 15, g4 = lane >> 4;
  const int tok_end = L;
  const int32_t* table = a.block_tables + (size_t)s * a.max_blocks;

  // tile addresses: a buffer descriptor over the 16-token tile, built in
  // scalar registers, plus a constant 32-bit per-lane byte offset, so no
  // per-tile address arithmetic runs on the vector ALU
  const size_t block_bytes = (size_t)a.num_kv_heads * BS * HD * sizeof(T);
  const char* kbase = static_cast<const char*>(a.k_cache) + (size_t)g * BS * HD * sizeof(T);
  const char* vbase = static_cast<const char*>(a.v_cache) + (size_t)g * BS * HD * sizeof(T);
  const uint32_t koff = (uint32_t)((n * HD + mfma_dim0<C>(0, g4)) * sizeof(T));
  const uint32_t voff = (uint32_t)(((4 * g4) * HD + n * DPL) * sizeof(T));

  f32x4 acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = st.acc[e];
  float m = st.m, l = st.l;
  int bad = st.bad;

  // passes of at most 64 of the wave's tiles: their table entries fit one VGPR
  if (kWaitQ && ta + first >= tb) __syncthreads();   // no tiles: the barrier alone
  for (int pass = ta + first; pass < tb; pass += kWave * stride) {
    const int mine = min(kWave, (tb - pass + stride - 1) / stride);
    int tbl = tbl0;
    if (pass != ta + first) {
      const int blk = min((pass + stride * lane) / TPB, a.max_blocks - 1);
      tbl = a.contiguous ? s * a.max_blocks + blk : table[blk];
    }

    // issue the loads of the wave's i-th tile of the pass: K in the A layout
    // (token row n, dims 32*kk + 8*g4 .. +8), V row-wise (tokens 4*g4 + r,
    // dims n*DPL .. +DPL)
    // (tiles i >= mine get an empty descriptor: their loads return zeros
    // without a memory access, so every step issues the same loads)
    auto load_tile = [&](int i, u32x4* ka, uint32_t (*vv)[VL]) {
      const bool live = i < mine;
      const int u = pass + stride * i;
      int phys = lane_value(tbl, i < kWave ? i : kWave - 1);
      if (live && (unsigned)phys >= (unsigned)a.num_blocks) bad = 1;
      if (!live || (unsigned)phys >= (unsigned)a.num_blocks) phys = 0;
      const size_t toff = (size_t)phys * block_bytes + (size_t)(u % TPB) * 16 * HD * sizeof(T);
      constexpr uint32_t kTileBytes = 16 * HD * sizeof(T);
      const uint32_t nbytes = live ? kTileBytes : 0u;
      const rsrc_t kt = make_rsrc(kbase + toff, nbytes);
      const rsrc_t vt = make_rsrc(vbase + toff, nbytes);
#pragma unroll
      for (int kk = 0; kk < KL; ++kk) ka[kk] = bld16<POL>(kt, koff, kk * (k8 ? 64 : 32) * sizeof(T));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (VL == 1) {
          vv[r][0] = bld4<POL>(vt, voff, r * HD * sizeof(T));
        } else if constexpr (VL == 2) {
          const u32x2 x = bld8<POL>(vt, voff, r * HD * sizeof(T));
          vv[r][0] = x[0];
          vv[r][1] = x[1];
        } else {
          const u32x4 x = bld16<POL>(vt, voff, r * HD * sizeof(T));
          vv[r][0] = x[0];
          vv[r][1] = x[1];
          vv[r][2] = x[2];
          vv[r][3] = x[3];
        }
      }
    };

    auto compute_tile = [&](int i, const u32x4* kl, uint32_t (*vl)[VL]) {
      const int u = pass + stride * i;
      // the tile's operands in E's 16-bit values (8-bit codes converted here,
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
      // read Q^T from LDS for this tile; the compiler barrier keeps the reads
      // from being hoisted out of the loop (which would pin Q in registers)
      __asm__ volatile("" ::: "memory");
      u32x4 qb[KSTEPS];
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) qb[kk] = q[kk][lane];
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) sacc = Ops::qk(ka[kk], qb[kk], sacc);
      float sc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = sacc[r] * a.scale_log2e;
      if (u * 16 + 16 > tok_end) {
        // the sequence's last tile: mask by index, and zero the value rows
        // past the context so a non-finite value there cannot reach the product
        const int t0 = u * 16 + 4 * g4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (t0 + r >= tok_end) {
            sc[r] = -INFINITY;
#pragma unroll
            for (int w = 0; w < VW; ++w) vv[r][w] = 0u;
          }
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

      // P^T in the B layout: tokens 4*g4 + r of head n
      const u32x2 pb = {Ops::pack2(p[0], p[1]), Ops::pack2(p[2], p[3])};
      u32x2 pr = {0u, 0u};
      if constexpr (Ops::kSplit) {
        pr[0] = Ops::pack2(p[0] - Ops::widen_lo(pb[0]), p[1] - Ops::widen_hi(pb[0]));
        pr[1] = Ops::pack2(p[2] - Ops::widen_lo(pb[1]), p[3] - Ops::widen_hi(pb[1]));
      }
      // V^T in the A layout, one MFMA per lane-dim e
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const u32x2 va = {pair_of(e, vv[0], vv[1]), pair_of(e, vv[2], vv[3])};
        acc[e] = Ops::pv(va, pb, acc[e]);
        if constexpr (Ops::kSplit) acc[e] = Ops::pv(va, pr, acc[e]);
      }
    };

    // NS register stages: the loads of tiles i+1 .. i+NS-1 are in flight
    // while tile i is computed
    u32x4 kb[NS][KL];
    uint32_t vb[NS][4][VL];
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) load_tile(j, kb[j], vb[j]);
    if (kWaitQ && pass == ta + first) __syncthreads();   // Q^T is in LDS
    for (int i0 = 0; i0 < mine; i0 += NS) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        load_tile(i0 + j + NS - 1, kb[(j + NS - 1) % NS], vb[(j + NS - 1) % NS]);
        if (i0 + j < mine) compute_tile(i0 + j, kb[j], vb[j]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) st.acc[e] = acc[e];
  st.m = m;
  st.l = l;
  st.bad = bad;
}

template <int DPL>
__device__ inline void mfma_state_init(MfmaState<DPL>& st) {
#pragma unroll
  for (int e = 0; e < DPL; ++e) st.acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
  st.bad = 0;
}

// Attention of the G query heads of KV head g of sequence s over its
// 16-token tiles [ta, tb) (tokens at or past L > 0 masked), by the four waves of the
// workgroup (tile round-robin), merged in LDS.  The merged states are
// normalised and rounded into `out` (the group's first head) when `out` is
// not null, else stored unnormalised to the partial states
// state0 + hh * hh_stride (hh < G).
template <typename E, typename C, int HD, int BS, int GMAX, int POL>
__device__ inline void mfma_piece(const DecodeArgs& a, int s, int g, int L, int ta, int tb,
                                  int tbl0, typename E::storage* out, size_t state0,
                                  size_t hh_stride, MfmaShared<HD, GMAX>& sm) {
  constexpr int NW = 4;
  constexpr int DPL = HD / 16;
  const int tid = threadIdx.x, wave = uniform(tid / kWave), lane = tid % kWave;
  const int n = lane & 15, g4 = lane >> 4;
  const int G = a.group;

  MfmaState<DPL> st;
  mfma_state_init(st);
  mfma_accumulate<E, C, HD, BS, true, kMfmaStages, POL>(a, s, g, L, ta, tb, wave, NW, tbl0, sm.q,
                                                        st);

  // the four token groups of a head column hold partial sums of l
  const float l = rows_sum(st.l);

  // merge the 4 waves in LDS
  if (n < G) {
    if (g4 == 0) {
      sm.m[wave][n] = st.m;
      sm.l[wave][n] = l;
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.o[wave][n][(4 * g4 + r) * DPL + e] = st.acc[e][r];
  }
  const int any_bad = __any(st.bad);
  if (lane == 0) sm.bad[wave] = any_bad;
  __syncthreads();

  const int all_bad = sm.bad[0] | sm.bad[1] | sm.bad[2] | sm.bad[3];
  for (int idx = tid; idx < G * (HD / 4); idx += 256) {
    const int hh = idx / (HD / 4), d = (idx % (HD / 4)) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.m[w][hh]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float Ls = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = fast_exp2(sm.m[w][hh] - Mu);
      Ls = __builtin_fmaf(wt, sm.l[w][hh], Ls);
      O += wt * *reinterpret_cast<const f32x4*>(&sm.o[w][hh][d]);
    }
    if constexpr (!__is_same(E, C)) O *= a.v_scale;   // 8-bit V: code units -> values
    if (all_bad) O = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    if (out) {
      const float inv = 1.f / Ls;
      float r[4] = {O[0] * inv, O[1] * inv, O[2] * inv, O[3] * inv};
      store_rounded<E, 4>(out + hh * HD + d, r);
    } else {
      const size_t stt = state0 + hh * hh_stride;
      *reinterpret_cast<f32x4*>(a.part_o + stt * HD + d) = O;
      if (d == 0) *reinterpret_cast<f32x2*>(a.part_ml + 2 * stt) = f32x2{M, Ls};
    }
  }
  __syncthreads();   // LDS is free for the next piece
}

// One workgroup per (work item, KV head g): the grid is described with
// DecodeArgs.
template <typename E, typename C, int HD, int BS, int GMAX, int POL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void decode_mfma_kernel(
    DecodeArgs a) {
  using T = typename E::storage;
  __shared__ MfmaShared<HD, GMAX> sm;
  __shared__ PlanScratch sm_plan;
  const WorkItem w = work_item(a, a.num_kv_heads, sm_plan);
  if (!w.valid) return;
  const int s = uniform(w.s), g = w.unit, G = a.group;
  const int wave = uniform(threadIdx.x / kWave);
  T* out = static_cast<T*>(a.out) + ((size_t)s * a.num_q_heads + (size_t)g * G) * HD;
  if (w.t1 <= w.t0) {   // empty context: zero row
    for (int i = threadIdx.x; i < G * HD; i += 256) out[i] = E::round(0.f);
    return;
  }
  // the query heads and the blocks of the first tiles are read together
  const int ta = w.t0 / 16, tb = (w.t1 + 15) / 16;
  const int tbl0 = mfma_first_blocks<BS>(a, s, ta, wave, 4);
  if (wave == 0) mfma_load_q<E, C, HD>(a, s, g, sm.q);
  const size_t state0 = ((size_t)s * a.num_q_heads + (size_t)g * G) * a.max_parts + w.part;
  mfma_piece<E, C, HD, BS, GMAX, POL>(a, s, g, w.t1, ta, tb, tbl0, w.n == 1 ? out : nullptr, state0,
                                 a.max_parts, sm);
}

template <typename E, typename C, int HD, int BS, int GMAX>
static void launch_mfma_g(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid = a.planned ? dim3(a.num_kv_heads * a.max_parts * a.num_seqs)
                              : dim3(a.num_kv_heads * a.max_parts, 1, a.num_seqs);
  if (a.cached_kv)
    hipLaunchKernelGGL((decode_mfma_kernel<E, C, HD, BS, GMAX, 0>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<E, C, HD, BS, GMAX, kStream>), grid, dim3(256), 0, st, a);
}

template <typename E, typename C, int HD, int BS>
static hipError_t launch_mfma_t(const DecodeArgs& a, hipStream_t st) {
  if (a.group <= 4)
    launch_mfma_g<E, C, HD, BS, 4>(a, st);
  else if (a.group <= 8)
    launch_mfma_g<E, C, HD, BS, 8>(a, st);
  else
    launch_mfma_g<E, C, HD, BS, 16>(a, st);
  return hipGetLastError();
}

template <typename E, typename C, int HD, int BS>
static int occupancy_t(int group) {
  int n = 0;
  const void* f =
      group <= 4 ? reinterpret_cast<const void*>(&decode_mfma_kernel<E, C, HD, BS, 4, kStream>)
      : group <= 8 ? reinterpret_cast<const void*>(&decode_mfma_kernel<E, C, HD, BS, 8, kStream>)
                   : reinterpret_cast<const void*>(&decode_mfma_kernel<E, C, HD, BS, 16, kStream>);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, 256, 0) != hipSuccess) return 0;
  return n;
}

template <typename E, typename C>
static int occupancy_e(int hd, int bs, int group) {
  switch (hd * 100 + bs) {
    case 6416: return occupancy_t<E, C, 64, 16>(group);
    case 6432: return occupancy_t<E, C, 64, 32>(group);
    case 12816: return occupancy_t<E, C, 128, 16>(group);
    case 12832: return occupancy_t<E, C, 128, 32>(group);
  }
  return 0;
}

int decode_mfma_occupancy(Elem e, bool kv_fp8, int hd, int bs, int group) {
  switch (e) {
    case Elem::F16:
      return kv_fp8 ? occupancy_e<F16, E4M3>(hd, bs, group) : occupancy_e<F16, F16>(hd, bs, group);
    case Elem::BF16:
      return kv_fp8 ? occupancy_e<BF16, E4M3>(hd, bs, group)
                    : occupancy_e<BF16, BF16>(hd, bs, group);
    default: break;
  }
  return 0;
}

template <typename E, typename C, int HD>
static hipError_t launch_mfma_hd(int bs, const DecodeArgs& a, hipStream_t st) {
  switch (bs) {
    case 16: return launch_mfma_t<E, C, HD, 16>(a, st);
    case 32: return launch_mfma_t<E, C, HD, 32>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename E, typename C>
static hipError_t launch_mfma_e(int hd, int bs, const DecodeArgs& a, hipStream_t st) {
  switch (hd) {
    case 64: return launch_mfma_hd<E, C, 64>(bs, a, st);
    case 128: return launch_mfma_hd<E, C, 128>(bs, a, st);
  }
  return hipErrorInvalidValue;
}

bool decode_mfma_supported(Elem e, int hd, int bs) {
  return (e == Elem::F16 || e == Elem::BF16) && (hd == 64 || hd == 128) && (bs == 16 || bs == 32);
}

hipError_t launch_decode_mfma(Elem e, bool kv_fp8, int hd, int bs, const DecodeArgs& a,
                              hipStream_t st) {
  switch (e) {
    case Elem::F16:
      return kv_fp8 ? launch_mfma_e<F16, E4M3>(hd, bs, a, st) : launch_mfma_e<F16, F16>(hd, bs, a, st);
    case Elem::BF16:
      return kv_fp8 ? launch_mfma_e<BF16, E4M3>(hd, bs, a, st)
                    : launch_mfma_e<BF16, BF16>(hd, bs, a, st);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
