// Paged decode attention, vector-ALU variant (one query head per workgroup).
//
// A workgroup (4 waves) computes one query head of one sequence over one
// partition of its context.  The sequence's KV lives in fixed-size physical
// blocks reached through its block table ("Memory Optimization in LLM
// Serving with PagedAttention", section "How PagedAttention Works"); only the
// last block is partly filled, and its tail is masked by token index.
//
// Work unit: UT consecutive tokens of one block (UT = CH * RPI, at most a
// whole block).  A wave reads a unit's K rows and V rows with CH 16-byte
// loads each: LPR lanes cover one token row of head_dim elements and one
// load instruction covers RPI whole rows, so every load is fully coalesced.
// Each lane keeps the 16 bytes of the query that match its columns; a row's
// dot product is LPR partial dot products (v_dot2 for 16-bit types) summed
// across the row with DPP.
//
// Latency hiding: wave w takes units w, w+4, w+8, ... of the partition.  The
// physical block of each of its units is fetched up front with one vector
// load (lane i holds the entry of the wave's i-th unit), so no unit waits on
// a table read, and the loads of unit i+1 are issued before unit i is
// computed (two register buffers), so every wave keeps loads in flight.
//
// Softmax: every row group of a wave keeps its own online state (running
// max m in log2 units, running sum l, unnormalised output o) over the tokens
// it sees; the states are merged across row groups with lane shuffles and
// across waves in LDS.  When the context is split into several partitions,
// each partition stores (m, l, o) in fp32 and attn_reduce.hip merges them.
#include "common.h"
#include "decode.h"

namespace pkv {

template <typename C, int HD, int BS>
struct ValuTiling {
  static constexpr int VEC = C::kVec;            // cache elements per 16-byte load
  static constexpr int LPR = HD / VEC;           // lanes per token row
  static constexpr int RPI = kWave / LPR;        // token rows per load instruction
  static constexpr int LPB = BS / RPI;           // load instructions per block
  static constexpr int CH = LPB < 4 ? LPB : 4;   // load instructions per unit
  static constexpr int UT = CH * RPI;            // tokens per unit
  static constexpr int UPB = BS / UT;            // units per block
  static_assert(RPI * LPR == kWave && BS % RPI == 0 && LPB % CH == 0, "unsupported shape");
};

int valu_unit_tokens(Elem e, bool kv_fp8, int head_dim, int block_size) {
  const int vec = kv_fp8 ? 16 : (e == Elem::F32 ? 4 : 8);
  const int rpi = kWave / (head_dim / vec);
  const int lpb = block_size / rpi;
  return (lpb < 4 ? lpb : 4) * rpi;
}

// LDS of one workgroup: the four waves' softmax states.
template <int HD>
struct ValuShared {
  float m[4], l[4];
  __attribute__((aligned(16))) float o[4][HD];
  int bad[4];
};

// One lane's online softmax state: running max m (log2 units), running sum
// l and unnormalised output o over its columns; bad is set when a table
// entry fell outside the pool.
template <int VEC>
struct ValuState {
  float m, l, o[VEC];
  int bad;
};

// What a wave must read before streaming a piece: its lane's query
// elements (QW 16-byte words: the VEC columns it covers) and the physical
// blocks of its first 64 units.
template <int QW>
struct ValuMeta {
  u32x4 q[QW];
  int tbl;
};

// Issue the loads of a piece's ValuMeta (units ta + first + stride*i).
template <typename E, typename C, int HD, int BS>
__device__ inline ValuMeta<KvDot<E, C>::QW> valu_meta(const DecodeArgs& a, int s, int h, int ta,
                                                      int first, int stride) {
  using T = typename E::storage;
  using Tl = ValuTiling<C, HD, BS>;
  constexpr int QW = KvDot<E, C>::QW;
  const int lane = threadIdx.x % kWave, col = lane % Tl::LPR;
  const T* qrow = static_cast<const T*>(a.q) + ((size_t)s * a.num_q_heads + h) * HD;
  ValuMeta<QW> mt;
#pragma unroll
  for (int j = 0; j < QW; ++j) mt.q[j] = ld16(qrow + col * Tl::VEC + j * (16 / sizeof(T)));
  const int blk = min((ta + first + stride * lane) / Tl::UPB, a.max_blocks - 1);
  mt.tbl = a.contiguous ? s * a.max_blocks + blk : a.block_tables[(size_t)s * a.max_blocks + blk];
  return mt;
}

// Fold units ta + first, ta + first + stride, ... (< tb) of query head h of
// sequence s (unit = UT tokens; tokens at or past L > 0 are masked) into the
// calling wave's state, given the piece's ValuMeta.  Row group `row` of the wave
// sees every RPI-th token.
template <typename E, typename C, int HD, int BS, int POL>
__device__ inline void valu_accumulate(const DecodeArgs& a, int s, int h, int L, int ta, int tb,
                                       int first, int stride,
                                       const ValuMeta<KvDot<E, C>::QW>& meta,
                                       ValuState<ValuTiling<C, HD, BS>::VEC>& st) {
  using T = typename C::storage;   // cache element
  using Tl = ValuTiling<C, HD, BS>;
  constexpr int VEC = Tl::VEC, LPR = Tl::LPR, RPI = Tl::RPI, CH = Tl::CH, UT = Tl::UT,
                UPB = Tl::UPB;
  const int lane = threadIdx.x % kWave;
  const int row = lane / LPR, col = lane % LPR;
  const int g = h / a.group;
  const int tok_end = L;

  // unit addresses: a buffer descriptor over the unit's tile rows, built in
  // scalar registers, plus a constant 32-bit per-lane byte offset, so no
  // per-unit address arithmetic runs on the vector ALU
  const size_t block_bytes = (size_t)a.num_kv_heads * BS * HD * sizeof(T);
  const char* kbase = static_cast<const char*>(a.k_cache) + (size_t)g * BS * HD * sizeof(T);
  const char* vbase = static_cast<const char*>(a.v_cache) + (size_t)g * BS * HD * sizeof(T);
  const uint32_t loff = (uint32_t)((row * HD + col * VEC) * sizeof(T));
  const int32_t* table = a.block_tables + (size_t)s * a.max_blocks;

  float m = st.m, l = st.l, o[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) o[e] = st.o[e];
  int bad = st.bad;

  // passes of at most 64 of the wave's units: their table entries fit one
  // VGPR (the first pass's come with the meta)
  for (int pass = ta + first; pass < tb; pass += kWave * stride) {
    const int mine = min(kWave, (tb - pass + stride - 1) / stride);
    int tbl = meta.tbl;
    if (pass != ta + first) {
      const int blk = min((pass + stride * lane) / UPB, a.max_blocks - 1);
      tbl = a.contiguous ? s * a.max_blocks + blk : table[blk];
    }

    // issue the loads of the wave's i-th unit of the pass
    auto load_unit = [&](int i, u32x4* kr, u32x4* vr) {
      const int u = pass + stride * i;
      int phys = lane_value(tbl, i);
      if ((unsigned)phys >= (unsigned)a.num_blocks) {
        bad = 1;
        phys = 0;
      }
      const size_t off = (size_t)phys * block_bytes + (size_t)(u % UPB) * UT * HD * sizeof(T);
      constexpr uint32_t kUnitBytes = UT * HD * sizeof(T);
      const rsrc_t kt = make_rsrc(kbase + off, kUnitBytes);
      const rsrc_t vt = make_rsrc(vbase + off, kUnitBytes);
#pragma unroll
      for (int c = 0; c < CH; ++c) kr[c] = bld16<POL>(kt, loff, c * RPI * HD * sizeof(T));
#pragma unroll
      for (int c = 0; c < CH; ++c) vr[c] = bld16<POL>(vt, loff, c * RPI * HD * sizeof(T));
    };

    // fold the wave's i-th unit into the online state
    auto compute_unit = [&](int i, const u32x4* kr, const u32x4* vr) {
      const int u = pass + stride * i;
      float sc[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c)
        sc[c] = group_sum<LPR>(KvDot<E, C>::dot(kr[c], meta.q)) * a.scale_log2e;
      if ((u + 1) * UT <= tok_end) {
        // every token of the unit is inside the context
        float mb = sc[0];
#pragma unroll
        for (int c = 1; c < CH; ++c) mb = fmaxf(mb, sc[c]);
        const float mn = fmaxf(m, mb);
        const float corr = fast_exp2(m - mn);
        m = mn;
        l *= corr;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] *= corr;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const float p = fast_exp2(sc[c] - mn);
          l += p;
          float vf[VEC];
          C::unpack16(vr[c], vf);
#pragma unroll
          for (int e = 0; e < VEC; ++e) o[e] = __builtin_fmaf(p, vf[e], o[e]);
        }
      } else {
        // the sequence's last unit: tokens at or past the context length are
        // masked by index, never by arithmetic, so whatever those slots hold
        // cannot reach the result
        const int t0 = u * UT + row;
        float mb = -INFINITY;
#pragma unroll
        for (int c = 0; c < CH; ++c)
          if (t0 + c * RPI < tok_end) mb = fmaxf(mb, sc[c]);
        const float mn = fmaxf(m, mb);
        const float mu = (mn == -INFINITY) ? 0.f : mn;
        const float corr = fast_exp2(m - mu);
        m = mn;
        l *= corr;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] *= corr;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          if (t0 + c * RPI < tok_end) {
            const float p = fast_exp2(sc[c] - mu);
            l += p;
            float vf[VEC];
            C::unpack16(vr[c], vf);
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] = __builtin_fmaf(p, vf[e], o[e]);
          }
        }
      }
    };

    // two register buffers: the loads of unit i+1 are in flight while unit i
    // is computed
    u32x4 kA[CH], vA[CH], kB[CH], vB[CH];
    load_unit(0, kA, vA);
    int i = 0;
    // steady state: the loads of the next unit are always issued, so the
    // wait before each unit's math covers only that unit's own loads
    for (; i + 2 < mine; i += 2) {
      load_unit(i + 1, kB, vB);
      compute_unit(i, kA, vA);
      load_unit(i + 2, kA, vA);
      compute_unit(i + 1, kB, vB);
    }
    if (i + 1 < mine) {
      load_unit(i + 1, kB, vB);
      compute_unit(i, kA, vA);
      compute_unit(i + 1, kB, vB);
    } else {
      compute_unit(i, kA, vA);
    }
  }
  st.m = m;
  st.l = l;
#pragma unroll
  for (int e = 0; e < VEC; ++e) st.o[e] = o[e];
  st.bad = bad;
}

// Merge the wave's RPI row groups (lanes that differ in `row`): afterwards
// every lane holds the wave's state for its columns.
template <int VEC, int LPR>
__device__ inline void valu_row_merge(ValuState<VEC>& st) {
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
    const float mo = __shfl_xor(st.m, off, 64);
    const float lo = __shfl_xor(st.l, off, 64);
    const float mn = fmaxf(st.m, mo);
    const float mu = (mn == -INFINITY) ? 0.f : mn;
    const float wa = fast_exp2(st.m - mu), wb = fast_exp2(mo - mu);
    st.l = st.l * wa + lo * wb;
#pragma unroll
    for (int e = 0; e < VEC; ++e) st.o[e] = st.o[e] * wa + __shfl_xor(st.o[e], off, 64) * wb;
    st.m = mn;
  }
}

// Store a merged state's VEC columns at col*VEC: normalised and rounded into
// out when out is not null, else unnormalised to po and (max, sum) to pml.
// kScaled: O is in code units of an 8-bit cache and is multiplied by the V
// scale first (a per-cache constant, so it commutes with every merge).
template <typename E, int VEC, bool kScaled>
__device__ inline void valu_emit(float M, float Ls, float* O, bool bad, int col, float v_scale,
                                 typename E::storage* out, float* po, float* pml) {
  if constexpr (kScaled) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) O[e] *= v_scale;
  }
  if (bad) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) O[e] = __builtin_nanf("");
  }
  if (out) {
    const float inv = 1.f / Ls;
#pragma unroll
    for (int e = 0; e < VEC; ++e) O[e] *= inv;
    store_rounded<E, VEC>(out + col * VEC, O);
  } else {
#pragma unroll
    for (int e = 0; e < VEC; e += 4)
      *reinterpret_cast<f32x4*>(po + col * VEC + e) = f32x4{O[e], O[e + 1], O[e + 2], O[e + 3]};
    if (col == 0) *reinterpret_cast<f32x2*>(pml) = f32x2{M, Ls};
  }
}

// Attention of query head h of sequence s over its units [ta, tb) (tokens
// at or past L > 0 masked), by the four waves of the workgroup (unit round-robin),
// merged in LDS.  Result as in valu_emit.
template <typename E, typename C, int HD, int BS, int POL>
__device__ inline void valu_piece(const DecodeArgs& a, int s, int h, int L, int ta, int tb,
                                  const ValuMeta<KvDot<E, C>::QW>& meta,
                                  typename E::storage* out, float* po, float* pml,
                                  ValuShared<HD>& sm) {
  using Tl = ValuTiling<C, HD, BS>;
  constexpr int VEC = Tl::VEC, LPR = Tl::LPR;
  constexpr int NW = 4;
  const int tid = threadIdx.x, wave = uniform(tid / kWave), lane = tid % kWave;
  const int row = lane / LPR, col = lane % LPR;
  ValuState<VEC> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int e = 0; e < VEC; ++e) st.o[e] = 0.f;
  st.bad = 0;
  valu_accumulate<E, C, HD, BS, POL>(a, s, h, L, ta, tb, wave, NW, meta, st);
  valu_row_merge<VEC, LPR>(st);

  // merge the 4 waves in LDS
  if (lane == 0) {
    sm.m[wave] = st.m;
    sm.l[wave] = st.l;
  }
  if (row == 0) {
#pragma unroll
    for (int e = 0; e < VEC; e += 4)
      *reinterpret_cast<f32x4*>(&sm.o[wave][col * VEC + e]) =
          f32x4{st.o[e], st.o[e + 1], st.o[e + 2], st.o[e + 3]};
  }
  const int any_bad = __any(st.bad);
  if (lane == 0) sm.bad[wave] = any_bad;
  __syncthreads();
  if (wave == 0 && row == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.m[w]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float wt[NW], Ls = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      wt[w] = fast_exp2(sm.m[w] - Mu);
      Ls = __builtin_fmaf(wt[w], sm.l[w], Ls);
    }
    float O[VEC];
#pragma unroll
    for (int e = 0; e < VEC; e += 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NW; ++w)
        acc += wt[w] * *reinterpret_cast<const f32x4*>(&sm.o[w][col * VEC + e]);
      O[e] = acc[0];
      O[e + 1] = acc[1];
      O[e + 2] = acc[2];
      O[e + 3] = acc[3];
    }
    valu_emit<E, VEC, !__is_same(E, C)>(M, Ls, O, sm.bad[0] | sm.bad[1] | sm.bad[2] | sm.bad[3],
                                        col, a.v_scale, out, po, pml);
  }
  __syncthreads();   // the LDS states are free for the next piece
}

// One workgroup per (work item, query head h): the grid is described with
// DecodeArgs.
// POL: cache policy of the K/V loads (kStream, or 0 when blocks are shared
// across the batch; DecodeArgs::cached_kv).
template <typename E, typename C, int HD, int BS, int POL>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
  using T = typename E::storage;
  constexpr int UT = ValuTiling<C, HD, BS>::UT;
  __shared__ ValuShared<HD> sm;
  __shared__ PlanScratch sm_plan;
  const WorkItem w = work_item(a, a.num_q_heads, sm_plan);
  if (!w.valid) return;
  const int s = uniform(w.s), h = w.unit;
  T* out = static_cast<T*>(a.out) + ((size_t)s * a.num_q_heads + h) * HD;
  if (w.t1 <= w.t0) {   // empty context: zero row
    for (int d = threadIdx.x; d < HD; d += 256) out[d] = E::round(0.f);
    return;
  }
  // the query slice and the blocks of the first units are read together
  const int ta = w.t0 / UT, tb = (w.t1 + UT - 1) / UT;
  const auto meta = valu_meta<E, C, HD, BS>(a, s, h, ta, uniform(threadIdx.x / kWave), 4);
  const size_t pidx = ((size_t)s * a.num_q_heads + h) * a.max_parts + w.part;
  valu_piece<E, C, HD, BS, POL>(a, s, h, w.t1, ta, tb, meta, w.n == 1 ? out : nullptr,
                           a.part_o + pidx * HD, a.part_ml + 2 * pidx, sm);
}

// ------------------------------------------------------------------ dispatch

// 8-bit caches need RPI = 64 / (HD / 16) rows per load to divide the block.
template <typename C, int HD, int BS>
constexpr bool valu_shape_ok() {
  return kWave % (HD / C::kVec) == 0 && BS % (kWave / (HD / C::kVec)) == 0;
}

template <typename E, typename C, int HD, int BS>
static hipError_t launch_valu_t(const DecodeArgs& a, hipStream_t st) {
  if constexpr (!valu_shape_ok<C, HD, BS>()) {
    return hipErrorInvalidValue;
  } else {
    const dim3 grid = a.planned ? dim3(a.num_q_heads * a.max_parts * a.num_seqs)
                                : dim3(a.num_q_heads * a.max_parts, 1, a.num_seqs);
    if (a.cached_kv)
      hipLaunchKernelGGL((decode_valu_kernel<E, C, HD, BS, 0>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((decode_valu_kernel<E, C, HD, BS, kStream>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
}

template <typename E, typename C, int HD, int BS>
static int occupancy_t() {
  if constexpr (!valu_shape_ok<C, HD, BS>()) {
    return 0;
  } else {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(&decode_valu_kernel<E, C, HD, BS, kStream>), 256, 0) !=
        hipSuccess)
      return 0;
    return n;
  }
}

template <typename E, typename C, int HD>
static hipError_t launch_valu_hd(int bs, const DecodeArgs& a, hipStream_t st) {
  switch (bs) {
    case 8: return launch_valu_t<E, C, HD, 8>(a, st);
    case 16: return launch_valu_t<E, C, HD, 16>(a, st);
    case 32: return launch_valu_t<E, C, HD, 32>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename E, typename C>
static hipError_t launch_valu_e(int hd, int bs, const DecodeArgs& a, hipStream_t st) {
  switch (hd) {
    case 64: return launch_valu_hd<E, C, 64>(bs, a, st);
    case 128: return launch_valu_hd<E, C, 128>(bs, a, st);
    case 256: return launch_valu_hd<E, C, 256>(bs, a, st);
  }
  return hipErrorInvalidValue;
}

template <typename E, typename C>
static int occupancy_e(int hd, int bs) {
  switch (hd * 100 + bs) {
    case 6408: return occupancy_t<E, C, 64, 8>();
    case 6416: return occupancy_t<E, C, 64, 16>();
    case 6432: return occupancy_t<E, C, 64, 32>();
    case 12808: return occupancy_t<E, C, 128, 8>();
    case 12816: return occupancy_t<E, C, 128, 16>();
    case 12832: return occupancy_t<E, C, 128, 32>();
    case 25608: return occupancy_t<E, C, 256, 8>();
    case 25616: return occupancy_t<E, C, 256, 16>();
    case 25632: return occupancy_t<E, C, 256, 32>();
  }
  return 0;
}

int decode_valu_occupancy(Elem e, bool kv_fp8, int hd, int bs) {
  switch (e) {
    case Elem::F32: return kv_fp8 ? occupancy_e<F32, E4M3>(hd, bs) : occupancy_e<F32, F32>(hd, bs);
    case Elem::F16: return kv_fp8 ? occupancy_e<F16, E4M3>(hd, bs) : occupancy_e<F16, F16>(hd, bs);
    case Elem::BF16:
      return kv_fp8 ? occupancy_e<BF16, E4M3>(hd, bs) : occupancy_e<BF16, BF16>(hd, bs);
  }
  return 0;
}

bool decode_valu_supported(Elem e, bool kv_fp8, int hd, int bs) {
  (void)e;
  if (!(hd == 64 || hd == 128 || hd == 256) || !(bs == 8 || bs == 16 || bs == 32)) return false;
  return !(kv_fp8 && hd == 64 && bs == 8);   // 16 rows per 8-bit load exceed the block
}

hipError_t launch_decode_valu(Elem e, bool kv_fp8, int hd, int bs, const DecodeArgs& a,
                              hipStream_t st) {
  switch (e) {
    case Elem::F32:
      return kv_fp8 ? launch_valu_e<F32, E4M3>(hd, bs, a, st) : launch_valu_e<F32, F32>(hd, bs, a, st);
    case Elem::F16:
      return kv_fp8 ? launch_valu_e<F16, E4M3>(hd, bs, a, st) : launch_valu_e<F16, F16>(hd, bs, a, st);
    case Elem::BF16:
      return kv_fp8 ? launch_valu_e<BF16, E4M3>(hd, bs, a, st)
                    : launch_valu_e<BF16, BF16>(hd, bs, a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
