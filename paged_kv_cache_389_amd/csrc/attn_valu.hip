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
#include "order.h"

namespace pkv {

template <typename E, int HD, int BS>
struct ValuTiling {
  static constexpr int VEC = E::kVec;            // elements per 16-byte load
  static constexpr int LPR = HD / VEC;           // lanes per token row
  static constexpr int RPI = kWave / LPR;        // token rows per load instruction
  static constexpr int LPB = BS / RPI;           // load instructions per block
  static constexpr int CH = LPB < 4 ? LPB : 4;   // load instructions per unit
  static constexpr int UT = CH * RPI;            // tokens per unit
  static constexpr int UPB = BS / UT;            // units per block
  static_assert(RPI * LPR == kWave && BS % RPI == 0 && LPB % CH == 0, "unsupported shape");
};

int valu_unit_tokens(Elem e, int head_dim, int block_size) {
  const int vec = e == Elem::F32 ? 4 : 8;
  const int rpi = kWave / (head_dim / vec);
  const int lpb = block_size / rpi;
  return (lpb < 4 ? lpb : 4) * rpi;
}

template <typename E, int HD, int BS>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
  using T = typename E::storage;
  using Tl = ValuTiling<E, HD, BS>;
  constexpr int VEC = Tl::VEC, LPR = Tl::LPR, RPI = Tl::RPI, CH = Tl::CH, UT = Tl::UT,
                UPB = Tl::UPB;
  constexpr int NW = 4;

  const int part = blockIdx.x, h = blockIdx.y;
  __shared__ OrderScratch sm_order;
  const int s = uniform(a.order_mode == 2 ? sorted_sequence(a.context_lens, a.num_seqs,
                                                            a.len_cap, blockIdx.z, sm_order)
                                          : sequence_of(a, blockIdx.z));
  const int tid = threadIdx.x, wave = uniform(tid / kWave), lane = tid % kWave;
  const int row = lane / LPR, col = lane % LPR;
  const int P = a.part_tokens;
  const int tok_begin = part * P;
  const int unit_begin = tok_begin / UT;
  const int g = h / a.group;

  // independent loads first: the length, the query slice, this wave's table entries
  int L = a.context_lens[s];
  const T* qrow = static_cast<const T*>(a.q) + ((size_t)s * a.num_q_heads + h) * HD;
  const u32x4 qv = ld16(qrow + col * VEC);
  int tbl;
  {
    const int blk = min((unit_begin + wave + NW * lane) / UPB, a.max_blocks - 1);
    tbl = a.contiguous ? s * a.max_blocks + blk : a.block_tables[(size_t)s * a.max_blocks + blk];
  }

  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  T* out = static_cast<T*>(a.out) + ((size_t)s * a.num_q_heads + h) * HD;
  if (L == 0) {
    if (part == 0)
      for (int d = tid; d < HD; d += 256) out[d] = E::round(0.f);
    return;
  }
  if (tok_begin >= L) return;
  const int tok_end = min(L, tok_begin + P);
  const int nparts = (L + P - 1) / P;
  const int n_units = (tok_end + UT - 1) / UT - unit_begin;   // <= 4 * 64
  const int mine = n_units > wave ? (n_units - wave + NW - 1) / NW : 0;

  // unit addresses: a buffer descriptor over the unit's tile rows, built in
  // scalar registers, plus a constant 32-bit per-lane byte offset, so no
  // per-unit address arithmetic runs on the vector ALU
  const size_t block_bytes = (size_t)a.num_kv_heads * BS * HD * sizeof(T);
  const char* kbase = static_cast<const char*>(a.k_cache) + (size_t)g * BS * HD * sizeof(T);
  const char* vbase = static_cast<const char*>(a.v_cache) + (size_t)g * BS * HD * sizeof(T);
  const uint32_t loff = (uint32_t)((row * HD + col * VEC) * sizeof(T));

  float m = -INFINITY, l = 0.f, o[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) o[e] = 0.f;
  int bad = 0;

  // issue the loads of the wave's i-th unit
  auto load_unit = [&](int i, u32x4* kr, u32x4* vr) {
    const int u = unit_begin + wave + NW * i;
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
    for (int c = 0; c < CH; ++c) kr[c] = bld16(kt, loff, c * RPI * HD * sizeof(T));
#pragma unroll
    for (int c = 0; c < CH; ++c) vr[c] = bld16(vt, loff, c * RPI * HD * sizeof(T));
  };

  // fold the wave's i-th unit into the online state
  auto compute_unit = [&](int i, const u32x4* kr, const u32x4* vr) {
    const int u = unit_begin + wave + NW * i;
    float sc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) sc[c] = group_sum<LPR>(E::dot16(kr[c], qv, 0.f)) * a.scale_log2e;
    if ((u + 1) * UT <= tok_end) {
      // every token of the unit is inside the partition
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
        E::unpack16(vr[c], vf);
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = __builtin_fmaf(p, vf[e], o[e]);
      }
    } else {
      // the partition's last unit: tokens at or past tok_end are masked by
      // index, never by arithmetic, so whatever those slots hold cannot
      // reach the result
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
          E::unpack16(vr[c], vf);
#pragma unroll
          for (int e = 0; e < VEC; ++e) o[e] = __builtin_fmaf(p, vf[e], o[e]);
        }
      }
    }
  };

  // two register buffers: the loads of unit i+1 are in flight while unit i
  // is computed
  u32x4 kA[CH], vA[CH], kB[CH], vB[CH];
  if (mine > 0) {
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

  // merge the wave's RPI row groups (lanes that differ in `row`)
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
    const float mo = __shfl_xor(m, off, 64);
    const float lo = __shfl_xor(l, off, 64);
    const float mn = fmaxf(m, mo);
    const float mu = (mn == -INFINITY) ? 0.f : mn;
    const float wa = fast_exp2(m - mu), wb = fast_exp2(mo - mu);
    l = l * wa + lo * wb;
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] = o[e] * wa + __shfl_xor(o[e], off, 64) * wb;
    m = mn;
  }

  // merge the 4 waves in LDS
  __shared__ float sm_m[NW], sm_l[NW];
  __shared__ __attribute__((aligned(16))) float sm_o[NW][HD];
  __shared__ int sm_bad[NW];
  if (lane == 0) {
    sm_m[wave] = m;
    sm_l[wave] = l;
  }
  if (row == 0) {
#pragma unroll
    for (int e = 0; e < VEC; e += 4)
      *reinterpret_cast<f32x4*>(&sm_o[wave][col * VEC + e]) = f32x4{o[e], o[e + 1], o[e + 2], o[e + 3]};
  }
  const int any_bad = __any(bad);
  if (lane == 0) sm_bad[wave] = any_bad;
  __syncthreads();
  if (wave != 0 || row != 0) return;

  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w]);
  float wt[NW], Ls = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    wt[w] = fast_exp2(sm_m[w] - M);   // M is finite: this partition has a token
    Ls = __builtin_fmaf(wt[w], sm_l[w], Ls);
  }
  float O[VEC];
#pragma unroll
  for (int e = 0; e < VEC; e += 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) acc += wt[w] * *reinterpret_cast<const f32x4*>(&sm_o[w][col * VEC + e]);
    O[e] = acc[0];
    O[e + 1] = acc[1];
    O[e + 2] = acc[2];
    O[e + 3] = acc[3];
  }
  if (sm_bad[0] | sm_bad[1] | sm_bad[2] | sm_bad[3]) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) O[e] = __builtin_nanf("");
  }
  if (nparts == 1) {
    const float inv = 1.f / Ls;
#pragma unroll
    for (int e = 0; e < VEC; ++e) O[e] *= inv;
    store_rounded<E, VEC>(out + col * VEC, O);
  } else {
    const size_t pidx = ((size_t)s * a.num_q_heads + h) * a.max_parts + part;
    float* po = a.part_o + pidx * HD + col * VEC;
#pragma unroll
    for (int e = 0; e < VEC; e += 4)
      *reinterpret_cast<f32x4*>(po + e) = f32x4{O[e], O[e + 1], O[e + 2], O[e + 3]};
    if (col == 0) *reinterpret_cast<f32x2*>(a.part_ml + 2 * pidx) = f32x2{M, Ls};
  }
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

}  // namespace pkv
