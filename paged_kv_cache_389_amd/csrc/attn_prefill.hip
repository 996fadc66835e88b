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
// A workgroup of four waves takes consecutive query tokens of one
// (sequence, KV head); a wave owns kPrefillGroups groups of 16 query
// columns, each 16/G query tokens times the G query heads of the KV head.
// Workgroups go out sequence by sequence, longest context first (batches of
// up to 64 sequences; larger ones in index order), and each sequence's
// chunks latest-first, so that the heaviest work starts early.
// The context is walked in tiles of 32 tokens (two 16-token units, each in
// its own block or half block), and each tile's K and V rows are loaded
// once for the workgroup, straight into LDS (16-byte buffer loads that
// write LDS): wave w loads unit w & 1 of K (w < 2) or of V (w >= 2).  Tiles
// are double-buffered with one barrier per tile: the loads of tile j + 1 are
// issued right after the barrier that opens tile j, so they have a whole
// tile of work to land.  The two buffers are separate LDS objects and the
// tile loop is unrolled by two, so that each read names its buffer at
// compile time and the compiler does not make it wait for the loads in
// flight into the other one.  The rows of a tile sit in LDS with their 16-byte
// chunks swizzled (chunk c of row r at c ^ swz(r)), so that the operand
// reads below touch distinct banks.  Per tile, the score products of every
// group are issued back to back (the tile's V reads go out among them), the
// column maxima follow, and whether any reference must move is decided once
// for the tile.  Per tile and group:
//
//   S^T = K Q^T       per unit, 16x16x32 MFMAs over the head dim (K rows as
//                     the A operand, read from LDS; Q^T, the B operand, held
//                     in the wave's registers for the whole kernel);
//   P = exp2(S^T c - m)   one FMA and one exp2 per score, c the positive
//                     softmax factor in log2 units (a negative scale is
//                     moved into Q, whose sign flip is exact), m a per-column
//                     reference maximum that moves only when a tile passes
//                     it by more than kPrefillSlack (the normalised result
//                     does not depend on the reference);
//   O^T += V^T P^T    one 16x16x32 MFMA per 16 output dims and group, whose
//                     32-deep contraction runs over both units of the tile:
//                     a lane's score registers hold tokens 4*g4 .. 4*g4 + 3
//                     of each unit, which is exactly its B operand; the same
//                     eight tokens' V values at one dim form its A operand,
//                     read by two transposing LDS reads (ds_read_b64_tr_b16)
//                     for 16-bit caches (output row n of product e is dim
//                     16*e + n), and for 8-bit codes widened from the lane's
//                     V rows at DPL consecutive dims and regrouped into token
//                     pairs per dim by v_perm (row n of product e: dim
//                     DPL*n + e); either way all of a tile's V reads are
//                     issued once its score products are, into the K
//                     operands' registers.
//
// The row sums take the probabilities as rounded for the product (a dot2
// against ones), so numerator and denominator use the same values.  Loads
// go through buffer descriptors whose range ends with the context, so rows
// past it read as zeros (and their scores are masked); the causal bound of
// each column masks by index only in the tiles that reach past the wave's
// smallest bound.  No cross-wave merge is needed: a wave owns its columns'
// whole context; a wave whose columns end before the workgroup's last tile
// keeps loading its share and skips the arithmetic.
#include "common.h"
#include "decode.h"
#include "mfma_ops.h"

namespace pkv {

// How far (log2 units) a tile's maximum may pass the reference maximum
// before the accumulators are rescaled: probabilities stay below 2^8.
constexpr float kPrefillSlack = 8.f;

// Column groups of 16 per wave: each K/V tile serves 4 * CG groups.
constexpr int kPrefillGroups = 3;

template <typename C, int HD>
struct PrefillShared {
  static constexpr int kTile = 32 * HD * (int)sizeof(typename C::storage);   // bytes of 32 rows
  __attribute__((aligned(16))) unsigned char kv[2][kTile];   // [K, V][32 swizzled rows]
};

__device__ inline float max3f(float x, float y, float z) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(x, y), z);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Position of the 16-byte chunks of tile row r in LDS: chunk c sits at
// c ^ swz(r).  With 16 chunks per row the rows of a 16-row unit get 16
// distinct values, so the K operand reads (16 rows, one chunk) and the V
// transposing reads (4 rows, 8 of their chunks) each touch distinct banks.
template <int NCH>
__device__ constexpr int swz(int r) {
  if constexpr (NCH == 16) return ((r & 7) << 1) | ((r >> 3) & 1);
  else return r & (NCH - 1);
}

// 16-byte buffer load that writes LDS: lane l's 16 bytes (at lane_off in
// the buffer) land at dst + 16 * l; dst must be wave-uniform.  Its wait is
// the vector-memory counter.  (A plain device function: the builtin has no
// host form, and a lambda body is also compiled for the host.)
__device__ inline void buffer_load_lds16(rsrc_t r, unsigned char* dst, uint32_t lane_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, lane_off, 0, 0, 0);
}
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) const u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) const uint32_t lds_u32;

// C is the cache element: E itself, or E4M3 codes (16 codes of a K row per
// read, feeding two k-steps; V rows at half width), widened to E right
// before the products, as in the decode MFMA kernel; the K scale is folded
// into scale_log2e and the V scale multiplies the output.
template <typename E, typename C, int HD, int BS, int CG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_mfma_kernel(
    PrefillArgs a) {
  using TQ = typename E::storage;   // query and output
  using T = typename C::storage;    // cache element
  using Ops = MfmaOps<E>;
  using SM = PrefillShared<C, HD>;
  constexpr bool k8 = sizeof(T) == 1;
  constexpr int KSTEPS = HD / 32;
  constexpr int DPL = HD / 16;                   // output dims per lane and column
  constexpr int VW = DPL / 2;                    // dwords of one V row's DPL dims (16-bit)
  constexpr int KL = k8 ? KSTEPS / 2 : KSTEPS;   // 16-byte K reads per unit
  constexpr int VL = k8 ? VW / 2 : VW;           // dwords of V read per row
  constexpr int TPB = BS / 16;                   // 16-token units per block
  constexpr int kRow = HD * (int)sizeof(T);      // bytes of one token row of one head
  constexpr int NCH = kRow / 16;                 // 16-byte chunks per row
  constexpr int LPU = 16 * kRow / 1024;          // 1 KiB loads per unit
  static_assert(HD % 32 == 0 && BS % 16 == 0 && (VW == 2 || VW == 4) && LPU >= 1,
                "unsupported shape");
  __shared__ SM sm0;
  __shared__ SM sm1;

  const int g = blockIdx.x % a.num_kv_heads;
  // heaviest query chunks (latest positions) first
  const int chunk = a.chunks - 1 - (int)(blockIdx.x / a.num_kv_heads);
  // sequences longest first (batches of up to 64 sequences): blockIdx.z
  // is the rank of the sequence's context length (ties by index)
  int s = blockIdx.z;
  if (a.num_seqs <= kWave) {
    const int li = threadIdx.x % kWave;
    const int Li = li < a.num_seqs ? a.context_lens[li] : INT32_MIN;
    int r = 0;
    for (int t = 0; t < a.num_seqs; ++t) {
      const int Lt = __builtin_amdgcn_readlane(Li, t);
      r += (Lt > Li || (Lt == Li && t < li)) ? 1 : 0;
    }
    const unsigned long long m = __ballot(li < a.num_seqs && r == (int)blockIdx.z);
    s = __builtin_ctzll(m);
  }
  const int lane = threadIdx.x % kWave, wave = uniform(threadIdx.x / kWave);
  const int n = lane & 15, g4 = lane >> 4;
  const int G = a.group, tpg = 16 / G, tpw = CG * tpg;   // query tokens per group / wave

  int q0 = load_uniform(a.query_start + s), q1 = load_uniform(a.query_start + s + 1);
  q0 = min(max(q0, 0), a.total_q);
  q1 = min(max(q1, q0), a.total_q);
  const int nq = q1 - q0;
  int L = load_uniform(a.context_lens + s);
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int wg_first = chunk * 4 * tpw;
  if (wg_first >= nq) return;   // the whole workgroup: no barrier has been reached
  // tokens the workgroup reads: up to the bound of its last query token
  const int wg_lim = max(0, L - nq + min(nq, wg_first + 4 * tpw));
  const int wg_units = (wg_lim + 15) / 16;
  const int wg_tiles = (wg_units + 1) / 2;
  const int first = wg_first + wave * tpw;   // the wave's first query token

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
  const int my_tiles = (lim_max + 31) / 32;   // tiles this wave computes (<= wg_tiles)

  int my_bad = INT32_MAX;   // first tile whose share this wave loaded named a block outside the pool
  // ---- this wave's share of every tile: unit `mu` of K (waves 0, 1) or V
  const int mu = wave & 1;
  const char* src = static_cast<const char*>(wave < 2 ? a.k_cache : a.v_cache) +
                    (size_t)g * BS * kRow;
  const size_t block_bytes = (size_t)a.num_kv_heads * BS * kRow;
  const int32_t* table = a.block_tables + (size_t)s * a.max_blocks;
  // lane l of load q writes LDS bytes q * 1024 + 16 * l of the unit, which
  // hold chunk (slot ^ swizzle) of row (q * 1024 + 16 * l) / kRow
  uint32_t src_off[LPU];
#pragma unroll
  for (int q = 0; q < LPU; ++q) {
    const int slot = q * 1024 + 16 * lane;
    const int row = slot / kRow, ch = (slot % kRow) / 16;
    src_off[q] = (uint32_t)(row * kRow + ((ch ^ swz<NCH>(16 * mu + row)) * 16));
  }
  // table entries of 64 units per window, one vector load each
  int wbase = 0;
  int tbl = table[min(lane / TPB, a.max_blocks - 1)];
  auto load_tile = [&](int j, SM& buf) {
    const int u = 2 * j + mu;
    if (u >= wbase + 64) {
      wbase += 64;
      tbl = table[min((wbase + lane) / TPB, a.max_blocks - 1)];
    }
    const bool live = u < wg_units;
    int phys = live ? lane_value(tbl, u - wbase) : 0;
    if (live && (unsigned)phys >= (unsigned)a.num_blocks) {
      my_bad = min(my_bad, j);
      phys = 0;
    }
    const uint32_t bytes = live ? (uint32_t)min(L - 16 * u, 16) * kRow : 0u;
    const rsrc_t r = make_rsrc(src + (size_t)phys * block_bytes + (size_t)(u % TPB) * 16 * kRow,
                               bytes);
    unsigned char* dst = &buf.kv[wave >> 1][mu * 16 * kRow];
#pragma unroll
    for (int q = 0; q < LPU; ++q)
      buffer_load_lds16(r, dst + q * 1024, src_off[q]);
  };

  if (wg_tiles > 0) load_tile(0, sm0);   // in flight while Q is staged

  // Q^T of the wave's columns (B layout) in registers for the whole kernel,
  // every load issued before the first use (columns past the queries read
  // row 0 and hold zeros); a negative factor is moved into Q (sign flip of
  // both halves of every word), and a zero one becomes the smallest normal
  // float: every visible score then weighs exp2(0) = 1 exactly, and a
  // masked one, -inf times it, 0
  const float cs = fmaxf(fabsf(a.scale_log2e), __FLT_MIN__);
  const float inv_cs = 1.f / cs;
  const uint32_t flip = a.scale_log2e < 0.f ? 0x80008000u : 0u;
  u32x4 qv[CG][KSTEPS];   // Q^T of the wave's columns in the B layout, for the whole kernel
  {
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      const TQ* qrow = static_cast<const TQ*>(a.q) +
                       ((size_t)(q0 + (valid[c] ? i[c] : 0)) * a.num_q_heads + h) * HD;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) qv[c][kk] = ld16(qrow + mfma_dim0<C>(kk, g4));
    }
#pragma unroll
    for (int c = 0; c < CG; ++c)
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
        qv[c][kk] = valid[c] ? (qv[c][kk] ^ flip) : u32x4{0, 0, 0, 0};
  }

  // ---- per-lane LDS offsets of the operands inside a 32-row tile
  // K (A operand of S^T): row 16 * hh + n, chunk 4 * kk + g4
  uint32_t k_at[2][KL];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int kk = 0; kk < KL; ++kk) {
      const int row = 16 * hh + n;
      k_at[hh][kk] = (uint32_t)(row * kRow + (((4 * kk + g4) ^ swz<NCH>(row)) * 16));
    }
  // 8-bit caches: the V codes of row 16 * hh + 4 * g4 + rr at the lane's DPL
  // dims (byte DPL * n of the row), widened and regrouped at the products
  uint32_t v_at[2][4];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = 16 * hh + 4 * g4 + rr;
      const int byte = n * DPL * (int)sizeof(T);
      v_at[hh][rr] = (uint32_t)(row * kRow + (((byte / 16) ^ swz<NCH>(row)) * 16) + byte % 16);
    }
  // 16-bit caches: V^T operands by transposing reads.  Lane 4 * k + q of a
  // 16-lane group names row 16 * hh + 4 * g4 + k at dims 16 * e + 4 * q .. + 3;
  // lane n of the group then holds those rows' values at dim 16 * e + n,
  // tokens in the order of its score registers (output row n of product e
  // is dim 16 * e + n).
  // Chunk 2 * e + (q >> 1) of a row stored at chunk (2 * e) ^ (q >> 1) ^ swz:
  // with rows a power of two of chunks, the byte offset is tr_at ^ (32 * e);
  // rows 16 .. 31 take the same swizzle as rows 0 .. 15, 16 rows further on.
  const int tr_q = n & 3, tr_row = 4 * g4 + (n >> 2);
  const uint32_t tr_at =
      (uint32_t)(tr_row * kRow + (((tr_q >> 1) ^ swz<NCH>(tr_row)) * 16) + (tr_q & 1) * 8);

  f32x4 acc[CG][DPL];
  float nmu[CG], thr[CG], l[CG];
#pragma unroll
  for (int c = 0; c < CG; ++c) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[c][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    nmu[c] = 0.f;         // minus the reference maximum (log2 units), 0 while there is none
    thr[c] = -INFINITY;   // raw score above which the reference must move
    l[c] = 0.f;
  }

  // S^T of both units of the current tile for group c
  auto scores = [&](const u32x4 (*ka)[KSTEPS], const u32x4* qb, float* sv) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) x = Ops::qk(ka[hh][kk], qb[kk], x);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sv[4 * hh + rr] = x[rr];
    }
  };

  auto tile = [&](int j, SM& cur, SM& nxt) {
    // this wave's share of tile j has landed; the barrier makes every
    // share visible and tells that every wave is done with tile j - 1,
    // whose buffer the loads of tile j + 1 then overwrite
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    if (j + 1 < wg_tiles) load_tile(j + 1, nxt);
    if (j >= my_tiles) return;   // this wave's columns end before the tile
    const unsigned char* kt = cur.kv[0];
    const unsigned char* vt = cur.kv[1];

    // ---- the tile's K rows as E values (8-bit codes widened here)
    u32x4 ka[2][KSTEPS];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int kk = 0; kk < KL; ++kk) {
        const u32x4 x = *(lds_u32x4*)(kt + k_at[hh][kk]);
        if constexpr (k8) {
          ka[hh][2 * kk] = u32x4{codes_to_pair<E, false>(x[0]), codes_to_pair<E, true>(x[0]),
                                 codes_to_pair<E, false>(x[1]), codes_to_pair<E, true>(x[1])};
          ka[hh][2 * kk + 1] = u32x4{codes_to_pair<E, false>(x[2]), codes_to_pair<E, true>(x[2]),
                                     codes_to_pair<E, false>(x[3]), codes_to_pair<E, true>(x[3])};
        } else {
          ka[hh][kk] = x;
        }
      }
    }

    auto read_va = [&](int e) {
      uint32_t w[4];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vt + (tr_at ^ (32u * e)) + hh * 16 * kRow));
        const u32x2 y = __builtin_bit_cast(u32x2, x);
        w[2 * hh] = y[0];
        w[2 * hh + 1] = y[1];
      }
      return u32x4{w[0], w[1], w[2], w[3]};
    };
    u32x4 vall[DPL];
    uint32_t vraw[2][4][VL];
    // ---- scores of every group, issued back to back; then the maxima and
    // one decision per tile on moving references
    const bool edge = 32 * j + 32 > lim_min;   // some column's bound or the context ends here
    const int t0 = 32 * j + 4 * g4;            // token of score row 0 of unit 0
    u32x4 pb[CG];
    float sv[CG][8];
#pragma unroll
    for (int c = 0; c < CG; ++c) scores(ka, qv[c], sv[c]);
    // every V operand of the tile, in the K operands' registers, while the
    // exponentials run (8-bit: the codes, widened at the products)
    if constexpr (!k8) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) vall[e] = read_va(e);
    } else {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          if constexpr (VL == 1) {
            vraw[hh][rr][0] = *(lds_u32*)(vt + v_at[hh][rr]);
          } else if constexpr (VL == 2) {
            const u32x2 y = *(lds_u32x2*)(vt + v_at[hh][rr]);
            vraw[hh][rr][0] = y[0];
            vraw[hh][rr][1] = y[1];
          } else {
            const u32x4 y = *(lds_u32x4*)(vt + v_at[hh][rr]);
#pragma unroll
            for (int w = 0; w < 4; ++w) vraw[hh][rr][w] = y[w];
          }
        }
    }
    float lm[CG];
    bool up = false;
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      if (edge) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (t0 + 16 * (k / 4) + (k % 4) >= limit[c]) sv[c][k] = -INFINITY;
      }
      lm[c] = max3f(max3f(sv[c][0], sv[c][1], sv[c][2]), max3f(sv[c][3], sv[c][4], sv[c][5]),
                    __builtin_elementwise_maximum(sv[c][6], sv[c][7]));
      up = up || lm[c] > thr[c];
    }
    if (__any(up)) {
#pragma unroll
      for (int c = 0; c < CG; ++c) {
        if (__any(lm[c] > thr[c])) {
          // move the reference to the column maximum (across the four token
          // groups of the column) and rescale what has been accumulated
          const float mo = thr[c] == -INFINITY ? -INFINITY : -nmu[c];   // none yet: -inf
          const float mn = fmaxf(mo, rows_max(lm[c]) * cs);
          const float corr = mo == -INFINITY ? 1.f : fast_exp2(mo - mn);
          if (mn != -INFINITY) {
            nmu[c] = -mn;
            thr[c] = (mn + kPrefillSlack) * inv_cs;
          }
          l[c] *= corr;
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[c][e] *= corr;
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      float p[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) p[k] = fast_exp2(__builtin_fmaf(sv[c][k], cs, nmu[c]));   // exp2(-inf) == 0
      pb[c] = u32x4{Ops::pack2(p[0], p[1]), Ops::pack2(p[2], p[3]), Ops::pack2(p[4], p[5]),
                    Ops::pack2(p[6], p[7])};
#pragma unroll
      for (int w = 0; w < 4; ++w) l[c] = Ops::sum2(pb[c][w], l[c]);
    }

    if constexpr (!k8) {
      // the value products (their operands read with the score products) at
      // raised wave priority: when both waves of the SIMD are ready to issue,
      // these go first (measured 0.5-1% faster)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int e = 0; e < DPL; ++e)
#pragma unroll
        for (int c = 0; c < CG; ++c) acc[c][e] = Ops::qk(vall[e], pb[c], acc[c][e]);
      __builtin_amdgcn_s_setprio(0);
      return;
    }
    // ---- 8-bit caches: one A operand per output dim e serves every group
    uint32_t vv[2][4][VW];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int w = 0; w < VL; ++w) {
          vv[hh][rr][2 * w] = codes_to_pair<E, false>(vraw[hh][rr][w]);
          vv[hh][rr][2 * w + 1] = codes_to_pair<E, true>(vraw[hh][rr][w]);
        }
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      const u32x4 va = {pair_of(e, vv[0][0], vv[0][1]), pair_of(e, vv[0][2], vv[0][3]),
                        pair_of(e, vv[1][0], vv[1][1]), pair_of(e, vv[1][2], vv[1][3])};
#pragma unroll
      for (int c = 0; c < CG; ++c) acc[c][e] = Ops::qk(va, pb[c], acc[c][e]);
    }
  };
  // two buffers, each its own LDS object named at compile time, so that
  // the reads of one tile need not wait for the loads into the other
  for (int j = 0; j < wg_tiles; j += 2) {
    tile(j, sm0, sm1);
    if (j + 1 < wg_tiles) tile(j + 1, sm1, sm0);
  }
  // the first tile any wave found naming a block outside the pool, through
  // the K/V buffers once every wave is done with them
  __syncthreads();
  int* bad = reinterpret_cast<int*>(&sm0.kv[0][0]);
  if (lane == 0) bad[wave] = my_bad;
  __syncthreads();
  const int bad_tile = min(min(bad[0], bad[1]), min(bad[2], bad[3]));
  const bool any_bad = bad_tile < my_tiles;   // a tile this wave read is among them
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    // the four token groups of a column hold partial sums of l
    const float lsum = rows_sum(l[c]);
    if (!valid[c]) continue;
    TQ* orow = static_cast<TQ*>(a.out) + ((size_t)(q0 + i[c]) * a.num_q_heads + h) * HD;
    // no visible token: zero row; 8-bit V: code units -> values
    const float inv = lsum > 0.f ? (k8 ? a.v_scale : 1.f) / lsum : 0.f;
    if constexpr (!k8) {
      // element rr of product e: dim 16 * e + 4 * g4 + rr
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        float o[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) o[rr] = any_bad ? __builtin_nanf("") : acc[c][e][rr] * inv;
        store_rounded<E, 4>(orow + 16 * e + 4 * g4, o);
      }
    } else {
      // element rr of product e: dim DPL * (4 * g4 + rr) + e
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float o[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] = any_bad ? __builtin_nanf("") : acc[c][e][rr] * inv;
        store_rounded<E, DPL>(orow + (4 * g4 + rr) * DPL, o);
      }
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
