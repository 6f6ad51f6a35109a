// tv_attn.hip -- tree_verify_attn: one target attention layer over a flattened tree.
//
// Graft (arXiv:2605.20104) §二, third gear: one parallel verification pass of
// the flattened tree under the tree mask. SpecOPD (arXiv:2611.02846) §02,
// proposal tree: all branches are scored in one pass that shares the trunk
// KV cache. D-cut (paper 2607.14647) technical summary §1 (verification of
// B x (D+1) tokens per step turns compute-bound as B grows) and §2 pipeline
// (each request keeps a contiguous prefix; the packed batch is verified).
//
// bf16 path (MFMA, gfx950). A workgroup of NW wavefronts owns one
// (request, kv head, row block, key split). Rows are the (node, query head)
// pairs of one GQA group, node-major, so all query heads that share a kv head
// and all tree nodes of the request are packed into the MFMA M/N dimension:
// every K/V byte staged in LDS serves up to 16*NW*RW rows.
//   S^T = K Q^T     v_mfma_f32_16x16x32_bf16, A = K tile from LDS [key][d],
//                   B = Q fragment held in VGPRs; lane (r, q) of the 16x16
//                   result holds row r, keys 4q..4q+3 of the subtile.
//   online softmax  fp32; the row max / sum over the 4 lanes of a row use
//                   v_permlane32_swap + v_permlane16_swap (no LDS trip);
//                   p = exp2(fma(s, scale*log2e, -m)); the ancestor mask is
//                   evaluated only on tiles holding tree keys or running past
//                   the end of the request.
//   O^T += V^T P^T  A = V^T from LDS (V transposed while staging), B = P
//                   converted to bf16 straight from the S^T accumulators.
// K/V tiles of 64 keys are gathered through the page table with 128-bit loads
// into two alternating register sets, so a tile's loads are issued two tiles
// before its turn; page-table entries are read three tiles ahead. Loads are
// unconditional: a position past the request's last key reads that last key
// instead (finite data, masked out of the softmax), so no branch guards them.
// Long prefixes are cut into key splits whose (m, l, o) partials are merged by
// a second kernel with the usual LSE weights.
//
// fp32 path (VALU): 4 lanes per row, a 64-key tile of K/V in LDS, same math.
//
// Cache layouts: K [page][kv_head][slot][head_dim], V [page][kv_head][head_dim][slot]
// (d-major V pages: 16 consecutive keys of one d are contiguous, which is the
// V^T operand layout of the PV product).
#include <algorithm>

#include "tv_internal.h"

namespace tv {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTile = 64;     // keys per tile
constexpr int kNumCUs = 256;  // MI355X compute units (the launch plan targets one pass over them)
constexpr int kMaxSplitPages = 4096;  // page ids one workgroup can stage (16-token pages: 64K keys)

struct Params {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const int32_t* block_table;
  const int32_t* prefix_len;
  const int32_t* cu_nodes;
  MaskDev mask;
  __bf16* out;
  float* lse;
  float* part_o;   // [splits][total_nodes*hq][D]
  float* part_ml;  // [splits][total_nodes*hq][2]  (m in log2 units, l)
  int32_t num_pages, max_pages, batch, total_nodes;
  int32_t hq, hkv, group, page_size;
  int32_t row_blocks, splits, keys_per_split;
  float scale_log2;  // softmax scale * log2(e), > 0
};

__device__ __forceinline__ uint32_t lo16x2(uint32_t a, uint32_t b) {  // {a.lo, b.lo}
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi16x2(uint32_t a, uint32_t b) {  // {a.hi, b.hi}
  return (a >> 16) | (b & 0xffff0000u);
}

// Max / sum over lanes l, l^16, l^32, l^48 (the 4 lanes holding one row of a
// 16x16 accumulator). Every one of the 4 lanes gets bit-identical results.
// v_permlane32_swap(x, y) leaves {x.lo | y.lo, x.hi | y.hi} in the two
// registers, so with y a copy of x the pair holds x_l and x_(l^32) in every
// lane (v_permlane16_swap likewise for rows of 16). The copy is hidden from
// the optimizer: given the same value twice it treats the two results as
// equal and drops one of them.
__device__ __forceinline__ void swap_pair(uint32_t u, bool rows32, uint32_t& a, uint32_t& b) {
  uint32_t w = u;
  asm volatile("" : "+v"(w));
  if (rows32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, w, false, false);
    a = r[0]; b = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(u, w, false, false);
    a = r[0]; b = r[1];
  }
}
__device__ __forceinline__ float row_max4(float v) {
  uint32_t a, b;
  swap_pair(__builtin_bit_cast(uint32_t, v), true, a, b);
  v = fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  swap_pair(__builtin_bit_cast(uint32_t, v), false, a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float row_sum4(float v) {
  uint32_t a, b;
  swap_pair(__builtin_bit_cast(uint32_t, v), true, a, b);
  v = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
  swap_pair(__builtin_bit_cast(uint32_t, v), false, a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// Direct-to-LDS 16-byte load of every lane (global_load_lds_dwordx4): lane
// l's 16 bytes from `src` land at LDS byte address lds + 16 l (lds must be
// wave-uniform). Issued through inline asm so that the compiler's wait-count
// insertion does not model it -- it would put a vmcnt(0) before any LDS read
// of the same array and drain the tile pipeline; the pipeline waits for
// these loads itself (counted vmcnt, then a barrier). M0 is restored.
__device__ __forceinline__ void lds_dma16(const void* src, const void* lds) {
  const uint32_t a = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(a), "v"(src)
      : "memory");
}

template <int D, int NW, int RW, bool WIDE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bf16_kernel(Params p) {
  constexpr int T = 64 * NW;           // threads
  constexpr int DS = D / 32;           // 32-wide d steps of S^T = K Q^T
  constexpr int DU = D / 16;           // 16-wide d subtiles of O^T
  constexpr int MBLK = 16 * NW * RW;   // rows per workgroup
  constexpr int CPR = D / 8;           // 16-byte chunks per K row
  constexpr int STAGES = 4;            // LDS ring depth: 3 tiles in flight
  constexpr int TILE_E = kTile * D;    // elements of one K (or V) tile
  constexpr int K_INS = D / 8;         // 1 KB direct-to-LDS loads per K tile
  constexpr int INS = 2 * K_INS;       // ... per K + V tile
  constexpr int IPW = INS / NW;        // ... per wave
  constexpr int RPI = 512 / D;         // K rows per load (1 KB / row bytes)
  constexpr int VPG = D / 32;          // V loads per 16-key group (32 d rows each)
  static_assert(INS % NW == 0, "load split");
  // Ring of STAGES tiles: K as [key][d] with 16-byte chunks XOR-swizzled by
  // key (conflict-free A-operand reads), V as [16-key group][d][16 keys] (the
  // V^T operand layout, copied as is from the d-major V pages).
  __shared__ __attribute__((aligned(16))) __bf16 sK[STAGES][TILE_E];
  __shared__ __attribute__((aligned(16))) __bf16 sV[STAGES][TILE_E];
  __shared__ int s_pages[kMaxSplitPages];  // page ids of this block's key range
  __shared__ int s_bounds[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int r16 = lane & 15, q4 = lane >> 4;

  int wg = blockIdx.x;
  const int split = wg % p.splits;
  wg /= p.splits;
  // later row blocks see more tree keys (causal trunks): dispatch them first
  const int rb = p.row_blocks - 1 - wg % p.row_blocks;
  wg /= p.row_blocks;
  const int g = wg % p.hkv;
  const int b = wg / p.hkv;

  const int n0 = clampi(p.cu_nodes[b], 0, p.total_nodes);
  const int n = clampi(p.cu_nodes[b + 1], n0, p.total_nodes) - n0;
  const int P = max(p.prefix_len[b], 0);
  const int G = p.group;
  const int rows = n * G;
  const int row0 = rb * MBLK;
  if (row0 >= rows) return;
  const int kv_end = P + n;
  const int ks = split * p.keys_per_split;
  if (ks >= kv_end) return;  // split absent for this request; the merge skips it
  // Ancestors-or-self have smaller indices, so no key past the block's last
  // node is visible to any of its rows.
  const int node_hi = min(n - 1, (row0 + MBLK - 1) / G);
  const int ke = min(min(ks + p.keys_per_split, kv_end), P + node_hi + 1);

  // ANCHOR form: block-wide bounds to skip tree tiles no row can see and to
  // treat tiles every row sees in full as unmasked.
  int ap_min = -1, ap_max = 0x7fffffff, br_lo = 0x7fffffff;
  const bool anchor = p.mask.kind == TV_MASK_ANCHOR;
  if (anchor) {
    if (tid == 0) { s_bounds[0] = 0x7fffffff; s_bounds[1] = -1; s_bounds[2] = 0x7fffffff; }
    __syncthreads();
    const int node_lo = row0 / G;
    for (int i = node_lo + tid; i <= node_hi; i += T) {
      const int a = p.mask.anchor_pos[n0 + i], d = p.mask.branch_depth[n0 + i];
      atomicMin(&s_bounds[0], a);
      atomicMax(&s_bounds[1], a);
      if (d > 0) atomicMin(&s_bounds[2], i - d + 1);
    }
    __syncthreads();
    ap_min = s_bounds[0]; ap_max = s_bounds[1]; br_lo = s_bounds[2];
  }
  // Tile [k0, k0+64): skipped when it holds no prefix key and no tree key any
  // row of the block can see; unmasked when all its keys are visible to all.
  auto skip_tile = [&](int k0) -> bool {
    if (!anchor || k0 < P) return false;
    const int j0 = k0 - P;
    return j0 > ap_max && j0 + kTile - 1 < br_lo;
  };
  auto full_tile = [&](int k0) -> bool {
    if (k0 + kTile > kv_end) return false;
    if (k0 + kTile <= P) return true;
    return anchor && (k0 + kTile - 1 - P) <= ap_min;
  };
  auto next_tile = [&](int k0) {
    int k = k0 + kTile;
    while (k < ke && skip_tile(k)) k += kTile;
    return k;
  };

  // Q fragments (B operand of S^T): lane (r16, q4) holds row r16 of its
  // subtile, d = 32s + 8q4 .. +7. Subtiles st = wave + NW r hold rows
  // row0 + 16 st ..; the first nv of them (a wave-uniform count) have a real
  // row. Padding rows carry zero Q and are never stored, so the MFMAs below
  // run unguarded.
  int nv = 0;
#pragma unroll
  for (int r = 0; r < RW; ++r) nv += (row0 + 16 * (wave + NW * r) < rows) ? 1 : 0;
  bf16x8 qf[RW][DS];
  int orow[RW], rnode[RW], rloc[RW];
  bool row_ok[RW];
  // per-row mask data kept in registers: ANCHOR (anchor_pos | branch_depth
  // << 32 in m_w0), BITS with <= 2 words (the two words in m_w0, m_w1);
  // wider BITS masks (the WIDE instantiation) are read per masked tile
  const bool bits_in_regs = !WIDE && !anchor;
  uint64_t m_w0[RW], m_w1[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int row = row0 + 16 * (wave + NW * r) + r16;
    row_ok[r] = row < rows;
    const int i = row_ok[r] ? row / G : 0;
    const int hl = row_ok[r] ? row % G : 0;
    rloc[r] = i;
    rnode[r] = n0 + i;
    orow[r] = (n0 + i) * p.hq + g * G + hl;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      if (row_ok[r]) {
        const uint4 u = *reinterpret_cast<const uint4*>(p.q + (size_t)orow[r] * D + 32 * s + 8 * q4);
        qf[r][s] = __builtin_bit_cast(bf16x8, u);
      } else {
        qf[r][s] = bf16x8{};
      }
    }
    m_w0[r] = 0ull; m_w1[r] = 0ull;
    if (row_ok[r]) {
      if (anchor) {
        m_w0[r] = (uint64_t)(uint32_t)p.mask.anchor_pos[rnode[r]] |
                  ((uint64_t)(uint32_t)p.mask.branch_depth[rnode[r]] << 32);
      } else if (bits_in_regs) {
        m_w0[r] = p.mask.bits[(size_t)rnode[r] * p.mask.words];
        if (p.mask.words == 2) m_w1[r] = p.mask.bits[(size_t)rnode[r] * 2 + 1];
      }
    }
    // keep these in registers: re-reading them inside the tile loop would
    // make its masked tiles wait for every load in flight, prefetch included
    asm volatile("" : "+v"(m_w0[r]), "+v"(m_w1[r]));
  }
  // Visibility of keys [k0, k0 + 64) for this lane's row of subtile r.
  auto row_visibility = [&](int r, int k0) -> uint64_t {
    if (!row_ok[r]) return 0ull;
    uint64_t v = range_bits(0, P - 1 - k0);
    if (k0 + kTile > P && k0 < kv_end) {
      const int j0 = k0 - P;  // > -64
      uint64_t t;
      if (anchor) {
        const int ap = (int)(uint32_t)m_w0[r], bd = (int)(uint32_t)(m_w0[r] >> 32);
        t = range_bits(-j0, ap - j0) | range_bits(rloc[r] - bd + 1 - j0, rloc[r] - j0);
      } else if (!WIDE) {
        if (j0 < 0) {
          t = m_w0[r] << (-j0);
        } else {
          const int sh = j0 & 63;
          const uint64_t lo = (j0 < 64) ? m_w0[r] : m_w1[r];
          const uint64_t hi = (j0 < 64) ? m_w1[r] : 0ull;
          t = sh ? ((lo >> sh) | (hi << (64 - sh))) : lo;
        }
      } else {
        return tile_visibility(p.mask, rnode[r], rloc[r], P, kv_end, k0);
      }
      v |= t & range_bits(P - k0, kv_end - 1 - k0);
    }
    return v;
  };

  f32x4 o[RW][DU];
  float m_run[RW], l_run[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
#pragma unroll
    for (int u = 0; u < DU; ++u) o[r][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- direct-to-LDS staging (lds_dma16). Load m of wave w is number
  // ins = w*IPW + m of the tile: ins < K_INS copies K rows [ins*RPI, +RPI)
  // (lane l: row ins*RPI + l/CPR, whose LDS chunk l%CPR receives K chunk
  // (l%CPR) ^ (row%CPR)); otherwise V 16-key group j = (ins-K_INS)/VPG,
  // d rows 32*((ins-K_INS)%VPG) + l/2, keys 8*(l%2) .. +7. The keys of one
  // load share a 16-key group and pages hold a power of two >= 16 keys, so a
  // load never crosses a page: its page id and slot are wave-uniform and
  // only a per-lane constant element offset differs between lanes.
  const int lp = __builtin_ctz(p.page_size);  // page_size == 1 << lp
  const int pmask = p.page_size - 1;
  long lane_off[IPW];
  int tile_off[IPW];
  int lds_off[IPW];  // element offset of the load inside one stage of sK / sV
#pragma unroll
  for (int m = 0; m < IPW; ++m) {
    const int ins = wave * IPW + m;
    if (ins < K_INS) {
      const int row = ins * RPI + lane / CPR;
      tile_off[m] = ins * RPI;
      lane_off[m] = (long)(lane / CPR) * D + 8 * ((lane % CPR) ^ (row % CPR));
      lds_off[m] = ins * RPI * D;
    } else {
      const int vi = ins - K_INS, jj = vi / VPG, dp = vi % VPG;
      tile_off[m] = 16 * jj;
      lane_off[m] = ((long)(32 * dp + lane / 2) << lp) + 8 * (lane % 2);
      lds_off[m] = jj * 16 * D + 32 * dp * 16;
    }
  }
  const int last = kv_end - 1;
  // Page ids of every key an issued tile can touch, [pg_lo, pg_hi], read
  // once into LDS (clamped into the pool) and looked up from there.
  const int pg_lo = ks >> lp;
  const int pg_hi = min((min(ke + kTile, kv_end) - 1) >> lp, p.max_pages - 1);
  const int n_pg = min(max(pg_hi - pg_lo + 1, 1), kMaxSplitPages);
  {
    const int32_t* row_tab = p.block_table + (size_t)b * p.max_pages;
    for (int i = tid; i < n_pg; i += T)
      s_pages[i] = clampi(row_tab[min(pg_lo + i, p.max_pages - 1)], 0, p.num_pages - 1);
  }
  // page id (wave-uniform) of tile position pos; positions past the
  // request's last key use the last key's page: tiles past the end read
  // valid memory that the softmax masks out or whose V is zeroed
  auto page_of = [&](int pos) -> int {
    const int i = min(max((min(pos, last) >> lp) - pg_lo, 0), n_pg - 1);
    return __builtin_amdgcn_readfirstlane(s_pages[i]);
  };
  auto issue = [&](int stage, int k0) {
#pragma unroll
    for (int m = 0; m < IPW; ++m) {
      const int ins = wave * IPW + m;
      const int pos0 = k0 + tile_off[m];
      const long blk = (long)(page_of(pos0) * p.hkv + g);
      const int slot0 = pos0 & pmask;
      if (ins < K_INS)
        lds_dma16(p.k + (((blk << lp) + slot0) * D + lane_off[m]), &sK[stage][lds_off[m]]);
      else
        lds_dma16(p.v + (((blk * D) << lp) + slot0 + lane_off[m]), &sV[stage][lds_off[m]]);
    }
  };

  // ---- S^T = K Q^T of the tile in stage `buf`
  auto qk = [&](int buf, f32x4 (&sacc)[RW][4]) {
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int t = 0; t < 4; ++t) sacc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (nv == 0) return;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int krow = 16 * t + r16;
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
            &sK[buf][krow * D + 8 * ((4 * s + q4) ^ (krow % CPR))]);
#pragma unroll
        for (int r = 0; r < RW; ++r)
          sacc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[r][s], sacc[r][t], 0, 0, 0);
      }
    }
  };

  // ---- online softmax of tile k0 from its scores, then O^T += V^T P^T
  auto softmax_pv = [&](int buf, int k0, f32x4 (&sacc)[RW][4]) {
    if (nv == 0) return;
    const bool masked = !full_tile(k0);
    bf16x8 pf[RW][2];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      float mx = -INFINITY;
      if (masked) {
        // this lane's 16 keys 16t + 4q4 + i as bits 4t + i of `own`
        const uint64_t sh = row_visibility(r, k0) >> (4 * q4);
        const uint32_t own = (uint32_t)(sh & 0xfu) | (uint32_t)((sh >> 12) & 0xf0u) |
                             (uint32_t)((sh >> 24) & 0xf00u) | (uint32_t)((sh >> 36) & 0xf000u);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = ((own >> (4 * t + i)) & 1u) ? sacc[r][t][i] : -INFINITY;
            sacc[r][t][i] = x;
            mx = fmaxf(mx, x);
          }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[r][t][i]);
      }
      mx = row_max4(mx) * p.scale_log2;
      const float m_new = fmaxf(m_run[r], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[r] - m_use);
      float part[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        part[t] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r][t][i], p.scale_log2, -m_use));
          sacc[r][t][i] = e;
          part[t] += e;
        }
      }
      const float sum = row_sum4((part[0] + part[1]) + (part[2] + part[3]));
      l_run[r] = l_run[r] * alpha + sum;
      // o is zero while m_run is -inf, and alpha == 1 when the max held:
      // rescale only if some row of the wave raised a finite running max
      const bool moved = m_run[r] != -INFINITY && m_new > m_run[r];
      m_run[r] = m_new;
      if (__any(moved)) {
#pragma unroll
        for (int u = 0; u < DU; ++u) o[r][u] *= alpha;
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[i] = static_cast<__bf16>(sacc[r][2 * kk][i]);
          f[4 + i] = static_cast<__bf16>(sacc[r][2 * kk + 1][i]);
        }
        pf[r][kk] = f;
      }
    }
    // logical k of lane group q4, element e: keys 32kk + 4q4 + e (e < 4)
    // and 32kk + 16 + 4q4 + (e - 4) (e >= 4)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int u = 0; u < DU; ++u) {
        // keys 32kk + 4q4 + e live in group 2kk, keys 32kk + 16 + .. in 2kk + 1
        const __bf16* vg = &sV[buf][(2 * kk) * 16 * D + (16 * u + r16) * 16 + 4 * q4];
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vg);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vg + 16 * D);
        const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int r = 0; r < RW; ++r)
          o[r][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[r][kk], o[r][u], 0, 0, 0);
      }
    }
  };

  // ---- pipeline. Tiles c0, c1, ... of the block; a step finishes tile c0
  // (softmax + PV, its scores already in registers) while the scores of c1
  // are computed -- independent MFMA work the scheduler interleaves with the
  // softmax -- and c2, c3 are in flight. Each wave waits (counted vmcnt) for
  // its own loads of c1 only, then a barrier makes every wave's loads
  // visible; the same barrier proves every wave is done with the stage the
  // step's new loads overwrite (tile c0 - 1's).
  constexpr int W_ALL = (15) | (3 << 14) | (7 << 4) | (15 << 8);  // s_waitcnt: no-op base
  auto wait_vm = [&](bool one_ahead) {  // wait until <= IPW (or 0) loads of this wave pend
    if (one_ahead) __builtin_amdgcn_s_waitcnt((W_ALL & ~0xC00F) | (IPW & 15) | ((IPW >> 4) << 14));
    else __builtin_amdgcn_s_waitcnt(W_ALL & ~0xC00F);
  };
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // zero the V columns of positions past the request's last key in a tile
  // that just landed (their K columns are masked; V must hold finite zeros
  // for P = 0 to contribute nothing)
  auto zero_tail = [&](int stage, int k0) {
    if (k0 >= ke || k0 + kTile <= kv_end) return;
    for (int e = tid; e < TILE_E; e += T) {
      const int key = 16 * (e / (16 * D)) + (e & 15);  // element (group, d, key%16)
      if (k0 + key >= kv_end) sV[stage][e] = static_cast<__bf16>(0.f);
    }
    __builtin_amdgcn_s_waitcnt(W_ALL & ~0x0F00);  // lgkmcnt(0): zeros written
    barrier();
  };
  int c0 = ks;
  while (c0 < ke && skip_tile(c0)) c0 += kTile;
  int c1 = next_tile(c0), c2 = next_tile(c1), c3 = next_tile(c2);
  // the page list (and Q, mask rows) land here; then it is visible to all
  __builtin_amdgcn_s_waitcnt(0);
  barrier();
  if (c0 < ke) issue(0, c0);
  if (c1 < ke) issue(1, c1);
  if (c2 < ke) issue(2, c2);
  f32x4 sA[RW][4], sB[RW][4];
  int it = 0;
  if (c0 < ke) {
    if (c1 >= ke) wait_vm(false);
    else if (c2 >= ke) wait_vm(true);
    else __builtin_amdgcn_s_waitcnt((W_ALL & ~0xC00F) | ((2 * IPW) & 15) | (((2 * IPW) >> 4) << 14));
    barrier();
    zero_tail(0, c0);
    qk(0, sA);
  }
  auto step = [&](f32x4 (&scur)[RW][4], f32x4 (&snext)[RW][4]) {
    wait_vm(c2 < ke);  // tile c1 has landed (c2 may still be in flight)
    barrier();
    zero_tail((it + 1) & (STAGES - 1), c1);
    if (c3 < ke) issue((it + 3) & (STAGES - 1), c3);
    if (c1 < ke) qk((it + 1) & (STAGES - 1), snext);
    softmax_pv(it & (STAGES - 1), c0, scur);
    c0 = c1; c1 = c2; c2 = c3; c3 = next_tile(c3);
    ++it;
  };
  while (c0 < ke) {
    step(sA, sB);
    if (c0 >= ke) break;
    step(sB, sA);
  }

  // ---- epilogue: lane (r16, q4) holds O[row r16][16u + 4q4 + i]
  const size_t R_tot = (size_t)p.total_nodes * p.hq;
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    if (!row_ok[r]) continue;
    if (p.splits == 1) {
      const float inv = l_run[r] > 0.f ? 1.f / l_run[r] : 0.f;
#pragma unroll
      for (int u = 0; u < DU; ++u) {
        bf16x4 h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = static_cast<__bf16>(o[r][u][i] * inv);
        *reinterpret_cast<bf16x4*>(p.out + (size_t)orow[r] * D + 16 * u + 4 * q4) = h;
      }
      if (p.lse && q4 == 0)
        p.lse[orow[r]] = l_run[r] > 0.f ? (m_run[r] + log2f(l_run[r])) * kLn2 : -INFINITY;
    } else {
      const size_t prow = (size_t)split * R_tot + orow[r];
#pragma unroll
      for (int u = 0; u < DU; ++u)
        *reinterpret_cast<f32x4*>(p.part_o + prow * D + 16 * u + 4 * q4) = o[r][u];
      if (q4 == 0) *reinterpret_cast<float2*>(p.part_ml + prow * 2) = float2{m_run[r], l_run[r]};
    }
  }
}

// Merge of split partials: m = max m_s, l = sum 2^(m_s - m) l_s,
// o = sum 2^(m_s - m) o_s / l, lse = (m + log2 l) ln 2. One row per D/4 lanes.
template <int D, typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      const int32_t* __restrict__ cu_nodes,
                                                      const int32_t* __restrict__ prefix_len,
                                                      int32_t batch, int32_t total_nodes, int32_t hq,
                                                      int32_t splits, int32_t keys_per_split,
                                                      OutT* __restrict__ out, float* __restrict__ lse) {
  constexpr int LPR = D / 4;               // lanes per row
  constexpr int RPB = 256 / LPR;           // rows per block
  const size_t R_tot = (size_t)total_nodes * hq;
  const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  if (row >= R_tot) return;
  const int node = (int)(row / hq);
  int lo = 0, hi = batch;  // request b with cu_nodes[b] <= node < cu_nodes[b+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_nodes[mid] <= node) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int kv_end = max(prefix_len[b], 0) + (cu_nodes[b + 1] - cu_nodes[b]);
  const int ns = min(splits, (kv_end + keys_per_split - 1) / keys_per_split);
  // pass 1: the split maxima (independent loads, 8 in flight)
  float m = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += 8) {
    float ms[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      ms[j] = (s0 + j < ns) ? part_ml[((size_t)(s0 + j) * R_tot + row) * 2] : -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, ms[j]);
  }
  // pass 2: weighted sums of l and o
  float l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ns; s0 += 8) {
    float2 ml[8];
    f32x4 os[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const size_t pr = (size_t)(s0 + j) * R_tot + row;
      ml[j] = (s0 + j < ns) ? *reinterpret_cast<const float2*>(part_ml + pr * 2) : float2{-INFINITY, 0.f};
      os[j] = (s0 + j < ns) ? *reinterpret_cast<const f32x4*>(part_o + pr * D + 4 * sub) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float w = (ml[j].x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ml[j].x - m);
      l += w * ml[j].y;
      acc += w * os[j];
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  OutT* dst = out + row * D + 4 * sub;
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = static_cast<OutT>(acc[i] * inv);
  if (lse && sub == 0) lse[row] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------- fp32 path --
// 4 lanes per (node, head) row, each owning d = 4j + sub; 16 rows per block.
struct ParamsF32 {
  const float* q;
  const float* k;
  const float* v;
  const int32_t* block_table;
  const int32_t* prefix_len;
  const int32_t* cu_nodes;
  MaskDev mask;
  float* out;
  float* lse;
  int32_t num_pages, max_pages, total_nodes, hq, hkv, group, page_size, row_blocks;
  float scale_log2;
};

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(ParamsF32 p) {
  constexpr int DL = D / 4;
  __shared__ float sK[kTile][D + 1];
  __shared__ float sV[kTile][D + 1];
  const int tid = threadIdx.x, sub = tid & 3, rloc = tid >> 2;
  int wg = blockIdx.x;
  const int rb = wg % p.row_blocks;
  wg /= p.row_blocks;
  const int g = wg % p.hkv;
  const int b = wg / p.hkv;
  const int n0 = clampi(p.cu_nodes[b], 0, p.total_nodes);
  const int n = clampi(p.cu_nodes[b + 1], n0, p.total_nodes) - n0;
  const int P = max(p.prefix_len[b], 0);
  const int G = p.group;
  const int rows = n * G;
  if (rb * 16 >= rows) return;
  const int row = rb * 16 + rloc;
  const bool ok = row < rows;
  const int i = ok ? row / G : 0;
  const int hl = ok ? row % G : 0;
  const int orow = (n0 + i) * p.hq + g * G + hl;
  const int kv_end = P + n;
  const int node_hi = min(n - 1, (rb * 16 + 15) / G);
  const int ke = min(kv_end, P + node_hi + 1);

  float qv[DL], acc[DL];
#pragma unroll
  for (int j = 0; j < DL; ++j) {
    qv[j] = ok ? p.q[(size_t)orow * D + 4 * j + sub] : 0.f;
    acc[j] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  for (int k0 = 0; k0 < ke; k0 += kTile) {
    __syncthreads();
    for (int e = tid; e < kTile * D; e += 64) {
      const int key = e / D, d = e % D;
      int pos = k0 + key;
      float kx = 0.f, vx = 0.f;
      if (pos < kv_end && pos / p.page_size < p.max_pages) {
        const int pg = clampi(p.block_table[(size_t)b * p.max_pages + pos / p.page_size], 0, p.num_pages - 1);
        const size_t kof = ((size_t)(pg * p.hkv + g) * p.page_size + pos % p.page_size) * D + d;
        const size_t vof = ((size_t)(pg * p.hkv + g) * D + d) * p.page_size + pos % p.page_size;
        kx = p.k[kof];
        vx = p.v[vof];
      }
      sK[key][d] = kx;
      sV[key][d] = vx;
    }
    __syncthreads();
    const uint64_t vis = ok ? tile_visibility(p.mask, n0 + i, i, P, kv_end, k0) : 0ull;
    float s[kTile];
    float mx = -INFINITY;
#pragma unroll
    for (int key = 0; key < kTile; ++key) {
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < DL; ++j) part += qv[j] * sK[key][4 * j + sub];
      part += __shfl_xor(part, 1, 64);
      part += __shfl_xor(part, 2, 64);
      const float x = ((vis >> key) & 1ull) ? part * p.scale_log2 : -INFINITY;
      s[key] = x;
      mx = fmaxf(mx, x);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
#pragma unroll
    for (int j = 0; j < DL; ++j) acc[j] *= alpha;
    float sum = 0.f;
#pragma unroll
    for (int key = 0; key < kTile; ++key) {
      const float e = __builtin_amdgcn_exp2f(s[key] - m_use);
      sum += e;
#pragma unroll
      for (int j = 0; j < DL; ++j) acc[j] += e * sV[key][4 * j + sub];
    }
    l_run = l_run * alpha + sum;
    m_run = m_new;
  }
  if (!ok) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
  for (int j = 0; j < DL; ++j) p.out[(size_t)orow * D + 4 * j + sub] = acc[j] * inv;
  if (p.lse && sub == 0) p.lse[orow] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
}

template <int D, int NW, int RW>
hipError_t run_bf16(const Params& prm, int grid, hipStream_t stream) {
  if (prm.mask.kind == TV_MASK_BITS && prm.mask.words > 2)
    hipLaunchKernelGGL((attn_bf16_kernel<D, NW, RW, true>), dim3(grid), dim3(64 * NW), 0, stream, prm);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, NW, RW, false>), dim3(grid), dim3(64 * NW), 0, stream, prm);
  return hipGetLastError();
}

template <int D>
hipError_t dispatch_bf16(const Params& prm, const AttnPlan& plan, int grid, hipStream_t stream) {
  if (plan.waves == 4) return run_bf16<D, 4, 1>(prm, grid, stream);
  if (plan.rw == 1) return run_bf16<D, 8, 1>(prm, grid, stream);
  return run_bf16<D, 8, 2>(prm, grid, stream);
}

}  // namespace

AttnPlan plan_attn(int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t max_prefix_len,
                   int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype) {
  AttnPlan pl{};
  const long G = hkv > 0 ? hq / hkv : 1;
  const long rows = (long)max_nodes * G;
  if (dtype == TV_F32) {
    pl.waves = 1;
    pl.rw = 1;
    pl.row_blocks = (int)((rows + 15) / 16);
    pl.splits = 1;
    pl.keys_per_split = max_prefix_len + max_nodes;
    pl.workspace = 0;
    return pl;
  }
  // rows of one kv head: <= 64 -> 4 waves x 1 subtile (64 rows per block),
  // <= 128 -> 8 waves x 1 (128 rows), else 8 waves x 2 (256 rows)
  if (rows <= 64) { pl.waves = 4; pl.rw = 1; }
  else if (rows <= 128) { pl.waves = 8; pl.rw = 1; }
  else { pl.waves = 8; pl.rw = 2; }
  const long mblk = 16L * pl.waves * pl.rw;
  pl.row_blocks = (int)((rows + mblk - 1) / mblk);
  const long kv = (long)max_prefix_len + max_nodes;
  const long tiles = (kv + kTile - 1) / kTile;
  const long base = (long)batch * hkv * pl.row_blocks;
  // One 128 KB-LDS workgroup fits a CU: cut the keys into splits until the
  // workgroups cover the CUs once; more splits only add partial traffic.
  const long cus = kNumCUs;
  long splits = std::max(1L, std::min(tiles, cus / base));
  // a split's pages must fit the block's LDS page list (16-token pages)
  const long max_tps = (long)(kMaxSplitPages - 8) * 16 / kTile;
  splits = std::max(splits, (tiles + max_tps - 1) / max_tps);
  const long tps = (tiles + splits - 1) / splits;
  pl.keys_per_split = (int)(tps * kTile);
  pl.splits = (int)((tiles + tps - 1) / tps);
  if (pl.splits > 1) {
    const size_t rtot = (size_t)total_nodes * hq;
    const size_t o_bytes = (size_t)pl.splits * rtot * head_dim * sizeof(float);
    const size_t ml_bytes = (size_t)pl.splits * rtot * 2 * sizeof(float);
    pl.workspace = ((o_bytes + 255) & ~(size_t)255) + ((ml_bytes + 255) & ~(size_t)255);
  } else {
    pl.workspace = 0;
  }
  return pl;
}

hipError_t launch_attn(const AttnArgs& a, const AttnPlan& plan, hipStream_t stream) {
  const int G = a.hq / a.hkv;
  if (a.dtype == TV_F32) {
    ParamsF32 p{};
    p.q = static_cast<const float*>(a.q);
    p.k = static_cast<const float*>(a.k_cache);
    p.v = static_cast<const float*>(a.v_cache);
    p.block_table = a.block_table;
    p.prefix_len = a.prefix_len;
    p.cu_nodes = a.cu_nodes;
    p.mask = a.mask;
    p.out = static_cast<float*>(a.out);
    p.lse = a.lse;
    p.num_pages = a.num_pages;
    p.max_pages = a.max_pages;
    p.total_nodes = a.total_nodes;
    p.hq = a.hq;
    p.hkv = a.hkv;
    p.group = G;
    p.page_size = a.page_size;
    p.row_blocks = plan.row_blocks;
    p.scale_log2 = a.scale * kLog2e;
    const int grid = a.batch * a.hkv * plan.row_blocks;
    if (a.head_dim == 64)
      hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(grid), dim3(64), 0, stream, p);
    else
      hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(grid), dim3(64), 0, stream, p);
    return hipGetLastError();
  }
  Params p{};
  p.q = static_cast<const __bf16*>(a.q);
  p.k = static_cast<const __bf16*>(a.k_cache);
  p.v = static_cast<const __bf16*>(a.v_cache);
  p.block_table = a.block_table;
  p.prefix_len = a.prefix_len;
  p.cu_nodes = a.cu_nodes;
  p.mask = a.mask;
  p.out = static_cast<__bf16*>(a.out);
  p.lse = a.lse;
  const size_t rtot = (size_t)a.total_nodes * a.hq;
  char* ws = static_cast<char*>(a.workspace);
  p.part_o = reinterpret_cast<float*>(ws);
  const size_t o_bytes = ((size_t)plan.splits * rtot * a.head_dim * sizeof(float) + 255) & ~(size_t)255;
  p.part_ml = plan.splits > 1 ? reinterpret_cast<float*>(ws + o_bytes) : nullptr;
  p.num_pages = a.num_pages;
  p.max_pages = a.max_pages;
  p.batch = a.batch;
  p.total_nodes = a.total_nodes;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.group = G;
  p.page_size = a.page_size;
  p.row_blocks = plan.row_blocks;
  p.splits = plan.splits;
  p.keys_per_split = plan.keys_per_split;
  p.scale_log2 = a.scale * kLog2e;
  const int grid = a.batch * a.hkv * plan.row_blocks * plan.splits;
  hipError_t e = (a.head_dim == 64) ? dispatch_bf16<64>(p, plan, grid, stream)
                                    : dispatch_bf16<128>(p, plan, grid, stream);
  if (e != hipSuccess || plan.splits == 1) return e;
  const int lpr = a.head_dim / 4, rpb = 256 / lpr;
  const int cgrid = (int)((rtot + rpb - 1) / rpb);
  if (a.head_dim == 64)
    hipLaunchKernelGGL((combine_kernel<64, __bf16>), dim3(cgrid), dim3(256), 0, stream, p.part_o,
                       p.part_ml, a.cu_nodes, a.prefix_len, a.batch, a.total_nodes, a.hq,
                       plan.splits, plan.keys_per_split, p.out, a.lse);
  else
    hipLaunchKernelGGL((combine_kernel<128, __bf16>), dim3(cgrid), dim3(256), 0, stream, p.part_o,
                       p.part_ml, a.cu_nodes, a.prefix_len, a.batch, a.total_nodes, a.hq,
                       plan.splits, plan.keys_per_split, p.out, a.lse);
  return hipGetLastError();
}

}  // namespace tv
