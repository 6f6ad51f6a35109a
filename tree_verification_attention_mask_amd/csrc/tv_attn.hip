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
#include <type_traits>

#include "tv_internal.h"

namespace tv {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTile = 64;     // keys per tile
constexpr int kMaxSplitPages = 4096;  // page ids one workgroup can stage (16-token pages: 64K keys)
constexpr int kMaxLptBatch = 256;   // requests the in-kernel longest-first order handles
constexpr float kLazyMax = 8.f;      // running-max slack before O is rescaled (log2 units)
constexpr float kLazySum = 256.f;    // 2^kLazyMax
// running max (log2 units) of a row before its first visible key: finite, so
// that the probabilities' offset needs no select, and far below any score
// (the first key raises it, with a rescale of the still-zero O and l by 0)
constexpr float kNoMax = -1e30f;

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
  __bf16* part_o;  // [splits][total_nodes*hq][D] the split's output over its own l
  float* part_ml;  // [splits][total_nodes*hq][2]  (m in log2 units, l)
  int32_t num_pages, max_pages, batch, total_nodes;
  int32_t hq, hkv, group, page_size;
  int32_t row_blocks, splits, keys_per_split;
  int32_t lpt;       // map block order onto requests longest first (batch <= kMaxLptBatch)
  float scale_log2;  // softmax scale * log2(e), > 0
};

// Sum / max over lanes l, l^16, l^32, l^48 (the 4 lanes holding one row of a
// 16x16 accumulator). Every one of the 4 lanes gets bit-identical results.
// v_permlane32_swap(x, y) leaves {x.lo | y.lo, x.hi | y.hi} in the two
// registers, so with y a copy of x the pair holds x_l and x_(l^32) in every
// lane (v_permlane16_swap likewise for rows of 16). The copy is hidden from
// the optimizer: given the same value twice it treats the two results as
// equal and drops one of them.
__device__ __forceinline__ void swap_pair(uint32_t u, bool rows32, uint32_t& a, uint32_t& b) {
  uint32_t w = u;
  asm("" : "+v"(w));
  if (rows32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, w, false, false);
    a = r[0]; b = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(u, w, false, false);
    a = r[0]; b = r[1];
  }
}
__device__ __forceinline__ float row_sum4(float v) {
  uint32_t a, b;
  swap_pair(__builtin_bit_cast(uint32_t, v), true, a, b);
  v = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
  swap_pair(__builtin_bit_cast(uint32_t, v), false, a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
// v_max_f32 / v_max3_f32 as written: fmaxf on values the compiler cannot
// prove quiet (integer bits from a lane swap, masked accumulators) first
// quiets each operand with one more v_max_f32; the scores are never
// signalling NaNs
__device__ __forceinline__ float fmax_bits(uint32_t a, uint32_t b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float fmax_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float fmax3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float row_max4(float v) {
  uint32_t a, b;
  swap_pair(__builtin_bit_cast(uint32_t, v), true, a, b);
  v = fmax_bits(a, b);
  swap_pair(__builtin_bit_cast(uint32_t, v), false, a, b);
  return fmax_bits(a, b);
}

// s_waitcnt operand that waits for nothing (gfx9 encoding: vmcnt bits 3:0
// and 15:14, expcnt 6:4, lgkmcnt 11:8), and a wait for vmcnt <= N.
constexpr int W_ALL = (15) | (3 << 14) | (7 << 4) | (15 << 8);
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((W_ALL & ~0xC00F) | (N & 15) | ((N >> 4) << 14));
}

// One wave's share of a K or V tile: N direct-to-LDS loads
// (global_load_lds_dwordx4), load m of lane l reading 16 bytes at
// base + voff[m] + 1024 m and writing them at LDS byte address
// lds + 1024 m + 16 l (the instruction's immediate offset adds to both
// addresses; base and lds are wave-uniform, voff[m] a per-lane 32-bit
// offset). One M0 setting serves the N loads; M0 is restored after them (the
// compiler reserves it). Issued through inline asm so that the compiler's
// wait-count insertion does not model the LDS writes -- it would put a
// vmcnt(0) before any LDS read of the same arrays and drain the tile
// pipeline; the pipeline waits for these loads itself (counted vmcnt, then a
// barrier).
template <int N>
__device__ __forceinline__ void dma_burst(const void* base, const uint32_t (&voff)[N], uint32_t lds) {
  uint32_t saved;
  if constexpr (N == 4) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %3, %2\n\t"
        "global_load_lds_dwordx4 %4, %2 offset:1024\n\t"
        "global_load_lds_dwordx4 %5, %2 offset:2048\n\t"
        "global_load_lds_dwordx4 %6, %2 offset:3072\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "s"(base), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3])
        : "memory");
  } else {
    static_assert(N == 2, "two or four loads per wave and tile");
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %3, %2\n\t"
        "global_load_lds_dwordx4 %4, %2 offset:1024\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "s"(base), "v"(voff[0]), "v"(voff[1])
        : "memory");
  }
}

// A single direct-to-LDS load (as dma_burst, N = 1, no step): 16 bytes of
// every lane from `src` to LDS byte address lds + 16 l.
__device__ __forceinline__ void dma_single(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(src)
      : "memory");
}

// LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// XOR swizzle of the 16-byte chunks of K row `row` in LDS: chunk c of the
// row is stored at position c ^ kswz(row). The S^T = K Q^T fragments read
// rows 32(t/2) + 8(r/4) + 4(t%2) + r%4 for the 16 lanes r of a column group,
// so the swizzle must take 16 different values on row bits {0, 1, 3, 4}
// (D = 128: 16 chunks per 256-byte row, every row on the same banks); the
// plain row % 16 takes only 8 there and makes those reads two-way bank
// conflicts (measured on gfx950: 127 against 215 bytes per clock for a
// conflict-free ds_read_b128 stream).
template <int D>
__device__ __forceinline__ int kswz(int row) {
  if constexpr (D == 128) return (row & 3) | ((row >> 1) & 12);
  else return row % (D / 8);
}

// Per-lane byte offsets (less 1 KB per load, as dma_burst adds it) and the
// LDS byte offset within a stage of load 0, for wave w's share of a tile.
// Load m of wave w is number ins = w*IPW + m of the tile: ins < K_INS copies
// K rows [ins*RPI, +RPI) (lane l: row ins*RPI + l/CPR, whose LDS chunk l%CPR
// receives K chunk (l%CPR) ^ kswz(row)); otherwise V 16-key group
// j = (ins-K_INS)/VPG, d rows 32*((ins-K_INS)%VPG) + l/2, keys 8*(l%2) .. +7.
// The first four waves load K, the others V; the loads of one wave cover one
// whole 16-key group, and pages hold a power of two >= 16 keys, so the group
// lies in one page: K rows are consecutive 1 KB steps of it, V's d rows step
// by 32 rows of page_size keys (>= 1 KB).
template <int D>
__device__ __forceinline__ void tile_load_offsets(int wave, int lane, int lp, int nw,
                                                  uint32_t (&voff)[(2 * D / 8) / 8],
                                                  uint32_t& lds0) {
  constexpr int K_INS = D / 8, INS = 2 * K_INS, IPW = INS / 8;
  constexpr int RPI = 512 / D, VPG = D / 32, CPR = D / 8;
  const bool k_wave = wave < nw / 2;
#pragma unroll
  for (int m = 0; m < IPW; ++m) {
    const int ins = wave * IPW + m;
    if (k_wave) {
      const int row = ins * RPI + lane / CPR;
      voff[m] = 2u * (uint32_t)((lane / CPR) * D + 8 * ((lane % CPR) ^ kswz<D>(row)));
    } else {
      const int vi = ins - K_INS, dp = vi % VPG;
      voff[m] = 2u * (uint32_t)(((32 * dp + lane / 2) << lp) + 8 * (lane % 2)) - 1024u * m;
    }
  }
  const int ins0 = wave * IPW;
  lds0 = k_wave ? 2u * (uint32_t)(ins0 * RPI * D)
                : 2u * (uint32_t)(((ins0 - K_INS) / VPG) * 16 * D + 32 * ((ins0 - K_INS) % VPG) * 16);
}

template <int D, int NW, int RW, bool WIDE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bf16_kernel(Params p) {
  static_assert(NW == 8, "two groups of four waves (one wave of each per SIMD)");
  constexpr int T = 64 * NW;           // threads
  constexpr int DS = D / 32;           // 32-wide d steps of S^T = K Q^T
  constexpr int DU = D / 16;           // 16-wide d subtiles of O^T
  constexpr int MBLK = 16 * NW * RW;   // rows per workgroup
  constexpr int STAGES = 4;            // LDS ring depth: 3 tiles in flight
  constexpr int TILE_E = kTile * D;    // elements of one K (or V) tile
  constexpr int K_INS = D / 8;         // 1 KB direct-to-LDS loads per K tile
  constexpr int INS = 2 * K_INS;       // ... per K + V tile
  constexpr int IPW = INS / NW;        // ... per wave
  constexpr int RPI = 512 / D;         // K rows per load (1 KB / row bytes)
  constexpr int VPG = D / 32;          // V loads per 16-key group (32 d rows each)
  constexpr int GPW = 1;               // 16-key groups one wave loads per tile
  constexpr int PPT = kMaxSplitPages / T;  // page-table entries per thread
  static_assert(INS % NW == 0 && IPW * RPI == 16 * GPW && IPW == VPG * GPW, "load split");
  // Ring of STAGES tiles: K as [key][d] with 16-byte chunks XOR-swizzled by
  // key (conflict-free A-operand reads), V as [16-key group][d][16 keys] (the
  // V^T operand layout, copied as is from the d-major V pages).
  __shared__ __attribute__((aligned(16))) __bf16 sK[STAGES][TILE_E];
  __shared__ __attribute__((aligned(16))) __bf16 sV[STAGES][TILE_E];
  __shared__ int s_pages[kMaxSplitPages];  // page ids of this block's key window
  __shared__ int s_bounds[NW][4];  // ANCHOR form: each wave's partial bounds
  __shared__ int s_len[kMaxLptBatch], s_order[kMaxLptBatch];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int r16 = lane & 15, q4 = lane >> 4;

  // block order: split fastest, then kv head, then request, row block
  // slowest and last first -- later row blocks see more tree keys (causal
  // trunks), so the longest workgroups of every head start first (with the
  // snake below, which keeps the four CU groups of an XCD evenly loaded)
  int wg = blockIdx.x;
  const int split = wg % p.splits;
  wg /= p.splits;
  const int g = wg % p.hkv;
  wg /= p.hkv;
  int b = wg % p.batch;
  // Dispatch position t of the row block (0 first): last row blocks first,
  // every other full group of four in reverse ("snake"), so that workgroups
  // dealt out in turn over four groups of CUs give each group a like share
  // of long and short blocks.
  int t = wg / p.batch;
  if (((t >> 2) & 1) && (t | 3) < p.row_blocks) t ^= 3;
  const int rb = p.row_blocks - 1 - t;
  if (p.lpt) {
    // Longest-first: when the grid takes several rounds of the CUs, blocks
    // of long requests are dispatched first (ranked by key count, ties by
    // index), so that short ones fill the tail. Each block ranks the batch
    // itself; this costs one dependent load before the page table.
    for (int i = tid; i < p.batch; i += T) {
      const int c0 = clampi(p.cu_nodes[i], 0, p.total_nodes);
      s_len[i] = max(p.prefix_len[i], 0) + clampi(p.cu_nodes[i + 1], c0, p.total_nodes) - c0;
    }
    __syncthreads();
    if (p.batch <= T / 8) {
      // eight lanes per request (batch <= 64), each counting the requests
      // ranked ahead of it among eight others; the counts are added across
      // the eight lanes
      const int i = tid >> 3, part = tid & 7;
      int cnt = 0;
      if (i < p.batch) {
        const int li = s_len[i];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int j = part * 8 + q;
          const int lj = j < p.batch ? s_len[j] : -1;
          cnt += (lj > li || (lj == li && j < i)) ? 1 : 0;
        }
      }
      cnt += __shfl_xor(cnt, 1, 8);
      cnt += __shfl_xor(cnt, 2, 8);
      cnt += __shfl_xor(cnt, 4, 8);
      if (i < p.batch && part == 0) s_order[cnt] = i;
    } else {
      for (int i = tid; i < p.batch; i += T) {
        const int li = s_len[i];
        int rank = 0;
        for (int j = 0; j < p.batch; ++j) {
          const int lj = s_len[j];
          rank += (lj > li || (lj == li && j < i)) ? 1 : 0;
        }
        s_order[rank] = i;
      }
    }
    __syncthreads();
    b = s_order[b];
  }
  const int ks = split * p.keys_per_split;

  // Page ids of the split's key window [ks, ks + keys_per_split + 64): their
  // loads do not depend on the request's bounds, so both are in flight at
  // once. Entries past the request's last page are never used for a key.
  const int lp = __builtin_ctz(p.page_size);  // page_size == 1 << lp
  const int pmask = p.page_size - 1;
  const int pg_lo = ks >> lp;
  const int n_pg = max(1, min(((ks + p.keys_per_split + kTile - 1) >> lp) - pg_lo + 1, kMaxSplitPages));
  int pgv[PPT];
  const int32_t* row_tab = p.block_table + (size_t)b * p.max_pages;
  // page ids of this wave's 16-key group of the block's first two tiles,
  // straight from the block table and loaded first, with the request's
  // bounds: the tiles go out as soon as those are known (an entry past the
  // request's pages is clamped into the pool; its keys are masked and its
  // V zeroed)
  int pgf[2];
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2)
    pgf[t2] = row_tab[min((ks + kTile * t2 + 16 * ((wave < NW / 2 ? wave : wave - NW / 2) * GPW)) >> lp,
                          p.max_pages - 1)];
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int i = tid + j * T;
    pgv[j] = (i < n_pg) ? row_tab[min(pg_lo + i, p.max_pages - 1)] : 0;
  }

  // the request's bounds and the first page ids in one round trip: held in
  // registers here, so that no load is moved past the early exits below
  // (where it would start a second round trip)
  int cu_lo = p.cu_nodes[b], cu_hi = p.cu_nodes[b + 1], p_len = p.prefix_len[b];
  asm volatile("" : "+s"(cu_lo), "+s"(cu_hi), "+s"(p_len), "+s"(pgf[0]), "+s"(pgf[1]));
  const int n0 = clampi(cu_lo, 0, p.total_nodes);
  const int n = clampi(cu_hi, n0, p.total_nodes) - n0;
  const int P = max(p_len, 0);
  const int G = p.group;
  const int rows = n * G;
  const int row0 = rb * MBLK;
  if (row0 >= rows) return;
  const int kv_end = P + n;
  if (ks >= kv_end) {
    // split absent for this request: mark its rows empty (m = -inf, l = 0)
    // so that the merge needs no per-request bounds
    if (p.splits > 1) {
      const size_t R_tot = (size_t)p.total_nodes * p.hq;
      for (int i = tid; i < min(MBLK, rows - row0); i += T) {
        const int row = row0 + i;
        const size_t orow_i = (size_t)(n0 + row / G) * p.hq + g * G + row % G;
        *reinterpret_cast<float2*>(p.part_ml + ((size_t)split * R_tot + orow_i) * 2) =
            float2{-INFINITY, 0.f};
      }
    }
    return;
  }
  // Ancestors-or-self have smaller indices, so no key past the block's last
  // node is visible to any of its rows.
  const int node_hi = min(n - 1, (row0 + MBLK - 1) / G);
  const int ke = min(min(ks + p.keys_per_split, kv_end), P + node_hi + 1);

  // ANCHOR form: block-wide bounds to skip tree tiles no row can see and to
  // treat tiles every row sees in full as unmasked: the min and max anchor
  // and the lowest branch start over the block's nodes (their loads go out
  // below, ahead of the Q, mask-row and first tile loads). Each wave folds
  // its nodes with a butterfly; the barrier publishes the waves' partial
  // bounds.
  int ap_min = -1, ap_max = 0x7fffffff, br_lo = 0x7fffffff;
  const bool anchor = p.mask.kind == TV_MASK_ANCHOR;

  // ---- direct-to-LDS staging (dma_burst, tile_load_offsets): the first
  // NW/2 waves load K, the others V, one 16-key group (one page segment) of
  // the tile each; its page id is looked up a step ahead.
  const bool k_wave = wave < NW / 2;
  // solo blocks (at most 16*NW/2 rows, so group B holds none; the tile loop
  // below tells how they differ)
  const bool solo = rows - row0 <= 16 * (NW / 2);
  const int gw = (k_wave ? wave : wave - NW / 2) * GPW;
  uint32_t voff[IPW], lds0;
  tile_load_offsets<D>(wave, lane, lp, NW, voff, lds0);
  lds0 += k_wave ? lds_u32(&sK[0][0]) : lds_u32(&sV[0][0]);
  constexpr uint32_t kStageBytes = TILE_E * sizeof(__bf16);
  // bytes of one (page, kv head) block of K or V, and this head's first one
  const size_t blk_bytes = (size_t)D * sizeof(__bf16) << lp;
  const char* kv_g = reinterpret_cast<const char*>(k_wave ? p.k : p.v) + (size_t)g * blk_bytes;
  const size_t pg_stride = blk_bytes * p.hkv;
  const int last = kv_end - 1;
  // page id (wave-uniform) of tile position pos; positions past the
  // request's last key use the last key's page: tiles past the end read
  // valid memory that the softmax masks out or whose V is zeroed
  auto page_of = [&](int pos) -> int {
    const int i = min(max((min(pos, last) >> lp) - pg_lo, 0), n_pg - 1);
    return __builtin_amdgcn_readfirstlane(s_pages[i]);
  };
  auto pages_for = [&](int k0, int (&pg)[GPW]) {
#pragma unroll
    for (int l = 0; l < GPW; ++l) pg[l] = page_of(k0 + 16 * (gw + l));
  };
  // the same lookup in two halves: the LDS read early, the result taken a
  // half-step later (no wait on the LDS latency in between)
  int pg_raw[GPW];
  auto pages_load = [&](int k0) {
#pragma unroll
    for (int l = 0; l < GPW; ++l) {
      const int pos = k0 + 16 * (gw + l);
      pg_raw[l] = s_pages[min(max((min(pos, last) >> lp) - pg_lo, 0), n_pg - 1)];
    }
  };
  auto pages_take = [&](int (&pg)[GPW]) {
#pragma unroll
    for (int l = 0; l < GPW; ++l) pg[l] = __builtin_amdgcn_readfirstlane(pg_raw[l]);
  };
  auto issue = [&](int stage, int k0, const int (&pg)[GPW]) {
    // the wave's group starts at position slot of its page (K rows of D
    // elements, V 16-key runs of each d row)
    const int slot = (k0 + 16 * gw) & pmask;
    const char* src = kv_g + (size_t)(uint32_t)pg[0] * pg_stride +
                      (uint32_t)(k_wave ? slot * D : slot) * sizeof(__bf16);
    const uint32_t lds = lds0 + (uint32_t)stage * kStageBytes;
    if (solo) {
      // blocks bound by HBM latency: the wave's loads one at a time, each
      // with its own M0 (four back-to-back loads were slower there, 102.9
      // against 99.2 us for 64 short chains; the blocks of both groups gain
      // from the burst's fewer scalar instructions)
#pragma unroll
      for (int m = 0; m < IPW; ++m) dma_single(src + voff[m] + 1024 * m, lds + 1024 * m);
    } else {
      dma_burst<IPW>(src, voff, lds);
    }
  };

  // Q fragments (B operand of S^T): lane (r16, q4) holds row r16 of its
  // subtile, d = 32s + 8q4 .. +7. Subtiles st = wave + NW r hold rows
  // row0 + 16 st ..; the first nv of them (a wave-uniform count) have a real
  // row. Padding rows carry the request's first row's Q and are never
  // stored, so the MFMAs below run unguarded. load_rows() issues these loads
  // and the mask rows'; they stay in flight while the block's first K/V
  // tiles are requested.
  int nv = 0;
#pragma unroll
  for (int r = 0; r < RW; ++r) nv += (row0 + 16 * (wave + NW * r) < rows) ? 1 : 0;
  bf16x8 qf[RW][DS];
  int orow[RW], rnode[RW], rloc[RW];
  bool row_ok[RW];
  // per-row mask data kept in registers: ANCHOR (anchor_pos and
  // branch_depth in m_ap, m_bd), BITS with <= 2 words (the two words in
  // m_w0, m_w1); wider BITS masks (the WIDE instantiation) are read per
  // masked tile. (Separate registers per form: one 64-bit value built from
  // either form's loads needed copies that waited for every load in flight.)
  const bool bits_in_regs = !WIDE && !anchor;
  uint64_t m_w0[RW], m_w1[RW];
  uint32_t m_ap[RW], m_bd[RW];
  auto load_rows = [&]() {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int row = row0 + 16 * (wave + NW * r) + r16;
      row_ok[r] = row < rows;
      const int i = row_ok[r] ? row / G : 0;
      const int hl = row_ok[r] ? row % G : 0;
      rloc[r] = i;
      rnode[r] = n0 + i;
      orow[r] = (n0 + i) * p.hq + g * G + hl;
      // unconditional loads whose values are first used after the first tiles
      // are requested: a padding row reads the request's first row (its scores
      // are computed, never stored, and no other row depends on them; its mask
      // is never consulted), and no select on the loaded values here, which
      // would wait for them before the tile requests. With one mask word the
      // second load reads the first again; bits past the last node are cut by
      // the request's key range.
      // (each form sets only its own registers: a constant written into a
      // register that the other form's load may still be filling would wait
      // for every load in flight)
      if (anchor) {
        m_ap[r] = (uint32_t)p.mask.anchor_pos[rnode[r]];
        m_bd[r] = (uint32_t)p.mask.branch_depth[rnode[r]];
      } else if (bits_in_regs) {
        m_w0[r] = p.mask.bits[(size_t)rnode[r] * p.mask.words];
        m_w1[r] = p.mask.bits[(size_t)rnode[r] * p.mask.words + (p.mask.words - 1)];
      }
  #pragma unroll
      for (int s = 0; s < DS; ++s) {
        const uint4 u = *reinterpret_cast<const uint4*>(p.q + (size_t)orow[r] * D + 32 * s + 8 * q4);
        qf[r][s] = __builtin_bit_cast(bf16x8, u);
      }
    }
  };

  // The block's first two tiles go out with its Q and mask rows, as soon as
  // the request's bounds are known, with the page ids loaded beside those.
  // BITS form: no tile is skipped, so they are tiles ks and ks + 64. ANCHOR
  // form: the same two are requested before the anchor bounds tell whether
  // they are skipped (tile ks is whenever a split starts inside the run no
  // row of the block sees); the anchor bounds' loads go out first, and a
  // wrong guess is requested again below once the bounds are known (its
  // stale loads land first: one wave's loads return in order). The page
  // list in LDS serves the later tiles.
  static_assert(GPW == 1, "one page id per wave and tile");
  int pgn[GPW];
  // ANCHOR: the block's nodes (at most 256, one per thread) for its bounds
  const int node_lo = row0 / G;
  const int a_node = min(node_lo + tid, node_hi);
  int a_ld = 0, d_ld = 0;
  if (anchor) {
    a_ld = p.mask.anchor_pos[n0 + a_node];
    d_ld = p.mask.branch_depth[n0 + a_node];
  }
  load_rows();
  if (ks < ke) { pgn[0] = clampi(pgf[0], 0, p.num_pages - 1); issue(0, ks, pgn); }
  if (ks + kTile < ke) { pgn[0] = clampi(pgf[1], 0, p.num_pages - 1); issue(1, ks + kTile, pgn); }

  if (anchor) {
    static_assert(MBLK <= T, "one node of the block per thread");
    int a_min = 0x7fffffff, a_max = -1, b_lo = 0x7fffffff;
    if (node_lo + tid <= node_hi) {
      a_min = a_ld;
      a_max = a_ld;
      if (d_ld > 0) b_lo = a_node - d_ld + 1;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      a_min = min(a_min, __shfl_xor(a_min, off, 64));
      a_max = max(a_max, __shfl_xor(a_max, off, 64));
      b_lo = min(b_lo, __shfl_xor(b_lo, off, 64));
    }
    if (lane == 0) { s_bounds[wave][0] = a_min; s_bounds[wave][1] = a_max; s_bounds[wave][2] = b_lo; }
  }
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int i = tid + j * T;
    if (i < n_pg) s_pages[i] = clampi(pgv[j], 0, p.num_pages - 1);
  }
  // V of stage STAGES-1 is read (times P = 0) by the first M cluster
  for (int c = tid; c < TILE_E / 8; c += T)
    reinterpret_cast<uint4*>(&sV[STAGES - 1][0])[c] = uint4{0u, 0u, 0u, 0u};
  // the page list, the partial bounds and the zeros are written; make them
  // visible (this waits for the page table's and the bounds' loads, and in
  // the BITS form for the first tiles and the Q and mask rows, which the
  // first step needs anyway)
  __builtin_amdgcn_s_waitcnt(W_ALL & ~0x0F00);
  __syncthreads();
  // Tile [k0, k0+64): skipped when it holds no prefix key and no tree key any
  // row of the block can see (tree position j0 = k0 - P past every anchor,
  // j0 + 63 before every branch start); unmasked when all its keys are
  // visible to all.
  // (unmasked: its keys lie before full_end = min(kv_end, P), or with the
  // ANCHOR form min(kv_end, max(P, P + ap_min + 1)), set with the bounds)
  int full_end = min(kv_end, P);
  auto full_tile = [&](int k0) -> bool { return k0 + kTile <= full_end; };
  // The skipped tiles of the split form one run of consecutive tile starts,
  // [skip_from, skip_to) (set once the bounds are known; none by default).
  int skip_from = 0x7fffffff, skip_to = 0x7fffffff;
  auto next_tile = [&](int k0) {
    const int k = k0 + kTile;
    return k == skip_from ? skip_to : k;
  };
  if (anchor) {
    int a_min = 0x7fffffff, a_max = -1, b_lo = 0x7fffffff;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      a_min = min(a_min, s_bounds[w][0]);
      a_max = max(a_max, s_bounds[w][1]);
      b_lo = min(b_lo, s_bounds[w][2]);
    }
    ap_min = a_min; ap_max = a_max; br_lo = b_lo;
    full_end = (int)min((long long)kv_end, max((long long)P, (long long)P + ap_min + 1));
    // tile starts ks + 64j skipped: from the first at or past
    // max(P, P + ap_max + 1) up to the last at or before P + br_lo - 64
    const long long lo = max((long long)P, (long long)P + ap_max + 1);
    const long long hi = (long long)P + br_lo - kTile;
    const long long f = ks + ((max(lo - ks, 0LL) + kTile - 1) / kTile) * kTile;
    if (f <= hi && f < ke) {
      skip_from = (int)f;
      skip_to = (int)min((long long)ks + ((hi - ks) / kTile + 1) * kTile, (long long)ke);
    }
  }
  // the block's first tiles (known before any tile is requested)
  int c_cur = ks == skip_from ? skip_to : ks;
  int c_prev = ke;  // tile m-1 (none yet)
  int c_n1 = next_tile(c_cur), c_n2 = next_tile(c_n1);

  // Visibility of keys [k0, k0 + 64) for this lane's row of subtile r.
  auto row_visibility = [&](int r, int k0) -> uint64_t {
    if (!row_ok[r]) return 0ull;
    uint64_t v = range_bits(0, P - 1 - k0);
    if (k0 + kTile > P && k0 < kv_end) {
      const int j0 = k0 - P;  // > -64
      uint64_t t;
      if (anchor) {
        const int ap = (int)m_ap[r], bd = (int)m_bd[r];
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
  // fp32 row sums of P: each lane sums its own 16 keys of a row per tile;
  // the 4 lanes of a row are added once, after the last tile
  float l_lane[RW];
  float m_run[RW], alpha[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    m_run[r] = kNoMax;
    l_lane[r] = 0.f;
    alpha[r] = 1.f;
#pragma unroll
    for (int u = 0; u < DU; ++u) o[r][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bool rescale = false;  // some row of the wave raised its running max: O *= alpha

  // ---- S^T = K Q^T of the tile in stage `buf`. Row 4c + i of subtile t of
  // S^T (the A-operand row fed from LDS) is key key_of(t, 4c + i) =
  // 32(t/2) + 8c + 4(t%2) + i, so the lane of query row r16 and column group
  // c = q4 ends up with keys 32kk + 8q4 .. +7 of each 32-key half kk: eight
  // consecutive keys, which is what its B operand of the PV product needs
  // and what one 16-byte LDS read of V supplies.
  auto key_of = [](int t, int m) { return 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3); };
  auto qk = [&](int buf, f32x4 (&sacc)[RW][4]) {
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int t = 0; t < 4; ++t) sacc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int krow = key_of(t, r16);
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
            &sK[buf][krow * D + 8 * ((4 * s + q4) ^ kswz<D>(krow))]);
#pragma unroll
        for (int r = 0; r < RW; ++r)
          sacc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[r][s], sacc[r][t], 0, 0, 0);
      }
    }
  };
  // ---- scores of keys a row may not see -> -inf
  auto apply_mask = [&](int k0, f32x4 (&sacc)[RW][4]) {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      // this lane's 16 keys key_of(t, 4q4 + i) as bits 4t + i of `own`
      const uint64_t sh = row_visibility(r, k0) >> (8 * q4);
      const uint32_t own = (uint32_t)(sh & 0xffu) | ((uint32_t)(sh >> 32) & 0xffu) << 8;
      // bit 4t + i of `own` spread over the score's 32 bits (one bit-field
      // extract), then the score or -inf by that mask (one bit-field insert)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t keep = (uint32_t)((int32_t)(own << (31 - (4 * t + i))) >> 31);
          const float sv = sacc[r][t][i];  // (a bit cast of a vector element
          const uint32_t sb = __builtin_bit_cast(uint32_t, sv);  // itself reads element 0)
          sacc[r][t][i] = __builtin_bit_cast(float, (sb & keep) | (0xff800000u & ~keep));
        }
    }
  };
  // ---- running max from a tile's (masked) scores. The max is raised only
  // when it grows by more than kLazyMax (log2 units), so rows rarely need
  // their O rescaled; probabilities stay <= 2^kLazyMax, exact in fp32 and
  // rounded to bf16 with the same relative error as any other value.
  auto row_update = [&](f32x4 (&sacc)[RW][4]) {
    bool up_any = false;
    // each lane's max of its 16 scores of a row subtile as a tree of v_max3
    // (depth 3 instead of a chain of 8), the row subtiles side by side
    float mx4[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const f32x4* v = sacc[r];
      const float a0 = fmax3_raw(v[0][0], v[0][1], v[0][2]);
      const float a1 = fmax3_raw(v[0][3], v[1][0], v[1][1]);
      const float a2 = fmax3_raw(v[1][2], v[1][3], v[2][0]);
      const float a3 = fmax3_raw(v[2][1], v[2][2], v[2][3]);
      const float a4 = fmax3_raw(v[3][0], v[3][1], v[3][2]);
      mx4[r] = fmax_raw(fmax3_raw(a0, a1, a2), fmax3_raw(a3, a4, v[3][3]));
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const float mx = row_max4(mx4[r]) * p.scale_log2;
      const bool up = mx > m_run[r] + kLazyMax;
      alpha[r] = up ? __builtin_amdgcn_exp2f(m_run[r] - mx) : 1.f;
      m_run[r] = up ? mx : m_run[r];
      up_any = up_any || up;
    }
    rescale = __builtin_amdgcn_ballot_w64(up_any) != 0;
  };
  // ---- probabilities of a tile against the running max, 2^(s*scale - m),
  // straight into the bf16 B operand of the PV product; `part` gets each
  // lane's fp32 sum of its 16 values per row. The scores are left as they are.
  auto probs = [&](const f32x4 (&sacc)[RW][4], float (&part)[RW], bf16x8 (&pf)[RW][2]) {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const float m_use = m_run[r];
      float pt[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r][t][i], p.scale_log2, -m_use));
          pf[r][t >> 1][4 * (t & 1) + i] = static_cast<__bf16>(e[i]);
        }
        pt[t] = (e[0] + e[1]) + (e[2] + e[3]);
      }
      part[r] = (pt[0] + pt[1]) + (pt[2] + pt[3]);
    }
  };
  // ---- O^T += V^T P^T of the tile in stage `buf`. Element e of lane group
  // q4 is key 32kk + 8q4 + e: 16-key group 2kk + q4/2, keys 8(q4%2) .. +7.
  auto pv = [&](int buf, const bf16x8 (&pf)[RW][2]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int u = 0; u < DU; ++u) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
            &sV[buf][(2 * kk + (q4 >> 1)) * 16 * D + (16 * u + r16) * 16 + 8 * (q4 & 1)]);
#pragma unroll
        for (int r = 0; r < RW; ++r)
          o[r][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[r][kk], o[r][u], 0, 0, 0);
      }
    }
  };

  // ---- pipeline ("ping-pong"). Tiles c(0), c(1), ... of the block; per
  // tile m two slots separated by barriers. The waves of group A
  // (0 .. NW/2-1) run the MFMA cluster M(m) = [O += V(m-1)^T P(m-1)^T,
  // S(m) = K(m) Q^T] in slot 2m and the VALU cluster V(m) = [mask, running
  // max, rescale, P(m) = exp2(...)] in slot 2m+1; group B (NW = 8 only) runs
  // the same clusters one slot later, so the two waves sharing a SIMD
  // (w, w + 4) keep its matrix and vector pipes busy at the same time.
  // Tile m+2 is requested at the start of slot 2m into the stage that tile
  // m-2 left (its last reader, B's M(m-1), ended before that barrier); tile m
  // must have landed by slot 2m: each wave waits (counted vmcnt) for its own
  // loads of tile m, then the barrier makes every wave's loads visible.
  // wait until at most `pending` loads of this wave are in flight
  auto wait_vm = [&](int pending) {
    if (pending >= 2 * IPW) wait_vmem<2 * IPW>();
    else if (pending >= IPW) wait_vmem<IPW>();
    else wait_vmem<0>();
  };
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // zero the V columns of positions past the request's last key in a tile
  // that just landed (their K columns are masked; V must hold finite zeros
  // for P = 0 to contribute nothing); the next barrier publishes them (the
  // first reader of V(m) is M(m+1), after the next step's first barrier)
  auto zero_tail = [&](int stage, int k0) {
    if (k0 + kTile <= kv_end) return;
    const int lim = kv_end - k0;  // tile keys >= lim are past the end
    // 16-byte chunks: 8 consecutive keys of one d (layout [group][d][16 keys])
    for (int c = tid; c < TILE_E / 8; c += T) {
      const int e = 8 * c;
      const int key0 = 16 * (e / (16 * D)) + (e & 15);
      if (key0 + 7 < lim) continue;
      bf16x8* ch = reinterpret_cast<bf16x8*>(&sV[stage][e]);
      bf16x8 v = *ch;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (key0 + i >= lim) ? static_cast<__bf16>(0.f) : v[i];
      *ch = v;
    }
    __builtin_amdgcn_s_waitcnt(W_ALL & ~0x0F00);  // lgkmcnt(0): zeros written
  };
  const bool grp_b = wave >= NW / 2;
  f32x4 sc[RW][4];
  bf16x8 pf[RW][2];
#pragma unroll
  for (int r = 0; r < RW; ++r) pf[r][0] = pf[r][1] = bf16x8{};
  // M(m) runs both products unconditionally (no branches, so no copies of
  // the accumulators at merge points): before the first tile P is zero and
  // the V stage it reads was zeroed; after the last, the scores are unused.
  auto cluster_m = [&](int m) {
    if (nv == 0) return;
    // the wave in its MFMA cluster issues first on its SIMD; the other
    // group's VALU cluster fills the matrix core's busy cycles
    __builtin_amdgcn_s_setprio(1);
    pv((m - 1) & (STAGES - 1), pf);
    qk(m & (STAGES - 1), sc);
    // software pipeline of the cluster: LDS fragment reads run kAhead
    // fragments ahead of the MFMAs that consume them (RW MFMAs each), which
    // hides LDS latency without holding every fragment in registers
    constexpr int NFRAG = 2 * DU + 4 * DS;
    constexpr int kAhead = 4;
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int f = 0; f < NFRAG - kAhead; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, RW, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, RW * kAhead, 0);
    __builtin_amdgcn_s_setprio(0);
  };
  // VALU cluster. Once the wave's rows hold a running max, the tile's
  // probabilities are first taken against it as it stands: if no lane's sum
  // of its 16 values of a row exceeds 2^kLazyMax, no value does, so no score
  // rose more than kLazyMax above the max and the running max would not have
  // moved -- the values are final, with no max of the tile taken at all.
  // Otherwise (and for a wave's first tile) the max is taken from the scores,
  // which the trial left in place, and raised with a rescale of O and l.
  bool max_set = false;  // wave-uniform: the running maxima have been taken once
  auto cluster_v = [&](int k0) {
    if (nv == 0) return;
    if (!full_tile(k0)) apply_mask(k0, sc);
    float part[RW];
    if (max_set) {
      probs(sc, part, pf);
      uint64_t big = 0;  // lanes with a sum past the slack (or NaN), one compare each
#pragma unroll
      for (int r = 0; r < RW; ++r) big |= __builtin_amdgcn_ballot_w64(!(part[r] <= kLazySum));
      if (big == 0) {
#pragma unroll
        for (int r = 0; r < RW; ++r) l_lane[r] += part[r];
        return;
      }
    }
    max_set = true;
    row_update(sc);
    if (rescale) {
#pragma unroll
      for (int r = 0; r < RW; ++r) {
#pragma unroll
        for (int u = 0; u < DU; ++u) o[r][u] *= alpha[r];
        l_lane[r] *= alpha[r];
      }
    }
    probs(sc, part, pf);
#pragma unroll
    for (int r = 0; r < RW; ++r) l_lane[r] += part[r];
  };

  // ANCHOR form: the first two tiles again where the bounds skip the guess
  if (anchor) {
    if (c_cur < ke && c_cur != ks) { pages_for(c_cur, pgn); issue(0, c_cur, pgn); }
    if (c_n1 < ke && c_n1 != ks + kTile) { pages_for(c_n1, pgn); issue(1, c_n1, pgn); }
  }
  // Solo blocks: the waves of group B hold no rows (at most 16*NW/2 rows),
  // so only group A reads the tiles and the stage of tile m-1 is free once
  // slot 2m ends. Tiles are then requested three ahead, in slot 2m+1, into
  // that stage (3 tiles in flight instead of 2: these blocks are bound by
  // HBM latency, not by the matrix cores).
  int c_n3 = solo ? next_tile(c_n2) : ke;  // tile to request in slot 2m+1 (solo)
  // Q fragments and mask rows are used from registers from here on (this
  // waits for them, and for the tiles requested above)
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    asm volatile("" : "+v"(m_w0[r]), "+v"(m_w1[r]), "+v"(m_ap[r]), "+v"(m_bd[r]));
#pragma unroll
    for (int s = 0; s < DS; ++s) asm volatile("" : "+v"(qf[r][s]));
  }
  if (solo) {
    if (c_n2 < ke) { pages_for(c_n2, pgn); issue(2, c_n2, pgn); }
    pages_for(c_n3, pgn);
  } else {
    pages_for(c_n2, pgn);
  }
  int m = 0;
  // start of slot 2m: tile m has landed and is visible; tile m+2 is
  // requested now (tile m+3 in slot 2m+1 for solo blocks)
  int c_nn = ke;  // successor of the tile requested in this step
  auto head = [&]() {
    if (c_cur < ke)
      wait_vm(solo ? (c_n2 < ke ? 2 * IPW : (c_n1 < ke ? IPW : 0)) : (c_n1 < ke ? IPW : 0));
    barrier();
    if (c_cur < ke) zero_tail(m & (STAGES - 1), c_cur);
  };
  // tile m+2 into the stage tile m-2 left (free since the barrier that
  // opened this step)
  auto request = [&]() {
    if (!solo) {
      if (c_n2 < ke) issue((m + 2) & (STAGES - 1), c_n2, pgn);
      c_nn = next_tile(c_n2);
      pages_load(c_nn);
    }
  };
  // The barrier between a step's two slots orders LDS only in solo blocks:
  // there the stage of tile m-1, which group A's M(m) reads, takes tile m+3
  // in slot 2m+1 (and the V waves of group B issue part of it). Otherwise
  // every stage a step writes was last read in an earlier step and every
  // tile it reads landed before the step's first barrier, so the two groups
  // run their clusters back to back: one wave's matrix cluster meets the
  // other's VALU cluster without either waiting for the slower side of each
  // slot.
  auto mid_barrier = [&]() {
    if (solo) barrier();
  };
  auto mid = [&]() {  // after the barrier that opens slot 2m+1
    if (solo) {
      if (c_n3 < ke) issue((m + 3) & (STAGES - 1), c_n3, pgn);
      c_nn = next_tile(c_n3);
      pages_load(c_nn);
    }
  };
  auto advance = [&]() {
    pages_take(pgn);
    // value selects (a conditional store would take the variables' address)
    const int n2 = solo ? c_n3 : c_nn, n3 = solo ? c_nn : c_n3;
    c_prev = c_cur; c_cur = c_n1; c_n1 = c_n2; c_n2 = n2; c_n3 = n3;
    ++m;
  };
  // Steady state of blocks of both groups (tiles m, m+1 and m+2 exist):
  // tile m is full (it ends before tile m+2 starts, at most at the last
  // key), so the step needs no tail zeros, and its wait count, request and
  // successor are fixed -- the scalar code between the clusters stays short.
  auto head_ss = [&]() {
    wait_vmem<IPW>();
    barrier();
  };
  auto request_ss = [&]() {
    issue((m + 2) & (STAGES - 1), c_n2, pgn);
    c_nn = next_tile(c_n2);
    pages_load(c_nn);
  };
  auto advance_ss = [&]() {
    pages_take(pgn);
    c_prev = c_cur; c_cur = c_n1; c_n1 = c_n2; c_n2 = c_nn;
    ++m;
  };
  // Each group runs straight loops (no per-slot branch between the two
  // clusters, which would force copies of the accumulators); both execute
  // 1 barrier per tile plus 1 at the end (2 and 2 in solo blocks), so the
  // steady-state loop and the general one may hand over at any step.
  if (!grp_b) {
    if (!solo) {
      while (c_n2 < ke) {
        head_ss();
        cluster_m(m);
        request_ss();
        cluster_v(c_cur);
        advance_ss();
      }
    }
    while (c_cur < ke) {
      head();
      cluster_m(m);
      mid_barrier();
      mid();
      request();
      cluster_v(c_cur);
      advance();
    }
    head();
    request();
    cluster_m(m);  // PV of the last tile
    mid_barrier();
  } else {
    if (c_cur < ke) {
      head();
      request();
      mid_barrier();
      mid();
      cluster_m(m);
      advance();
    }
    if (!solo) {
      while (c_n2 < ke) {
        head_ss();
        request_ss();
        cluster_v(c_prev);
        cluster_m(m);
        advance_ss();
      }
    }
    while (c_cur < ke) {
      head();
      request();
      cluster_v(c_prev);
      mid_barrier();
      mid();
      cluster_m(m);
      advance();
    }
    head();
    request();
    if (c_prev < ke) cluster_v(c_prev);
    mid_barrier();
    cluster_m(m);  // PV of the last tile
  }

  // ---- epilogue: lane (r16, q4) holds O[row r16][16u + 4q4 + i]
  const size_t R_tot = (size_t)p.total_nodes * p.hq;
  float l_run[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) l_run[r] = row_sum4(l_lane[r]);
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
      // the split's own softmax average in bf16 (the merge weights it by l):
      // half the bytes of the raw fp32 sums, one more rounding of O
      const size_t prow = (size_t)split * R_tot + orow[r];
      const float inv = l_run[r] > 0.f ? 1.f / l_run[r] : 0.f;
#pragma unroll
      for (int u = 0; u < DU; ++u) {
        bf16x4 h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = static_cast<__bf16>(o[r][u][i] * inv);
        __builtin_nontemporal_store(h, reinterpret_cast<bf16x4*>(p.part_o + prow * D + 16 * u + 4 * q4));
      }
      if (q4 == 0) {
        __builtin_nontemporal_store(l_run[r] > 0.f ? m_run[r] : -INFINITY, p.part_ml + prow * 2);
        __builtin_nontemporal_store(l_run[r], p.part_ml + prow * 2 + 1);
      }
    }
  }
}

// ---- short splits: every tile of the split in LDS at once ("one-shot").
// When a split holds at most kShortTiles key tiles (short prefixes cut over
// many workgroups, e.g. a 60-node tree behind a 2048-key prefix), the tile
// loop's per-tile barriers and pipeline fill cost more than its arithmetic.
// Here a workgroup of 8 waves (16 rows each, 128 rows) requests Q and all of
// its tiles in one round trip (Q through LDS as well, so that every wait is
// a counted one), and every wave takes each tile through S = K Q^T, an
// online-softmax step (the tile loop's lazy running max and trial
// probabilities) and O += V^T P^T as soon as the tile has landed.
//
// Blocks are numbered split-major over groups padded to a multiple of 8, so
// every split of one (request, kv head, row block) -- and, when batch * Hkv
// is a multiple of 8, every row block of one kv head -- is dispatched to the
// same XCD (workgroups go round-robin over the 8 XCDs): the group's Q and
// K/V tiles are fetched from HBM once and then hit that XCD's L2.
//
// With key splits, every split stores its partial (its own softmax
// average in bf16, m and l) and the merge kernel combines them, as for the
// tile loop. (Merging inside this kernel -- by the last split to arrive, or
// by merge workgroups at the end of the grid -- was measured slower on this
// GPU: the acknowledged partial stores and the arrival atomics cost more
// than the kernel boundary they save.)
constexpr int kShortTiles = 4;

template <int D, bool WIDE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bf16_short_kernel(Params p) {
  constexpr int NW = 8;
  constexpr int T = 64 * NW;
  constexpr int DS = D / 32;           // 32-wide d steps of S^T = K Q^T
  constexpr int DU = D / 16;           // 16-wide d subtiles of O^T
  constexpr int MBLK = 16 * NW;        // rows per workgroup
  constexpr int TILE_E = kTile * D;
  constexpr int K_INS = D / 8;         // 1 KB direct-to-LDS loads per K tile
  constexpr int INS = 2 * K_INS;
  constexpr int IPW = INS / NW;        // loads per wave per tile
  constexpr int RPI = 512 / D;         // K rows per load
  constexpr int VPG = D / 32;          // V loads per 16-key group
  static_assert(IPW * RPI == 16 && IPW == VPG, "one 16-key group per wave and tile");
  __shared__ __attribute__((aligned(16))) __bf16 sK[kShortTiles][TILE_E];
  __shared__ __attribute__((aligned(16))) __bf16 sV[kShortTiles][TILE_E];
  // each wave's Q fragments, fragment s of lane l at [wave][s][8 l]
  __shared__ __attribute__((aligned(16))) __bf16 sQ[NW][DS][64 * 8];

  const int ng = p.batch * p.hkv * p.row_blocks;
  const int ng_pad = (ng + 7) & ~7;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q4 = lane >> 4;
  const int gi = blockIdx.x % ng_pad;
  const int split = blockIdx.x / ng_pad;
  if (gi >= ng) return;
  const int g = gi % p.hkv;
  const int b = (gi / p.hkv) % p.batch;
  const int rb = gi / (p.hkv * p.batch);
  const int ks = split * p.keys_per_split;

  // this wave's 16-key group of every tile and its page id: table reads that
  // do not wait for the request's bounds (entries past the request's pages
  // are clamped into the pool; their keys are masked and their V zeroed)
  const int lp = __builtin_ctz(p.page_size);
  const int pmask = p.page_size - 1;
  const bool k_wave = wave < NW / 2;
  const int gw = k_wave ? wave : wave - NW / 2;
  const int32_t* row_tab = p.block_table + (size_t)b * p.max_pages;
  int pg[kShortTiles];
#pragma unroll
  for (int t = 0; t < kShortTiles; ++t)
    pg[t] = row_tab[min((ks + kTile * t + 16 * gw) >> lp, p.max_pages - 1)];

  const int n0 = clampi(p.cu_nodes[b], 0, p.total_nodes);
  const int n = clampi(p.cu_nodes[b + 1], n0, p.total_nodes) - n0;
  const int P = max(p.prefix_len[b], 0);
  const int G = p.group;
  const int rows = n * G;
  const int row0 = rb * MBLK;
  if (row0 >= rows) return;
  const int kv_end = P + n;
  // Keys [ks, ke): none when the split starts past the request's keys or
  // past what the block's last node can see (the split then contributes
  // an empty partial, m = -inf, l = 0).
  const int node_hi = min(n - 1, (row0 + MBLK - 1) / G);
  const int ke = min(min(ks + p.keys_per_split, kv_end), P + node_hi + 1);
  const int nt = ke > ks ? (ke - ks + kTile - 1) / kTile : 0;  // tiles in range, 0 .. kShortTiles

  // ---- Q fragments, staged through LDS and requested before the tiles so
  // they land first (their wait is counted below, as the tiles' are; padding
  // rows read the request's first row)
  const int row = row0 + 16 * wave + r16;
  const bool row_ok = row < rows;
  const bool has_rows = row0 + 16 * wave < rows;  // wave-uniform
  const int li = row_ok ? row / G : 0;
  const int rnode = n0 + li;
  const int orow = rnode * p.hq + g * G + (row_ok ? row % G : 0);
  const bool anchor = p.mask.kind == TV_MASK_ANCHOR;
#pragma unroll
  for (int s = 0; s < DS; ++s)
    dma_single(p.q + (size_t)orow * D + 32 * s + 8 * q4, lds_u32(&sQ[wave][s][0]));

  // ---- all tiles of the split, straight into LDS (layouts as in the tile loop)
  uint32_t voff[IPW], lds0;
  tile_load_offsets<D>(wave, lane, lp, NW, voff, lds0);
  lds0 += k_wave ? lds_u32(&sK[0][0]) : lds_u32(&sV[0][0]);
  const size_t blk_bytes = (size_t)D * sizeof(__bf16) << lp;
  const char* kv_g = reinterpret_cast<const char*>(k_wave ? p.k : p.v) + (size_t)g * blk_bytes;
#pragma unroll
  for (int t = 0; t < kShortTiles; ++t) {
    if (t >= nt) break;
    const int slot = (ks + kTile * t + 16 * gw) & pmask;
    const uint32_t pgt = __builtin_amdgcn_readfirstlane(clampi(pg[t], 0, p.num_pages - 1));
    const char* src = kv_g + (size_t)pgt * (blk_bytes * p.hkv) +
                      (uint32_t)(k_wave ? slot * D : slot) * sizeof(__bf16);
    dma_burst<IPW>(src, voff, lds0 + (uint32_t)(t * TILE_E * sizeof(__bf16)));
  }
  // this wave's Q fragments: its loads of them have landed once at most its
  // tile loads are in flight (loads return in order); only this wave reads them
  if (nt >= 4) wait_vmem<4 * IPW>();
  else if (nt == 3) wait_vmem<3 * IPW>();
  else if (nt == 2) wait_vmem<2 * IPW>();
  else if (nt == 1) wait_vmem<IPW>();
  else wait_vmem<0>();
  asm volatile("" ::: "memory");
  bf16x8 qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(&sQ[wave][s][8 * lane]);
  // mask rows, requested after the tiles: the first use of a plain load waits
  // for every load in flight, and they are first used in a tile that reaches
  // the tree keys (the last tiles of the request). Each form sets only the
  // words it reads (a zero written into a register that the other form's load
  // may still be filling would wait for every load in flight).
  uint64_t m_w0, m_w1;
  if (anchor) {
    m_w0 = (uint64_t)(uint32_t)p.mask.anchor_pos[rnode] |
           ((uint64_t)(uint32_t)p.mask.branch_depth[rnode] << 32);
  } else if (!WIDE) {
    m_w0 = p.mask.bits[(size_t)rnode * p.mask.words];
    m_w1 = p.mask.bits[(size_t)rnode * p.mask.words + (p.mask.words - 1)];
  }

  // visibility of keys [k0, k0 + 64) for this lane's row (as in the tile loop)
  auto row_visibility = [&](int k0) -> uint64_t {
    if (!row_ok) return 0ull;
    uint64_t v = range_bits(0, P - 1 - k0);
    if (k0 + kTile > P && k0 < kv_end) {
      const int j0 = k0 - P;
      uint64_t t;
      if (anchor) {
        const int ap = (int)(uint32_t)m_w0, bd = (int)(uint32_t)(m_w0 >> 32);
        t = range_bits(-j0, ap - j0) | range_bits(li - bd + 1 - j0, li - j0);
      } else if (!WIDE) {
        if (j0 < 0) {
          t = m_w0 << (-j0);
        } else {
          const int sh = j0 & 63;
          const uint64_t lo = (j0 < 64) ? m_w0 : m_w1;
          const uint64_t hi = (j0 < 64) ? m_w1 : 0ull;
          t = sh ? ((lo >> sh) | (hi << (64 - sh))) : lo;
        }
      } else {
        return tile_visibility(p.mask, rnode, li, P, kv_end, k0);
      }
      v |= t & range_bits(P - k0, kv_end - 1 - k0);
    }
    return v;
  };
  // ---- S^T = K Q^T of tile t (score rows permuted as in the tile loop: the
  // lane of row r16, column group q4 holds keys 32kk + 8q4 .. +7)
  auto key_of = [](int t, int m) { return 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3); };
  f32x4 sc[4];
  auto qk = [&](int t) {
#pragma unroll
    for (int u = 0; u < 4; ++u) sc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int krow = key_of(u, r16);
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
            &sK[t][krow * D + 8 * ((4 * s + q4) ^ kswz<D>(krow))]);
        sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], sc[u], 0, 0, 0);
      }
    }
  };
  // ---- online softmax over the split's tiles, one tile at a time as it
  // lands (running max in log2 units, raised lazily as in the tile loop)
  float m_run = kNoMax, l_lane = 0.f;
  bool max_set = false;  // wave-uniform: the running max has been taken once
  bf16x8 pf[2];
  f32x4 o[DU];
#pragma unroll
  for (int u = 0; u < DU; ++u) o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mask_tile = [&](int k0) {
    const uint64_t sh = row_visibility(k0) >> (8 * q4);
    const uint32_t own = (uint32_t)(sh & 0xffu) | ((uint32_t)(sh >> 32) & 0xffu) << 8;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[u][i] = ((own >> (4 * u + i)) & 1u) ? sc[u][i] : -INFINITY;
  };
  // probabilities against the running max, straight into the bf16 B operand
  // of the PV product; returns this lane's fp32 sum of its 16 values
  auto probs = [&]() -> float {
    float pt[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][i], p.scale_log2, -m_run));
        pf[u >> 1][4 * (u & 1) + i] = static_cast<__bf16>(e[i]);
      }
      pt[u] = (e[0] + e[1]) + (e[2] + e[3]);
    }
    return (pt[0] + pt[1]) + (pt[2] + pt[3]);
  };
  auto softmax_step = [&]() {
    if (max_set) {
      const float part = probs();
      if (__builtin_amdgcn_ballot_w64(!(part <= kLazySum)) == 0) {
        l_lane += part;
        return;
      }
    }
    max_set = true;
    const float a0 = fmax3_raw(sc[0][0], sc[0][1], sc[0][2]);
    const float a1 = fmax3_raw(sc[0][3], sc[1][0], sc[1][1]);
    const float a2 = fmax3_raw(sc[1][2], sc[1][3], sc[2][0]);
    const float a3 = fmax3_raw(sc[2][1], sc[2][2], sc[2][3]);
    const float a4 = fmax3_raw(sc[3][0], sc[3][1], sc[3][2]);
    const float mx = row_max4(fmax_raw(fmax3_raw(a0, a1, a2), fmax3_raw(a3, a4, sc[3][3]))) * p.scale_log2;
    const bool up = mx > m_run + kLazyMax;
    if (__builtin_amdgcn_ballot_w64(up) != 0) {
      const float alpha = up ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
#pragma unroll
      for (int u = 0; u < DU; ++u) o[u] *= alpha;
      l_lane *= alpha;
      m_run = up ? mx : m_run;
    }
    l_lane += probs();
  };
  // ---- O^T += V^T P^T of tile t
  auto pv = [&](int t) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int u = 0; u < DU; ++u) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
            &sV[t][(2 * kk + (q4 >> 1)) * 16 * D + (16 * u + r16) * 16 + 8 * (q4 & 1)]);
        o[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[kk], o[u], 0, 0, 0);
      }
    }
  };

  // ---- tiles land in order: wait for this wave's loads of tile t (counted
  // vmcnt), then the barrier publishes every wave's part of it; each wave
  // then takes the tile through S, the softmax step and O
  const bool tail = nt > 0 && ks + kTile * nt > kv_end;
#pragma unroll
  for (int t = 0; t < kShortTiles; ++t) {
    if (t >= nt) break;
    const int later = nt - 1 - t;  // tiles requested after this one
    if (later >= 3) wait_vmem<3 * IPW>();
    else if (later == 2) wait_vmem<2 * IPW>();
    else if (later == 1) wait_vmem<IPW>();
    else wait_vmem<0>();
    __builtin_amdgcn_s_barrier();
    if (t == nt - 1 && tail) {
      // V of the positions past the request's last key (cache slots the
      // caller never wrote) must be finite zeros: P = 0 there. Published by
      // a second barrier, before the PV product of this tile.
      const int lim = kv_end - (ks + kTile * t);
      for (int c = tid; c < TILE_E / 8; c += T) {
        const int e = 8 * c;
        const int key0 = 16 * (e / (16 * D)) + (e & 15);
        if (key0 + 7 < lim) continue;
        bf16x8* ch = reinterpret_cast<bf16x8*>(&sV[t][e]);
        bf16x8 v = *ch;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (key0 + i >= lim) ? static_cast<__bf16>(0.f) : v[i];
        *ch = v;
      }
      __builtin_amdgcn_s_waitcnt(W_ALL & ~0x0F00);
      __builtin_amdgcn_s_barrier();
    }
    if (has_rows) {
      const int k0 = ks + kTile * t;
      qk(t);
      if (k0 + kTile > P) mask_tile(k0);
      softmax_step();
      pv(t);
    }
  }
  const float l_row = row_sum4(l_lane);
  const float m_row = l_row > 0.f ? m_run : -INFINITY;

  // ---- epilogue: lane (r16, q4) holds O[row r16][16u + 4q4 + i]. The
  // wave's 16 rows go through its own Q stage in LDS (no longer read; 16-byte
  // chunks XOR-swizzled by row), so that each store instruction writes whole
  // rows, 16 bytes a lane, instead of 8-byte pieces of 16 rows.
  constexpr int CPR16 = D / 8;         // 16-byte chunks per row
  constexpr int RPS = 64 / CPR16;      // rows per store instruction
  auto swz = [](int rr) { return rr & (CPR16 - 1); };
  const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
  char* ep = reinterpret_cast<char*>(&sQ[wave][0][0]);
  if (p.splits == 1 || nt > 0) {
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      bf16x4 h;
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = static_cast<__bf16>(o[u][i] * inv);
      const int c = 2 * u + (q4 >> 1);
      *reinterpret_cast<bf16x4*>(ep + r16 * (2 * D) + ((c ^ swz(r16)) << 4) + 8 * (q4 & 1)) = h;
    }
  }
  const size_t obase = p.splits == 1 ? 0 : (size_t)split * p.total_nodes * p.hq;
  // row rr of the wave's 16 and the 16-byte chunk c of it that this lane
  // stores in store instruction m; false past the request's rows
  auto chunk = [&](int m, size_t& off, bf16x8& v) -> bool {
    const int rr = RPS * m + lane / CPR16, c = lane % CPR16;
    const int rw = row0 + 16 * wave + rr;
    off = (obase + (size_t)(n0 + rw / G) * p.hq + g * G + rw % G) * D + 8 * c;
    v = *reinterpret_cast<const bf16x8*>(ep + rr * (2 * D) + ((c ^ swz(rr)) << 4));
    return rw < rows;
  };
  if (p.splits == 1) {
#pragma unroll
    for (int m = 0; m < 16 / RPS; ++m) {
      size_t off;
      bf16x8 v;
      if (chunk(m, off, v)) *reinterpret_cast<bf16x8*>(p.out + off) = v;
    }
  } else if (nt > 0) {
    // partials: nontemporal (less dirty L2 to write back when the kernel ends)
#pragma unroll
    for (int m = 0; m < 16 / RPS; ++m) {
      size_t off;
      bf16x8 v;
      if (chunk(m, off, v)) __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(p.part_o + off));
    }
    // (keeps the compiler from sinking the last store of each loop into one
    // shared store, which drops the nontemporal hint)
    asm volatile("; partial rows stored" ::: "memory");
  }
  if (!row_ok || q4 != 0) return;
  if (p.splits == 1) {
    if (p.lse) p.lse[orow] = l_row > 0.f ? (m_row + log2f(l_row)) * kLn2 : -INFINITY;
    return;
  }
  // partials for the merge kernel, [split][total_nodes * hq] rows; a split
  // with no key for this block stores only its empty marker (m = -inf,
  // l = 0: the merge never reads that split's o)
  typedef __attribute__((ext_vector_type(2))) float f32x2;
  __builtin_nontemporal_store(f32x2{m_row, l_row},
                              reinterpret_cast<f32x2*>(p.part_ml + (obase + orow) * 2));
}

// Merge of split partials: m = max m_s, l = sum 2^(m_s - m) l_s,
// o = sum 2^(m_s - m) l_s o_s / l (o_s the split's own average, bf16),
// lse = (m + log2 l) ln 2. One row per D/4 lanes; the partials of CH splits
// (CH >= splits when splits <= 16) are loaded at once, unconditionally (a
// chunk's positions past the last split reload the last split and count as
// empty), so every load of a chunk is in flight together: one round trip.
// Longer split lists are folded in chunks with the same online rescaling.
// Every (split, row) pair holds a partial or an empty marker (m = -inf),
// whose o is never read into the sums.
template <int D, int CH, typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(const __bf16* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      int64_t R_tot, int32_t splits,
                                                      OutT* __restrict__ out, float* __restrict__ lse) {
  constexpr int LPR = D / 4;               // lanes per row
  constexpr int RPB = 256 / LPR;           // rows per block
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  if (row >= R_tot) return;
  float m = -INFINITY, l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += CH) {
    float2 ml[CH];
    bf16x4 os[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int64_t pr = (int64_t)min(s0 + j, splits - 1) * R_tot + row;
      ml[j] = *reinterpret_cast<const float2*>(part_ml + pr * 2);
      os[j] = *reinterpret_cast<const bf16x4*>(part_o + pr * D + 4 * sub);
    }
#pragma unroll
    for (int j = 0; j < CH; ++j)
      if (s0 + j >= splits) ml[j].x = -INFINITY;
    // (no early exit for an all-empty chunk: a branch on the maxima would
    // hold the other loads back until they are known, a second round trip)
    float mc = m;
#pragma unroll
    for (int j = 0; j < CH; ++j) mc = fmaxf(mc, ml[j].x);
    const float a = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mc);
    l *= a;
    acc *= a;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const bool live = ml[j].x != -INFINITY;
      const float w = live ? __builtin_amdgcn_exp2f(ml[j].x - mc) : 0.f;
      const float wl = w * ml[j].y;
      l += live ? wl : 0.f;
      f32x4 o4;
#pragma unroll
      for (int i = 0; i < 4; ++i) o4[i] = static_cast<float>(os[j][i]);
      acc = live ? acc + wl * o4 : acc;
    }
    m = mc;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  OutT* dst = out + row * D + 4 * sub;
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = static_cast<OutT>(acc[i] * inv);
  if (lse && sub == 0) lse[row] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

// The same merge for many rows (at least 16,384, so that the blocks still
// fill the GPU): 8 elements (16 bytes) a lane, half the lanes and loads.
template <int D, int CH>
__global__ __launch_bounds__(256) void combine_wide_kernel(const __bf16* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           int64_t R_tot, int32_t splits,
                                                           __bf16* __restrict__ out, float* __restrict__ lse) {
  constexpr int LPR = D / 8;               // lanes per row
  constexpr int RPB = 256 / LPR;           // rows per block
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  if (row >= R_tot) return;
  float m = -INFINITY, l = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += CH) {
    float2 ml[CH];
    bf16x8 os[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int64_t pr = (int64_t)min(s0 + j, splits - 1) * R_tot + row;
      ml[j] = *reinterpret_cast<const float2*>(part_ml + pr * 2);
      os[j] = *reinterpret_cast<const bf16x8*>(part_o + pr * D + 8 * sub);
    }
#pragma unroll
    for (int j = 0; j < CH; ++j)
      if (s0 + j >= splits) ml[j].x = -INFINITY;
    float mc = m;
#pragma unroll
    for (int j = 0; j < CH; ++j) mc = fmaxf(mc, ml[j].x);
    const float a = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mc);
    l *= a;
    acc0 *= a;
    acc1 *= a;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const bool live = ml[j].x != -INFINITY;
      const float w = live ? __builtin_amdgcn_exp2f(ml[j].x - mc) : 0.f;
      const float wl = w * ml[j].y;
      l += live ? wl : 0.f;
      f32x4 o0, o1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o0[i] = static_cast<float>(os[j][i]);
        o1[i] = static_cast<float>(os[j][4 + i]);
      }
      acc0 = live ? acc0 + wl * o0 : acc0;
      acc1 = live ? acc1 + wl * o1 : acc1;
    }
    m = mc;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  bf16x8 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = static_cast<__bf16>(acc0[i] * inv);
    h[4 + i] = static_cast<__bf16>(acc1[i] * inv);
  }
  *reinterpret_cast<bf16x8*>(out + row * D + 8 * sub) = h;
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
  if (plan.short_splits) {
    if (prm.mask.kind == TV_MASK_BITS && prm.mask.words > 2)
      hipLaunchKernelGGL((attn_bf16_short_kernel<D, true>), dim3(grid), dim3(512), 0, stream, prm);
    else
      hipLaunchKernelGGL((attn_bf16_short_kernel<D, false>), dim3(grid), dim3(512), 0, stream, prm);
    return hipGetLastError();
  }
  if (plan.rw == 1) return run_bf16<D, 8, 1>(prm, grid, stream);
  return run_bf16<D, 8, 2>(prm, grid, stream);
}

}  // namespace

AttnPlan plan_attn(int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t max_prefix_len,
                   int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype, int32_t num_cus) {
  AttnPlan pl{};
  pl.num_cus = num_cus > 0 ? num_cus : 1;
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
  // 8 waves (two groups sharing the SIMDs) x 1 subtile (128 rows per block);
  // 8 x 2 (256 rows) when a kv head has more rows and keys enough for the
  // larger block to amortise its longer per-tile step
  const long kv = (long)max_prefix_len + max_nodes;
  const long tiles = (kv + kTile - 1) / kTile;
  pl.waves = 8;
  pl.rw = (rows > 128 && tiles >= 48) ? 2 : 1;
  const long mblk = 16L * pl.waves * pl.rw;
  pl.row_blocks = (int)((rows + mblk - 1) / mblk);
  const long base = (long)batch * hkv * pl.row_blocks;
  // One 128 KB-LDS workgroup fits a CU: cut the keys into splits until the
  // workgroups cover the CUs once; more splits only add partial traffic.
  const long cus = pl.num_cus;
  long splits = std::max(1L, std::min(tiles, cus / base));
  // a split's pages must fit the block's LDS page list (16-token pages)
  const long max_tps = (long)(kMaxSplitPages - 8) * 16 / kTile;
  splits = std::max(splits, (tiles + max_tps - 1) / max_tps);
  const long tps = (tiles + splits - 1) / splits;
  // whole 64-key tiles per split: the kernels mask only keys past the
  // request's end, so a split ending inside a tile would also count the next
  // split's keys in that tile
  pl.keys_per_split = (int)(tps * kTile);
  pl.splits = (int)((tiles + tps - 1) / tps);
  // splits of a few tiles take the one-shot kernel (128-row blocks)
  pl.short_splits = (pl.rw == 1 && tps <= kShortTiles) ? 1 : 0;
  if (pl.splits > 1) {
    const size_t rtot = (size_t)total_nodes * hq;
    const size_t o_bytes = (size_t)pl.splits * rtot * head_dim * sizeof(__bf16);
    const size_t ml_bytes = (size_t)pl.splits * rtot * 2 * sizeof(float);
    pl.part_ml_offset = (o_bytes + 255) & ~(size_t)255;
    pl.workspace = pl.part_ml_offset + ((ml_bytes + 255) & ~(size_t)255);
  } else {
    pl.part_ml_offset = 0;
    pl.workspace = 0;
  }
  return pl;
}
// the merge with the smallest chunk that holds every split (16 at most)
template <int D>
hipError_t launch_combine(const Params& p, int splits, int64_t rtot, float* lse, hipStream_t stream) {
  if (rtot >= 16384 && splits <= 4) {
    constexpr int rpw = 256 / (D / 8);
    const int wgrid = (int)((rtot + rpw - 1) / rpw);
    if (splits <= 2)
      hipLaunchKernelGGL((combine_wide_kernel<D, 2>), dim3(wgrid), dim3(256), 0, stream, p.part_o,
                         p.part_ml, rtot, splits, p.out, lse);
    else
      hipLaunchKernelGGL((combine_wide_kernel<D, 4>), dim3(wgrid), dim3(256), 0, stream, p.part_o,
                         p.part_ml, rtot, splits, p.out, lse);
    return hipGetLastError();
  }
  constexpr int rpb = 256 / (D / 4);
  const int cgrid = (int)((rtot + rpb - 1) / rpb);
  if (splits <= 2)
    hipLaunchKernelGGL((combine_kernel<D, 2, __bf16>), dim3(cgrid), dim3(256), 0, stream, p.part_o,
                       p.part_ml, rtot, splits, p.out, lse);
  else if (splits <= 4)
    hipLaunchKernelGGL((combine_kernel<D, 4, __bf16>), dim3(cgrid), dim3(256), 0, stream, p.part_o,
                       p.part_ml, rtot, splits, p.out, lse);
  else if (splits <= 8)
    hipLaunchKernelGGL((combine_kernel<D, 8, __bf16>), dim3(cgrid), dim3(256), 0, stream, p.part_o,
                       p.part_ml, rtot, splits, p.out, lse);
  else
    hipLaunchKernelGGL((combine_kernel<D, 16, __bf16>), dim3(cgrid), dim3(256), 0, stream, p.part_o,
                       p.part_ml, rtot, splits, p.out, lse);
  return hipGetLastError();
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
  p.part_o = plan.splits > 1 ? reinterpret_cast<__bf16*>(ws) : nullptr;
  p.part_ml = plan.splits > 1 ? reinterpret_cast<float*>(ws + plan.part_ml_offset) : nullptr;
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
  const int ng = a.batch * a.hkv * plan.row_blocks;
  const int grid = plan.short_splits ? ((ng + 7) & ~7) * plan.splits : ng * plan.splits;
  p.lpt = (!plan.short_splits && a.batch >= 2 && a.batch <= kMaxLptBatch && grid > plan.num_cus) ? 1 : 0;
  hipError_t e = (a.head_dim == 64) ? dispatch_bf16<64>(p, plan, grid, stream)
                                    : dispatch_bf16<128>(p, plan, grid, stream);
  if (e != hipSuccess || plan.splits == 1) return e;
  return (a.head_dim == 64) ? launch_combine<64>(p, plan.splits, rtot, a.lse, stream)
                            : launch_combine<128>(p, plan.splits, rtot, a.lse, stream);
}

}  // namespace tv
