// tv_attn.hip -- tree_verify_attn: one target attention layer over a flattened tree.
//
// Graft (arXiv:2605.20104) §二, third gear: one parallel verification pass of
// the flattened tree under the tree mask. SpecOPD (arXiv:2611.02846) §02,
// proposal tree: all branches are scored in one pass that shares the trunk
// KV cache. D-cut (paper 2607.14647) technical summary §1 (verification of
// B x (D+1) tokens per step turns compute-bound as B grows) and §2 pipeline
// (each request keeps a contiguous prefix; the packed batch is verified).
//
// bf16 path (MFMA, gfx950). A workgroup (4 wavefronts) owns one
// (request, kv head, row block, key split). Rows are the (node, query head)
// pairs of one GQA group, node-major, so all query heads that share a kv head
// and all tree nodes of the request are packed into the MFMA M/N dimension
// and every K/V byte brought into LDS is used by up to 64*rw rows.
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16, A = K tile from LDS [key][d],
//                 B = Q fragment kept in VGPRs; lane (r, q) of the 16x16
//                 result holds row r, keys 4q..4q+3 of the subtile.
//   online softmax in fp32, exp2 with the scale folded into log2(e); the
//                 ancestor mask is evaluated only on tiles that hold tree keys
//                 (or run past the end of the request).
//   O^T += V^T P^T  A = V^T from LDS (V transposed while staging), B = P
//                 converted to bf16 straight from the S^T accumulators.
// K/V tiles of 64 keys are gathered through the page table with 128-bit
// loads into registers one tile ahead and stored into a double-buffered LDS.
// Long prefixes are cut into key splits whose (m, l, o) partials are merged
// by a second kernel with the usual LSE weights.
//
// fp32 path (VALU): 4 lanes per row, a 64-key tile of K/V in LDS, same math.
#include <algorithm>

#include "tv_internal.h"

namespace tv {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTile = 64;        // keys per tile
constexpr int kWaves = 4;        // wavefronts per workgroup (bf16 path)
constexpr int kThreads = 64 * kWaves;

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
  float scale_log2;
};

__device__ __forceinline__ uint32_t lo16x2(uint32_t a, uint32_t b) {  // {a.lo, b.lo}
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi16x2(uint32_t a, uint32_t b) {  // {a.hi, b.hi}
  return (a >> 16) | (b & 0xffff0000u);
}

// Element offset of (position pos, kv head g) in a [page][hkv][page_size][D]
// cache, or -1 when the position is past the request's keys or its table.
template <int D>
__device__ __forceinline__ long kv_offset(const Params& p, int b, int g, int pos, int kv_end) {
  if (pos >= kv_end) return -1;
  const int pi = pos / p.page_size;
  if (pi >= p.max_pages) return -1;
  const int pg = clampi(p.block_table[(size_t)b * p.max_pages + pi], 0, p.num_pages - 1);
  return ((long)(pg * p.hkv + g) * p.page_size + pos % p.page_size) * D;
}

template <int D, int RW>
__global__ __launch_bounds__(kThreads) void attn_bf16_kernel(Params p) {
  constexpr int KSTR = D + 8;          // K tile row stride in LDS (elements)
  constexpr int VSTR = kTile + 8;      // V^T tile row stride in LDS (elements)
  constexpr int DS = D / 32;           // 32-wide d steps of S^T = K Q^T
  constexpr int DU = D / 16;           // 16-wide d subtiles of O^T
  constexpr int MBLK = 16 * kWaves * RW;
  __shared__ __attribute__((aligned(16))) __bf16 sK[2][kTile * KSTR];
  __shared__ __attribute__((aligned(16))) __bf16 sV[2][D * VSTR];
  __shared__ int s_bounds[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int r16 = lane & 15, q4 = lane >> 4;

  int wg = blockIdx.x;
  const int split = wg % p.splits;
  wg /= p.splits;
  const int rb = wg % p.row_blocks;
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
    for (int i = node_lo + tid; i <= node_hi; i += kThreads) {
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

  // Q fragments (B operand of S^T): lane (r16, q4) holds row r16 of its
  // subtile, d = 32s + 8q4 .. +7.
  // Subtiles st = wave + 4r hold rows row0 + 16 st ..; the first nv of them
  // (a wave-uniform count) have at least one real row. Padding rows carry
  // zero Q and are never stored, so the MFMAs below run unguarded.
  int nv = 0;
#pragma unroll
  for (int r = 0; r < RW; ++r) nv += (row0 + 16 * (wave + kWaves * r) < rows) ? 1 : 0;
  bf16x8 qf[RW][DS];
  bool sub_ok[RW];
  int orow[RW], rnode[RW], rloc[RW];
  bool row_ok[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int st = wave + kWaves * r;
    sub_ok[r] = r < nv;
    const int row = row0 + 16 * st + r16;
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
  }

  f32x4 o[RW][DU];
  float m_run[RW], l_run[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
#pragma unroll
    for (int u = 0; u < DU; ++u) o[r][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Staging unit = 4 consecutive keys x 8 elements (one 16-byte chunk per key).
  // A tile has 16 key groups x D/8 chunks units per tensor. K units are
  // numbered chunk-fastest (a wave reads whole 256-byte rows), V units key-
  // group-fastest (a wave's transposed LDS stores fill whole V^T row
  // segments). head_dim 128: each thread moves one K and one V unit;
  // head_dim 64: threads 0..127 move K, threads 128..255 move V.
  constexpr int CPR = D / 8;
  constexpr int UNITS = 16 * CPR;
  static_assert(UNITS == kThreads || 2 * UNITS == kThreads, "staging map");
  constexpr bool BOTH = UNITS == kThreads;
  const bool do_k = BOTH || tid < UNITS;
  const bool do_v = BOTH || tid >= UNITS;
  const int ku = tid, vu = BOTH ? tid : tid - UNITS;
  const int kc = ku % CPR, kkg = ku / CPR;
  const int vkg = vu % 16, vc = vu / 16;
  uint4 kreg[4], vreg[4];
  auto gload = [&](int k0) {
    if (do_k) {
      const long ko = kv_offset<D>(p, b, g, k0 + 4 * kkg, kv_end);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bool ok = ko >= 0 && k0 + 4 * kkg + k < kv_end;
        kreg[k] = ok ? *reinterpret_cast<const uint4*>(p.k + ko + k * D + 8 * kc) : uint4{0, 0, 0, 0};
      }
    }
    if (do_v) {
      const long vo = kv_offset<D>(p, b, g, k0 + 4 * vkg, kv_end);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bool ok = vo >= 0 && k0 + 4 * vkg + k < kv_end;
        vreg[k] = ok ? *reinterpret_cast<const uint4*>(p.v + vo + k * D + 8 * vc) : uint4{0, 0, 0, 0};
      }
    }
  };
  auto sstore = [&](int buf) {
    if (do_k) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *reinterpret_cast<uint4*>(&sK[buf][(4 * kkg + k) * KSTR + 8 * kc]) = kreg[k];
    }
    if (!do_v) return;
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vreg[1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vreg[2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vreg[3]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int h = e >> 1;
      uint2 t;
      if (e & 1) { t.x = hi16x2(w0[h], w1[h]); t.y = hi16x2(w2[h], w3[h]); }
      else       { t.x = lo16x2(w0[h], w1[h]); t.y = lo16x2(w2[h], w3[h]); }
      *reinterpret_cast<uint2*>(&sV[buf][(8 * vc + e) * VSTR + 4 * vkg]) = t;
    }
  };

  auto next_tile = [&](int k0) {
    int k = k0 + kTile;
    while (k < ke && skip_tile(k)) k += kTile;
    return k;
  };

  int k0 = ks;
  while (k0 < ke && skip_tile(k0)) k0 += kTile;
  int buf = 0;
  if (k0 < ke) {
    gload(k0);
    sstore(0);
  }
  __syncthreads();

  for (; k0 < ke;) {
    const int kn = next_tile(k0);
    if (kn < ke) gload(kn);
    const bool masked = !full_tile(k0);

    if (nv > 0) {
    // ---- S^T = K Q^T for every row subtile of this wave
    f32x4 sacc[RW][4];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int t = 0; t < 4; ++t) sacc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&sK[buf][(16 * t + r16) * KSTR + 32 * s + 8 * q4]);
#pragma unroll
        for (int r = 0; r < RW; ++r)
          sacc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[r][s], sacc[r][t], 0, 0, 0);
      }
    }

    // ---- online softmax (row r16 of each subtile; this lane has keys 16t + 4q4 + i)
    bf16x8 pf[RW][2];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      // this lane's 16 keys 16t + 4q4 + i as bits 4t + i of `own`
      uint32_t own = 0xffffu;
      if (masked) {
        const uint64_t vis = row_ok[r] ? tile_visibility(p.mask, rnode[r], rloc[r], P, kv_end, k0) : 0ull;
        const uint64_t sh = vis >> (4 * q4);
        own = (uint32_t)(sh & 0xfu) | (uint32_t)((sh >> 12) & 0xf0u) |
              (uint32_t)((sh >> 24) & 0xf00u) | (uint32_t)((sh >> 36) & 0xf000u);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = sacc[r][t][i] * p.scale_log2;
          if (!((own >> (4 * t + i)) & 1u)) x = -INFINITY;
          sacc[r][t][i] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[r], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[r] - m_use);
      float sum = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(sacc[r][t][i] - m_use);
          sacc[r][t][i] = e;
          sum += e;
        }
      sum += __shfl_xor(sum, 16, 64);
      sum += __shfl_xor(sum, 32, 64);
      l_run[r] = l_run[r] * alpha + sum;
      m_run[r] = m_new;
#pragma unroll
      for (int u = 0; u < DU; ++u) o[r][u] *= alpha;
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

    // ---- O^T += V^T P^T; logical k of lane group q4, element e:
    //      keys 32kk + 4q4 + e (e < 4) and 32kk + 16 + 4q4 + (e - 4) (e >= 4)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int u = 0; u < DU; ++u) {
        const __bf16* vrow = &sV[buf][(16 * u + r16) * VSTR + 32 * kk + 4 * q4];
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + 16);
        const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int r = 0; r < RW; ++r)
          o[r][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[r][kk], o[r][u], 0, 0, 0);
      }
    }
    }  // nv > 0

    if (kn < ke) sstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    k0 = kn;
  }

  // ---- epilogue: lane (r16, q4) holds O[row r16][16u + 4q4 + i]
  const size_t R_tot = (size_t)p.total_nodes * p.hq;
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    if (!sub_ok[r] || !row_ok[r]) continue;
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
  float m = -INFINITY;
  for (int s = 0; s < ns; ++s) m = fmaxf(m, part_ml[((size_t)s * R_tot + row) * 2]);
  float l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < ns; ++s) {
    const float ms = part_ml[((size_t)s * R_tot + row) * 2];
    if (ms == -INFINITY) continue;
    const float w = __builtin_amdgcn_exp2f(ms - m);
    l += w * part_ml[((size_t)s * R_tot + row) * 2 + 1];
    const f32x4 os = *reinterpret_cast<const f32x4*>(part_o + ((size_t)s * R_tot + row) * D + 4 * sub);
    acc += w * os;
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
        const size_t off = ((size_t)(pg * p.hkv + g) * p.page_size + pos % p.page_size) * D + d;
        kx = p.k[off];
        vx = p.v[off];
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

template <int D, int RW>
hipError_t run_bf16(const Params& prm, const AttnPlan& plan, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_bf16_kernel<D, RW>), dim3(grid), dim3(kThreads), 0, stream, prm);
  return hipGetLastError();
}

template <int D>
hipError_t dispatch_bf16(const Params& prm, const AttnPlan& plan, int grid, hipStream_t stream) {
  if (plan.rw == 1) return run_bf16<D, 1>(prm, plan, grid, stream);
  return run_bf16<D, 2>(prm, plan, grid, stream);
}

}  // namespace

AttnPlan plan_attn(int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t max_prefix_len,
                   int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype) {
  AttnPlan pl{};
  const long G = hkv > 0 ? hq / hkv : 1;
  const long rows = (long)max_nodes * G;
  if (dtype == TV_F32) {
    pl.rw = 1;
    pl.row_blocks = (int)((rows + 15) / 16);
    pl.splits = 1;
    pl.keys_per_split = max_prefix_len + max_nodes;
    pl.workspace = 0;
    return pl;
  }
  pl.rw = rows <= 64 ? 1 : 2;
  const long mblk = 64L * pl.rw;
  pl.row_blocks = (int)((rows + mblk - 1) / mblk);
  const long kv = (long)max_prefix_len + max_nodes;
  const long tiles = (kv + kTile - 1) / kTile;
  const long base = (long)batch * hkv * pl.row_blocks;
  // Enough workgroups to cover the 256 CUs several times over, but no split
  // shorter than 2 tiles (each split re-reads Q and writes a partial row).
  const long target = 1024;
  long splits = (target + base - 1) / base;
  splits = std::min(splits, std::max(1L, tiles / 2));
  splits = std::max(1L, splits);
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
