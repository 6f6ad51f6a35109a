// tv_internal.h -- what the attention kernel compiles against: the mask as the
// kernels see it, tile visibility, and the attention launch plan. Nothing here
// is part of the C ABI; the other kernels' launchers are in tv_launch.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "treeverify.h"

namespace tv {

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Mask as the attention kernels see it (a copy of tv_mask_t).
struct MaskDev {
  int32_t kind;
  int32_t words;
  const uint64_t* bits;
  const int32_t* anchor_pos;
  const int32_t* branch_depth;
};

// Bits [lo, hi] of a 64-bit word (clipped to 0..63; empty when lo > hi).
__device__ __forceinline__ uint64_t range_bits(int lo, int hi) {
  lo = lo < 0 ? 0 : lo;
  hi = hi > 63 ? 63 : hi;
  if (lo > hi) return 0ull;
  const uint64_t upto = (hi == 63) ? ~0ull : ((1ull << (hi + 1)) - 1ull);
  return upto & ~((1ull << lo) - 1ull);
}

// Visibility of the 64 key positions [k0, k0 + 64) for local tree node i
// (flattened node index node) of a request with prefix P and kv_end = P + n:
// bit t set <=> position k0 + t is a prefix key, or a tree key P + j with j
// visible to i under the mask. Positions >= kv_end are never visible.
__device__ __forceinline__ uint64_t tile_visibility(const MaskDev& mk, int node, int i, int P,
                                                    int kv_end, int k0) {
  uint64_t v = range_bits(0, P - 1 - k0);
  if (k0 + 64 > P && k0 < kv_end) {
    const int j0 = k0 - P;  // tree index of tile position 0, > -64
    uint64_t t;
    if (mk.kind == TV_MASK_BITS) {
      const uint64_t* row = mk.bits + (size_t)node * mk.words;
      if (j0 >= 0) {
        const int w = j0 >> 6, sh = j0 & 63;
        const uint64_t lo = w < mk.words ? row[w] : 0ull;
        const uint64_t hi = (w + 1) < mk.words ? row[w + 1] : 0ull;
        t = sh ? ((lo >> sh) | (hi << (64 - sh))) : lo;
      } else {
        t = row[0] << (-j0);
      }
    } else {
      const int ap = mk.anchor_pos[node], bd = mk.branch_depth[node];
      t = range_bits(-j0, ap - j0) | range_bits(i - bd + 1 - j0, i - j0);
    }
    v |= t & range_bits(P - k0, kv_end - 1 - k0);
  }
  return v;
}

struct AttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  int32_t num_pages;
  const int32_t* block_table;
  int32_t max_pages;
  const int32_t* prefix_len;
  const int32_t* cu_nodes;
  int32_t batch, total_nodes, max_nodes, max_prefix_len;
  int32_t hq, hkv, head_dim, page_size, dtype;
  float scale;
  MaskDev mask;
  void* out;
  float* lse;
  void* workspace;
};

// Launch plan of the bf16 path: rows per block, key splits. A pure function
// of host scalars, shared by the workspace query and the launch.
struct AttnPlan {
  int num_cus;         // compute units the plan was made for
  int waves;           // wavefronts per workgroup (8)
  int rw;              // 16-row subtiles per wave (block rows = 16 * waves * rw)
  int row_blocks;      // blocks over the node*group rows of one kv head
  int splits;          // key splits
  int keys_per_split;  // multiple of 64
  int short_splits;    // 1: splits of at most a few tiles, one-shot kernel
  size_t part_ml_offset;  // byte offset of the (m, l) partials (o partials at 0)
  size_t workspace;    // bytes of split partials (0 when splits == 1)
};
// num_cus: compute units of the device the call runs on (the split count
// aims at one workgroup per compute unit).
AttnPlan plan_attn(int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t max_prefix_len,
                   int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype, int32_t num_cus);
// returns the launch's hipError_t
hipError_t launch_attn(const AttnArgs& a, const AttnPlan& plan, hipStream_t stream);

}  // namespace tv
