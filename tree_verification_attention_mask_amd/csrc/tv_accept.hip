// tv_accept.hip -- tree_accept: greedy acceptance of the longest matching root path.
//
// SpecOPD (arXiv:2611.02846) §01: drafted tokens that agree with the target are
// accepted and the draft is cut at the first divergence. Graft
// (arXiv:2605.20104) introduction and §二 third gear: the target checks the
// whole tree at once and keeps the path that goes furthest, applying the same
// rule to draft and retrieved nodes. BlockPilot (arXiv:2606.31315) §八:
// accepted length = survival length of the prefix.
//
// One wavefront per request; nodes are visited in chunks of 64 in index
// order. Since parent[i] < i, a node whose parent lies in an earlier chunk
// reads the parent's final state from LDS; a node whose parent lies in the
// same chunk is resolved by pointer jumping over the lanes (6 shuffle rounds
// for 64 lanes). state(i) = depth(i) if i is accepted, else -1. The deepest
// accepted node (ties: smallest index) wins a wave max-reduction.
#include "tv_launch.h"

namespace tv {
namespace {

constexpr int kIdxBits = 13;  // TV_MAX_ACCEPT_NODES = 8192 = 2^13

__global__ __launch_bounds__(64) void accept_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ draft_tok,
    const int32_t* __restrict__ target_tok, const int32_t* __restrict__ cu_nodes,
    int32_t total_nodes, int32_t cap, int32_t max_depth, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ path, int32_t* __restrict__ bonus_tok) {
  extern __shared__ int32_t lds[];  // parent[cap], state[cap], target[cap]
  int32_t* s_par = lds;
  int32_t* s_state = lds + cap;
  int32_t* s_tgt = lds + 2 * cap;
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int n0 = clampi(cu_nodes[b], 0, total_nodes);
  const int n = min(clampi(cu_nodes[b + 1], n0, total_nodes) - n0, cap);

  int best_key = -1;  // (depth << kIdxBits) | (2^kIdxBits - 1 - index)
  for (int c0 = 0; c0 < n; c0 += 64) {
    const int i = c0 + lane;
    const bool live = i < n;
    // clamp malformed parents into [0, i) so every walk moves strictly upward
    int p = live ? parent[n0 + i] : -1;
    p = (i == 0) ? -1 : clampi(p, 0, i - 1);
    // every node's target token is loaded once, with its parent and draft
    // token; a child reads its parent's from a lane (same chunk) or from LDS
    const int tgt = live ? target_tok[n0 + i] : -1;
    const int dft = live ? draft_tok[n0 + i] : 0;
    const int tp_lane = __shfl(tgt, (p >= c0) ? p - c0 : lane, 64);
    const int tp = (p >= c0) ? tp_lane : (p >= 0 ? s_tgt[p] : -1);
    const bool match = live && (i == 0 || dft == tp);
    // (ok, d, link): ok/d cover the path from i up to (excluding) lane link
    int ok, d, link;
    if (!live || i == 0) {
      ok = live; d = 0; link = -1;
    } else if (p < c0) {
      const int ps = s_state[p];
      ok = match && ps >= 0; d = ps + 1; link = -1;
    } else {
      ok = match; d = 1; link = p - c0;
    }
#pragma unroll
    for (int r = 0; r < 6; ++r) {
      const int src = link < 0 ? lane : link;
      const int ok2 = __shfl(ok, src, 64);
      const int d2 = __shfl(d, src, 64);
      const int l2 = __shfl(link, src, 64);
      if (link >= 0) { ok &= ok2; d += d2; link = l2; }
    }
    const int state = ok ? d : -1;
    if (live) { s_par[i] = p; s_state[i] = state; s_tgt[i] = tgt; }
    if (live && state >= 0)
      best_key = max(best_key, (state << kIdxBits) | ((1 << kIdxBits) - 1 - i));
    __syncthreads();
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) best_key = max(best_key, __shfl_xor(best_key, off, 64));

  const int best = (best_key < 0) ? 0 : (1 << kIdxBits) - 1 - (best_key & ((1 << kIdxBits) - 1));
  const int best_depth = (best_key < 0) ? 0 : (best_key >> kIdxBits);
  // Path root..best, staged in the (now unused) state array by lane 0.
  if (lane == 0 && n > 0) {
    for (int j = best, t = best_depth; j >= 0 && t >= 0; j = s_par[j], --t) s_state[t] = j;
  }
  __syncthreads();
  int32_t* prow = path + (size_t)b * (max_depth + 1);
  for (int t = lane; t <= max_depth; t += 64) prow[t] = (n > 0 && t <= best_depth) ? s_state[t] : -1;
  if (lane == 0) {
    accept_len[b] = best_depth;
    if (bonus_tok) bonus_tok[b] = n > 0 ? s_tgt[best] : -1;
  }
}

}  // namespace

hipError_t launch_accept(const int32_t* parent, const int32_t* draft_tok, const int32_t* target_tok,
                         const int32_t* cu_nodes, int32_t batch, int32_t total_nodes,
                         int32_t max_nodes, int32_t max_depth, int32_t* accept_len, int32_t* path,
                         int32_t* bonus_tok, hipStream_t stream) {
  const int cap = max_nodes < 1 ? 1 : max_nodes;
  const size_t lds = 3 * sizeof(int32_t) * (size_t)cap;
  // allow > 64 KiB dynamic LDS for the largest trees
  hipError_t e = raise_dynamic_lds(reinterpret_cast<const void*>(&accept_kernel),
                                   (int)(3 * sizeof(int32_t) * TV_MAX_ACCEPT_NODES));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_kernel, dim3(batch), dim3(64), lds, stream, parent, draft_tok,
                     target_tok, cu_nodes, total_nodes, cap, max_depth, accept_len, path,
                     bonus_tok);
  return hipGetLastError();
}

}  // namespace tv
