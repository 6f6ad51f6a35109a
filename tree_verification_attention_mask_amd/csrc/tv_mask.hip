// tv_mask.hip -- tree_mask_build: parent[] -> depth and the ancestor-only tree mask.
//
// Graft (arXiv:2605.20104) §二, third gear: the flattened hybrid tree gets its
// tree position ids and tree mask rebuilt before the verification pass.
// SpecOPD (arXiv:2611.02846) §02, attention table (full attention / GQA): the
// mask is the ancestor relation -- own root path plus shared trunk only.
//
// One workgroup per request. BITS form: every node's ancestor set is built
// by pointer jumping in LDS (round k doubles the covered path length), so the
// number of rounds is ceil(log2(depth)) whatever the tree's shape; trees of
// at most 64 nodes use one wavefront and lane shuffles instead. ANCHOR
// form: the trunk length is a block-wide min, and each branch node finds its
// branch start with a block-wide running-max scan.
#include "tv_launch.h"

namespace tv {
namespace {

constexpr int kMaskThreads = 256;
constexpr int kMaxNodesPerThread = (64 * TV_MAX_MASK_WORDS) / kMaskThreads;  // 4

// Validity of one request's parent array, as a block-wide OR of violations:
// parent[0] == -1 and 0 <= parent[i] < i for i > 0 (so no cycle can exist).
__device__ bool block_tree_invalid(const int32_t* par, int n) {
  int bad = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int p = par[i];
    bad |= (i == 0) ? (p != -1) : (p < 0 || p >= i);
  }
  return __syncthreads_or(bad) != 0;
}

__global__ __launch_bounds__(kMaskThreads) void mask_bits_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ cu_nodes, int32_t total_nodes,
    int32_t words, uint64_t* __restrict__ bits, int32_t* __restrict__ depth,
    int32_t* __restrict__ err) {
  extern __shared__ uint64_t smem[];  // [cap][words] ancestor bits, then jump[cap]
  const int b = blockIdx.x;
  const int n0 = clampi(cu_nodes[b], 0, total_nodes);
  const int n = clampi(cu_nodes[b + 1], n0, total_nodes) - n0;
  const int cap = 64 * words;
  const int32_t* par = parent + n0;
  uint64_t* sb = smem;
  int32_t* jump = reinterpret_cast<int32_t*>(smem + (size_t)cap * words);

  const bool bad = n <= 0 || n > cap || block_tree_invalid(par, n);
  if (bad) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      for (int w = 0; w < words; ++w) bits[(size_t)(n0 + i) * words + w] = 0ull;
      depth[n0 + i] = -1;
    }
    if (threadIdx.x == 0) err[b] = 1;
    return;
  }

  // Round 0: node i covers itself and its parent; jump[i] = parent.
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int p = par[i];
    for (int w = 0; w < words; ++w) sb[i * words + w] = 0ull;
    sb[i * words + (i >> 6)] |= 1ull << (i & 63);
    if (p >= 0) sb[i * words + (p >> 6)] |= 1ull << (p & 63);
    jump[i] = p;
  }
  __syncthreads();

  // Round k: bits(i) |= bits(jump(i)); jump(i) = jump(jump(i)). After the
  // round, bits(i) holds every ancestor within distance 2^(k+1).
  for (;;) {
    uint64_t nb[kMaxNodesPerThread][TV_MAX_MASK_WORDS];
    int nj[kMaxNodesPerThread];
    int active = 0;
#pragma unroll
    for (int k = 0; k < kMaxNodesPerThread; ++k) {
      const int i = threadIdx.x + k * kMaskThreads;
      nj[k] = -1;
      if (i < n && jump[i] >= 0) {
        const int j = jump[i];
        active = 1;
#pragma unroll
        for (int w = 0; w < TV_MAX_MASK_WORDS; ++w)
          if (w < words) nb[k][w] = sb[j * words + w];
        nj[k] = jump[j];
      }
    }
    if (!__syncthreads_or(active)) break;
#pragma unroll
    for (int k = 0; k < kMaxNodesPerThread; ++k) {
      const int i = threadIdx.x + k * kMaskThreads;
      if (i < n && jump[i] >= 0) {
#pragma unroll
        for (int w = 0; w < TV_MAX_MASK_WORDS; ++w)
          if (w < words) sb[i * words + w] |= nb[k][w];
        jump[i] = nj[k];
      }
    }
    __syncthreads();
  }

  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    int pop = 0;
    for (int w = 0; w < words; ++w) {
      const uint64_t x = sb[i * words + w];
      bits[(size_t)(n0 + i) * words + w] = x;
      pop += __popcll(x);
    }
    depth[n0 + i] = pop - 1;
  }
  if (threadIdx.x == 0) err[b] = 0;
}

// Trees that fit one mask word (<= 64 nodes): one wavefront per request,
// lane i owns node i. Validation is one ballot; the ancestor sets are built
// by the same pointer jumping as above, over the lanes with shuffles (at most
// 6 rounds), so there is no LDS and no barrier.
constexpr int kWavesPerBlock = 4;
__global__ __launch_bounds__(64 * kWavesPerBlock) void mask_bits1_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ cu_nodes, int32_t batch,
    int32_t total_nodes, uint64_t* __restrict__ bits, int32_t* __restrict__ depth,
    int32_t* __restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (b >= batch) return;
  const int n0 = clampi(cu_nodes[b], 0, total_nodes);
  const int n = clampi(cu_nodes[b + 1], n0, total_nodes) - n0;
  const bool live = lane < n;
  const int p = live ? parent[n0 + lane] : -1;
  const bool viol = live && ((lane == 0) ? (p != -1) : (p < 0 || p >= lane));
  if (n <= 0 || n > 64 || __ballot(viol) != 0) {
    for (int i = lane; i < n; i += 64) {
      bits[n0 + i] = 0ull;
      depth[n0 + i] = -1;
    }
    if (lane == 0) err[b] = 1;
    return;
  }
  // bits(i) = {i, parent(i)}, jump(i) = parent(i); then
  // bits(i) |= bits(jump(i)), jump(i) = jump(jump(i)) until every jump is -1
  uint64_t m = live ? ((1ull << lane) | (p >= 0 ? (1ull << p) : 0ull)) : 0ull;
  int j = p;
  while (__any(j >= 0)) {
    const int src = j >= 0 ? j : lane;
    const uint64_t mj = __shfl(m, src, 64);
    const int jj = __shfl(j, src, 64);
    if (j >= 0) { m |= mj; j = jj; }
  }
  if (live) {
    bits[n0 + lane] = m;
    depth[n0 + lane] = __popcll(m) - 1;
  }
  if (lane == 0) err[b] = 0;
}

// Block-wide inclusive running max over one value per thread (256 threads).
__device__ int block_scan_max(int v, int* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v = max(v, o);
  }
  if (lane == 63) wave_tot[wave] = v;
  __syncthreads();
  for (int w = 0; w < wave; ++w) v = max(v, wave_tot[w]);
  __syncthreads();
  return v;
}

__global__ __launch_bounds__(kMaskThreads) void mask_anchor_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ cu_nodes, int32_t total_nodes,
    int32_t* __restrict__ anchor_pos, int32_t* __restrict__ branch_depth,
    int32_t* __restrict__ depth, int32_t* __restrict__ err) {
  __shared__ int s_trunk;
  __shared__ int s_wave[kMaskThreads / 64];
  const int b = blockIdx.x;
  const int n0 = clampi(cu_nodes[b], 0, total_nodes);
  const int n = clampi(cu_nodes[b + 1], n0, total_nodes) - n0;
  const int32_t* par = parent + n0;

  int e = (n <= 0 || block_tree_invalid(par, n)) ? 1 : 0;
  // Trunk length T: first k >= 1 whose parent is not k - 1 (else n).
  if (threadIdx.x == 0) s_trunk = n;
  __syncthreads();
  if (!e)
    for (int k = 1 + threadIdx.x; k < n; k += blockDim.x)
      if (par[k] != k - 1) atomicMin(&s_trunk, k);
  __syncthreads();
  const int T = s_trunk;
  // Every node past the trunk must start a branch (parent < T) or continue
  // the previous node's branch (parent == i - 1).
  int shape_bad = 0;
  if (!e)
    for (int i = T + threadIdx.x; i < n; i += blockDim.x)
      shape_bad |= !(par[i] < T || par[i] == i - 1);
  if (__syncthreads_or(shape_bad) && !e) e = 2;

  if (e) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      anchor_pos[n0 + i] = -1;
      branch_depth[n0 + i] = 0;
      depth[n0 + i] = -1;
    }
    if (threadIdx.x == 0) err[b] = e;
    return;
  }
  for (int i = threadIdx.x; i < T; i += blockDim.x) {
    anchor_pos[n0 + i] = i;
    branch_depth[n0 + i] = 0;
    depth[n0 + i] = i;
  }
  // Branch start of node i = the latest node s <= i with parent[s] < T.
  int carry = -1;
  for (int c0 = T; c0 < n; c0 += blockDim.x) {
    const int i = c0 + threadIdx.x;
    const int is_start = (i < n && par[i] < T) ? i : -1;
    const int s = max(carry, block_scan_max(is_start, s_wave));
    if (i < n) {
      const int a = par[s];
      anchor_pos[n0 + i] = a;
      branch_depth[n0 + i] = i - s + 1;
      depth[n0 + i] = a + 1 + (i - s);
    }
    // the block's last thread holds the running max over this chunk
    if ((threadIdx.x >> 6) == (kMaskThreads / 64) - 1 && (threadIdx.x & 63) == 63) s_wave[0] = s;
    __syncthreads();
    carry = max(carry, s_wave[0]);
    __syncthreads();
  }
  if (threadIdx.x == 0) err[b] = 0;
}

// The same ANCHOR-form decision for requests of at most kAnchorCap nodes
// (the host's max_nodes): the request's parent array is read into LDS at once
// (every thread's loads in flight together) and each thread then handles a
// contiguous run of kAnchorPerThread nodes, so validation, the trunk length,
// the shape check and the branch-start scan cost one memory round trip, not
// one per strided pass; the outputs are written in the strided order. A
// request past kAnchorCap nodes (more than max_nodes allows) is reported
// malformed.
constexpr int kAnchorThreads = 1024;
constexpr int kAnchorPerThread = 8;
constexpr int kAnchorCap = kAnchorThreads * kAnchorPerThread;

__global__ __launch_bounds__(kAnchorThreads) void mask_anchor_small_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ cu_nodes, int32_t total_nodes,
    int32_t* __restrict__ anchor_pos, int32_t* __restrict__ branch_depth,
    int32_t* __restrict__ depth, int32_t* __restrict__ err) {
  __shared__ int s_par[kAnchorCap];
  __shared__ int s_start[kAnchorCap];  // branch start of each branch node
  __shared__ int s_incl[kAnchorThreads];
  __shared__ int s_wave[kAnchorThreads / 64];
  __shared__ int s_trunk;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int n0 = clampi(cu_nodes[b], 0, total_nodes);
  const int n = clampi(cu_nodes[b + 1], n0, total_nodes) - n0;
  const int32_t* par = parent + n0;
  const int m = min(n, kAnchorCap);
  int pv[kAnchorPerThread];
#pragma unroll
  for (int j = 0; j < kAnchorPerThread; ++j) {
    const int i = tid + j * kAnchorThreads;
    pv[j] = i < m ? par[i] : 0;
  }
#pragma unroll
  for (int j = 0; j < kAnchorPerThread; ++j) {
    const int i = tid + j * kAnchorThreads;
    if (i < m) s_par[i] = pv[j];
  }
  if (tid == 0) s_trunk = n;
  __syncthreads();
  // this thread's run [i0, i0 + kAnchorPerThread): parent validity, and the
  // first k >= 1 whose parent is not k - 1 (the trunk length T, else n)
  const int i0 = tid * kAnchorPerThread;
  int bad = 0, tk = n;
#pragma unroll
  for (int j = 0; j < kAnchorPerThread; ++j) {
    const int i = i0 + j;
    if (i < m) {
      const int p = s_par[i];
      bad |= (i == 0) ? (p != -1) : (p < 0 || p >= i);
      if (i >= 1 && p != i - 1) tk = min(tk, i);
    }
  }
  if (tk < n) atomicMin(&s_trunk, tk);
  int e = (__syncthreads_or(bad) || n <= 0 || n > kAnchorCap) ? 1 : 0;
  const int T = s_trunk;
  // every node past the trunk starts a branch (parent < T) or continues the
  // previous node's branch (parent == i - 1)
  int shape_bad = 0;
  if (!e) {
#pragma unroll
    for (int j = 0; j < kAnchorPerThread; ++j) {
      const int i = i0 + j;
      if (i >= T && i < n) {
        const int p = s_par[i];
        shape_bad |= !(p < T || p == i - 1);
      }
    }
  }
  if (__syncthreads_or(shape_bad) && !e) e = 2;
  if (e) {
    for (int i = tid; i < n; i += kAnchorThreads) {
      anchor_pos[n0 + i] = -1;
      branch_depth[n0 + i] = 0;
      depth[n0 + i] = -1;
    }
    if (tid == 0) err[b] = e;
    return;
  }
  // branch start of node i = the latest s <= i with parent[s] < T: a running
  // max of (i if it starts a branch, else -1), within the run and then over
  // the runs of earlier threads
  int run = -1;
#pragma unroll
  for (int j = 0; j < kAnchorPerThread; ++j) {
    const int i = i0 + j;
    if (i >= T && i < n && s_par[i] < T) run = i;
  }
  s_incl[tid] = block_scan_max(run, s_wave);
  __syncthreads();
  // each branch node's start into LDS, then the outputs in the strided
  // order (consecutive threads, consecutive nodes: whole cache lines)
  int st = tid > 0 ? s_incl[tid - 1] : -1;
#pragma unroll
  for (int j = 0; j < kAnchorPerThread; ++j) {
    const int i = i0 + j;
    if (i >= T && i < n) {
      if (s_par[i] < T) st = i;
      s_start[i] = st;
    }
  }
  __syncthreads();
  for (int i = tid; i < n; i += kAnchorThreads) {
    if (i < T) {
      anchor_pos[n0 + i] = i;
      branch_depth[n0 + i] = 0;
      depth[n0 + i] = i;
    } else {
      const int s = s_start[i];
      const int a = s_par[s];
      anchor_pos[n0 + i] = a;
      branch_depth[n0 + i] = i - s + 1;
      depth[n0 + i] = a + 1 + (i - s);
    }
  }
  if (tid == 0) err[b] = 0;
}

}  // namespace

hipError_t launch_mask_bits(const int32_t* parent, const int32_t* cu_nodes, int32_t batch,
                            int32_t total_nodes, int32_t words, uint64_t* bits, int32_t* depth,
                            int32_t* err, hipStream_t stream) {
  if (words == 1) {
    const int grid = (batch + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(mask_bits1_kernel, dim3(grid), dim3(64 * kWavesPerBlock), 0, stream, parent,
                       cu_nodes, batch, total_nodes, bits, depth, err);
    return hipGetLastError();
  }
  const size_t cap = 64 * (size_t)words;
  const size_t lds = cap * words * sizeof(uint64_t) + cap * sizeof(int32_t);
  // allow > 64 KiB dynamic LDS (words > 11)
  const size_t max_lds = 64 * TV_MAX_MASK_WORDS * (TV_MAX_MASK_WORDS * sizeof(uint64_t) + sizeof(int32_t));
  hipError_t e = raise_dynamic_lds(reinterpret_cast<const void*>(&mask_bits_kernel), (int)max_lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mask_bits_kernel, dim3(batch), dim3(kMaskThreads), lds, stream, parent,
                     cu_nodes, total_nodes, words, bits, depth, err);
  return hipGetLastError();
}

hipError_t launch_mask_anchor(const int32_t* parent, const int32_t* cu_nodes, int32_t batch,
                              int32_t total_nodes, int32_t max_nodes, int32_t* anchor_pos,
                              int32_t* branch_depth, int32_t* depth, int32_t* err,
                              hipStream_t stream) {
  if (max_nodes <= kAnchorCap)
    hipLaunchKernelGGL(mask_anchor_small_kernel, dim3(batch), dim3(kAnchorThreads), 0, stream,
                       parent, cu_nodes, total_nodes, anchor_pos, branch_depth, depth, err);
  else
    hipLaunchKernelGGL(mask_anchor_kernel, dim3(batch), dim3(kMaskThreads), 0, stream, parent,
                       cu_nodes, total_nodes, anchor_pos, branch_depth, depth, err);
  return hipGetLastError();
}

}  // namespace tv
