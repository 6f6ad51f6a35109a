// tv_sampled.hip -- tv_tree_accept_sampled: stochastic tree verification.
//
// The pages verify at temperature 1 (BlockPilot §五, D-cut §4) and give the
// one-token rule (SpecOPD §03.2: exact rejection sampling accepts a drafted
// token with the overlap of the target's and the draft's distributions). The
// rule for a tree is recursive rejection sampling (Jeon et al. 2024,
// "Recursive Speculative Decoding"): SpecInfer's multi-step speculative
// sampling with siblings drawn without replacement. At the current node the
// children are tried in index order; the child with token x is accepted iff
// u * q(x) < p(x); on a rejection p becomes the normalised residual
// max(0, p - q) and x leaves q, which is renormalised; when no child is
// accepted the bonus token is drawn from the current p by inverse transform
// in token order.
//
// With the node's softmax values P(v) = 2^(c a_v - Lp), Q(v) = 2^(c b_v - Lq)
// (a, b the target's and the draft's logits, c = log2(e) / T) and the tokens
// x_0..x_{i-1} rejected so far:
//   q_j(v) = Q(v) / M_j unless v is one of x_0..x_{j-1}, then 0
//            (M_j = the draft mass left after j rejections, M_0 = 1);
//   p_0 = P, p_{j+1}(v) = max(0, p_j(v) - q_j(v)) / Z_j
//            (Z_j = sum_v max(0, p_j(v) - q_j(v)); p stays when Z_j = 0).
// A child's test needs p_i and q_i at its token only; a rejection adds Z_i and
// M_{i+1}, two sums over the vocabulary.
//
// sampled_norm_kernel: one 512-thread workgroup per node: Lp and Lq (NaN
//   logits count as -inf), into the caller's workspace.
// sampled_walk_kernel: one 1024-thread workgroup per request walks its tree
//   from the root. The request's parent array sits in LDS; at each node the
//   children are gathered in index order, their tokens, uniforms and the two
//   logits at those tokens are read in parallel, and the children are tried
//   with scalar arithmetic that every thread repeats. A rejection costs one
//   pass over the node's two logit rows; the bonus costs one pass (per-thread
//   runs of tokens in order, a block scan, then a rescan of the one run that
//   holds the draw).
#include "tv_vocab.h"

namespace tv {
namespace {

constexpr int kNormThreads = 512;
constexpr int kNormUnroll = 4;
constexpr int kWalkThreads = 1024;
constexpr int kWalkWaves = kWalkThreads / 64;
constexpr float kLog2eS = 1.4426950408889634f;

__device__ __forceinline__ float nan_to_ninf(float x) { return (x == x) ? x : -INFINITY; }

template <typename T, bool VEC>
__global__ __launch_bounds__(kNormThreads) void sampled_norm_kernel(const T* __restrict__ tl,
                                                                    const T* __restrict__ dl,
                                                                    int64_t vocab, float c,
                                                                    float2* __restrict__ norm) {
  constexpr int W = VocabUnit<T, VEC>::W;
  __shared__ MaxSum s_ms[kNormThreads / 64];
  const int64_t node = blockIdx.x;
  const T* a = tl + node * vocab;
  const T* b = dl + node * vocab;
  const int64_t units = vocab / W;  // VEC only when vocab % W == 0
  MaxSum ra{-INFINITY, 0.f}, rb{-INFINITY, 0.f};
  int64_t j = threadIdx.x;
  for (; j + (kNormUnroll - 1) * kNormThreads < units; j += kNormUnroll * kNormThreads) {
    float ya[kNormUnroll][W], yb[kNormUnroll][W];
#pragma unroll
    for (int u = 0; u < kNormUnroll; ++u) {
      VocabUnit<T, VEC>::load(a + (j + u * kNormThreads) * W, ya[u]);
      VocabUnit<T, VEC>::load(b + (j + u * kNormThreads) * W, yb[u]);
    }
#pragma unroll
    for (int u = 0; u < kNormUnroll; ++u) {
#pragma unroll
      for (int e = 0; e < W; ++e) {
        ya[u][e] = nan_to_ninf(ya[u][e]);
        yb[u][e] = nan_to_ninf(yb[u][e]);
      }
      fold(ra, ya[u], c);
      fold(rb, yb[u], c);
    }
  }
  for (; j < units; j += kNormThreads) {
    float ya[W], yb[W];
    VocabUnit<T, VEC>::load(a + j * W, ya);
    VocabUnit<T, VEC>::load(b + j * W, yb);
#pragma unroll
    for (int e = 0; e < W; ++e) {
      ya[e] = nan_to_ninf(ya[e]);
      yb[e] = nan_to_ninf(yb[e]);
    }
    fold(ra, ya, c);
    fold(rb, yb, c);
  }
  ra = block_merge<kNormThreads / 64>(ra, s_ms);
  rb = block_merge<kNormThreads / 64>(rb, s_ms);
  if (threadIdx.x == 0) norm[node] = make_float2(ra.m + __log2f(ra.s), rb.m + __log2f(rb.s));
}

struct WalkArgs {
  const int32_t* parent;
  const int32_t* draft_tok;
  const int32_t* cu_nodes;
  int32_t total_nodes, max_nodes, max_children, max_depth;
  int64_t vocab;
  float c;
  const float* u_accept;
  const float* u_bonus;
  const float2* norm;
  int32_t* accept_len;
  int32_t* path;
  int32_t* bonus_tok;
};

// Inclusive prefix sum over the block of one value per thread, in thread
// order; s_w holds kWalkWaves floats. Returns the thread's inclusive sum and
// the block total.
__device__ float block_inclusive_sum(float v, float* s_w, float& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o = __shfl_up(x, off, 64);
    if (lane >= off) x += o;
  }
  if (lane == 63) s_w[wave] = x;
  __syncthreads();
  float before = 0.f;
  total = 0.f;
#pragma unroll
  for (int w = 0; w < kWalkWaves; ++w) {
    const float t = s_w[w];
    before += (w < wave) ? t : 0.f;
    total += t;
  }
  __syncthreads();
  return before + x;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kWalkThreads) void sampled_walk_kernel(WalkArgs w,
                                                                    const T* __restrict__ tl,
                                                                    const T* __restrict__ dl) {
  constexpr int W = VocabUnit<T, VEC>::W;
  extern __shared__ int32_t s_dyn[];
  const int cap = w.max_nodes, cc = w.max_children;
  int32_t* s_par = s_dyn;                                 // [cap] request-local parents
  int32_t* s_kid = s_par + cap;                           // [cc] children of the current node
  int32_t* s_tok = s_kid + cc;                            // [cc] their tokens (-1: outside the vocabulary)
  float* s_u = reinterpret_cast<float*>(s_tok + cc);      // [cc] their uniforms
  float* s_a = s_u + cc;                                  // [cc] target logit at each token
  float* s_b = s_a + cc;                                  // [cc] draft logit at each token
  int32_t* s_rx = reinterpret_cast<int32_t*>(s_b + cc);   // [cc] rejected tokens, in order
  float* s_iz = reinterpret_cast<float*>(s_rx + cc);      // [cc] 1 / Z_j (0: Z_j = 0)
  float* s_im = s_iz + cc;                                // [cc + 1] 1 / M_j (0: no draft mass left)
  __shared__ float s_red[2][kWalkWaves];
  __shared__ int s_cnt[kWalkWaves];
  __shared__ float s_incl[kWalkWaves];
  __shared__ int s_pick, s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  const int lo = clampi(w.cu_nodes[b], 0, w.total_nodes);
  const int hi = clampi(w.cu_nodes[b + 1], lo, w.total_nodes);
  const int n = min(hi - lo, cap);
  const int prow = w.max_depth + 1;
  int32_t* path = w.path + (size_t)b * prow;
  for (int i = tid; i < n; i += kWalkThreads) s_par[i] = w.parent[lo + i];
  for (int d = tid; d < prow; d += kWalkThreads) path[d] = (d == 0 && n > 0) ? 0 : -1;
  if (n == 0) {  // an empty request (uniform over the block)
    if (tid == 0) {
      w.accept_len[b] = 0;
      w.bonus_tok[b] = -1;
    }
    return;
  }
  __syncthreads();

  // p_i(v) and q_i(v) after i rejections, from P(v), Q(v); `rej` = index of
  // v's first rejection among 0..i-1, or i. Every thread gets the same values
  // for the same inputs (LDS reads only).
  auto chain = [&](int v, float P, float Q, int i, float& p, float& q, int& rej) {
    rej = i;
    for (int l = 0; l < i; ++l)
      if (s_rx[l] == v) {
        rej = l;
        break;
      }
    p = P;
    for (int j = 0; j < i; ++j) {
      const float qj = (rej < j) ? 0.f : Q * s_im[j];
      const float iz = s_iz[j];
      p = (iz > 0.f) ? fmaxf(0.f, p - qj) * iz : p;
    }
    q = (rej < i) ? 0.f : Q * s_im[i];
  };
  const int64_t units = w.vocab / W;

  int node = 0, depth = 0;
  for (;;) {
    const float2 L = w.norm[lo + node];
    const int64_t row = (int64_t)(lo + node) * w.vocab;
    // children of `node`, in index order (the first cc of them)
    int m = 0;
    for (int base = node + 1; base < n; base += kWalkThreads) {
      const int ci = base + tid;
      const bool is = ci < n && s_par[ci] == node;
      const uint64_t bal = __ballot(is);
      if (lane == 0) s_cnt[wave] = __popcll(bal);
      __syncthreads();
      int off = m, tot = 0;
#pragma unroll
      for (int x = 0; x < kWalkWaves; ++x) {
        const int cnt = s_cnt[x];
        off += (x < wave) ? cnt : 0;
        tot += cnt;
      }
      const int pos = off + __popcll(bal & ((1ull << lane) - 1));
      if (is && pos < cc) s_kid[pos] = ci;
      m += tot;
      __syncthreads();
    }
    m = min(m, cc);
    for (int k = tid; k < m; k += kWalkThreads) {
      const int g = lo + s_kid[k];
      const int x = w.draft_tok[g];
      const bool ok = x >= 0 && (int64_t)x < w.vocab;
      s_tok[k] = ok ? x : -1;
      s_u[k] = w.u_accept[g];
      s_a[k] = ok ? nan_to_ninf(load_one(tl + row + x)) : -INFINITY;
      s_b[k] = ok ? nan_to_ninf(load_one(dl + row + x)) : -INFINITY;
    }
    if (tid == 0) s_im[0] = 1.f;
    __syncthreads();

    // try the children in order
    int i = 0, next = -1;
    for (int k = 0; k < m; ++k) {
      const int x = s_tok[k];
      if (x < 0) continue;  // not a token of the vocabulary: passed over
      const float P = __builtin_amdgcn_exp2f(__builtin_fmaf(s_a[k], w.c, -L.x));
      const float Q = __builtin_amdgcn_exp2f(__builtin_fmaf(s_b[k], w.c, -L.y));
      float p, q;
      int rej;
      chain(x, P, Q, i, p, q, rej);
      if (s_u[k] * q < p) {
        next = s_kid[k];
        break;
      }
      // rejected: Z_i and M_{i+1} over the vocabulary
      if (tid == 0) s_rx[i] = x;
      __syncthreads();
      float zs = 0.f, ms = 0.f;
      for (int64_t j = tid; j < units; j += kWalkThreads) {
        float ya[W], yb[W];
        VocabUnit<T, VEC>::load(tl + row + j * W, ya);
        VocabUnit<T, VEC>::load(dl + row + j * W, yb);
#pragma unroll
        for (int e = 0; e < W; ++e) {
          const int v = (int)(j * W + e);
          const float Pv = __builtin_amdgcn_exp2f(__builtin_fmaf(nan_to_ninf(ya[e]), w.c, -L.x));
          const float Qv = __builtin_amdgcn_exp2f(__builtin_fmaf(nan_to_ninf(yb[e]), w.c, -L.y));
          float pv, qv;
          int rv;
          chain(v, Pv, Qv, i, pv, qv, rv);
          zs += fmaxf(0.f, pv - qv);
          ms += (rv == i && v != x) ? Qv : 0.f;
        }
      }
      zs = block_sum<kWalkWaves>(zs, s_red[0]);
      ms = block_sum<kWalkWaves>(ms, s_red[1]);
      if (tid == 0) {
        s_iz[i] = zs > 0.f ? 1.f / zs : 0.f;
        s_im[i + 1] = ms > 0.f ? 1.f / ms : 0.f;
      }
      __syncthreads();
      ++i;
    }

    if (next >= 0) {
      node = next;
      ++depth;
      if (tid == 0 && depth <= w.max_depth) path[depth] = node;
      continue;
    }

    // bonus token: inverse transform of p_i in token order
    const int64_t per = (units + kWalkThreads - 1) / kWalkThreads;
    const int64_t j0 = min(units, (int64_t)tid * per), j1 = min(units, j0 + per);
    auto p_at = [&](int64_t j, float (&pv)[W]) {
      float ya[W], yb[W];
      VocabUnit<T, VEC>::load(tl + row + j * W, ya);
      VocabUnit<T, VEC>::load(dl + row + j * W, yb);
#pragma unroll
      for (int e = 0; e < W; ++e) {
        const float Pv = __builtin_amdgcn_exp2f(__builtin_fmaf(nan_to_ninf(ya[e]), w.c, -L.x));
        const float Qv = __builtin_amdgcn_exp2f(__builtin_fmaf(nan_to_ninf(yb[e]), w.c, -L.y));
        float qv;
        int rv;
        chain((int)(j * W + e), Pv, Qv, i, pv[e], qv, rv);
      }
    };
    float s = 0.f;
    for (int64_t j = j0; j < j1; ++j) {
      float pv[W];
      p_at(j, pv);
#pragma unroll
      for (int e = 0; e < W; ++e) s += pv[e];
    }
    float total;
    const float incl = block_inclusive_sum(s, s_red[0], total);
    // the previous thread's inclusive sum: a shuffle within the wave, LDS
    // across waves, so the runs [excl, incl) tile [0, total) exactly
    if (lane == 63) s_incl[wave] = incl;
    if (tid == 0) {
      s_pick = -1;
      s_last = -1;
    }
    __syncthreads();
    float excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = (wave == 0) ? 0.f : s_incl[wave - 1];
    const float target = w.u_bonus[b] * total;
    // exactly one run holds the draw unless rounding put it at or past the
    // total
    if (excl <= target && target < incl) {
      float r = excl;
      int pick = -1, last = -1;
      for (int64_t j = j0; j < j1 && pick < 0; ++j) {
        float pv[W];
        p_at(j, pv);
#pragma unroll
        for (int e = 0; e < W; ++e) {
          if (pick >= 0) break;
          if (pv[e] > 0.f) last = (int)(j * W + e);
          r += pv[e];
          if (r > target && pv[e] > 0.f) pick = (int)(j * W + e);
        }
      }
      s_pick = pick >= 0 ? pick : last;
    }
    if (s > 0.f) atomicMax(&s_last, tid);
    __syncthreads();
    if (s_pick < 0 && tid == s_last) {
      // the draw fell at or past the total: the last token with mass
      int last = -1;
      for (int64_t j = j0; j < j1; ++j) {
        float pv[W];
        p_at(j, pv);
#pragma unroll
        for (int e = 0; e < W; ++e)
          if (pv[e] > 0.f) last = (int)(j * W + e);
      }
      s_pick = last;
    }
    __syncthreads();
    if (tid == 0) {
      w.bonus_tok[b] = s_pick;
      w.accept_len[b] = depth;
    }
    return;
  }
}

template <typename T, bool VEC>
hipError_t run_sampled(const WalkArgs& a, const void* tl, const void* dl, int32_t batch,
                       int32_t total_nodes, float c, hipStream_t stream) {
  const T* t = static_cast<const T*>(tl);
  const T* d = static_cast<const T*>(dl);
  if (total_nodes > 0)
    hipLaunchKernelGGL((sampled_norm_kernel<T, VEC>), dim3(total_nodes), dim3(kNormThreads), 0,
                       stream, t, d, a.vocab, c, const_cast<float2*>(a.norm));
  if (batch > 0) {
    // s_par [max_nodes], seven per-child arrays [max_children] and s_im [max_children + 1]
    const size_t lds = ((size_t)a.max_nodes + (size_t)8 * a.max_children + 1) * 4;
    hipLaunchKernelGGL((sampled_walk_kernel<T, VEC>), dim3(batch), dim3(kWalkThreads), lds, stream,
                       a, t, d);
  }
  return hipGetLastError();
}

}  // namespace

size_t sampled_workspace(int32_t total_nodes) {
  return ((size_t)total_nodes * sizeof(float2) + 255) / 256 * 256;
}

hipError_t launch_accept_sampled(const int32_t* parent, const int32_t* draft_tok,
                                 const int32_t* cu_nodes, int32_t batch, int32_t total_nodes,
                                 int32_t max_nodes, int32_t max_children, int32_t max_depth,
                                 const void* target_logits, const void* draft_logits,
                                 int32_t dtype, int32_t vocab, float temperature,
                                 const float* u_accept, const float* u_bonus,
                                 int32_t* accept_len, int32_t* path, int32_t* bonus_tok,
                                 void* workspace, hipStream_t stream) {
  WalkArgs a;
  a.parent = parent;
  a.draft_tok = draft_tok;
  a.cu_nodes = cu_nodes;
  a.total_nodes = total_nodes;
  a.max_nodes = max_nodes;
  a.max_children = max_children < 1 ? 1 : max_children;
  a.max_depth = max_depth;
  a.vocab = vocab;
  a.c = kLog2eS / temperature;
  a.u_accept = u_accept;
  a.u_bonus = u_bonus;
  a.norm = static_cast<const float2*>(workspace);
  a.accept_len = accept_len;
  a.path = path;
  a.bonus_tok = bonus_tok;
  if (dtype == TV_BF16) {
    const bool vec = vocab_vec<__bf16>(target_logits, vocab) && vocab_vec<__bf16>(draft_logits, vocab);
    return vec ? run_sampled<__bf16, true>(a, target_logits, draft_logits, batch, total_nodes, a.c, stream)
               : run_sampled<__bf16, false>(a, target_logits, draft_logits, batch, total_nodes, a.c, stream);
  }
  const bool vec = vocab_vec<float>(target_logits, vocab) && vocab_vec<float>(draft_logits, vocab);
  return vec ? run_sampled<float, true>(a, target_logits, draft_logits, batch, total_nodes, a.c, stream)
             : run_sampled<float, false>(a, target_logits, draft_logits, batch, total_nodes, a.c, stream);
}

}  // namespace tv
