// tv_e2etv.hip -- tv_e2e_tv_stats: SpecOPD's E2E-TV statistics over a vocabulary.
//
// SpecOPD (arXiv:2611.02846) §02 stage 4 and §03.2: with exact rejection
// sampling the drafted token at a node is accepted with probability
// alpha = sum_v min(p_v, q_v) = 1 - TV(p, q), p and q being the target's and
// the draft's next-token distributions there; a branch is accepted token by
// token, so the chance of accepting its first k tokens is the product of their
// alphas, and the expected run of accepted tokens is the sum of those products.
//
// alpha_kernel: one workgroup per node streams its two logit rows twice.
//   pass 1: per row, the log2-domain maximum and sum of 2^(y - max), with
//           y = logit * log2(e) / T; 8 values share one rescale, so each value
//           costs one fma and one exp2; the block merges the (max, sum) pairs;
//   pass 2: alpha = sum_v 2^min(ya_v - La, yb_v - Lb) with L = max + log2(sum):
//           the min of the two probabilities taken on their logarithms, one
//           exp2 per vocabulary entry. The second pass re-reads rows the
//           first pass just brought through L2 / the last-level cache.
// branch_kernel: one thread per branch, prefix products and their sum.
#include "tv_vocab.h"

namespace tv {
namespace {

constexpr int kTvThreads = 512;
constexpr int kTvWaves = kTvThreads / 64;
constexpr int kUnroll = 4;  // 16-byte groups per row each thread keeps in flight
constexpr float kLog2eF = 1.4426950408889634f;

template <typename T, bool VEC>
__global__ __launch_bounds__(kTvThreads) void alpha_kernel(const T* __restrict__ tl,
                                                           const T* __restrict__ dl, int64_t vocab,
                                                           float c, float* __restrict__ alpha) {
  __shared__ MaxSum s_ms[kTvWaves];
  __shared__ float s_f[kTvWaves];
  constexpr int W = VocabUnit<T, true>::W;
  const int64_t node = blockIdx.x;
  const T* a = tl + node * vocab;
  const T* b = dl + node * vocab;
  const int tid = threadIdx.x;
  const int64_t nvec = VEC ? vocab / W : 0;  // whole W-groups (rows 16-byte aligned)
  const int64_t tail0 = nvec * W;

  // pass 1 (kUnroll groups per thread in flight, then one at a time)
  MaxSum ra{-INFINITY, 0.f}, rb{-INFINITY, 0.f};
  int64_t j = tid;
  for (; j + (kUnroll - 1) * kTvThreads < nvec; j += kUnroll * kTvThreads) {
    float ya[kUnroll][W], yb[kUnroll][W];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      VocabUnit<T, true>::load(a + (j + u * kTvThreads) * W, ya[u]);
      VocabUnit<T, true>::load(b + (j + u * kTvThreads) * W, yb[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      fold(ra, ya[u], c);
      fold(rb, yb[u], c);
    }
  }
  for (; j < nvec; j += kTvThreads) {
    float ya[W], yb[W];
    VocabUnit<T, true>::load(a + j * W, ya);
    VocabUnit<T, true>::load(b + j * W, yb);
    fold(ra, ya, c);
    fold(rb, yb, c);
  }
  for (int64_t v = tail0 + tid; v < vocab; v += kTvThreads) {
    const float ya[1] = {load_one<T>(a + v)}, yb[1] = {load_one<T>(b + v)};
    fold(ra, ya, c);
    fold(rb, yb, c);
  }
  ra = block_merge<kTvWaves>(ra, s_ms);
  rb = block_merge<kTvWaves>(rb, s_ms);
  const float La = ra.m + __log2f(ra.s), Lb = rb.m + __log2f(rb.s);

  // pass 2
  float acc = 0.f;
  auto overlap = [&](const float (&ya)[W], const float (&yb)[W]) {
#pragma unroll
    for (int i = 0; i < W; ++i)
      acc += __builtin_amdgcn_exp2f(fminf(__builtin_fmaf(ya[i], c, -La), __builtin_fmaf(yb[i], c, -Lb)));
  };
  j = tid;
  for (; j + (kUnroll - 1) * kTvThreads < nvec; j += kUnroll * kTvThreads) {
    float ya[kUnroll][W], yb[kUnroll][W];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      VocabUnit<T, true>::load(a + (j + u * kTvThreads) * W, ya[u]);
      VocabUnit<T, true>::load(b + (j + u * kTvThreads) * W, yb[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) overlap(ya[u], yb[u]);
  }
  for (; j < nvec; j += kTvThreads) {
    float ya[W], yb[W];
    VocabUnit<T, true>::load(a + j * W, ya);
    VocabUnit<T, true>::load(b + j * W, yb);
    overlap(ya, yb);
  }
  for (int64_t v = tail0 + tid; v < vocab; v += kTvThreads)
    acc += __builtin_amdgcn_exp2f(fminf(__builtin_fmaf(load_one<T>(a + v), c, -La),
                                        __builtin_fmaf(load_one<T>(b + v), c, -Lb)));
  acc = block_sum<kTvWaves>(acc, s_f);
  if (tid == 0) alpha[node] = acc;
}

__global__ __launch_bounds__(256) void branch_kernel(const float* __restrict__ alpha,
                                                     const int32_t* __restrict__ cu, int32_t nb,
                                                     int32_t num_nodes, float* __restrict__ prefix,
                                                     float* __restrict__ expected) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nb) return;
  const int lo = clampi(cu[b], 0, num_nodes), hi = clampi(cu[b + 1], lo, num_nodes);
  // the same left-to-right products; eight alphas requested at a time (a
  // loop of one load per step waited for each)
  float run = 1.f, sum = 0.f;
  int i = lo;
  for (; i + 8 <= hi; i += 8) {
    float a8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) a8[j] = alpha[i + j];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      run *= a8[j];
      prefix[i + j] = run;
      sum += run;
    }
  }
  for (; i < hi; ++i) {
    run *= alpha[i];
    prefix[i] = run;
    sum += run;
  }
  expected[b] = sum;
}

template <typename T>
hipError_t run_alpha(const void* tl, const void* dl, int32_t n, int32_t vocab, float c,
                     float* alpha, hipStream_t stream) {
  const T* a = static_cast<const T*>(tl);
  const T* b = static_cast<const T*>(dl);
  const bool vec = vocab_vec<T>(a, vocab) && vocab_vec<T>(b, vocab);
  if (vec)
    hipLaunchKernelGGL((alpha_kernel<T, true>), dim3(n), dim3(kTvThreads), 0, stream, a, b,
                       (int64_t)vocab, c, alpha);
  else
    hipLaunchKernelGGL((alpha_kernel<T, false>), dim3(n), dim3(kTvThreads), 0, stream, a, b,
                       (int64_t)vocab, c, alpha);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_e2e_tv(const void* target_logits, const void* draft_logits, int32_t dtype,
                         int32_t num_nodes, int32_t vocab, float temperature,
                         const int32_t* cu_branches, int32_t num_branches, float* alpha,
                         float* prefix_prob, float* expected_len, hipStream_t stream) {
  const float c = kLog2eF / temperature;
  hipError_t e = (dtype == TV_BF16)
                     ? run_alpha<__bf16>(target_logits, draft_logits, num_nodes, vocab, c, alpha, stream)
                     : run_alpha<float>(target_logits, draft_logits, num_nodes, vocab, c, alpha, stream);
  if (e != hipSuccess || num_branches == 0) return e;
  hipLaunchKernelGGL(branch_kernel, dim3((num_branches + 255) / 256), dim3(256), 0, stream, alpha,
                     cu_branches, num_branches, num_nodes, prefix_prob, expected_len);
  return hipGetLastError();
}

}  // namespace tv
