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
#include "tv_launch.h"

namespace tv {
namespace {

constexpr int kTvThreads = 512;
constexpr int kTvWaves = kTvThreads / 64;
constexpr int kUnroll = 4;  // 16-byte groups per row each thread keeps in flight
constexpr float kLog2eF = 1.4426950408889634f;

struct MaxSum {
  float m, s;  // log2-domain max and sum of 2^(y - m)
};
__device__ __forceinline__ MaxSum merge(MaxSum a, MaxSum b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return MaxSum{m, 0.f};
  return MaxSum{m, a.s * __builtin_amdgcn_exp2f(a.m - m) + b.s * __builtin_amdgcn_exp2f(b.m - m)};
}
// fold a group of raw logits x into a running (max, sum) of y = c x (log2
// units, c = log2(e) / T > 0, so the max of y is c times the max of x)
template <int N>
__device__ __forceinline__ void fold(MaxSum& r, const float (&x)[N], float c) {
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) mx = fmaxf(mx, x[i]);
  const float m = fmaxf(r.m, mx * c);
  float acc = (r.m == -INFINITY) ? 0.f : r.s * __builtin_amdgcn_exp2f(r.m - m);
#pragma unroll
  for (int i = 0; i < N; ++i) acc += __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], c, -m));
  r = MaxSum{m, acc};
}

// Block-wide merge of one value per thread; every thread gets the result.
__device__ MaxSum block_merge(MaxSum v, MaxSum* s_red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    MaxSum o{__shfl_xor(v.m, off, 64), __shfl_xor(v.s, off, 64)};
    v = merge(v, o);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  MaxSum r = s_red[0];
#pragma unroll
  for (int w = 1; w < kTvWaves; ++w) r = merge(r, s_red[w]);
  __syncthreads();
  return r;
}
__device__ float block_sum(float v, float* s_red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int w = 0; w < kTvWaves; ++w) r += s_red[w];
  __syncthreads();
  return r;
}

// Values of a row in groups of W (16-byte loads when VEC), converted to fp32.
template <typename T>
struct Row;
template <>
struct Row<__bf16> {
  static constexpr int W = 8;
  __device__ static void load(const __bf16* p, float (&y)[W]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[2 * i] = __uint_as_float(w[i] << 16);
      y[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static float one(const __bf16* p) { return static_cast<float>(*p); }
};
template <>
struct Row<float> {
  static constexpr int W = 4;
  __device__ static void load(const float* p, float (&y)[W]) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    y[0] = u.x; y[1] = u.y; y[2] = u.z; y[3] = u.w;
  }
  __device__ static float one(const float* p) { return *p; }
};

template <typename T, bool VEC>
__global__ __launch_bounds__(kTvThreads) void alpha_kernel(const T* __restrict__ tl,
                                                           const T* __restrict__ dl, int64_t vocab,
                                                           float c, float* __restrict__ alpha) {
  __shared__ MaxSum s_ms[kTvWaves];
  __shared__ float s_f[kTvWaves];
  constexpr int W = Row<T>::W;
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
      Row<T>::load(a + (j + u * kTvThreads) * W, ya[u]);
      Row<T>::load(b + (j + u * kTvThreads) * W, yb[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      fold(ra, ya[u], c);
      fold(rb, yb[u], c);
    }
  }
  for (; j < nvec; j += kTvThreads) {
    float ya[W], yb[W];
    Row<T>::load(a + j * W, ya);
    Row<T>::load(b + j * W, yb);
    fold(ra, ya, c);
    fold(rb, yb, c);
  }
  for (int64_t v = tail0 + tid; v < vocab; v += kTvThreads) {
    const float ya[1] = {Row<T>::one(a + v)}, yb[1] = {Row<T>::one(b + v)};
    fold(ra, ya, c);
    fold(rb, yb, c);
  }
  ra = block_merge(ra, s_ms);
  rb = block_merge(rb, s_ms);
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
      Row<T>::load(a + (j + u * kTvThreads) * W, ya[u]);
      Row<T>::load(b + (j + u * kTvThreads) * W, yb[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) overlap(ya[u], yb[u]);
  }
  for (; j < nvec; j += kTvThreads) {
    float ya[W], yb[W];
    Row<T>::load(a + j * W, ya);
    Row<T>::load(b + j * W, yb);
    overlap(ya, yb);
  }
  for (int64_t v = tail0 + tid; v < vocab; v += kTvThreads)
    acc += __builtin_amdgcn_exp2f(fminf(__builtin_fmaf(Row<T>::one(a + v), c, -La),
                                        __builtin_fmaf(Row<T>::one(b + v), c, -Lb)));
  acc = block_sum(acc, s_f);
  if (tid == 0) alpha[node] = acc;
}

__global__ __launch_bounds__(256) void branch_kernel(const float* __restrict__ alpha,
                                                     const int32_t* __restrict__ cu, int32_t nb,
                                                     int32_t num_nodes, float* __restrict__ prefix,
                                                     float* __restrict__ expected) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nb) return;
  const int lo = clampi(cu[b], 0, num_nodes), hi = clampi(cu[b + 1], lo, num_nodes);
  float run = 1.f, sum = 0.f;
  for (int i = lo; i < hi; ++i) {
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
  constexpr int W = Row<T>::W;
  const bool vec = (vocab % W) == 0 && (reinterpret_cast<uintptr_t>(a) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(b) & 15) == 0;
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
