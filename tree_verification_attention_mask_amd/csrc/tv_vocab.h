// tv_vocab.h -- device helpers for kernels that stream vocabulary-sized logit
// rows: row loaders and a log2-domain running (max, sum) for softmax
// normalisers. Nothing here is part of the C ABI.
#pragma once

#include "tv_launch.h"

namespace tv {

// One unit of a logits row converted to fp32: a 16-byte group (8 bf16 or
// 4 fp32 values) when VEC -- rows 16-byte aligned and the vocabulary a
// multiple of W -- else a single value.
template <typename T, bool VEC>
struct VocabUnit;
// `fetch` returns the unit's raw bits and `unpack` converts them, so that a
// kernel can keep many units in flight in few registers.
template <>
struct VocabUnit<__bf16, true> {
  static constexpr int W = 8;
  using Raw = uint4;
  __device__ static Raw fetch(const __bf16* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ static void unpack(const Raw& u, float (&y)[W]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[2 * i] = __uint_as_float(w[i] << 16);
      y[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static void load(const __bf16* p, float (&y)[W]) { unpack(fetch(p), y); }
};
template <>
struct VocabUnit<float, true> {
  static constexpr int W = 4;
  using Raw = float4;
  __device__ static Raw fetch(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static void unpack(const Raw& u, float (&y)[W]) {
    y[0] = u.x; y[1] = u.y; y[2] = u.z; y[3] = u.w;
  }
  __device__ static void load(const float* p, float (&y)[W]) { unpack(fetch(p), y); }
};
template <typename T>
struct VocabUnit<T, false> {
  static constexpr int W = 1;
  using Raw = T;
  __device__ static Raw fetch(const T* p) { return *p; }
  __device__ static void unpack(const Raw& u, float (&y)[W]) { y[0] = static_cast<float>(u); }
  __device__ static void load(const T* p, float (&y)[W]) { y[0] = static_cast<float>(*p); }
};
template <typename T>
__device__ __forceinline__ float load_one(const T* p) {
  return static_cast<float>(*p);
}

// Whether a row of `vocab` logits at `p` takes 16-byte units.
template <typename T>
inline bool vocab_vec(const void* p, int64_t vocab) {
  return (reinterpret_cast<uintptr_t>(p) & 15) == 0 && vocab % VocabUnit<T, true>::W == 0;
}

// log2-domain running max m and sum s of 2^(y - m)
struct MaxSum {
  float m, s;
};
__device__ __forceinline__ MaxSum merge(MaxSum a, MaxSum b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return MaxSum{m, 0.f};
  return MaxSum{m, a.s * __builtin_amdgcn_exp2f(a.m - m) + b.s * __builtin_amdgcn_exp2f(b.m - m)};
}
// fold a group of raw logits x into a running (max, sum) of y = c x (log2
// units, c = log2(e) / T > 0, so the max of y is c times the max of x).
// -inf logits add nothing, also when the whole group and the running max are
// -inf (the shift then stays finite).
template <int N>
__device__ __forceinline__ void fold(MaxSum& r, const float (&x)[N], float c) {
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) mx = fmaxf(mx, x[i]);
  const float m = fmaxf(r.m, mx * c);
  const float shift = (m == -INFINITY) ? 0.f : m;
  float acc = (r.m == -INFINITY) ? 0.f : r.s * __builtin_amdgcn_exp2f(r.m - m);
#pragma unroll
  for (int i = 0; i < N; ++i) acc += __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], c, -shift));
  r = MaxSum{m, acc};
}

// Wave-wide DPP helpers (64 lanes, no LDS round trip). dpp_from: the value
// of the lane that DPP control CTRL names, `old` where there is none (a
// shift past the row's or the wave's edge, or a row ROWS leaves out).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_from(float old, float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), CTRL, ROWS, 0xf, false));
}
// Inclusive prefix sum in lane order: shifts by 1, 2, 4, 8 inside each row of
// 16 lanes, then a row's last lane added into the rows after it (row_bcast:15
// into rows 1 and 3, row_bcast:31 into rows 2 and 3).
__device__ __forceinline__ float wave_incl_sum(float x) {
  x += dpp_from<0x111, 0xf>(0.f, x);
  x += dpp_from<0x112, 0xf>(0.f, x);
  x += dpp_from<0x114, 0xf>(0.f, x);
  x += dpp_from<0x118, 0xf>(0.f, x);
  x += dpp_from<0x142, 0xa>(0.f, x);
  x += dpp_from<0x143, 0xc>(0.f, x);
  return x;
}
// The previous lane's value (wave_shr:1), 0 in lane 0.
__device__ __forceinline__ float wave_prev(float x) { return dpp_from<0x138, 0xf>(0.f, x); }
__device__ __forceinline__ float lane_value(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}
// Sum and maximum over the wave, the same value in every lane.
__device__ __forceinline__ float wave_sum(float x) { return lane_value(wave_incl_sum(x), 63); }
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_from<0x111, 0xf>(x, x));
  x = fmaxf(x, dpp_from<0x112, 0xf>(x, x));
  x = fmaxf(x, dpp_from<0x114, 0xf>(x, x));
  x = fmaxf(x, dpp_from<0x118, 0xf>(x, x));
  x = fmaxf(x, dpp_from<0x142, 0xa>(x, x));
  x = fmaxf(x, dpp_from<0x143, 0xc>(x, x));
  return lane_value(x, 63);
}
// (max, sum) merge over the wave: the maximum, then every lane's sum
// rescaled to it and added up (-inf maxima add nothing).
__device__ __forceinline__ MaxSum wave_merge(MaxSum v) {
  const float m = wave_max(v.m);
  if (m == -INFINITY) return MaxSum{m, 0.f};
  const float t = (v.m == -INFINITY) ? 0.f : v.s * __builtin_amdgcn_exp2f(v.m - m);
  return MaxSum{m, wave_sum(t)};
}

// Block-wide merge of one value per thread over NW waves; every thread gets
// the result. s_red holds NW entries; the trailing barrier lets the next call
// reuse it.
template <int NW>
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
  for (int w = 1; w < NW; ++w) r = merge(r, s_red[w]);
  __syncthreads();
  return r;
}
template <int NW>
__device__ float block_sum(float v, float* s_red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) r += s_red[w];
  __syncthreads();
  return r;
}

}  // namespace tv
