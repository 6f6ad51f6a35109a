// tv_dcut.hip -- tv_dcut_select: the D-cut verification budget on the device.
//
// D-cut (paper 2607.14647) technical summary §2, cross-request pruning and the
// pipeline's scoring & ranking and packing steps: every draft position is
// scored by the product of its block's draft confidences up to it, all
// positions of the batch are ranked together, the best are verified, and
// because scores only fall along a block each request keeps a prefix, which
// is packed densely for the verification pass.
//
// One workgroup of 1024 threads (the ranked set is at most 32768 positions,
// held in LDS as fp32 bit patterns -- non-negative floats order like their
// bits):
//   1. scores: the confidences come into LDS in one round trip (every load in
//      flight), then each thread walks its requests' blocks left to right in
//      fp32, the products replacing the confidences;
//   2. threshold: the R-th largest score (R = budget - batch ranked slots) by
//      a radix select, 8 bits per pass from the top, with an LDS histogram
//      (two alternating, two barriers a pass);
//   3. per request: positions above the threshold, plus positions equal to it
//      handed out in request order (a block scan) -- the tie rule;
//   4. cu_nodes by a second block scan, then the packed chains and tokens:
//      with one request per thread (at most 1024), every packed slot finds
//      its request by a binary search over the requests' first slots and
//      loads its token, all at once; beyond, each thread packs its requests.
// Threads own contiguous runs of requests, so scans keep request order.
#include "tv_launch.h"

namespace tv {
namespace {

constexpr int kDcutThreads = 1024;
constexpr int kDcutWaves = kDcutThreads / 64;

// Exclusive prefix sum over the block of one value per thread, in thread
// order; the block total is returned in `total`. s_wave holds kDcutWaves + 1
// ints; the trailing barrier lets the next call reuse it.
__device__ int block_exclusive_sum(int v, int* s_wave, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(x, off, 64);
    if (lane >= off) x += o;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < kDcutWaves; ++w) {
      const int t = s_wave[w];
      s_wave[w] = acc;
      acc += t;
    }
    s_wave[kDcutWaves] = acc;
  }
  __syncthreads();
  const int r = s_wave[wave] + x - v;
  total = s_wave[kDcutWaves];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kDcutThreads) void dcut_select_kernel(
    const float* __restrict__ conf, const int32_t* __restrict__ tokens, int32_t batch,
    int32_t D, int32_t budget, int32_t* __restrict__ n_keep, int32_t* __restrict__ cu_nodes,
    int32_t* __restrict__ parent, int32_t* __restrict__ packed_tokens) {
  extern __shared__ uint32_t s_key[];  // [batch * D] score bits, request-major
  __shared__ int s_hist[2][256];  // two passes' histograms alternate
  __shared__ int s_wave[kDcutWaves + 1];
  __shared__ uint32_t s_digit[2];
  __shared__ int s_rem[2];
  const int tid = threadIdx.x;
  const int M = batch * D;
  const int R = budget - batch;  // slots ranked among the draft positions
  const int chunk = (batch + kDcutThreads - 1) / kDcutThreads;
  const int b_lo = min(batch, tid * chunk), b_hi = min(batch, b_lo + chunk);
  if (tid == 0) { s_digit[0] = s_digit[1] = 0; s_rem[0] = s_rem[1] = 0; }
  if (tid < 256) s_hist[0][tid] = 0;  // the first pass's histogram

  // 1. scores, left to right along each block (confidences are probabilities):
  // the confidences come into the score array in one round trip (every load
  // in flight), then each block's products replace them in place
  for (int i = tid; i < M; i += kDcutThreads) s_key[i] = __float_as_uint(conf[i]);
  __syncthreads();
  auto clamp01 = [](uint32_t bits) {
    const float c = __uint_as_float(bits);
    return (c > 0.f) ? fminf(c, 1.f) : 0.f;  // NaN -> 0
  };
  for (int b = b_lo; b < b_hi; ++b) {
    float s = 1.f;
    uint32_t* row = s_key + b * D;
    int k = 0;
    for (; k + 4 <= D; k += 4) {
      uint32_t c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = row[k + j];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s = __fmul_rn(s, clamp01(c[j]));
        row[k + j] = __float_as_uint(s);
      }
    }
    for (; k < D; ++k) {
      s = __fmul_rn(s, clamp01(row[k]));
      row[k] = __float_as_uint(s);
    }
  }
  __syncthreads();

  // 2. the R-th largest key: tau, and how many keys equal to tau are taken
  uint32_t tau = 0;
  int rem = 0;
  const bool some = R > 0 && R < M;
  if (some) {
    uint32_t prefix = 0, hmask = 0;
    int remaining = R;  // keys still to take among those matching prefix
    // two barriers a pass: the next pass's histogram is cleared while this
    // one fills (it was last read before this pass began), and the picked
    // digit alternates between two slots
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      const int buf = pass & 1;
      for (int i = tid; i < M; i += kDcutThreads) {
        const uint32_t key = s_key[i];
        if ((key & hmask) == prefix) atomicAdd(&s_hist[buf][(key >> shift) & 255u], 1);
      }
      if (tid < 256) s_hist[buf ^ 1][tid] = 0;
      __syncthreads();
      if (tid < 64) {
        // lane l owns digits 255-4l .. 252-4l, largest first; the lane whose
        // group crosses `remaining` in descending digit order picks the digit
        int c[4], loc = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[j] = s_hist[buf][255 - 4 * tid - j];
          loc += c[j];
        }
        int x = loc;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int o = __shfl_up(x, off, 64);
          if (tid >= off) x += o;
        }
        int acc = x - loc;
        if (acc < remaining && remaining <= x) {
          for (int j = 0; j < 4; ++j) {
            if (acc + c[j] >= remaining) {
              s_digit[buf] = (uint32_t)(255 - 4 * tid - j);
              s_rem[buf] = remaining - acc;
              break;
            }
            acc += c[j];
          }
        }
      }
      __syncthreads();
      prefix |= s_digit[buf] << shift;
      hmask |= 0xffu << shift;
      remaining = s_rem[buf];
    }
    tau = prefix;
    rem = remaining;
  }
  // kept draft positions of request b: those above tau, then `take` of the
  // ones equal to tau (ties to the smaller request; within a request the
  // equal scores are consecutive, so smaller positions come first)
  auto counts = [&](int b, int& gt, int& eq) {
    gt = 0;
    eq = 0;
    if (R >= M) { gt = D; return; }
    if (!some) return;
    const uint32_t* row = s_key + b * D;
    int k = 0;
    for (; k + 4 <= D; k += 4) {
      uint32_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = row[k + j];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        gt += v[j] > tau ? 1 : 0;
        eq += v[j] == tau ? 1 : 0;
      }
    }
    for (; k < D; ++k) {
      gt += row[k] > tau ? 1 : 0;
      eq += row[k] == tau ? 1 : 0;
    }
  };

  // 3. ties in request order
  int local_eq = 0;
  for (int b = b_lo; b < b_hi; ++b) {
    int gt, eq;
    counts(b, gt, eq);
    local_eq += eq;
  }
  int total;
  const int eq_before = block_exclusive_sum(local_eq, s_wave, total);
  auto kept = [&](int b, int& eq_run) {
    int gt, eq;
    counts(b, gt, eq);
    const int take = min(eq, max(0, rem - eq_run));
    eq_run += eq;
    return 1 + gt + take;
  };
  int local_n = 0;
  {
    int eq_run = eq_before;
    for (int b = b_lo; b < b_hi; ++b) local_n += kept(b, eq_run);
  }

  // 4. offsets, then the packed chains and tokens
  const int n_before = block_exclusive_sum(local_n, s_wave, total);
  if (chunk != 1) {
    // several requests per thread: each packs its own in order
    int eq_run = eq_before, off = n_before;
    for (int b = b_lo; b < b_hi; ++b) {
      const int n = kept(b, eq_run);
      n_keep[b] = n;
      cu_nodes[b] = off;
      for (int k = 0; k < n && off + k < budget; ++k) {  // (bounded whatever the counts)
        parent[off + k] = k - 1;
        packed_tokens[off + k] = tokens[(size_t)b * (D + 1) + k];
      }
      off += n;
    }
    if (tid == 0) cu_nodes[batch] = total;
    return;
  }
  // one request per thread: the requests' first slots replace the scores in
  // LDS, and every packed slot finds its request by a binary search and loads
  // its token (every slot's load in flight at once)
  if (b_lo < b_hi) {
    int eq_run = eq_before;
    n_keep[b_lo] = kept(b_lo, eq_run);
    cu_nodes[b_lo] = n_before;
  }
  __syncthreads();  // every count has read the scores
  if (b_lo < b_hi) s_key[b_lo] = (uint32_t)n_before;
  __syncthreads();
  const int slots = min(total, budget);
  for (int o = tid; o < slots; o += kDcutThreads) {
    int lo = 0, hi = batch - 1;  // the last request whose first slot is <= o
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int)s_key[mid] <= o) lo = mid; else hi = mid - 1;
    }
    const int k = o - (int)s_key[lo];
    parent[o] = k - 1;
    packed_tokens[o] = tokens[(size_t)lo * (D + 1) + k];
  }
  if (tid == 0) cu_nodes[batch] = total;
}

}  // namespace

hipError_t launch_dcut_select(const float* conf, const int32_t* tokens, int32_t batch,
                              int32_t draft_len, int32_t budget, int32_t* n_keep,
                              int32_t* cu_nodes, int32_t* parent, int32_t* packed_tokens,
                              hipStream_t stream) {
  // the score array may exceed 64 KiB
  hipError_t e = raise_dynamic_lds(reinterpret_cast<const void*>(&dcut_select_kernel),
                                   (int)(TV_MAX_DCUT_DRAFT_POSITIONS * sizeof(uint32_t)));
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)batch * draft_len * sizeof(uint32_t);
  hipLaunchKernelGGL(dcut_select_kernel, dim3(1), dim3(kDcutThreads), lds, stream, conf, tokens,
                     batch, draft_len, budget, n_keep, cu_nodes, parent, packed_tokens);
  return hipGetLastError();
}

}  // namespace tv
