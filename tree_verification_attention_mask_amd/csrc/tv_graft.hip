// tv_graft.hip -- Graft's retrieval table on the device: tv_graft_retrieve and
// tv_graft_update.
//
// Graft (arXiv:2605.20104) §二, second gear: a table in GPU memory holds, for
// every vocabulary token, its k most likely successors; slots freed by
// pruning are filled by expanding a template rooted at the current token, one
// row lookup per template node. Third gear and §五 (online update): after the
// verification pass the row of every verified token is replaced by the
// target's most likely next tokens at that position.
//
// graft_retrieve_kernel: one wavefront per request, lane j = template node j
//   (at most 64). The template travels in the kernel arguments; the tree is
//   expanded one depth level at a time (the lookups of a level depend on the
//   tokens of the level above, handed over by lane shuffles): one gather per
//   level.
// graft_share_kernel + graft_lists_kernel (the online update of bf16 rows,
//   16-byte aligned, the vocabulary a multiple of 8 and up to 64 / k shares
//   of 40,960 entries): each node's row is cut into shares, one 256-thread
//   workgroup each with every load of its share in flight at once, so that
//   the few rows of one verification pass still fill the chip. A share
//   bounds its k best from below by a value T taken from integer keys of the
//   raw bf16 bits, lists the few elements >= T in LDS and ranks them by
//   counting; one wavefront per node ranks the shares' lists.
// graft_topk_kernel + graft_merge_kernel (every other row: fp32, unaligned,
//   other vocabularies): contiguous shares of at most one sweep of 16-byte or
//   one-value loads, one 256-thread workgroup each. Every wavefront keeps the
//   k best (logit, id) pairs it has seen, ordered by logit then smaller id,
//   one per lane (WaveTopK): its first batch of 64 values is ranked by
//   counting, later batches are filtered against the k-th best with one
//   compare and a ballot, and the rare survivors are inserted by lane
//   shifts. The workgroup ranks its waves' lists; the merge kernel ranks the
//   shares' lists and writes the row.
// Both write a row only when no later node carries the same token, so every
// row has one writer.
#include "tv_vocab.h"

namespace tv {
namespace {

struct GraftTemplate {
  int32_t nodes, max_depth;
  // node j: parent (+1, 0 = the current token) | rank << 8 | depth << 16
  uint32_t node[TV_MAX_GRAFT_TEMPLATE];
};

constexpr int kRetrieveWaves = 4;

__global__ __launch_bounds__(64 * kRetrieveWaves) void graft_retrieve_kernel(
    const int32_t* __restrict__ adj, int32_t vocab, int32_t k, const int32_t* __restrict__ roots,
    int32_t batch, GraftTemplate t, int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * kRetrieveWaves + (threadIdx.x >> 6);
  if (b >= batch) return;
  const int root = roots[b];
  const uint32_t code = lane < t.nodes ? t.node[lane] : 0u;
  const int par = (int)(code & 0xffu) - 1;      // -1: the current token
  const int rank = (int)((code >> 8) & 0xffu);
  const int depth = (int)(code >> 16);
  int tok = -1;
  for (int d = 1; d <= t.max_depth; ++d) {
    const int from = __shfl(tok, par >= 0 ? par : lane, 64);
    if (lane < t.nodes && depth == d) {
      const int src = par >= 0 ? from : root;
      int x = -1;
      if (src >= 0 && src < vocab) x = adj[(size_t)src * k + rank];
      tok = (x >= 0 && x < vocab) ? x : -1;
    }
  }
  if (lane < t.nodes) out[(size_t)b * t.nodes + lane] = tok;
}

constexpr int kUpdateThreads = 256;
constexpr int kUpdateWaves = kUpdateThreads / 64;
constexpr int kUpdateUnroll = 8;  // loads per thread in flight
constexpr int kMaxSplits = 32;    // workgroups sharing one logits row
constexpr int kMergeThreads = 256;

// (value, id) order: larger value first, then smaller id -- a total order, so
// the k best do not depend on the order the values are seen in
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return (va > vb) | ((va == vb) & (ia < ib));
}
__device__ __forceinline__ float rank_key(float x) { return (x == x) ? x : -INFINITY; }
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// Maximum over the wave: DPP within rows of 16 (pairs, quads, half rows,
// rows), then the four row results by scalar reads.
__device__ __forceinline__ float wave_max(float v) {
  auto step = [](float x, float y) { return fmaxf(x, y); };
  v = step(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0xB1, 0xf, 0xf, false)));  // quad_perm 1,0,3,2
  v = step(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x4E, 0xf, 0xf, false)));  // quad_perm 2,3,0,1
  v = step(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x141, 0xf, 0xf, false))); // row_half_mirror
  v = step(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x140, 0xf, 0xf, false))); // row_mirror
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

// Whether this node writes its token's row: the token is in range and no later
// node carries it. Uniform over the block (every thread reads the same token).
__device__ bool owns_row(const int32_t* node_tokens, int num_nodes, int node, int tok, int vocab) {
  if (tok < 0 || tok >= vocab) return false;
  int later = 0;
  for (int j = node + 1 + (int)threadIdx.x; j < num_nodes; j += (int)blockDim.x)
    later |= (node_tokens[j] == tok);
  return !__syncthreads_or(later);
}

// The wave's k best (logit, id) pairs so far, best first, one per lane in
// lanes 0..k-1. It starts with distinct stand-ins that lose to every real
// entry (ids above any token). `thr` is a value no entry of the k best can
// fall below: elements under it are dropped by one compare.
struct WaveTopK {
  float mv, thr;
  int mi, k, lane;
  uint64_t kmask;
  __device__ WaveTopK(int k_, int tid)
      : mv(-INFINITY), thr(-INFINITY), mi(0x7fffffff - tid), k(k_), lane(tid & 63),
        kmask(k_ >= 64 ? ~0ull : ((1ull << k_) - 1)) {}
  // Offers element e of every lane's unit (ids uid + e; lanes outside vmask
  // hold no element). Survivors of the compare (NaN passes and is ranked as
  // -inf here) are inserted one at a time: scalar broadcasts and a one-lane
  // DPP shift of the list's tail (k <= 16: one DPP row). Control flow is
  // uniform over the wave.
  __device__ __forceinline__ void offer(float x, uint64_t vmask, int uid, int e) {
    uint64_t cand = __ballot(!(x < thr)) & vmask;
    if (cand == 0) return;
    do {
      const int src = __builtin_ctzll(cand);
      cand &= cand - 1;
      const float cv = rank_key(readlane_f(x, src));
      const int ci = __builtin_amdgcn_readlane(uid, src) + e;
      const uint64_t beats = __ballot(better(cv, ci, mv, mi)) & kmask;
      if (beats == 0) continue;  // not among the k best
      const int pos = __builtin_ctzll(beats);
      // row_shr:1 -- lane l (1..15) reads lane l-1 of its row
      const float uv = __int_as_float(
          __builtin_amdgcn_update_dpp(__float_as_int(mv), __float_as_int(mv), 0x111, 0xf, 0xf, false));
      const int ui = __builtin_amdgcn_update_dpp(mi, mi, 0x111, 0xf, 0xf, false);
      if (lane > pos) { mv = uv; mi = ui; }
      if (lane == pos) { mv = cv; mi = ci; }
    } while (cand);
    thr = fmaxf(thr, readlane_f(mv, k - 1));
  }
};

// graft_topk_kernel: workgroup (node, split) finds the k best (logit, id) of
// its contiguous share of the node's row (at least one unit). With one split
// it writes the table row itself; otherwise its sorted k best go to
// part[node][split][k] for graft_merge_kernel.
template <typename T, bool VEC>
__global__ __launch_bounds__(kUpdateThreads) void graft_topk_kernel(
    int32_t* __restrict__ adj, int32_t vocab, int32_t k, const T* __restrict__ logits,
    int32_t num_nodes, const int32_t* __restrict__ node_tokens, int32_t splits,
    int2* __restrict__ part) {
  constexpr int UW = VocabUnit<T, VEC>::W;
  __shared__ float s_v[kUpdateWaves * 16];
  __shared__ int s_i[kUpdateWaves * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int node = blockIdx.x, split = blockIdx.y;
  const int tok = node_tokens[node];
  if (!owns_row(node_tokens, num_nodes, node, tok, vocab)) return;

  const int64_t units = vocab / UW;  // VEC only when vocab % W == 0
  const int64_t per = (units + splits - 1) / splits;
  const int64_t u0 = (int64_t)split * per;
  const int64_t n = min(units, u0 + per) - u0;  // >= 1 (the launch drops empty splits)
  const T* row = logits + (int64_t)node * vocab + u0 * UW;
  WaveTopK top(k, tid);
  auto offer = [&](float x, uint64_t vmask, int uid, int e) { top.offer(x, vmask, uid, e); };

  // First chunk: every thread's first kUpdateUnroll units, all loads in
  // flight together. The k-th largest of the wave's 64 lane maxima is
  // reached by k distinct elements, so it starts `thr`: about k elements of
  // the chunk pass the compare.
  const int64_t n_r = (n + kUpdateThreads - 1) / kUpdateThreads * kUpdateThreads;
  {
    float y[kUpdateUnroll][UW];
#pragma unroll
    for (int u = 0; u < kUpdateUnroll; ++u)
      VocabUnit<T, VEC>::load(row + min((int64_t)(u * kUpdateThreads + tid), n - 1) * UW, y[u]);
    float lm = -INFINITY;  // max ignores NaN
#pragma unroll
    for (int u = 0; u < kUpdateUnroll; ++u) {
      const bool ok = u * kUpdateThreads + tid < n;
#pragma unroll
      for (int e = 0; e < UW; ++e) lm = fmaxf(lm, ok ? y[u][e] : -INFINITY);
    }
    int ge = 0;  // lane maxima >= this lane's
#pragma unroll
    for (int s = 0; s < 64; ++s) ge += (readlane_f(lm, s) >= lm) ? 1 : 0;
    top.thr = wave_max(ge >= k ? lm : -INFINITY);
#pragma unroll
    for (int u = 0; u < kUpdateUnroll; ++u) {
      if (u * kUpdateThreads >= n) break;  // uniform: no unit of this sweep is in the share
      const int idx = u * kUpdateThreads + tid;
      const uint64_t vmask = __ballot(idx < n);
      const int uid = (int)((u0 + idx) * UW);
#pragma unroll
      for (int e = 0; e < UW; ++e) offer(y[u][e], vmask, uid, e);
    }
  }

  // The rest of the share in sweeps of the whole block (padded to whole
  // sweeps so that every lane takes part; loads from a clamped index).
  int64_t base = kUpdateUnroll * kUpdateThreads;
  for (; base + (kUpdateUnroll - 1) * kUpdateThreads < n_r; base += kUpdateUnroll * kUpdateThreads) {
    float y[kUpdateUnroll][UW];
#pragma unroll
    for (int u = 0; u < kUpdateUnroll; ++u)
      VocabUnit<T, VEC>::load(row + min(base + u * kUpdateThreads + tid, n - 1) * UW, y[u]);
#pragma unroll
    for (int u = 0; u < kUpdateUnroll; ++u) {
      const int64_t idx = base + u * kUpdateThreads + tid;
      const uint64_t vmask = __ballot(idx < n);
      const int uid = (int)((u0 + idx) * UW);
#pragma unroll
      for (int e = 0; e < UW; ++e) offer(y[u][e], vmask, uid, e);
    }
  }
  for (; base < n_r; base += kUpdateThreads) {
    float y[UW];
    const int64_t idx = base + tid;
    VocabUnit<T, VEC>::load(row + min(idx, n - 1) * UW, y);
    const uint64_t vmask = __ballot(idx < n);
    const int uid = (int)((u0 + idx) * UW);
#pragma unroll
    for (int e = 0; e < UW; ++e) offer(y[e], vmask, uid, e);
  }

  // Merge the waves' lists: wave 0 ranks the 4k entries by counting (they are
  // distinct, so ranks 0..k-1 are taken once each).
  if (lane < 16) {
    s_v[wave * 16 + lane] = top.mv;
    s_i[wave * 16 + lane] = top.mi;
  }
  __syncthreads();
  if (wave != 0) return;
  const int E = kUpdateWaves * k;
  float ev = -INFINITY;
  int ei = 0x7fffffff;
  if (lane < E) {
    ev = s_v[(lane / k) * 16 + lane % k];
    ei = s_i[(lane / k) * 16 + lane % k];
  }
  int rank = 0;
  for (int s = 0; s < E; ++s)
    rank += better(readlane_f(ev, s), __builtin_amdgcn_readlane(ei, s), ev, ei) ? 1 : 0;
  if (lane < E && rank < k) {
    if (splits == 1) adj[(size_t)tok * k + rank] = ei;
    else part[((size_t)node * splits + split) * k + rank] = make_int2(__float_as_int(ev), ei);
  }
}

// graft_share_kernel + graft_lists_kernel (bf16 rows, 16-byte aligned, the
// vocabulary a multiple of 8): each node's row is cut into the fewest
// shares of at most kShareUnits 16-byte units a thread (at most
// kListLanes / k shares), one 256-thread workgroup each, every unit of the
// share requested at once and before the ownership test's tokens are back.
// A row needs several compute units at a time: one compute unit alone
// streams a 151,936-entry row in about 10 us.
//
// Selection in a share: each unit gets a 16-bit key that orders like its
// largest value -- the raw bf16 bits compared as signed integers where the
// values that matter are above +0, else bits whose magnitude field is
// flipped for negative values (monotone in the value over all non-NaN bf16).
// A lane's largest key stands for an element no smaller than that value, so
// the k-th largest lane key of a wave stands for a value T with k elements at
// or above it: every element of the share's k best is >= T. With T the
// largest such value over the waves, units whose key falls below T's are
// skipped with one compare, and the few elements of the rest that are >= T
// are appended to a list in LDS and ranked by counting. A share whose T does
// not bound the list (ties, fewer than k finite values) takes the wave lists
// of WaveTopK instead, which handle every case. One share writes the table
// row itself; otherwise each writes its k best to part[node][share][k] and
// graft_lists_kernel, one wavefront per node, ranks the lists (at most 64
// entries, one a lane) and writes the row.
constexpr int kShareThreads = 256;
constexpr int kShareWaves = kShareThreads / 64;
constexpr int kShareUnits = 20;                 // units a thread
constexpr int kShareCap = 256;                  // listed elements (>= 16 per wave)
constexpr int kListLanes = 64;                  // shares * k at most: one entry a lane of graft_lists_kernel
constexpr int kKeyLo = -32768;                  // below every key

using short2v = short __attribute__((ext_vector_type(2)));
__device__ __forceinline__ short2v as_s2(uint32_t w) { return __builtin_bit_cast(short2v, w); }
// flip the magnitude bits of negative bf16 halves: signed 16-bit order = value
// order for non-NaN values (-0 sits just below +0)
__device__ __forceinline__ uint32_t monotone_bits(uint32_t w) {
  const uint32_t neg = __builtin_bit_cast(uint32_t, as_s2(w) >> (short)15);
  return w ^ (neg & 0x7fff7fffu);
}
template <bool MONO>
__device__ __forceinline__ int unit_key(const uint4& u) {
  const uint32_t a = MONO ? monotone_bits(u.x) : u.x, b = MONO ? monotone_bits(u.y) : u.y;
  const uint32_t c = MONO ? monotone_bits(u.z) : u.z, d = MONO ? monotone_bits(u.w) : u.w;
  const short2v m = __builtin_elementwise_max(__builtin_elementwise_max(as_s2(a), as_s2(b)),
                                              __builtin_elementwise_max(as_s2(c), as_s2(d)));
  return max((int)m.x, (int)m.y);
}

__global__ __launch_bounds__(kShareThreads) void graft_share_kernel(
    int32_t* __restrict__ adj, int32_t vocab, int32_t k, const __bf16* __restrict__ logits,
    int32_t num_nodes, const int32_t* __restrict__ node_tokens, int32_t shares,
    int2* __restrict__ part) {
  __shared__ float s_cv[kShareCap];
  __shared__ int s_ci[kShareCap];
  __shared__ int s_tq[kShareWaves];
  __shared__ int s_cnt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int node = blockIdx.x, share = blockIdx.y;
  const int n = vocab / 8;  // units in the row
  const int per = (n + shares - 1) / shares;
  const int u0 = share * per;
  const int ns = min(n, u0 + per) - u0;  // >= 1 (the launch leaves no share empty)
  const int tok = node_tokens[node];
  const int j0 = node + 1 + tid;
  const int tj = j0 < num_nodes ? node_tokens[j0] : -1;
  const __bf16* src = logits + (int64_t)node * vocab + (int64_t)u0 * 8;
  // every load issued (units past the share reload its last unit and are
  // masked by their key), so that the waits below can be counted
  uint4 raw[kShareUnits];
#pragma unroll
  for (int u = 0; u < kShareUnits; ++u)
    raw[u] = *reinterpret_cast<const uint4*>(src + (int64_t)min(u * kShareThreads + tid, ns - 1) * 8);
  if (tid == 0) s_cnt = 0;
  int later = (tj == tok);
  for (int j = j0 + kShareThreads; j < num_nodes; j += kShareThreads) later |= (node_tokens[j] == tok);
  if (tok < 0 || tok >= vocab) return;  // uniform
  if (__syncthreads_or(later)) return;  // a later node writes this row

  // Pass over the units with one of the two keys; returns whether its T
  // bounds the list (then the list holds every element >= T).
  auto listed = [&](auto mono) -> bool {
    constexpr bool MONO = decltype(mono)::value;
    // the keys that stand for a value: +0 .. +inf (plain bits), or -inf ..
    // +inf (flipped bits; 0xff80 flips to 0x807f)
    constexpr int lo = MONO ? (int)(short)0x807f : 0, hi = 0x7f80;
    int uk[kShareUnits];
    int lk = kKeyLo;
#pragma unroll
    for (int u = 0; u < kShareUnits; ++u) {
      int key = unit_key<MONO>(raw[u]);
      if (u * kShareThreads + tid >= ns) key = kKeyLo;
      uk[u] = key;
      lk = max(lk, key);
    }
    // q = 1 + (key - lo) for a lane whose largest key is a value, else 0; the
    // wave's k-th largest q by bisection over its 16 bits
    const int q = (lk >= lo && lk <= hi) ? lk - lo + 1 : 0;
    int pfx = 0;
#pragma unroll
    for (int b = 15; b >= 0; --b) {
      const int cand = pfx | (1 << b);
      if (__builtin_popcountll(__ballot(q >= cand)) >= k) pfx = cand;
    }
    if (lane == 0) s_tq[wave] = pfx;
    __syncthreads();
    int tq = 0;
#pragma unroll
    for (int w = 0; w < kShareWaves; ++w) tq = max(tq, s_tq[w]);
    // T must be finite and, with plain bits, above +0 (-0's plain key is
    // below every positive value's)
    if (tq < 2) return false;
    const int tkey = tq - 1 + lo;
    const uint32_t tb = (MONO && tkey < 0) ? (uint32_t)((tkey ^ 0x7fff) & 0xffff) : (uint32_t)tkey;
    const float T = __uint_as_float(tb << 16);
    // one key below T's also takes -0 when T is +0
    const int tk = tkey - 1;
#pragma unroll
    for (int u = 0; u < kShareUnits; ++u) {
      if (uk[u] >= tk) {
        float y[8];
        VocabUnit<__bf16, true>::unpack(raw[u], y);
        const int id0 = (u0 + u * kShareThreads + tid) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (y[e] >= T) {
            const int slot = atomicAdd(&s_cnt, 1);
            if (slot < kShareCap) {
              s_cv[slot] = y[e];
              s_ci[slot] = id0 + e;
            }
          }
        }
      }
    }
    __syncthreads();
    const int cnt = s_cnt;
    if (cnt <= kShareCap) return true;
    __syncthreads();  // every thread has read the count
    if (tid == 0) s_cnt = 0;
    return false;
  };

  int S;
  bool ok = listed(std::integral_constant<bool, false>{});
  if (!ok) {
    __syncthreads();
    ok = listed(std::integral_constant<bool, true>{});
  }
  if (ok) {
    S = s_cnt;
  } else {
    // every element through the wave lists
    WaveTopK top(k, tid);
#pragma unroll
    for (int u = 0; u < kShareUnits; ++u) {
      if (u * kShareThreads >= ns) break;  // uniform
      float y[8];
      VocabUnit<__bf16, true>::unpack(raw[u], y);
      const uint64_t vmask = __ballot(u * kShareThreads + tid < ns);
      const int uid = (u0 + u * kShareThreads + tid) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) top.offer(y[e], vmask, uid, e);
    }
    __syncthreads();  // the last pass's readers of the list are done
    if (lane < k) {
      s_cv[wave * k + lane] = top.mv;
      s_ci[wave * k + lane] = top.mi;
    }
    __syncthreads();
    S = kShareWaves * k;
  }
  // rank by counting (the listed elements are distinct by id)
  for (int i = tid; i < S; i += kShareThreads) {
    const float v = rank_key(s_cv[i]);
    const int id = s_ci[i];
    int rank = 0;
    for (int j = 0; j < S; ++j) rank += better(rank_key(s_cv[j]), s_ci[j], v, id) ? 1 : 0;
    if (rank >= k) continue;
    if (shares == 1) adj[(size_t)tok * k + rank] = id;
    else part[((size_t)node * shares + share) * k + rank] = make_int2(__float_as_int(v), id);
  }
}

// graft_lists_kernel: one wavefront per node ranks the shares' k best
// (shares * k <= 64 entries, one a lane, distinct) and writes the row. The
// lists and the tokens of the ownership test are read in one round trip.
__global__ __launch_bounds__(64) void graft_lists_kernel(
    int32_t* __restrict__ adj, int32_t vocab, int32_t k, int32_t num_nodes,
    const int32_t* __restrict__ node_tokens, int32_t shares, const int2* __restrict__ part) {
  const int lane = threadIdx.x, node = blockIdx.x;
  const int E = shares * k;
  const int2 e = part[(size_t)node * E + min(lane, E - 1)];
  const int tok = node_tokens[node];
  const int j0 = node + 1 + lane;
  const int tj = j0 < num_nodes ? node_tokens[j0] : -1;
  if (tok < 0 || tok >= vocab) return;
  int later = (tj == tok);
  for (int j = j0 + 64; j < num_nodes; j += 64) later |= (node_tokens[j] == tok);
  if (__ballot(later) != 0) return;
  const float v = __int_as_float(e.x);
  int rank = 0;
  for (int s = 0; s < E; ++s)
    rank += better(readlane_f(v, s), __builtin_amdgcn_readlane(e.y, s), v, e.y) ? 1 : 0;
  if (lane < E && rank < k) adj[(size_t)tok * k + rank] = e.y;
}

// graft_merge_kernel: one workgroup per node ranks the splits' partial lists
// (at most kMaxSplits * k entries, distinct) by counting and writes the row.
__global__ __launch_bounds__(kMergeThreads) void graft_merge_kernel(
    int32_t* __restrict__ adj, int32_t vocab, int32_t k, int32_t num_nodes,
    const int32_t* __restrict__ node_tokens, int32_t splits, const int2* __restrict__ part) {
  constexpr int kPer = kMaxSplits * TV_MAX_GRAFT_K / kMergeThreads;  // entries per thread
  __shared__ int2 s_e[kMaxSplits * TV_MAX_GRAFT_K];
  const int node = blockIdx.x, tid = threadIdx.x;
  const int E = splits * k;
  // the partial lists are read before the ownership test so that the two
  // reads overlap (a row nobody owns leaves its entries unused)
  const int2* p = part + (size_t)node * E;
  int2 mine[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = q * kMergeThreads + tid;
    mine[q] = i < E ? p[i] : make_int2(0, 0);
  }
  const int tok = node_tokens[node];
  if (!owns_row(node_tokens, num_nodes, node, tok, vocab)) return;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = q * kMergeThreads + tid;
    if (i < E) s_e[i] = mine[q];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = q * kMergeThreads + tid;
    if (q * kMergeThreads >= E) break;  // uniform
    const float v = __int_as_float(mine[q].x);
    const int id = mine[q].y;
    int rank = 0;
    for (int s = 0; s < E; ++s) {
      const int2 o = s_e[s];
      rank += better(__int_as_float(o.x), o.y, v, id) ? 1 : 0;
    }
    if (i < E && rank < k) adj[(size_t)tok * k + rank] = id;
  }
}

// Workgroups per row: shares of at most one sweep of loads (each thread's
// loads all in flight at once) while the grid stays within kMaxUpdateGroups;
// beyond that, enough shares to cover the chip about twice.
constexpr int64_t kMaxUpdateGroups = 8 * 256;
int update_splits(int32_t num_nodes, int64_t units) {
  if (units < 1 || num_nodes < 1) return 1;
  const int64_t sweep = (int64_t)kUpdateThreads * kUpdateUnroll;
  const int64_t by_len = (units + sweep - 1) / sweep;
  int64_t s = by_len;
  if (s * num_nodes > kMaxUpdateGroups) {
    s = (2 * 256 + (int64_t)num_nodes - 1) / num_nodes;
    if (s > by_len) s = by_len;
  }
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  const int64_t per = (units + s - 1) / s;
  return (int)((units + per - 1) / per);  // no empty split
}

}  // namespace

hipError_t launch_graft_retrieve(const int32_t* adj, int32_t vocab, int32_t k,
                                 const int32_t* root_tokens, int32_t batch,
                                 const int32_t* tmpl_parent, const int32_t* tmpl_rank,
                                 int32_t tmpl_nodes, int32_t* out_tokens, hipStream_t stream) {
  GraftTemplate t{};
  t.nodes = tmpl_nodes;
  int depth[TV_MAX_GRAFT_TEMPLATE];
  for (int j = 0; j < tmpl_nodes; ++j) {
    depth[j] = tmpl_parent[j] < 0 ? 1 : depth[tmpl_parent[j]] + 1;
    t.max_depth = depth[j] > t.max_depth ? depth[j] : t.max_depth;
    t.node[j] = (uint32_t)(tmpl_parent[j] + 1) | ((uint32_t)tmpl_rank[j] << 8) |
                ((uint32_t)depth[j] << 16);
  }
  const int grid = (batch + kRetrieveWaves - 1) / kRetrieveWaves;
  hipLaunchKernelGGL(graft_retrieve_kernel, dim3(grid), dim3(64 * kRetrieveWaves), 0, stream, adj,
                     vocab, k, root_tokens, batch, t, out_tokens);
  return hipGetLastError();
}

// Shares of the bf16 share kernel for this row length: the fewest with no
// more than kShareUnits units a thread (more shares, tried for rows that
// leave compute units idle, lengthened the list kernel more than they
// shortened the loads); 0 where the list kernel cannot hold that many lists
// (those rows take graft_topk_kernel).
static int graft_shares(int32_t vocab, int32_t dtype, bool vec, int32_t k) {
  if (!vec || dtype != TV_BF16 || vocab % 8 != 0) return 0;
  const int64_t n = vocab / 8, cap = (int64_t)kShareUnits * kShareThreads;
  const int64_t s = (n + cap - 1) / cap;
  if (s * k > kListLanes) return 0;
  const int64_t per = (n + s - 1) / s;
  return (int)((n + per - 1) / per);  // no empty share
}

size_t graft_update_workspace(int32_t num_nodes, int32_t vocab, int32_t k, int32_t dtype,
                              bool vec) {
  const int w = !vec ? 1 : (dtype == TV_BF16 ? 8 : 4);
  if (vocab % w != 0) return 0;  // that path is never taken for this vocabulary
  const int sh = graft_shares(vocab, dtype, vec, k);
  if (sh == 1) return 0;
  if (sh > 1) return ((size_t)num_nodes * sh * k * sizeof(int2) + 255) / 256 * 256;
  const int s = update_splits(num_nodes, vocab / w);
  if (s <= 1) return 0;
  return ((size_t)num_nodes * s * k * sizeof(int2) + 255) / 256 * 256;
}

namespace {
template <typename T, bool VEC>
hipError_t run_update(int32_t* adj, int32_t vocab, int32_t k, const T* lg, int32_t num_nodes,
                      const int32_t* node_tokens, int2* part, hipStream_t stream) {
  const int s = update_splits(num_nodes, vocab / VocabUnit<T, VEC>::W);
  hipLaunchKernelGGL((graft_topk_kernel<T, VEC>), dim3(num_nodes, s), dim3(kUpdateThreads), 0,
                     stream, adj, vocab, k, lg, num_nodes, node_tokens, s, part);
  if (s > 1)
    hipLaunchKernelGGL(graft_merge_kernel, dim3(num_nodes), dim3(kMergeThreads), 0, stream, adj,
                       vocab, k, num_nodes, node_tokens, s, part);
  return hipGetLastError();
}
}  // namespace

bool graft_update_vec(const void* logits, int32_t dtype, int32_t vocab) {
  return dtype == TV_BF16 ? vocab_vec<__bf16>(logits, vocab) : vocab_vec<float>(logits, vocab);
}

hipError_t launch_graft_update(int32_t* adj, int32_t vocab, int32_t k, const void* logits,
                               int32_t dtype, int32_t num_nodes, const int32_t* node_tokens,
                               void* workspace, hipStream_t stream) {
  const bool vec = graft_update_vec(logits, dtype, vocab);
  int2* part = static_cast<int2*>(workspace);
  const int sh = graft_shares(vocab, dtype, vec, k);
  if (sh > 0) {
    hipLaunchKernelGGL(graft_share_kernel, dim3(num_nodes, sh), dim3(kShareThreads), 0, stream,
                       adj, vocab, k, static_cast<const __bf16*>(logits), num_nodes, node_tokens,
                       sh, part);
    if (sh > 1)
      hipLaunchKernelGGL(graft_lists_kernel, dim3(num_nodes), dim3(64), 0, stream, adj, vocab, k,
                         num_nodes, node_tokens, sh, part);
    return hipGetLastError();
  }
  if (dtype == TV_BF16) {
    const __bf16* lg = static_cast<const __bf16*>(logits);
    return vec ? run_update<__bf16, true>(adj, vocab, k, lg, num_nodes, node_tokens, part, stream)
               : run_update<__bf16, false>(adj, vocab, k, lg, num_nodes, node_tokens, part, stream);
  }
  const float* lg = static_cast<const float*>(logits);
  return vec ? run_update<float, true>(adj, vocab, k, lg, num_nodes, node_tokens, part, stream)
             : run_update<float, false>(adj, vocab, k, lg, num_nodes, node_tokens, part, stream);
}

}  // namespace tv
