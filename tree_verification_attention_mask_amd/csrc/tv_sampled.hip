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
// One parameter per step. With the node's softmax values P(v), Q(v) and the
// draft mass M_r left after r rejections (M_0 = 1), every token not yet
// rejected has
//   p_r(v) = max(0, P(v) - beta_r Q(v)) / gamma_r,   q_r(v) = Q(v) / M_r,
// with beta_0 = 0, gamma_0 = 1 and, writing F(beta) = sum_v max(0, P(v) -
// beta Q(v)),
//   beta_{r+1} = beta_r + gamma_r / M_r,   gamma_{r+1} = F(beta_{r+1})
// (by induction: subtracting q_r from p_r and renormalising shifts beta and
// rescales). A rejected token has q = 0 from then on and its residual is
// already 0 (it was rejected because p <= u q < q), so F can sum over every
// token. When F(beta_{r+1}) = 0 the residual is empty and p stays (beta,
// gamma kept); when M_r = 0, q is zero and p stays too. So a node's whole
// chain is a few evaluations of F, each a sum over the vocabulary, and the
// bonus distribution after m rejections is max(0, P - beta_m Q) / gamma_m.
//
// Kernels (every node of the batch in parallel; each node's rows are cut into
// S shares, one 256-thread workgroup each):
//   pass 0:   share partials of both softmax normalisers; share 0 also lists
//             the node's children (index order, tokens in the vocabulary)
//             with their uniforms.
//   pass k:   (k = 1 .. max_children) combine the shares' partials of the pass
//             before and fix (beta_{k-1}, gamma_{k-1}) with each share's sum of
//             that state's residual (the partial of F over F); then, for a
//             node with m >= k children, share partials of F(beta_k) (pass 1
//             also the draft mass outside the children's tokens).
//   walk:     one 1024-thread workgroup per request: at each node one parallel
//             read of its children and steps, the tests in order with scalar
//             arithmetic every thread repeats; at the last node it fixes the
//             final step from the last pass's partials, finds the share that
//             holds the bonus draw from the share sums and inverts the CDF
//             inside it (per-thread runs in token order, a block scan, then a
//             rescan of the one run). The bonus distribution after the last
//             step needs no sweep of its own: its share sums are the last
//             F partials over F.
#include "tv_launch.h"
#include "tv_vocab.h"

namespace tv {
namespace {

constexpr int kPassThreads = 256;
constexpr int kPassWaves = kPassThreads / 64;
constexpr int kPassUnroll = 8;  // units per thread in flight (a share is one sweep at 16,384 tokens)
constexpr int kWalkThreads = 1024;
constexpr int kWalkWaves = kWalkThreads / 64;
constexpr int kMaxShares = 32;
constexpr float kLog2eS = 1.4426950408889634f;

struct NodeInfo {
  float lp, lq;  // log2 normalisers: P(v) = 2^(c a_v - lp), Q(v) = 2^(c b_v - lq)
  float snc;     // draft mass outside the children's tokens
  int32_t m;     // children kept (tokens in the vocabulary), at most max_children
};
struct ChildInfo {
  int32_t tok, local;  // token, request-local node index
  float P, Q, u;       // target / draft probability of the token, the child's uniform
  int32_t dup;         // earlier child with the same token, or -1
  int32_t pad[2];
};
struct Step {
  float beta, gamma;
};

struct SArgs {
  const int32_t* parent;
  const int32_t* draft_tok;
  const int32_t* cu_nodes;
  const float* u_accept;
  const float* u_bonus;
  int32_t batch, total_nodes, max_nodes, max_depth;
  int32_t C, S;  // children kept per node, shares per row
  int64_t vocab;
  float c;
  NodeInfo* node;    // [N]
  ChildInfo* child;  // [N][C]
  Step* step;        // [N][C + 1]
  float4* part;      // [2][N][S] share partials, by pass parity
  float* bonus;      // [N][S] share sums of the bonus distribution
  int32_t* accept_len;
  int32_t* path;
  int32_t* bonus_tok;
};

__device__ __forceinline__ float nan_to_ninf(float x) { return (x == x) ? x : -INFINITY; }
// softmax value 2^(c x - L); a NaN logit gives 0 (max returns its non-NaN operand)
__device__ __forceinline__ float prob(float x, float c, float L) {
  return fmaxf(__builtin_amdgcn_exp2f(__builtin_fmaf(x, c, -L)), 0.f);
}

// 1 / (draft mass left after the first r children are rejected): the mass
// outside every child's token plus each remaining distinct token's; 1 for
// r = 0 and 0 when nothing is left.
__device__ float inv_mass(float snc, const ChildInfo* ch, int m, int r) {
  if (r == 0) return 1.f;
  float M = snc;
  for (int j = r; j < m; ++j)
    if (ch[j].dup < 0) M += ch[j].Q;
  return M > 0.f ? 1.f / M : 0.f;
}

// Share s of a row of `units` units: [u0, u1).
__device__ __forceinline__ void share(int64_t units, int S, int s, int64_t& u0, int64_t& u1) {
  const int64_t per = (units + S - 1) / S;
  u0 = min(units, (int64_t)s * per);
  u1 = min(units, u0 + per);
}

// Visit the units [u0, u1) of two rows, kPassUnroll units per thread in
// flight at once (loads from a clamped index, so that a thread's loads are
// issued together); fn(ya, yb, unit, valid).
template <typename T, bool VEC, typename Fn>
__device__ __forceinline__ void for_units(const T* ra, const T* rb, int64_t u0, int64_t u1, Fn&& fn) {
  constexpr int W = VocabUnit<T, VEC>::W;
  for (int64_t base = u0; base < u1; base += kPassUnroll * kPassThreads) {
    float ya[kPassUnroll][W], yb[kPassUnroll][W];
#pragma unroll
    for (int u = 0; u < kPassUnroll; ++u) {
      const int64_t j = min(base + u * kPassThreads + (int64_t)threadIdx.x, u1 - 1);
      VocabUnit<T, VEC>::load(ra + j * W, ya[u]);
      VocabUnit<T, VEC>::load(rb + j * W, yb[u]);
    }
#pragma unroll
    for (int u = 0; u < kPassUnroll; ++u) {
      const int64_t j = base + u * kPassThreads + threadIdx.x;
      fn(ya[u], yb[u], j, j < u1);
    }
  }
}

// Sum over a pass workgroup of two values per thread.
__device__ float2 pass_sum2(float x, float y, float2* s_red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    x += __shfl_xor(x, off, 64);
    y += __shfl_xor(y, off, 64);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s_red[wave] = make_float2(x, y);
  __syncthreads();
  float2 r = s_red[0];
#pragma unroll
  for (int w = 1; w < kPassWaves; ++w) {
    r.x += s_red[w].x;
    r.y += s_red[w].y;
  }
  __syncthreads();
  return r;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kPassThreads) void sampled_prep_kernel(SArgs a, const T* __restrict__ tl,
                                                                       const T* __restrict__ dl) {
  constexpr int W = VocabUnit<T, VEC>::W;
  __shared__ MaxSum s_ms[kPassWaves];
  __shared__ int s_cnt[kPassWaves];
  const int g = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t units = a.vocab / W;  // VEC only when vocab % W == 0
  int64_t u0, u1;
  share(units, a.S, s, u0, u1);
  const T* ra = tl + (int64_t)g * a.vocab;
  const T* rb = dl + (int64_t)g * a.vocab;
  MaxSum mp{-INFINITY, 0.f}, mq{-INFINITY, 0.f};
  for_units<T, VEC>(ra, rb, u0, u1, [&](float (&ya)[W], float (&yb)[W], int64_t, bool valid) {
    if (!valid) return;
#pragma unroll
    for (int e = 0; e < W; ++e) {
      ya[e] = nan_to_ninf(ya[e]);
      yb[e] = nan_to_ninf(yb[e]);
    }
    fold(mp, ya, a.c);
    fold(mq, yb, a.c);
  });
  mp = block_merge<kPassWaves>(mp, s_ms);
  mq = block_merge<kPassWaves>(mq, s_ms);
  if (tid == 0) a.part[(size_t)g * a.S + s] = make_float4(mp.m, mp.s, mq.m, mq.s);
  if (s != 0) return;

  // the node's request (cu_nodes ascending: cu[b] <= g < cu[b + 1]) and its
  // children in index order
  int lo = 0, hi = a.batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu_nodes[mid] <= g) lo = mid;
    else hi = mid;
  }
  const int r0 = clampi(a.cu_nodes[lo], 0, a.total_nodes);
  const int r1 = clampi(a.cu_nodes[lo + 1], r0, a.total_nodes);
  const int n = min(r1 - r0, a.max_nodes);
  const int local = g - r0;
  int m = 0;
  if (local >= 0 && local < n) {  // (uniform; false only for malformed offsets)
    ChildInfo* ch = a.child + (size_t)g * a.C;
    for (int base = local + 1; base < n; base += kPassThreads) {
      const int ci = base + tid;
      int x = -1;
      bool is = false;
      if (ci < n && a.parent[r0 + ci] == local) {
        x = a.draft_tok[r0 + ci];
        is = x >= 0 && (int64_t)x < a.vocab;  // a token outside the vocabulary is passed over
      }
      const uint64_t bal = __ballot(is);
      if (lane == 0) s_cnt[wave] = __popcll(bal);
      __syncthreads();
      int off = m, tot = 0;
#pragma unroll
      for (int w = 0; w < kPassWaves; ++w) {
        const int cnt = s_cnt[w];
        off += (w < wave) ? cnt : 0;
        tot += cnt;
      }
      const int pos = off + __popcll(bal & ((1ull << lane) - 1));
      if (is && pos < a.C) {
        ChildInfo c{};
        c.tok = x;
        c.local = ci;
        c.u = a.u_accept[r0 + ci];
        c.dup = -1;
        ch[pos] = c;
      }
      m += tot;
      __syncthreads();
    }
  }
  if (tid == 0) {
    NodeInfo ni{};
    ni.m = min(m, a.C);
    a.node[g] = ni;
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kPassThreads) void sampled_pass_kernel(SArgs a, int k,
                                                                      const T* __restrict__ tl,
                                                                      const T* __restrict__ dl) {
  constexpr int W = VocabUnit<T, VEC>::W;
  __shared__ float2 s_red[kPassWaves];
  __shared__ ChildInfo s_ch[TV_MAX_SAMPLED_CHILDREN];
  const int g = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const bool lead = (s == 0 && tid == 0);
  NodeInfo ni = a.node[g];
  const int m = ni.m;
  if (k > (m > 1 ? m : 1)) return;  // pass 1 for every node, then while steps remain (uniform)
  const int S = a.S;
  const float4* prev = a.part + (size_t)((k - 1) & 1) * a.total_nodes * S + (size_t)g * S;
  ChildInfo* ch = a.child + (size_t)g * a.C;
  Step* st = a.step + (size_t)g * (a.C + 1);
  const T* ra = tl + (int64_t)g * a.vocab;
  const T* rb = dl + (int64_t)g * a.vocab;

  if (k == 1) {
    // normalisers from the shares, in share order (every workgroup alike)
    MaxSum mp{-INFINITY, 0.f}, mq{-INFINITY, 0.f};
    for (int i = 0; i < S; ++i) {
      const float4 p = prev[i];
      mp = merge(mp, MaxSum{p.x, p.y});
      mq = merge(mq, MaxSum{p.z, p.w});
    }
    ni.lp = mp.m + __log2f(mp.s);
    ni.lq = mq.m + __log2f(mq.s);
  } else if (k == 2) {
    float snc = 0.f;
    for (int i = 0; i < S; ++i) snc += prev[i].y;
    ni.snc = snc;
  }
  // the children: pass 1 fills in the probabilities of their tokens and the
  // repeated tokens, later passes read them
  for (int j = tid; j < m; j += kPassThreads) {
    ChildInfo c = ch[j];
    if (k == 1) {
      c.P = prob(load_one(ra + c.tok), a.c, ni.lp);
      c.Q = prob(load_one(rb + c.tok), a.c, ni.lq);
      c.dup = -1;
      for (int i = 0; i < j; ++i)
        if (ch[i].tok == c.tok) {
          c.dup = i;
          break;
        }
    }
    s_ch[j] = c;
  }
  __syncthreads();
  if (s == 0 && k == 1)
    for (int j = tid; j < m; j += kPassThreads) ch[j] = s_ch[j];
  if (lead && k <= 2) a.node[g] = ni;

  // (beta_{k-1}, gamma_{k-1})
  Step cur{0.f, 1.f};
  float F = 0.f;
  if (k >= 2) {
    const Step pk = st[k - 2];
    const float beta = pk.beta + pk.gamma * inv_mass(ni.snc, s_ch, m, k - 2);
    for (int i = 0; i < S; ++i) F += prev[i].x;
    cur = (F > 0.f) ? Step{beta, F} : pk;
  }
  if (lead) st[k - 1] = cur;
  // this share's sum of the state's residual max(0, P - beta Q) / gamma, kept
  // for the walk's bonus draw when a node's last step leaves p unchanged
  if (tid == 0) {
    float* bs = a.bonus + (size_t)g * S + s;
    if (k == 1) {
      const float4 p0 = prev[s];  // this share's (max, sum) of the target's exponents
      *bs = (p0.x == -INFINITY) ? 0.f : p0.y * __builtin_amdgcn_exp2f(p0.x - ni.lp);
    } else if (F > 0.f) {
      *bs = prev[s].x / F;
    }
  }

  const int64_t units = a.vocab / W;
  int64_t u0, u1;
  share(units, S, s, u0, u1);
  if (k <= m) {
    // share partial of F(beta_k); pass 1 also the draft mass outside the children
    const float beta = cur.beta + cur.gamma * inv_mass(ni.snc, s_ch, m, k - 1);
    float f = 0.f, snc = 0.f;
    for_units<T, VEC>(ra, rb, u0, u1, [&](float (&ya)[W], float (&yb)[W], int64_t j, bool valid) {
      if (!valid) return;
      float Q[W];
#pragma unroll
      for (int e = 0; e < W; ++e) {
        const float P = prob(ya[e], a.c, ni.lp);
        Q[e] = prob(yb[e], a.c, ni.lq);
        f += fmaxf(0.f, __builtin_fmaf(-beta, Q[e], P));
      }
      if (k == 1) {
        // draft mass outside the children's tokens: a unit holding none of
        // them adds all its values, else value by value
        bool hit = false;
        for (int i = 0; i < m; ++i) hit |= (s_ch[i].tok / W == j);
        if (!hit) {
#pragma unroll
          for (int e = 0; e < W; ++e) snc += Q[e];
        } else {
#pragma unroll
          for (int e = 0; e < W; ++e) {
            const int v = (int)(j * W + e);
            bool child = false;
            for (int i = 0; i < m; ++i) child |= (s_ch[i].tok == v);
            snc += child ? 0.f : Q[e];
          }
        }
      }
    });
    const float2 r = pass_sum2(f, snc, s_red);
    if (tid == 0)
      a.part[(size_t)(k & 1) * a.total_nodes * S + (size_t)g * S + s] = make_float4(r.x, r.y, 0.f, 0.f);
  }
}

// Inclusive prefix sum over the walk block of one value per thread, in thread
// order; returns the thread's inclusive sum and the block total.
__device__ float walk_inclusive_sum(float v, float* s_w, float& total) {
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

// Walk storage in dynamic LDS: K node slots of children [K][C], steps
// [K][C + 1], node info [K], share sums [K][S] and the share partials of F of
// both pass parities [K][2][S]. K = the request's node cap
// when that fits (everything is read once, up front), else 1 (one node read
// per level).
__host__ __device__ inline size_t walk_slot_bytes(int C, int S) {
  return (size_t)C * sizeof(ChildInfo) + (size_t)(C + 1) * sizeof(Step) + sizeof(NodeInfo) +
         (size_t)3 * S * sizeof(float);
}
constexpr size_t kWalkPreloadBytes = 48 * 1024;

template <typename T, bool VEC>
__global__ __launch_bounds__(kWalkThreads) void sampled_walk_kernel(SArgs a, int preload,
                                                                    const T* __restrict__ tl,
                                                                    const T* __restrict__ dl) {
  constexpr int W = VocabUnit<T, VEC>::W;
  extern __shared__ float4 s_dyn4[];
  __shared__ float s_w[kWalkWaves], s_incl[kWalkWaves];
  __shared__ int s_pick, s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  const int lo = clampi(a.cu_nodes[b], 0, a.total_nodes);
  const int hi = clampi(a.cu_nodes[b + 1], lo, a.total_nodes);
  const int n = min(hi - lo, a.max_nodes);
  const int prow = a.max_depth + 1;
  int32_t* path = a.path + (size_t)b * prow;
  for (int d = tid; d < prow; d += kWalkThreads) path[d] = (d == 0 && n > 0) ? 0 : -1;
  if (n == 0) {  // an empty request (uniform)
    if (tid == 0) {
      a.accept_len[b] = 0;
      a.bonus_tok[b] = -1;
    }
    return;
  }
  const int C = a.C, S = a.S;
  const int K = preload ? a.max_nodes : 1;
  ChildInfo* s_chs = reinterpret_cast<ChildInfo*>(s_dyn4);
  Step* s_sts = reinterpret_cast<Step*>(s_chs + (size_t)K * C);
  NodeInfo* s_nis = reinterpret_cast<NodeInfo*>(s_sts + (size_t)K * (C + 1));
  float* s_shs = reinterpret_cast<float*>(s_nis + K);
  float* s_pms = s_shs + (size_t)K * S;
  // copy nodes [first, first + cnt) of the request into slots [0, cnt)
  auto fetch = [&](int first, int cnt) {
    const size_t g0 = (size_t)lo + first;
    for (int i = tid; i < cnt * C; i += kWalkThreads) s_chs[i] = a.child[g0 * C + i];
    for (int i = tid; i < cnt * (C + 1); i += kWalkThreads) s_sts[i] = a.step[g0 * (C + 1) + i];
    for (int i = tid; i < cnt; i += kWalkThreads) s_nis[i] = a.node[g0 + i];
    for (int i = tid; i < cnt * S; i += kWalkThreads) s_shs[i] = a.bonus[g0 * S + i];
    for (int i = tid; i < 2 * cnt * S; i += kWalkThreads) {
      const int par = i / (cnt * S), r = i % (cnt * S);  // [parity][node][share] -> slot [node][parity][share]
      s_pms[(r / S) * 2 * S + par * S + r % S] =
          a.part[(size_t)par * a.total_nodes * S + g0 * S + r].x;
    }
  };
  if (preload) fetch(0, n);
  __syncthreads();
  const int64_t units = a.vocab / W;

  int node = 0, depth = 0;
  for (;;) {
    const int g = lo + node;
    if (!preload) {  // one round trip for the node, all its slots
      fetch(node, 1);
      __syncthreads();
    }
    const int slot = preload ? node : 0;
    const ChildInfo* s_ch = s_chs + (size_t)slot * C;
    const Step* s_st = s_sts + (size_t)slot * (C + 1);
    const float* s_share = s_shs + (size_t)slot * S;
    const NodeInfo ni = s_nis[slot];
    const int m = ni.m;
    const float* s_pm = s_pms + ((size_t)slot * 2 + (m & 1)) * S;  // the last pass's partials
    // the children in order (every thread takes the same decisions)
    int next = -1;
    for (int l = 0; l < m; ++l) {
      const ChildInfo c = s_ch[l];
      float p, q;
      if (c.dup >= 0) {  // its token was rejected before: q is 0, the residual frozen
        q = 0.f;
        p = fmaxf(0.f, __builtin_fmaf(-s_st[c.dup + 1].beta, c.Q, c.P)) / s_st[l].gamma;
      } else {
        q = c.Q * inv_mass(ni.snc, s_ch, m, l);
        p = fmaxf(0.f, __builtin_fmaf(-s_st[l].beta, c.Q, c.P)) / s_st[l].gamma;
      }
      if (c.u * q < p) {
        next = c.local;
        break;
      }
    }
    if (next > node && next < n) {
      node = next;
      ++depth;
      if (tid == 0 && depth <= a.max_depth) path[depth] = node;
      if (!preload) __syncthreads();  // slot 0 is refilled for the next node
      continue;
    }

    // bonus. The node's last step is fixed here from the last pass's share
    // partials of F (as a pass would fix it); the state's per-share sums are
    // those partials over F, or, when the step left p unchanged, the sums the
    // passes kept.
    Step fin{0.f, 1.f};
    float Fm = 0.f;
    if (m >= 1) {
      const Step pk = s_st[m - 1];
      const float beta = pk.beta + pk.gamma * inv_mass(ni.snc, s_ch, m, m - 1);
      for (int i = 0; i < S; ++i) Fm += s_pm[i];
      fin = (Fm > 0.f) ? Step{beta, Fm} : pk;
    }
    const bool fresh = Fm > 0.f;
    auto share_sum = [&](int i) { return fresh ? s_pm[i] / Fm : s_share[i]; };
    const float ig = 1.f / fin.gamma;
    float total = 0.f;
    for (int i = 0; i < S; ++i) total += share_sum(i);
    const float target = a.u_bonus[b] * total;
    int sh = -1, last_sh = -1;
    float before = 0.f, acc = 0.f;
    for (int i = 0; i < S; ++i) {
      const float si = share_sum(i);
      const float nx = acc + si;
      if (si > 0.f) last_sh = i;
      if (sh < 0 && acc <= target && target < nx) {
        sh = i;
        before = acc;
      }
      acc = nx;
    }
    const bool past = sh < 0;  // at or past the total: the last token with mass
    if (past) sh = last_sh;
    int pick = -1;
    if (sh >= 0) {
      int64_t u0, u1;
      share(units, S, sh, u0, u1);
      const int64_t per = (u1 - u0 + kWalkThreads - 1) / kWalkThreads;
      const int64_t j0 = min(u1, u0 + (int64_t)tid * per), j1 = min(u1, j0 + per);
      const T* ra = tl + (int64_t)g * a.vocab;
      const T* rb = dl + (int64_t)g * a.vocab;
      auto p_at = [&](int64_t j, float (&pv)[W]) {
        float ya[W], yb[W];
        VocabUnit<T, VEC>::load(ra + j * W, ya);
        VocabUnit<T, VEC>::load(rb + j * W, yb);
#pragma unroll
        for (int e = 0; e < W; ++e) {
          const float P = prob(ya[e], a.c, ni.lp);
          const float Q = prob(yb[e], a.c, ni.lq);
          pv[e] = fmaxf(0.f, __builtin_fmaf(-fin.beta, Q, P)) * ig;
        }
      };
      float run = 0.f;
      for (int64_t j = j0; j < j1; ++j) {
        float pv[W];
        p_at(j, pv);
#pragma unroll
        for (int e = 0; e < W; ++e) run += pv[e];
      }
      float stotal;
      const float incl = walk_inclusive_sum(run, s_w, stotal);
      // the previous thread's inclusive sum: a shuffle within the wave, LDS
      // across waves, so the runs [excl, incl) tile [0, stotal) exactly
      if (lane == 63) s_incl[wave] = incl;
      if (tid == 0) {
        s_pick = -1;
        s_last = -1;
      }
      __syncthreads();
      float excl = __shfl_up(incl, 1, 64);
      if (lane == 0) excl = (wave == 0) ? 0.f : s_incl[wave - 1];
      const float t = past ? INFINITY : target - before;
      if (excl <= t && t < incl) {
        float r = excl;
        int pk = -1, last = -1;
        for (int64_t j = j0; j < j1 && pk < 0; ++j) {
          float pv[W];
          p_at(j, pv);
#pragma unroll
          for (int e = 0; e < W; ++e) {
            if (pk >= 0) break;
            if (pv[e] > 0.f) last = (int)(j * W + e);
            r += pv[e];
            if (r > t && pv[e] > 0.f) pk = (int)(j * W + e);
          }
        }
        s_pick = pk >= 0 ? pk : last;
      }
      if (run > 0.f) atomicMax(&s_last, tid);
      __syncthreads();
      if (s_pick < 0 && tid == s_last) {
        // rounding left the draw outside every run: the last token with mass
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
      pick = s_pick;
    }
    if (tid == 0) {
      a.bonus_tok[b] = pick;
      a.accept_len[b] = depth;
    }
    return;
  }
}

template <typename T, bool VEC>
hipError_t run_sampled(const SArgs& a, const void* tl, const void* dl, hipStream_t stream) {
  const T* t = static_cast<const T*>(tl);
  const T* d = static_cast<const T*>(dl);
  if (a.total_nodes > 0) {
    const dim3 grid(a.total_nodes, a.S);
    hipLaunchKernelGGL((sampled_prep_kernel<T, VEC>), grid, dim3(kPassThreads), 0, stream, a, t, d);
    for (int k = 1; k <= a.C; ++k)
      hipLaunchKernelGGL((sampled_pass_kernel<T, VEC>), grid, dim3(kPassThreads), 0, stream, a, k,
                         t, d);
  }
  const size_t slot = walk_slot_bytes(a.C, a.S);
  const int preload = (size_t)a.max_nodes * slot <= kWalkPreloadBytes ? 1 : 0;
  const size_t lds = (preload ? (size_t)a.max_nodes : 1) * slot;
  hipLaunchKernelGGL((sampled_walk_kernel<T, VEC>), dim3(a.batch), dim3(kWalkThreads), lds, stream, a,
                     preload, t, d);
  return hipGetLastError();
}

}  // namespace

SampledLayout sampled_layout(int32_t total_nodes, int32_t max_children, int32_t vocab) {
  SampledLayout L{};
  L.C = max_children < 1 ? 1 : max_children;
  // shares per row: about four workgroups per CU over the batch's rows, at
  // least 16,384 tokens a share
  const int64_t nodes = total_nodes > 0 ? total_nodes : 1;
  int64_t s = (4 * 256 + nodes - 1) / nodes;
  const int64_t by_len = ((int64_t)vocab + 16383) / 16384;
  if (s > by_len) s = by_len;
  if (s > kMaxShares) s = kMaxShares;
  if (s < 1) s = 1;
  L.S = (int)s;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t N = total_nodes > 0 ? (size_t)total_nodes : 0;
  L.node = 0;
  L.child = L.node + up(N * sizeof(NodeInfo));
  L.step = L.child + up(N * L.C * sizeof(ChildInfo));
  L.part = L.step + up(N * (L.C + 1) * sizeof(Step));
  L.bonus = L.part + up(2 * N * L.S * sizeof(float4));
  L.total = L.bonus + up(N * L.S * sizeof(float));
  return L;
}

hipError_t launch_accept_sampled(const int32_t* parent, const int32_t* draft_tok,
                                 const int32_t* cu_nodes, int32_t batch, int32_t total_nodes,
                                 int32_t max_nodes, int32_t max_children, int32_t max_depth,
                                 const void* target_logits, const void* draft_logits,
                                 int32_t dtype, int32_t vocab, float temperature,
                                 const float* u_accept, const float* u_bonus,
                                 int32_t* accept_len, int32_t* path, int32_t* bonus_tok,
                                 void* workspace, hipStream_t stream) {
  const SampledLayout L = sampled_layout(total_nodes, max_children, vocab);
  char* ws = static_cast<char*>(workspace);
  SArgs a;
  a.parent = parent;
  a.draft_tok = draft_tok;
  a.cu_nodes = cu_nodes;
  a.u_accept = u_accept;
  a.u_bonus = u_bonus;
  a.batch = batch;
  a.total_nodes = total_nodes;
  a.max_nodes = max_nodes;
  a.max_depth = max_depth;
  a.C = L.C;
  a.S = L.S;
  a.vocab = vocab;
  a.c = kLog2eS / temperature;
  a.node = reinterpret_cast<NodeInfo*>(ws + L.node);
  a.child = reinterpret_cast<ChildInfo*>(ws + L.child);
  a.step = reinterpret_cast<Step*>(ws + L.step);
  a.part = reinterpret_cast<float4*>(ws + L.part);
  a.bonus = reinterpret_cast<float*>(ws + L.bonus);
  a.accept_len = accept_len;
  a.path = path;
  a.bonus_tok = bonus_tok;
  if (dtype == TV_BF16) {
    const bool vec = vocab_vec<__bf16>(target_logits, vocab) && vocab_vec<__bf16>(draft_logits, vocab);
    return vec ? run_sampled<__bf16, true>(a, target_logits, draft_logits, stream)
               : run_sampled<__bf16, false>(a, target_logits, draft_logits, stream);
  }
  const bool vec = vocab_vec<float>(target_logits, vocab) && vocab_vec<float>(draft_logits, vocab);
  return vec ? run_sampled<float, true>(a, target_logits, draft_logits, stream)
             : run_sampled<float, false>(a, target_logits, draft_logits, stream);
}

}  // namespace tv
