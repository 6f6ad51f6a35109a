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
//   pass 0:   share partials of both softmax normalisers; one more workgroup
//             a row lists the node's children (index order, tokens in the
//             vocabulary) with their uniforms, repeated tokens and both
//             logits at each child's token.
//   pass k:   (k = 1 .. max_children) combine the shares' partials of the pass
//             before and fix (beta_{k-1}, gamma_{k-1}) with each share's sum of
//             that state's residual (the partial of F over F); then, for a
//             node with m >= k children, share partials of F(beta_k) (pass 1
//             also the draft mass outside the children's tokens). A node's
//             last pass (k = max(m, 1)) knows the state every child meets and
//             takes all the children's tests at once (one lane each: a test
//             depends on no earlier outcome), storing the first that passes.
//   walk:     one 1024-thread workgroup per request: its tables copied into
//             LDS in one round trip, the first wave follows the stored
//             accepted child level by level; at the last node it fixes the
//             final step from the last pass's partials and finds, with a wave
//             scan of the share sums, the share that holds the bonus draw;
//             the block inverts the CDF inside it (per-thread runs in token
//             order, a block scan, then a rescan of the one run). The bonus
//             distribution after the last step needs no sweep of its own: its
//             share sums are the last F partials over F.
#include "tv_launch.h"
#include "tv_vocab.h"

namespace tv {
namespace {

constexpr int kPassThreads = 256;
constexpr int kPassWaves = kPassThreads / 64;
constexpr int kPassUnroll = 8;  // units per thread in flight (a share is one sweep at 16,384 tokens)
constexpr int kWalkThreads = 1024;
constexpr int kWalkWaves = kWalkThreads / 64;
constexpr int kFetchUnroll = 8;  // words a walk thread has in flight while copying tables
constexpr int kWalkCache = 2;    // bonus units a walk thread keeps in registers
constexpr int kMaxShares = 32;
constexpr float kLog2eS = 1.4426950408889634f;

struct NodeInfo {
  float lp, lq;  // log2 normalisers: P(v) = 2^(c a_v - lp), Q(v) = 2^(c b_v - lq)
  float snc;     // draft mass outside the children's tokens
  int32_t m;     // children kept (tokens in the vocabulary), at most max_children
  int32_t next;  // the first child that passes its test (request-local index), or -1
};
struct ChildInfo {
  int32_t tok, local;  // token, request-local node index
  float P, Q, u;       // target / draft probability of the token, the child's uniform
  int32_t dup;         // earlier child with the same token, or -1
  float xa, xb;        // target / draft logit of the token
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

// One batch of a pass sweep: units base + u * kPassThreads + thread, u <
// kPassUnroll, of two rows, loaded from a clamped index (a thread's loads
// are issued together; base < u1).
template <typename T, bool VEC>
__device__ __forceinline__ void load_batch(const T* ra, const T* rb, int64_t base, int64_t u1,
                                           float (&ya)[kPassUnroll][VocabUnit<T, VEC>::W],
                                           float (&yb)[kPassUnroll][VocabUnit<T, VEC>::W]) {
  constexpr int W = VocabUnit<T, VEC>::W;
#pragma unroll
  for (int u = 0; u < kPassUnroll; ++u) {
    const int64_t j = min(base + u * kPassThreads + (int64_t)threadIdx.x, u1 - 1);
    VocabUnit<T, VEC>::load(ra + j * W, ya[u]);
    VocabUnit<T, VEC>::load(rb + j * W, yb[u]);
  }
}
// fn(ya, yb, unit, valid) over a loaded batch.
template <int W, typename Fn>
__device__ __forceinline__ void visit_batch(float (&ya)[kPassUnroll][W], float (&yb)[kPassUnroll][W],
                                            int64_t base, int64_t u1, Fn&& fn) {
#pragma unroll
  for (int u = 0; u < kPassUnroll; ++u) {
    const int64_t j = base + u * kPassThreads + threadIdx.x;
    fn(ya[u], yb[u], j, j < u1);
  }
}

// Visit the units [u0, u1) of two rows, kPassUnroll units per thread in
// flight at once; fn(ya, yb, unit, valid).
template <typename T, bool VEC, typename Fn>
__device__ __forceinline__ void for_units(const T* ra, const T* rb, int64_t u0, int64_t u1, Fn&& fn) {
  constexpr int W = VocabUnit<T, VEC>::W;
  for (int64_t base = u0; base < u1; base += kPassUnroll * kPassThreads) {
    float ya[kPassUnroll][W], yb[kPassUnroll][W];
    load_batch<T, VEC>(ra, rb, base, u1, ya, yb);
    visit_batch<W>(ya, yb, base, u1, fn);
  }
}

// Sum over a pass workgroup of two values per thread.
__device__ float2 pass_sum2(float x, float y, float2* s_red) {
  x = wave_sum(x);
  y = wave_sum(y);
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
  __shared__ MaxSum s_ms[kPassWaves], s_mq[kPassWaves];
  __shared__ int s_cnt[kPassWaves];
  __shared__ int32_t s_tok[TV_MAX_SAMPLED_CHILDREN], s_loc[TV_MAX_SAMPLED_CHILDREN];
  const int g = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const T* ra = tl + (int64_t)g * a.vocab;
  const T* rb = dl + (int64_t)g * a.vocab;
  if (s < a.S) {
    // share partials of both softmax normalisers
    const int64_t units = a.vocab / W;  // VEC only when vocab % W == 0
    int64_t u0, u1;
    share(units, a.S, s, u0, u1);
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
    mp = wave_merge(mp);
    mq = wave_merge(mq);
    if (lane == 0) {
      s_ms[wave] = mp;
      s_mq[wave] = mq;
    }
    __syncthreads();
    if (tid == 0) {
      MaxSum rp = s_ms[0], rq = s_mq[0];
#pragma unroll
      for (int w = 1; w < kPassWaves; ++w) {
        rp = merge(rp, s_ms[w]);
        rq = merge(rq, s_mq[w]);
      }
      a.part[(size_t)g * a.S + s] = make_float4(rp.m, rp.s, rq.m, rq.s);
    }
    return;
  }

  // the extra workgroup of the row: the node's request (cu_nodes ascending:
  // cu[b] <= g < cu[b + 1]), its children in index order with their
  // uniforms, repeated tokens and both logits at each child's token
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
        s_tok[pos] = x;
        s_loc[pos] = ci;
      }
      m += tot;
      __syncthreads();
    }
  }
  m = min(m, a.C);
  ChildInfo* ch = a.child + (size_t)g * a.C;
  for (int j = tid; j < m; j += kPassThreads) {
    ChildInfo c;
    c.tok = s_tok[j];
    c.local = s_loc[j];
    c.P = 0.f;
    c.Q = 0.f;
    c.u = a.u_accept[r0 + c.local];
    c.dup = -1;
    for (int i = 0; i < j; ++i)
      if (s_tok[i] == c.tok) {
        c.dup = i;
        break;
      }
    c.xa = load_one(ra + c.tok);
    c.xb = load_one(rb + c.tok);
    ch[j] = c;
  }
  if (tid == 0) {
    NodeInfo ni{};
    ni.m = m;
    ni.next = -1;
    a.node[g] = ni;
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kPassThreads) void sampled_pass_kernel(SArgs a, int k,
                                                                      const T* __restrict__ tl,
                                                                      const T* __restrict__ dl) {
  constexpr int W = VocabUnit<T, VEC>::W;
  __shared__ float2 s_red[kPassWaves];
  __shared__ float4 s_prev[kMaxShares];
  __shared__ ChildInfo s_ch[TV_MAX_SAMPLED_CHILDREN];
  __shared__ Step s_st[TV_MAX_SAMPLED_CHILDREN];
  __shared__ int32_t s_tin[TV_MAX_SAMPLED_CHILDREN];  // pass 1: children's tokens inside the share
  __shared__ int s_nin;
  const int g = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const bool lead = (s == 0 && tid == 0);
  NodeInfo ni = a.node[g];
  const int m = ni.m;
  const int last = m > 1 ? m : 1;
  if (k > last) return;  // pass 1 for every node, then while steps remain (uniform)
  // the node's last pass fixes (beta_{m-1}, gamma_{m-1}): after it every
  // child's test is known, and share 0 takes them
  const bool tests = (s == 0 && k == last);
  const bool sweep = k <= m;  // a share partial of F(beta_k) to take
  const int S = a.S;
  const float4* prev = a.part + (size_t)((k - 1) & 1) * a.total_nodes * S + (size_t)g * S;
  ChildInfo* ch = a.child + (size_t)g * a.C;
  Step* st = a.step + (size_t)g * (a.C + 1);
  const T* ra = tl + (int64_t)g * a.vocab;
  const T* rb = dl + (int64_t)g * a.vocab;
  const int64_t units = a.vocab / W;
  int64_t u0, u1;
  share(units, S, s, u0, u1);

  // the sweep's first batch is requested before the tables, so that both
  // round trips overlap
  float ya[kPassUnroll][W], yb[kPassUnroll][W];
  const bool early = sweep && u0 < u1;
  if (early) load_batch<T, VEC>(ra, rb, u0, u1, ya, yb);
  // the tables: the pass before's share partials, the children, the steps so far
  if (tid < S) s_prev[tid] = prev[tid];
  for (int j = tid; j < m; j += kPassThreads) s_ch[j] = ch[j];
  for (int l = tid; l < k - 1; l += kPassThreads) s_st[l] = st[l];
  if (tid == 0) s_nin = 0;
  __syncthreads();
  // every wave combines the shares' partials itself (lane i holds share i;
  // S <= 64): the same operations in every wave and every workgroup
  const float4 pv = lane < S ? s_prev[lane] : make_float4(-INFINITY, 0.f, -INFINITY, 0.f);

  if (k == 1) {
    // normalisers from the shares, in share order (every workgroup alike),
    // then the probabilities of the children's tokens
    const MaxSum mp = wave_merge(MaxSum{pv.x, pv.y});
    const MaxSum mq = wave_merge(MaxSum{pv.z, pv.w});
    ni.lp = mp.m + __log2f(mp.s);
    ni.lq = mq.m + __log2f(mq.s);
    for (int j = tid; j < m; j += kPassThreads) {
      const int t = s_ch[j].tok;
      if (t >= u0 * W && t < u1 * W) s_tin[atomicAdd(&s_nin, 1)] = t;
      const float P = prob(s_ch[j].xa, a.c, ni.lp);
      const float Q = prob(s_ch[j].xb, a.c, ni.lq);
      s_ch[j].P = P;
      s_ch[j].Q = Q;
      if (s == 0) {
        ch[j].P = P;
        ch[j].Q = Q;
      }
    }
    __syncthreads();
  } else if (k == 2) {
    ni.snc = wave_sum(lane < S ? pv.y : 0.f);
  }
  if (lead && k <= 2) a.node[g] = ni;

  // (beta_{k-1}, gamma_{k-1})
  Step cur{0.f, 1.f};
  float F = 0.f;
  if (k >= 2) {
    const Step pk = s_st[k - 2];
    const float beta = pk.beta + pk.gamma * inv_mass(ni.snc, s_ch, m, k - 2);
    F = wave_sum(lane < S ? pv.x : 0.f);
    cur = (F > 0.f) ? Step{beta, F} : pk;
  }
  if (lead) st[k - 1] = cur;
  // this share's sum of the state's residual max(0, P - beta Q) / gamma, kept
  // for the walk's bonus draw when a node's last step leaves p unchanged
  if (tid == 0) {
    float* bs = a.bonus + (size_t)g * S + s;
    if (k == 1) {
      const float4 p0 = s_prev[s];  // this share's (max, sum) of the target's exponents
      *bs = (p0.x == -INFINITY) ? 0.f : p0.y * __builtin_amdgcn_exp2f(p0.x - ni.lp);
    } else if (F > 0.f) {
      *bs = s_prev[s].x / F;
    }
  }
  if (tests) {
    // the children's tests, one lane each (a test depends on no earlier
    // outcome, only on the state its child meets); the first that passes
    if (tid == 0) s_st[k - 1] = cur;
    __syncthreads();
    if (wave == 0) {
      int first = -1;
      for (int l0 = 0; l0 < m; l0 += 64) {
        const int l = l0 + lane;
        bool acc = false;
        if (l < m) {
          const ChildInfo c = s_ch[l];
          const Step sl = s_st[l];
          float p, q;
          if (c.dup >= 0) {  // its token was rejected before: q is 0, the residual frozen
            q = 0.f;
            p = fmaxf(0.f, __builtin_fmaf(-s_st[c.dup + 1].beta, c.Q, c.P)) / sl.gamma;
          } else {
            q = c.Q * inv_mass(ni.snc, s_ch, m, l);
            p = fmaxf(0.f, __builtin_fmaf(-sl.beta, c.Q, c.P)) / sl.gamma;
          }
          acc = c.u * q < p;
        }
        const uint64_t bal = __ballot(acc);
        if (bal != 0) {
          first = s_ch[l0 + __ffsll((unsigned long long)bal) - 1].local;
          break;
        }
      }
      if (lane == 0) a.node[g].next = first;
    }
  }

  if (sweep) {
    // share partial of F(beta_k); pass 1 also the draft mass outside the children
    const float beta = cur.beta + cur.gamma * inv_mass(ni.snc, s_ch, m, k - 1);
    const int nin = (k == 1) ? s_nin : 0;
    float f = 0.f, snc = 0.f;
    auto visit = [&](float (&ya)[W], float (&yb)[W], int64_t j, bool valid) {
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
        for (int i = 0; i < nin; ++i) hit |= (s_tin[i] / W == j);
        if (!hit) {
#pragma unroll
          for (int e = 0; e < W; ++e) snc += Q[e];
        } else {
#pragma unroll
          for (int e = 0; e < W; ++e) {
            const int v = (int)(j * W + e);
            bool child = false;
            for (int i = 0; i < nin; ++i) child |= (s_tin[i] == v);
            snc += child ? 0.f : Q[e];
          }
        }
      }
    };
    if (early) {
      visit_batch<W>(ya, yb, u0, u1, visit);
      for_units<T, VEC>(ra, rb, u0 + kPassUnroll * kPassThreads, u1, visit);
    }
    const float2 r = pass_sum2(f, snc, s_red);
    if (tid == 0)
      a.part[(size_t)(k & 1) * a.total_nodes * S + (size_t)g * S + s] = make_float4(r.x, r.y, 0.f, 0.f);
  }
}

// Inclusive prefix sum over the walk block of one value per thread, in thread
// order; returns the thread's inclusive sum, the block total and, in `excl`,
// the previous thread's inclusive sum (0 for thread 0), formed by the same
// additions, so that the runs [excl, incl) tile [0, total) exactly.
__device__ float walk_inclusive_sum(float v, float* s_w, float& total, float& excl) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float x = wave_incl_sum(v);
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
  // lane 0's predecessor is lane 63 of the wave before, whose inclusive sum
  // is that wave's `before` plus its lane-63 value: exactly this `before`
  const float xp = wave_prev(x);
  excl = (lane == 0) ? before : before + xp;
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

// What the walk's first wave hands the block for the bonus draw.
struct BonusPick {
  int32_t node, slot, depth;  // the last node (request-local), its slot, the accepted length
  int32_t sh;                 // the share that holds the draw (-1: none)
  float beta, ig;           // the final state: residual max(0, P - beta Q) * ig
  float t;                  // the draw's offset inside share `sh` (+inf: the last token with mass)
};

template <typename T, bool VEC>
__global__ __launch_bounds__(kWalkThreads) void sampled_walk_kernel(SArgs a, int preload,
                                                                    const T* __restrict__ tl,
                                                                    const T* __restrict__ dl) {
  constexpr int W = VocabUnit<T, VEC>::W;
  extern __shared__ float4 s_dyn4[];
  __shared__ float s_w[kWalkWaves];
  __shared__ int s_lastw[kWalkWaves];
  __shared__ int s_pick, s_fb;
  __shared__ BonusPick s_bp;
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
  const float ub = a.u_bonus[b];  // read now: its latency hides under the table copy
  const int C = a.C, S = a.S;
  const int K = preload ? a.max_nodes : 1;
  ChildInfo* s_chs = reinterpret_cast<ChildInfo*>(s_dyn4);
  Step* s_sts = reinterpret_cast<Step*>(s_chs + (size_t)K * C);
  NodeInfo* s_nis = reinterpret_cast<NodeInfo*>(s_sts + (size_t)K * (C + 1));
  float* s_shs = reinterpret_cast<float*>(s_nis + K);
  float* s_pms = s_shs + (size_t)K * S;
  // copy nodes [first, first + cnt) of the request into slots [0, cnt): the
  // five tables are one run of 32-bit words (the F partials' .x of both
  // parities last), copied kFetchUnroll words a thread at a time with every
  // load issued before the first LDS store, so the copy is one round trip
  auto fetch = [&](int first, int cnt) {
    const size_t g0 = (size_t)lo + first;
    const uint32_t* src_ch = reinterpret_cast<const uint32_t*>(a.child + g0 * C);
    const uint32_t* src_st = reinterpret_cast<const uint32_t*>(a.step + g0 * (C + 1));
    const uint32_t* src_ni = reinterpret_cast<const uint32_t*>(a.node + g0);
    const uint32_t* src_sh = reinterpret_cast<const uint32_t*>(a.bonus + g0 * S);
    const uint32_t* src_pm = reinterpret_cast<const uint32_t*>(a.part + g0 * S);
    const size_t par_words = (size_t)a.total_nodes * S * 4;  // float4 words of one parity
    const int cs = cnt * S;
    const int e_ch = cnt * C * (int)(sizeof(ChildInfo) / 4);
    const int e_st = e_ch + cnt * (C + 1) * (int)(sizeof(Step) / 4);
    const int e_ni = e_st + cnt * (int)(sizeof(NodeInfo) / 4);
    const int e_sh = e_ni + cs;
    const int total = e_sh + 2 * cs;
    uint32_t* dst_ch = reinterpret_cast<uint32_t*>(s_chs);
    uint32_t* dst_st = reinterpret_cast<uint32_t*>(s_sts);
    uint32_t* dst_ni = reinterpret_cast<uint32_t*>(s_nis);
    uint32_t* dst_sh = reinterpret_cast<uint32_t*>(s_shs);
    uint32_t* dst_pm = reinterpret_cast<uint32_t*>(s_pms);
    for (int base = tid; base < total; base += kWalkThreads * kFetchUnroll) {
      uint32_t v[kFetchUnroll];
#pragma unroll
      for (int u = 0; u < kFetchUnroll; ++u) {
        const int i = min(base + u * kWalkThreads, total - 1);  // clamped: every load in bounds
        const uint32_t* src;
        if (i < e_ch) src = src_ch + i;
        else if (i < e_st) src = src_st + (i - e_ch);
        else if (i < e_ni) src = src_ni + (i - e_st);
        else if (i < e_sh) src = src_sh + (i - e_ni);
        else {
          const int r = i - e_sh, par = r >= cs ? 1 : 0;
          src = src_pm + par * par_words + (size_t)(r - par * cs) * 4;
        }
        v[u] = *src;
      }
#pragma unroll
      for (int u = 0; u < kFetchUnroll; ++u) {
        const int i = base + u * kWalkThreads;
        if (i >= total) break;
        uint32_t* dst;
        if (i < e_ch) dst = dst_ch + i;
        else if (i < e_st) dst = dst_st + (i - e_ch);
        else if (i < e_ni) dst = dst_ni + (i - e_st);
        else if (i < e_sh) dst = dst_sh + (i - e_ni);
        else {  // [parity][node][share] -> slot [node][parity][share]
          const int r = i - e_sh, par = r >= cs ? 1 : 0, q = r - par * cs;
          dst = dst_pm + (q / S) * 2 * S + par * S + q % S;
        }
        *dst = v[u];
      }
    }
  };

  // First wave only. The bonus draw at the node in `slot`: the node's last
  // step is fixed from the last pass's share partials of F (as a pass would
  // fix it); the state's share sums are those partials over F or, when the
  // step left p unchanged, the sums the passes kept; a wave scan of the share
  // sums (S <= 64) finds the share that holds u * total.
  auto pick_share = [&](int node, int slot, int depth) {
    const ChildInfo* s_ch = s_chs + (size_t)slot * C;
    const Step* s_st = s_sts + (size_t)slot * (C + 1);
    const float* s_share = s_shs + (size_t)slot * S;
    const NodeInfo ni = s_nis[slot];
    const int m = ni.m;
    const float* s_pm = s_pms + ((size_t)slot * 2 + (m & 1)) * S;  // the last pass's partials
    const float pm = lane < S ? s_pm[lane] : 0.f;
    Step fin{0.f, 1.f};
    float Fm = 0.f;
    if (m >= 1) {
      const Step pk = s_st[m - 1];
      const float beta = pk.beta + pk.gamma * inv_mass(ni.snc, s_ch, m, m - 1);
      Fm = wave_sum(pm);
      fin = (Fm > 0.f) ? Step{beta, Fm} : pk;
    }
    const float si = lane < S ? ((Fm > 0.f) ? pm / Fm : s_share[lane]) : 0.f;
    const float incl = wave_incl_sum(si);
    const float excl = wave_prev(incl);
    const float total = lane_value(incl, 63);
    const float target = ub * total;
    const uint64_t in = __ballot(excl <= target && target < incl);
    const uint64_t mass = __ballot(si > 0.f);
    int sh = -1;
    float t = INFINITY;
    if (in != 0) {
      sh = __ffsll((unsigned long long)in) - 1;
      t = target - lane_value(excl, sh);
    } else if (mass != 0) {  // at or past the total: the last token with mass
      sh = 63 - __clzll((unsigned long long)mass);
    }
    if (lane == 0) s_bp = BonusPick{node, slot, depth, sh, fin.beta, 1.f / fin.gamma, t};
  };

  if (preload) fetch(0, n);
  __syncthreads();
  int node = 0, depth = 0;
  if (preload) {
    // the whole walk in the first wave, from the copied tables
    if (wave == 0) {
      for (;;) {
        const int next = s_nis[node].next;
        if (!(next > node && next < n)) break;
        node = next;
        ++depth;
        if (lane == 0 && depth <= a.max_depth) path[depth] = node;
      }
      pick_share(node, node, depth);
    }
  } else {
    for (;;) {  // one node's tables a level, read by the block
      fetch(node, 1);
      __syncthreads();
      const int next = s_nis[0].next;
      __syncthreads();  // every thread has read slot 0 before it is refilled
      if (!(next > node && next < n)) break;
      node = next;
      ++depth;
      if (tid == 0 && depth <= a.max_depth) path[depth] = node;
    }
    if (wave == 0) pick_share(node, 0, depth);
  }
  if (tid == 0) {
    s_pick = -1;
    s_fb = -1;
  }
  __syncthreads();
  const BonusPick bp = s_bp;
  const int g = lo + bp.node;
  int pick = -1;
  if (bp.sh >= 0) {
    const NodeInfo ni = s_nis[bp.slot];
    const int64_t units = a.vocab / W;
    int64_t u0, u1;
    share(units, S, bp.sh, u0, u1);
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
        pv[e] = fmaxf(0.f, __builtin_fmaf(-bp.beta, Q, P)) * bp.ig;
      }
    };
    // per-thread runs in token order; the thread's first kWalkCache units
    // stay in registers for the rescan (a clamped load of unit 0 stands in
    // past the run's end, then zeroed)
    float pc[kWalkCache][W];
    float run = 0.f;
#pragma unroll
    for (int c = 0; c < kWalkCache; ++c) {
      const bool ok = j0 + c < j1;
      p_at(ok ? j0 + c : 0, pc[c]);
#pragma unroll
      for (int e = 0; e < W; ++e) {
        pc[c][e] = ok ? pc[c][e] : 0.f;
        run += pc[c][e];
      }
    }
    for (int64_t j = j0 + kWalkCache; j < j1; ++j) {
      float pv[W];
      p_at(j, pv);
#pragma unroll
      for (int e = 0; e < W; ++e) run += pv[e];
    }
    const uint64_t has = __ballot(run > 0.f);
    if (lane == 0) s_lastw[wave] = has ? wave * 64 + 63 - __clzll((unsigned long long)has) : -1;
    float stotal, excl;
    const float incl = walk_inclusive_sum(run, s_w, stotal, excl);
    if (excl <= bp.t && bp.t < incl) {
      // the same additions in the same order as the run's sum
      float r = excl;
      int pk = -1, last = -1;
      auto visit = [&](int64_t j, const float (&pv)[W]) {
#pragma unroll
        for (int e = 0; e < W; ++e) {
          if (pk >= 0) break;
          if (pv[e] > 0.f) last = (int)(j * W + e);
          r += pv[e];
          if (r > bp.t && pv[e] > 0.f) pk = (int)(j * W + e);
        }
      };
#pragma unroll
      for (int c = 0; c < kWalkCache; ++c)
        if (j0 + c < j1 && pk < 0) visit(j0 + c, pc[c]);
      for (int64_t j = j0 + kWalkCache; j < j1 && pk < 0; ++j) {
        float pv[W];
        p_at(j, pv);
        visit(j, pv);
      }
      s_pick = pk >= 0 ? pk : last;
    }
    __syncthreads();
    pick = s_pick;  // not written again: the fallback has its own slot
    if (pick < 0) {  // (uniform)
      // the draw fell outside every run (+inf, or rounding): the last token
      // with mass, in the last run that has some
      int lt = -1;
#pragma unroll
      for (int w = 0; w < kWalkWaves; ++w) lt = max(lt, s_lastw[w]);
      if (tid == lt) {
        int last = -1;
#pragma unroll
        for (int c = 0; c < kWalkCache; ++c)
#pragma unroll
          for (int e = 0; e < W; ++e)
            if (pc[c][e] > 0.f) last = (int)((j0 + c) * W + e);
        for (int64_t j = j0 + kWalkCache; j < j1; ++j) {
          float pv[W];
          p_at(j, pv);
#pragma unroll
          for (int e = 0; e < W; ++e)
            if (pv[e] > 0.f) last = (int)(j * W + e);
        }
        s_fb = last;
      }
      __syncthreads();
      pick = s_fb;
    }
  }
  if (tid == 0) {
    a.bonus_tok[b] = pick;
    a.accept_len[b] = bp.depth;
  }
}

template <typename T, bool VEC>
hipError_t run_sampled(const SArgs& a, const void* tl, const void* dl, hipStream_t stream) {
  const T* t = static_cast<const T*>(tl);
  const T* d = static_cast<const T*>(dl);
  if (a.total_nodes > 0) {
    const dim3 grid(a.total_nodes, a.S);
    // one more workgroup a row in pass 0 lists the node's children
    hipLaunchKernelGGL((sampled_prep_kernel<T, VEC>), dim3(a.total_nodes, a.S + 1), dim3(kPassThreads), 0,
                       stream, a, t, d);
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
