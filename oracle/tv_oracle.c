/*
 * tv_oracle.c -- plain, slow CPU oracle for tree-verification attention.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this library. It shares no source, header, table or
 * helper with the GPU library, and nothing in the GPU library calls it.
 *
 * Everything here is the definition written out, one row / one node at a time,
 * in double precision (inputs are float32 arrays that hold exactly the values
 * the GPU receives; bf16 inputs are upcast exactly before they get here).
 * One exception: the D-cut scores decide an integer (which positions are
 * kept), so they are formed in fp32 as [D-cut] technical summary §2 defines
 * them -- the product of a block's confidences up to the position, taken left
 * to right along the block -- and the decision is taken on those values.
 *
 * Sources (the four web pages on candidate-tree speculative decoding):
 *   [Graft]      Graft, arXiv:2605.20104 (163.com article "浙江大学、阿里巴巴联手破解AI推理瓶颈")
 *   [BlockPilot] BlockPilot, arXiv:2606.31315 (zhengruan.com article on dynamic block size)
 *   [D-cut]      "D-cut: Adaptive Verification Depth Pruning for Batched Speculative Decoding"
 *                (gist.science summary of paper 2607.14647)
 *   [SpecOPD]    SpecOPD, arXiv:2611.02846 (lewlh.github.io blog post)
 *
 * Conventions shared with every caller (they are the library's documented data
 * layout, restated here, not included from anywhere):
 *   - request b owns flattened nodes [cu_nodes[b], cu_nodes[b+1]); parent[] holds
 *     request-local indices, the root is local node 0 with parent -1;
 *   - the K/V of local tree node j of request b sits at logical cache position
 *     prefix_len[b] + j, right after that request's prefix;
 *   - logical position p of request b lives in page block_table[b*max_pages + p/page_size],
 *     slot p % page_size; the K cache is laid out [page][kv_head][slot][head_dim]
 *     and the V cache [page][kv_head][head_dim][slot] (d-major pages);
 *   - query head h reads kv head h / (Hq / Hkv) (contiguous GQA groups);
 *   - q and out are [node][q_head][head_dim], lse is [node][q_head].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Tree topology and the ancestor mask.                                      */
/* [Graft] §二 third gear: the hybrid tree is flattened into a sequence and   */
/* tree positions plus the tree mask are rebuilt before one parallel pass.   */
/* [SpecOPD] §02 attention table, full-attention row: the mask is the        */
/* topological ancestor relation -- a node sees its own ancestor path and    */
/* the shared trunk, never a sibling branch or a later trunk token.          */
/* ------------------------------------------------------------------------ */

/* Validate one request's parent array: the root is node 0 (parent -1) and
 * every other node names an earlier node as parent, so the walk to the root
 * always terminates. Returns 0 if valid, 1 otherwise. */
static int orc_tree_invalid(const int32_t* par, int n) {
  if (n <= 0) return 1;
  if (par[0] != -1) return 1;
  for (int i = 1; i < n; ++i)
    if (par[i] < 0 || par[i] >= i) return 1;
  return 0;
}

/* BITS form: bit j of node i's mask is set iff j is i itself or one of its
 * ancestors; depth(i) = number of ancestors excluding i. A request with an
 * invalid parent array gets err[b] = 1, all-zero masks and depth -1. */
void orc_mask_bits(const int32_t* parent, const int32_t* cu_nodes, int32_t batch,
                   int32_t words, uint64_t* bits, int32_t* depth, int32_t* err) {
  for (int b = 0; b < batch; ++b) {
    int n0 = cu_nodes[b], n = cu_nodes[b + 1] - cu_nodes[b];
    const int32_t* par = parent + n0;
    int bad = orc_tree_invalid(par, n) || n > 64 * words;
    err[b] = bad;
    for (int i = 0; i < n; ++i) {
      uint64_t* row = bits + (size_t)(n0 + i) * words;
      for (int w = 0; w < words; ++w) row[w] = 0;
      depth[n0 + i] = -1;
      if (bad) continue;
      int d = -1;
      for (int j = i; j != -1; j = par[j]) {  /* walk up to the root */
        row[j / 64] |= (uint64_t)1 << (j % 64);
        ++d;
      }
      depth[n0 + i] = d;
    }
  }
}

/* ANCHOR form for trunk-plus-chain-branch trees ([SpecOPD] §02 anchor
 * sampling and proposal tree: branches hang off trunk anchor positions).
 * Trunk length T = largest t with parent[k] = k-1 for every 1 <= k < t.
 * Trunk node i: anchor_pos = i, branch_depth = 0.
 * Node i >= T either starts a branch (parent[i] < T: anchor = parent[i],
 * branch_depth = 1) or continues the previous node's branch
 * (parent[i] = i-1 >= T: same anchor, branch_depth + 1). Anything else
 * cannot be written in this form: err[b] = 2 (err[b] = 1 for an invalid tree).
 * Tree key j is then visible to node i iff j <= anchor_pos[i] or
 * i - branch_depth[i] < j <= i. */
void orc_mask_anchor(const int32_t* parent, const int32_t* cu_nodes, int32_t batch,
                     int32_t* anchor_pos, int32_t* branch_depth, int32_t* depth,
                     int32_t* err) {
  for (int b = 0; b < batch; ++b) {
    int n0 = cu_nodes[b], n = cu_nodes[b + 1] - cu_nodes[b];
    const int32_t* par = parent + n0;
    int e = orc_tree_invalid(par, n) ? 1 : 0;
    int T = 1;
    if (!e)
      while (T < n && par[T] == T - 1) ++T;
    for (int i = 0; i < n && !e; ++i) {
      if (i < T) {
        anchor_pos[n0 + i] = i;
        branch_depth[n0 + i] = 0;
        depth[n0 + i] = i;
      } else if (par[i] < T) {
        anchor_pos[n0 + i] = par[i];
        branch_depth[n0 + i] = 1;
        depth[n0 + i] = par[i] + 1;
      } else if (par[i] == i - 1) {
        anchor_pos[n0 + i] = anchor_pos[n0 + i - 1];
        branch_depth[n0 + i] = branch_depth[n0 + i - 1] + 1;
        depth[n0 + i] = depth[n0 + i - 1] + 1;
      } else {
        e = 2;
      }
    }
    err[b] = e;
    if (e)
      for (int i = 0; i < n; ++i) {
        anchor_pos[n0 + i] = -1;
        branch_depth[n0 + i] = 0;
        depth[n0 + i] = -1;
      }
  }
}

/* ------------------------------------------------------------------------ */
/* Attention of one tree node against the shared prefix plus its ancestors. */
/* [Graft] §二 third gear (one verification pass over the flattened tree);  */
/* [SpecOPD] §02 proposal tree (the target shares the trunk KV cache and    */
/* scores every branch under the tree mask); [D-cut] technical summary §2,  */
/* pipeline (the packed batch is verified by the target in one pass).       */
/* ------------------------------------------------------------------------ */

typedef struct {
  const float* q;          /* [N_tot][Hq][D] */
  const float* k_cache;    /* [num_pages][Hkv][page][D] */
  const float* v_cache;    /* [num_pages][Hkv][D][page] */
  const int32_t* block_table; /* [batch][max_pages] */
  const int32_t* prefix_len;  /* [batch] */
  const int32_t* cu_nodes;    /* [batch+1] */
  const int32_t* parent;      /* [N_tot] local */
  int32_t batch, max_pages, hq, hkv, d, page;
  double scale;
} orc_attn_args;

static const float* orc_k_row(const orc_attn_args* a, int b, int pos, int g) {
  int page = a->block_table[(size_t)b * a->max_pages + pos / a->page];
  int slot = pos % a->page;
  return a->k_cache + (((size_t)page * a->hkv + g) * a->page + slot) * a->d;
}

static double orc_v_at(const orc_attn_args* a, int b, int pos, int g, int t) {
  int page = a->block_table[(size_t)b * a->max_pages + pos / a->page];
  int slot = pos % a->page;
  return (double)a->v_cache[(((size_t)page * a->hkv + g) * a->d + t) * a->page + slot];
}

static double orc_dot(const float* x, const float* y, int d) {
  double s = 0.0;
  for (int t = 0; t < d; ++t) s += (double)x[t] * (double)y[t];
  return s;
}

/* Masked-dense formulation: score every key position of the request,
 * prefix and tree alike, and drop the tree keys that are not ancestors-or-self
 * of the querying node (visibility from the parent walk). Softmax is the
 * two-pass textbook one: m = max score, w = exp(s - m), o = sum w v / sum w,
 * lse = m + ln(sum w). */
static void orc_attn_row_dense(const orc_attn_args* a, int b, int i, int h,
                               double* out, double* lse, double* scores,
                               uint8_t* vis) {
  int n0 = a->cu_nodes[b], n = a->cu_nodes[b + 1] - n0, P = a->prefix_len[b];
  int g = h / (a->hq / a->hkv);
  const float* qrow = a->q + ((size_t)(n0 + i) * a->hq + h) * a->d;
  const int32_t* par = a->parent + n0;
  for (int j = 0; j < n; ++j) vis[j] = 0;
  for (int j = i; j != -1; j = par[j]) vis[j] = 1;
  int nk = P + n;
  double m = -INFINITY;
  for (int p = 0; p < nk; ++p) {
    int visible = p < P || vis[p - P];
    if (!visible) { scores[p] = -INFINITY; continue; }
    scores[p] = a->scale * orc_dot(qrow, orc_k_row(a, b, p, g), a->d);
    if (scores[p] > m) m = scores[p];
  }
  double l = 0.0;
  for (int t = 0; t < a->d; ++t) out[t] = 0.0;
  for (int p = 0; p < nk; ++p) {
    if (scores[p] == -INFINITY) continue;
    double w = exp(scores[p] - m);
    l += w;
    for (int t = 0; t < a->d; ++t) out[t] += w * orc_v_at(a, b, p, g, t);
  }
  for (int t = 0; t < a->d; ++t) out[t] /= l;
  *lse = m + log(l);
}

/* Path-gather formulation: collect the key list explicitly -- prefix
 * positions 0..P-1, then the root-to-node path in root-first order -- and run
 * unmasked softmax attention over exactly that list. */
static void orc_attn_row_path(const orc_attn_args* a, int b, int i, int h,
                              double* out, double* lse, int32_t* keys,
                              double* scores) {
  int n0 = a->cu_nodes[b], P = a->prefix_len[b];
  int g = h / (a->hq / a->hkv);
  const float* qrow = a->q + ((size_t)(n0 + i) * a->hq + h) * a->d;
  const int32_t* par = a->parent + n0;
  int plen = 0;
  for (int j = i; j != -1; j = par[j]) ++plen;
  int nk = P + plen;
  for (int p = 0; p < P; ++p) keys[p] = p;
  int pos = nk - 1;
  for (int j = i; j != -1; j = par[j]) keys[pos--] = P + j;
  double m = -INFINITY;
  for (int t = 0; t < nk; ++t) {
    scores[t] = a->scale * orc_dot(qrow, orc_k_row(a, b, keys[t], g), a->d);
    if (scores[t] > m) m = scores[t];
  }
  double l = 0.0;
  for (int t = 0; t < a->d; ++t) out[t] = 0.0;
  for (int t = 0; t < nk; ++t) {
    double w = exp(scores[t] - m);
    l += w;
    for (int e = 0; e < a->d; ++e) out[e] += w * orc_v_at(a, b, keys[t], g, e);
  }
  for (int e = 0; e < a->d; ++e) out[e] /= l;
  *lse = m + log(l);
}

/* Row selection: rows == NULL means every (node, head) of every request, in
 * [node][head] order; otherwise rows holds n_rows (global node, head) pairs
 * and out / lse are [n_rows][D] / [n_rows]. Returns 0, or -1 on bad input. */
static int orc_attn_run(const orc_attn_args* a, int formulation,
                        const int32_t* rows, int32_t n_rows, double* out,
                        double* lse) {
  if (a->hkv <= 0 || a->hq % a->hkv) return -1;
  int n_tot = a->cu_nodes[a->batch];
  int max_keys = 0;
  for (int b = 0; b < a->batch; ++b) {
    int nk = a->prefix_len[b] + a->cu_nodes[b + 1] - a->cu_nodes[b];
    if (nk > max_keys) max_keys = nk;
  }
  double* scores = (double*)malloc(sizeof(double) * (max_keys + 1));
  int32_t* keys = (int32_t*)malloc(sizeof(int32_t) * (max_keys + 1));
  uint8_t* vis = (uint8_t*)malloc(max_keys + 1);
  if (!scores || !keys || !vis) { free(scores); free(keys); free(vis); return -1; }
  int total = rows ? n_rows : n_tot * a->hq;
  for (int r = 0; r < total; ++r) {
    int node = rows ? rows[2 * r] : r / a->hq;
    int h = rows ? rows[2 * r + 1] : r % a->hq;
    int b = 0;
    while (b + 1 <= a->batch && a->cu_nodes[b + 1] <= node) ++b;
    int i = node - a->cu_nodes[b];
    if (formulation == 0)
      orc_attn_row_dense(a, b, i, h, out + (size_t)r * a->d, lse + r, scores, vis);
    else
      orc_attn_row_path(a, b, i, h, out + (size_t)r * a->d, lse + r, keys, scores);
  }
  free(scores); free(keys); free(vis);
  return 0;
}

int orc_tree_attn(int32_t formulation, const float* q, const float* k_cache,
                  const float* v_cache, const int32_t* block_table, int32_t max_pages,
                  const int32_t* prefix_len, const int32_t* cu_nodes,
                  const int32_t* parent, int32_t batch, int32_t hq, int32_t hkv,
                  int32_t d, int32_t page_size, double scale, const int32_t* rows,
                  int32_t n_rows, double* out, double* lse) {
  orc_attn_args a = {q, k_cache, v_cache, block_table, prefix_len, cu_nodes, parent,
                     batch, max_pages, hq, hkv, d, page_size, scale};
  return orc_attn_run(&a, formulation, rows, n_rows, out, lse);
}

/* ------------------------------------------------------------------------ */
/* Greedy acceptance.                                                        */
/* [SpecOPD] §01: tokens that agree with the target are accepted, the draft  */
/* is cut at the first divergence and everything after it is discarded.      */
/* [Graft] introduction: the target checks the whole tree at once and keeps  */
/* the path that goes furthest; §二 third gear: draft and retrieved nodes    */
/* face the same rule.                                                       */
/* Node i > 0 matches iff draft_tok[i] equals the target's greedy token at   */
/* its parent, target_tok[parent[i]]. A node is accepted iff every node on   */
/* its root path matches (the root always is). The answer is the accepted    */
/* node of greatest depth, ties to the smallest local index; accept_len is   */
/* its depth, path lists root..best (then -1), bonus = target_tok[best].     */
/* Brute force: every node's whole root path is checked edge by edge.        */
/* ------------------------------------------------------------------------ */
void orc_accept(const int32_t* parent, const int32_t* draft_tok,
                const int32_t* target_tok, const int32_t* cu_nodes, int32_t batch,
                int32_t max_depth, int32_t* accept_len, int32_t* path,
                int32_t* bonus_tok) {
  for (int b = 0; b < batch; ++b) {
    int n0 = cu_nodes[b], n = cu_nodes[b + 1] - n0;
    const int32_t* par = parent + n0;
    const int32_t* dr = draft_tok + n0;
    const int32_t* tg = target_tok + n0;
    int32_t* prow = path + (size_t)b * (max_depth + 1);
    for (int t = 0; t <= max_depth; ++t) prow[t] = -1;
    if (n <= 0) {
      /* no tree, so no root: nothing accepted, no path, no bonus token */
      accept_len[b] = 0;
      bonus_tok[b] = -1;
      continue;
    }
    int best = 0, best_depth = 0;
    for (int v = 0; v < n; ++v) {
      int ok = 1, dep = 0;
      for (int j = v; par[j] != -1; j = par[j]) {
        if (dr[j] != tg[par[j]]) ok = 0;
        ++dep;
      }
      if (ok && dep > best_depth) { best = v; best_depth = dep; }
    }
    accept_len[b] = best_depth;
    bonus_tok[b] = tg[best];
    for (int j = best, t = best_depth; j != -1; j = par[j], --t)
      if (t <= max_depth) prow[t] = j;
  }
}

/* ------------------------------------------------------------------------ */
/* D-cut verification budget.                                                */
/* [D-cut] technical summary §2, cross-request pruning and the pipeline's    */
/* scoring & ranking and packing steps: each draft position is scored by the */
/* product of the draft confidences up to it (the chance the block survives  */
/* to that depth); all positions of the batch are ranked together, the best  */
/* ones are verified, and since scores only fall along a block each request  */
/* keeps a prefix, packed densely. Position 0 of every request (its current  */
/* token) is always verified; the other budget - batch slots are ranked.     */
/* Ties: smaller request, then smaller position. Returns 1 on a bad budget.  */
/* ------------------------------------------------------------------------ */
typedef struct {
  float s;
  int32_t b, k;
} orc_dcut_pos;

static int orc_dcut_cmp(const void* x, const void* y) {
  const orc_dcut_pos* a = (const orc_dcut_pos*)x;
  const orc_dcut_pos* c = (const orc_dcut_pos*)y;
  if (a->s != c->s) return a->s > c->s ? -1 : 1;
  if (a->b != c->b) return a->b < c->b ? -1 : 1;
  return a->k < c->k ? -1 : (a->k > c->k);
}

int orc_dcut_select(const float* conf, const int32_t* tokens, int32_t batch,
                    int32_t draft_len, int32_t budget, int32_t* n_keep, int32_t* cu_nodes,
                    int32_t* parent, int32_t* packed_tokens) {
  const int D = draft_len;
  if (batch < 1 || D < 1 || budget < batch || budget > batch * (D + 1)) return 1;
  orc_dcut_pos* pos = (orc_dcut_pos*)malloc(sizeof(orc_dcut_pos) * (size_t)batch * D);
  for (int b = 0; b < batch; ++b) {
    float s = 1.0f;                       /* position 0: the empty product */
    for (int k = 1; k <= D; ++k) {
      float c = conf[(size_t)b * D + (k - 1)];
      if (!(c > 0.0f)) c = 0.0f;          /* a probability: NaN and negatives -> 0 */
      if (c > 1.0f) c = 1.0f;
      s = s * c;                          /* fp32, left to right along the block */
      orc_dcut_pos* e = &pos[(size_t)b * D + (k - 1)];
      e->s = s; e->b = b; e->k = k;
    }
  }
  qsort(pos, (size_t)batch * D, sizeof(orc_dcut_pos), orc_dcut_cmp);
  for (int b = 0; b < batch; ++b) n_keep[b] = 1;
  for (int r = 0; r < budget - batch; ++r) n_keep[pos[r].b] += 1;
  free(pos);
  int off = 0;
  for (int b = 0; b < batch; ++b) {
    cu_nodes[b] = off;
    for (int k = 0; k < n_keep[b]; ++k) {
      parent[off + k] = k - 1;
      packed_tokens[off + k] = tokens[(size_t)b * (D + 1) + k];
    }
    off += n_keep[b];
  }
  cu_nodes[batch] = off;
  return 0;
}
