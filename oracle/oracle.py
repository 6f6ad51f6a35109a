"""ctypes front end of the plain-C oracle (``tv_oracle.c``) -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s
CPU-baseline leg may import this module.  It shares no code with the HIP
library: it compiles its own C source with gcc and hands it numpy arrays.

All floating point in the C code is double precision; float inputs arrive as
float32 arrays holding exactly the values the GPU gets (bf16 values upcast).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point the front end at a deliberately mutated build of the same
# source (to show the pins catch planted mistakes); nothing else sets this.
_LIB_OVERRIDE = os.environ.get("TV_ORACLE_LIB")
_lib = None


def build_oracle(force: bool = True) -> str:
    """Compile ``tv_oracle.c`` into ``liboracle.so`` (plain gcc, IEEE math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Werror",
             "-fno-fast-math", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build_oracle(force=True)
            lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int32
        lib.orc_mask_bits.argtypes = [P, P, I, I, P, P, P]
        lib.orc_mask_bits.restype = None
        lib.orc_mask_anchor.argtypes = [P, P, I, P, P, P, P]
        lib.orc_mask_anchor.restype = None
        lib.orc_tree_attn.argtypes = [I, P, P, P, P, I, P, P, P, I, I, I, I, I,
                                      ctypes.c_double, P, I, P, P]
        lib.orc_tree_attn.restype = ctypes.c_int
        lib.orc_accept.argtypes = [P, P, P, P, I, I, P, P, P]
        lib.orc_accept.restype = None
        lib.orc_dcut_select.argtypes = [P, P, I, I, I, P, P, P, P]
        lib.orc_dcut_select.restype = ctypes.c_int
        _lib = lib
    return _lib


def _np(x, dtype):
    """torch tensor or array-like -> C-contiguous numpy array of ``dtype``."""
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if str(x.dtype) == "torch.bfloat16":
            x = x.float()
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x), dtype=dtype)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def mask_bits(parent, cu_nodes, words: int):
    """Ancestor bitmask per node: returns (bits uint64 [N, words], depth int32 [N], err int32 [B])."""
    lib = _load()
    parent = _np(parent, np.int32)
    cu = _np(cu_nodes, np.int32)
    batch = len(cu) - 1
    n = int(cu[-1])
    bits = np.zeros((n, words), np.uint64)
    depth = np.zeros(n, np.int32)
    err = np.zeros(batch, np.int32)
    lib.orc_mask_bits(_p(parent), _p(cu), batch, words, _p(bits), _p(depth), _p(err))
    return bits, depth, err


def mask_anchor(parent, cu_nodes):
    """Anchor form: returns (anchor_pos, branch_depth, depth, err), int32."""
    lib = _load()
    parent = _np(parent, np.int32)
    cu = _np(cu_nodes, np.int32)
    batch = len(cu) - 1
    n = int(cu[-1])
    ap = np.zeros(n, np.int32)
    bd = np.zeros(n, np.int32)
    depth = np.zeros(n, np.int32)
    err = np.zeros(batch, np.int32)
    lib.orc_mask_anchor(_p(parent), _p(cu), batch, _p(ap), _p(bd), _p(depth), _p(err))
    return ap, bd, depth, err


def tree_attn(q, k_cache, v_cache, block_table, prefix_len, cu_nodes, parent,
              num_q_heads: int, num_kv_heads: int, scale: float, rows=None,
              formulation: str = "dense"):
    """Attention of every (node, head) row -- or of the listed ``rows`` -- in fp64.

    ``q`` is [N, Hq, D]; the K cache is [pages, Hkv, page_size, D] and the V
    cache [pages, Hkv, D, page_size] (d-major pages); ``rows`` is an
    optional int array [R, 2] of (global node, q head).  Returns
    (out float64 [N, Hq, D] or [R, D], lse float64 [N, Hq] or [R]).
    """
    lib = _load()
    q = _np(q, np.float32)
    kc = _np(k_cache, np.float32)
    vc = _np(v_cache, np.float32)
    bt = _np(block_table, np.int32)
    pl = _np(prefix_len, np.int32)
    cu = _np(cu_nodes, np.int32)
    par = _np(parent, np.int32)
    batch = len(cu) - 1
    n = int(cu[-1])
    d = q.shape[-1]
    page = kc.shape[2]
    assert q.shape == (n, num_q_heads, d)
    assert kc.shape[1] == num_kv_heads and kc.shape[3] == d
    assert vc.shape == (kc.shape[0], num_kv_heads, d, page)
    assert bt.ndim == 2 and bt.shape[0] == batch
    if rows is None:
        out = np.zeros((n, num_q_heads, d), np.float64)
        lse = np.zeros((n, num_q_heads), np.float64)
        rp, nr = None, 0
    else:
        rows = _np(rows, np.int32).reshape(-1, 2)
        out = np.zeros((rows.shape[0], d), np.float64)
        lse = np.zeros(rows.shape[0], np.float64)
        rp, nr = _p(rows), rows.shape[0]
    form = {"dense": 0, "path": 1}[formulation]
    rc = lib.orc_tree_attn(form, _p(q), _p(kc), _p(vc), _p(bt), bt.shape[1], _p(pl),
                           _p(cu), _p(par), batch, num_q_heads, num_kv_heads, d, page,
                           float(scale), rp, nr, _p(out), _p(lse))
    if rc != 0:
        raise ValueError("oracle rejected the attention arguments")
    return out, lse


def accept(parent, draft_tok, target_tok, cu_nodes, max_depth: int):
    """Greedy acceptance: returns (accept_len [B], path [B, max_depth+1], bonus [B])."""
    lib = _load()
    par = _np(parent, np.int32)
    dr = _np(draft_tok, np.int32)
    tg = _np(target_tok, np.int32)
    cu = _np(cu_nodes, np.int32)
    batch = len(cu) - 1
    al = np.zeros(batch, np.int32)
    path = np.zeros((batch, max_depth + 1), np.int32)
    bonus = np.zeros(batch, np.int32)
    lib.orc_accept(_p(par), _p(dr), _p(tg), _p(cu), batch, max_depth, _p(al), _p(path),
                   _p(bonus))
    return al, path, bonus


def dcut_select(conf, tokens, budget: int):
    """D-cut selection: ``conf`` float32 [B, D], ``tokens`` int32 [B, D+1].

    Returns (n_keep [B], cu_nodes [B+1], parent [budget], packed_tokens [budget]),
    int32; raises ValueError on a budget outside [B, B*(D+1)].
    """
    lib = _load()
    conf = _np(conf, np.float32)
    tok = _np(tokens, np.int32)
    batch, d = conf.shape
    assert tok.shape == (batch, d + 1)
    n_keep = np.zeros(batch, np.int32)
    cu = np.zeros(batch + 1, np.int32)
    par = np.zeros(max(budget, 1), np.int32)
    ptok = np.zeros(max(budget, 1), np.int32)
    if lib.orc_dcut_select(_p(conf), _p(tok), batch, d, int(budget), _p(n_keep), _p(cu),
                           _p(par), _p(ptok)) != 0:
        raise ValueError("budget must lie in [batch, batch * (draft_len + 1)]")
    return n_keep, cu, par[:budget], ptok[:budget]


def e2e_tv_stats(target_logits, draft_logits, cu_branches, temperature: float = 1.0):
    """SpecOPD E2E-TV statistics, in float64 with numpy (no C needed).

    SpecOPD §02 stage 4 and §03.2: the chance that exact rejection sampling
    accepts the drafted token at a node is the overlap of the target's and
    the draft's next-token distributions, alpha = sum_v min(p_v, q_v)
    = 1 - TV(p, q); a branch's tokens are accepted consecutively, so the
    chance of accepting its first k tokens is the product of their alphas,
    and the expected run of accepted tokens is the sum of those products.

    ``target_logits``, ``draft_logits``: [N, V] (any float dtype; bf16 tensors
    are upcast exactly); p = softmax(target / T), q = softmax(draft / T).
    ``cu_branches`` [B+1]: branch b is the chain of nodes [cu[b], cu[b+1]).
    Returns (alpha [N], prefix_prob [N], expected_len [B]), float64.
    """
    t = _np(target_logits, np.float64) / float(temperature)
    d = _np(draft_logits, np.float64) / float(temperature)
    cu = _np(cu_branches, np.int64)
    n = t.shape[0]
    alpha = np.zeros(n, np.float64)
    for i in range(n):
        p = np.exp(t[i] - t[i].max())
        p /= p.sum()
        q = np.exp(d[i] - d[i].max())
        q /= q.sum()
        alpha[i] = np.minimum(p, q).sum()
    prefix = np.zeros(n, np.float64)
    expected = np.zeros(len(cu) - 1, np.float64)
    for b in range(len(cu) - 1):
        run = 1.0
        for i in range(int(cu[b]), int(cu[b + 1])):
            run *= alpha[i]
            prefix[i] = run
            expected[b] += run
    return alpha, prefix, expected


def graft_retrieve(adj, root_tokens, tmpl_parent, tmpl_rank):
    """Graft retrieval (Graft §二, second gear): expand a template from each
    request's current token through the adjacency table.

    ``adj`` int32 [V, k]: row t = the k most likely successors of token t
    (-1 = empty). Template node j hangs under template node tmpl_parent[j]
    (-1 = the current token) and takes that token's tmpl_rank[j]-th
    successor; a node whose parent has no token, or whose table entry is
    empty or out of range, has no token (-1). Returns int32 [B, T].
    """
    adj = _np(adj, np.int32)
    roots = _np(root_tokens, np.int32)
    par = [int(x) for x in tmpl_parent]
    rank = [int(x) for x in tmpl_rank]
    v, k = adj.shape
    out = np.full((len(roots), len(par)), -1, np.int32)
    for b, root in enumerate(roots):
        for j in range(len(par)):
            src = int(root) if par[j] < 0 else int(out[b, par[j]])
            if 0 <= src < v and 0 <= rank[j] < k:
                t = int(adj[src, rank[j]])
                out[b, j] = t if 0 <= t < v else -1
    return out


def graft_update(adj, target_logits, node_tokens):
    """Graft online update (Graft §二 third gear, §五): after verification the
    row of every verified node's token is replaced by the target's k most
    likely next tokens at that node (larger logit first, ties to the smaller
    token id); when several nodes carry the same token the later node's row
    is kept. Tokens outside [0, V) update nothing; NaN logits rank as -inf.
    Returns the new table."""
    adj = _np(adj, np.int32).copy()
    logits = _np(target_logits, np.float32)
    tok = _np(node_tokens, np.int32)
    v, k = adj.shape
    ids = np.arange(v)
    for i in range(len(tok)):              # in node order: a later node overwrites
        t = int(tok[i])
        if not (0 <= t < v):
            continue
        key = np.where(np.isnan(logits[i]), -np.inf, logits[i]).astype(np.float64)
        order = np.lexsort((ids, -key))     # by logit descending, then token id
        adj[t] = order[:k]
    return adj


def _dist(logits_row, temperature):
    """softmax(logits / T) in float64, NaN logits as -inf."""
    y = np.where(np.isnan(logits_row), -np.inf, logits_row).astype(np.float64) / temperature
    e = np.exp(y - y.max())
    return e / e.sum()


def accept_sampled(parent, draft_tok, cu_nodes, target_logits, draft_logits, temperature,
                   u_accept, u_bonus, max_depth: int):
    """Stochastic tree verification, in float64 with numpy (no C needed).

    The pages verify at temperature 1 (BlockPilot §五, D-cut §4) and fix the
    one-token rule (SpecOPD §03.2: exact rejection sampling accepts a drafted
    token with the overlap of the two distributions) but not the rule for a
    tree. This follows recursive rejection sampling (Jeon et al. 2024,
    "Recursive Speculative Decoding"; SpecInfer's multi-step speculative
    sampling extended to siblings drawn without replacement):

    at the current node (starting at the root), with p = softmax(target / T)
    and q = softmax(draft / T) there, its children are tried in index order.
    Child c with token x is accepted iff u_accept[c] * q(x) < p(x) (i.e. with
    probability min(1, p(x) / q(x)); q(x) = 0 < p(x) accepts, p(x) = 0
    rejects); on acceptance the walk moves to c. On rejection p becomes the
    normalised residual max(0, p - q) (unchanged if that is all zero) and
    x's mass is removed from q, which is renormalised. A child whose token
    is outside [0, V) is skipped. When no child is accepted, the bonus token
    is drawn from the current p by inverse transform in token order: the
    smallest v with cumsum(p)[v] > u_bonus[b] * sum(p).

    ``target_logits``, ``draft_logits``: [N, V], row i = the next-token
    logits after node i (the draft's row is the distribution node i's
    children were drawn from); ``u_accept`` [N], ``u_bonus`` [B] in [0, 1).
    Returns (accept_len [B], path [B, max_depth+1] local ids root..last
    accepted then -1, bonus [B], margin [B]); an empty request gives 0, a
    path of -1 and bonus -1. margin is the smallest distance
    of any decision from its boundary (|u q(x) - p(x)| for a child test, the
    distance of u_bonus * sum(p) to the nearest cumulative boundary for the
    bonus), so a test can tell a rounding-level tie from a disagreement.
    """
    par = _np(parent, np.int64)
    tok = _np(draft_tok, np.int64)
    cu = _np(cu_nodes, np.int64)
    tl = _np(target_logits, np.float64)
    dl = _np(draft_logits, np.float64)
    ua = _np(u_accept, np.float64)
    ub = _np(u_bonus, np.float64)
    T = float(temperature)
    v = tl.shape[1]
    batch = len(cu) - 1
    al = np.zeros(batch, np.int32)
    path = np.full((batch, max_depth + 1), -1, np.int32)
    bonus = np.zeros(batch, np.int32)
    margin = np.full(batch, np.inf)
    for b in range(batch):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi <= lo:                             # an empty request: nothing to verify
            bonus[b] = -1
            continue
        node, depth = 0, 0
        path[b, 0] = 0
        while True:
            p = _dist(tl[lo + node], T)
            q = _dist(dl[lo + node], T)
            nxt = None
            for c in range(node + 1, hi - lo):
                if par[lo + c] != node:
                    continue
                x = int(tok[lo + c])
                if not 0 <= x < v:
                    continue
                lhs, rhs = ua[lo + c] * q[x], p[x]
                margin[b] = min(margin[b], abs(lhs - rhs))
                if lhs < rhs:
                    nxt = c
                    break
                r = np.maximum(p - q, 0.0)
                if r.sum() > 0:
                    p = r / r.sum()
                q = q.copy()
                q[x] = 0.0
                if q.sum() > 0:
                    q = q / q.sum()
            if nxt is None:
                cdf = np.cumsum(p)
                t = ub[b] * cdf[-1]
                k = int(np.searchsorted(cdf, t, side="right"))
                k = min(k, v - 1)
                while p[k] == 0 and k > 0:       # u_bonus ~ 1: the last token with mass
                    k -= 1
                bonus[b] = k
                below = cdf[k - 1] if k > 0 else 0.0
                margin[b] = min(margin[b], t - below, cdf[k] - t)
                break
            node = nxt
            depth += 1
            if depth <= max_depth:
                path[b, depth] = node
        al[b] = depth
    return al, path, bonus, margin
