"""Seeded synthetic inputs shaped like the pages' verification workloads.

Every draw comes from one ``numpy.random.Generator(PCG64(seed))`` per
workload, in a fixed order: per-config structure (trees, prefix lengths,
confidences), then per request the draft and target token ids, then the page
permutation, then Q, K and V (standard normal, float32, rounded to the
workload's dtype).  Nothing here computes a mask, an attention output or an
acceptance result.

Sources (pages on candidate-tree speculative decoding):
  Graft      arXiv:2605.20104 (163.com article)
  D-cut      paper 2607.14647 (gist.science summary)
  SpecOPD    arXiv:2611.02846 (lewlh.github.io blog)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Sequence

import numpy as np
import torch

QWEN3_VOCAB = 151936
PAGE_SIZE = 16

CONFIG_NAMES = {
    1: "tiny-15node-fp32",
    2: "graft-60node-p2048",
    3: "dcut-b64-chains",
    4: "long-32k-b8-60node",
    5: "specopd-trunk4096-32x16",
}

# The 60-slot hybrid tree of a depth-5 prune (Graft §二, second gear: 40 draft
# nodes kept + 20 retrieved nodes).  Draft part: levels of 1, 3, 9, 9, 9, 9
# nodes (the 3 best nodes of each level expand 3 children each).  Retrieved
# part, grafted under the first depth-5 node (31): its top-4 successors
# (40..43); rank 1 heads a greedy chain that keeps 3 successors per level for
# 4 more levels (44.., 51.., 54.., 57..), ranks 2..4 keep 2, 1, 1 children.
# Breadth-first order, request-local indices, root = 0.
GRAFT_TREE_PARENT = (
    [-1, 0, 0, 0]
    + [1] * 3 + [2] * 3 + [3] * 3
    + [4] * 3 + [5] * 3 + [6] * 3
    + [13] * 3 + [14] * 3 + [15] * 3
    + [22] * 3 + [23] * 3 + [24] * 3
    + [31] * 4
    + [40] * 3 + [41] * 2 + [42] + [43]
    + [44] * 3
    + [51] * 3
    + [54] * 3
)
assert len(GRAFT_TREE_PARENT) == 60


@dataclass
class Workload:
    """One batch of verification inputs, host-side (numpy / CPU torch)."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    dtype: str                     # "f32" or "bf16"
    parent: np.ndarray             # int32 [N_tot], request-local, root 0 = -1
    cu_nodes: np.ndarray           # int32 [B+1]
    prefix_len: np.ndarray         # int32 [B]
    block_table: np.ndarray        # int32 [B, max_pages], -1 past the end
    num_pages: int
    q: torch.Tensor                # [N_tot, Hq, D]
    k_cache: torch.Tensor          # [num_pages, Hkv, page, D]
    v_cache: torch.Tensor          # [num_pages, Hkv, D, page] (d-major pages)
    draft_tok: np.ndarray | None   # int32 [N_tot]
    target_tok: np.ndarray | None  # int32 [N_tot]
    max_depth: int                 # deepest node over the batch
    mask_kind: str = "bits"        # "bits" or "anchor"
    vocab: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def total_nodes(self) -> int:
        return int(self.cu_nodes[-1])

    @property
    def nodes_per_request(self) -> np.ndarray:
        return np.diff(self.cu_nodes)

    @property
    def max_nodes(self) -> int:
        return int(self.nodes_per_request.max())

    @property
    def max_prefix_len(self) -> int:
        return int(self.prefix_len.max())

    @property
    def words_per_node(self) -> int:
        return max(1, (self.max_nodes + 63) // 64)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


def _depths(parent: Sequence[int]) -> np.ndarray:
    d = np.zeros(len(parent), np.int64)
    for i in range(1, len(parent)):
        d[i] = d[parent[i]] + 1
    return d


def _children(parent: Sequence[int]) -> list[list[int]]:
    ch: list[list[int]] = [[] for _ in parent]
    for i in range(1, len(parent)):
        ch[parent[i]].append(i)
    return ch


def _distinct(rng: np.random.Generator, k: int, vocab: int, exclude=()) -> list[int]:
    out: list[int] = []
    taken = set(exclude)
    while len(out) < k:
        t = int(rng.integers(vocab))
        if t not in taken:
            taken.add(t)
            out.append(t)
    return out


def _tree_tokens(rng, parent, vocab, match_p):
    """Draft ids (siblings distinct) and target greedy ids for one tree.

    match_p[i] is the probability that the target's greedy token at node i
    equals the draft token of one of i's children (chosen uniformly);
    otherwise it is uniform over the vocabulary minus the children's tokens.
    Leaves get a uniform target token.
    """
    n = len(parent)
    ch = _children(parent)
    draft = np.zeros(n, np.int32)
    draft[0] = int(rng.integers(vocab))
    for i in range(n):
        if ch[i]:
            # distinct siblings when the vocabulary allows it (tiny test vocabularies
            # with more children than tokens repeat tokens among siblings)
            if len(ch[i]) <= vocab:
                toks = _distinct(rng, len(ch[i]), vocab)
            else:
                toks = [int(t) for t in rng.integers(vocab, size=len(ch[i]))]
            for c, t in zip(ch[i], toks):
                draft[c] = t
    target = np.zeros(n, np.int32)
    for i in range(n):
        taken = {int(draft[c]) for c in ch[i]}
        if ch[i] and rng.random() < match_p[i]:
            target[i] = draft[ch[i][int(rng.integers(len(ch[i])))]]
        elif ch[i] and len(taken) < vocab:
            target[i] = _distinct(rng, 1, vocab, exclude=taken)[0]
        else:
            target[i] = int(rng.integers(vocab))
    return draft, target


def _normal(rng: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    """Standard-normal tensor of ``shape`` rounded to ``dtype`` (drawn in float32 chunks)."""
    out = torch.empty(shape, dtype=dtype)
    flat = out.view(-1)
    chunk = 1 << 24
    for s in range(0, flat.numel(), chunk):
        e = min(flat.numel(), s + chunk)
        flat[s:e] = torch.from_numpy(rng.standard_normal(e - s, dtype=np.float32)).to(dtype)
    return out


def build_workload(name: str, trees: Sequence[Sequence[int]], prefix_len: Sequence[int],
                   num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: str,
                   rng: np.random.Generator | int, *, page_size: int = PAGE_SIZE,
                   permute_pages: bool = False, vocab: int = 1000,
                   match_p: float | Callable[[int, np.ndarray], np.ndarray] = 0.7,
                   tokens: bool = True, mask_kind: str = "bits",
                   spare_pages: int = 0, meta: dict | None = None) -> Workload:
    """Draw a workload for the given trees and prefix lengths.

    ``match_p`` is a float or ``f(request, depths) -> per-node probability``.
    The K/V of request b's tree node j sits at logical position
    prefix_len[b] + j. K pages are [Hkv, page, D], V pages [Hkv, D, page].  Pages are handed out request by request (identity
    table) or, with ``permute_pages``, through a seeded permutation of the
    whole pool.  ``spare_pages`` adds unused pages to the pool.
    """
    if not isinstance(rng, np.random.Generator):
        rng = np.random.Generator(np.random.PCG64(int(rng)))
    assert len(trees) == len(prefix_len)
    batch = len(trees)
    sizes = [len(t) for t in trees]
    cu = np.zeros(batch + 1, np.int32)
    cu[1:] = np.cumsum(sizes)
    parent = np.concatenate([np.asarray(t, np.int32) for t in trees]) if batch else np.zeros(0, np.int32)
    depths = [_depths(t) for t in trees]
    max_depth = int(max((int(d.max()) if d.size else 0) for d in depths)) if batch else 0

    draft = target = None
    if tokens:
        dl, tl = [], []
        for b, t in enumerate(trees):
            p = match_p(b, depths[b]) if callable(match_p) else np.full(len(t), float(match_p))
            dr, tg = _tree_tokens(rng, t, vocab, p)
            dl.append(dr)
            tl.append(tg)
        draft = np.concatenate(dl).astype(np.int32)
        target = np.concatenate(tl).astype(np.int32)

    kv_len = [int(prefix_len[b]) + sizes[b] for b in range(batch)]
    npages = [(L + page_size - 1) // page_size for L in kv_len]
    num_pages = int(sum(npages)) + int(spare_pages)
    perm = rng.permutation(num_pages).astype(np.int32) if permute_pages else np.arange(num_pages, dtype=np.int32)
    max_pages = max(npages) if batch else 1
    table = np.full((batch, max(1, max_pages)), -1, np.int32)
    off = 0
    for b in range(batch):
        table[b, :npages[b]] = perm[off:off + npages[b]]
        off += npages[b]

    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    n_tot = int(cu[-1])
    q = _normal(rng, (n_tot, num_q_heads, head_dim), tdt)
    k = _normal(rng, (num_pages, num_kv_heads, page_size, head_dim), tdt)
    v = _normal(rng, (num_pages, num_kv_heads, head_dim, page_size), tdt)
    return Workload(name=name, batch=batch, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, page_size=page_size, dtype=dtype, parent=parent,
                    cu_nodes=cu, prefix_len=np.asarray(prefix_len, np.int32), block_table=table,
                    num_pages=num_pages, q=q, k_cache=k, v_cache=v, draft_tok=draft,
                    target_tok=target, max_depth=max_depth, mask_kind=mask_kind, vocab=vocab,
                    meta=dict(meta or {}))


def random_tree(rng: np.random.Generator, n: int, max_children: int | None = None) -> list[int]:
    """Random topologically ordered tree: parent[i] uniform over earlier nodes
    (optionally over those with fewer than ``max_children`` children)."""
    par = [-1]
    nch = [0]
    for i in range(1, n):
        while True:
            p = int(rng.integers(i))
            if max_children is None or nch[p] < max_children:
                break
        par.append(p)
        nch[p] += 1
        nch.append(0)
    return par


def trunk_branch_tree(trunk: int, anchors: Sequence[int], width: int) -> list[int]:
    """SpecOPD proposal tree (SpecOPD §02, anchor sampling and proposal tree):
    a causal trunk 0..trunk-1 (parent i-1), then one chain branch of ``width``
    nodes per anchor, in anchor order; a branch's first node hangs off its
    anchor trunk node, so the branch sees trunk[0..anchor] and its own chain."""
    par = [-1] + list(range(trunk - 1))
    for a in anchors:
        assert 0 <= a < trunk
        start = len(par)
        par.append(int(a))
        par.extend(range(start, start + width - 1))
    return par


# ---------------------------------------------------------------- configs --

def _cfg1(seed: int, prefix: int = 128, **kw) -> Workload:
    """Tiny: batch 1, 8 q / 2 kv heads, head_dim 64, fp32, prefix 128, 15 nodes of
    depth 4 whose root has exactly 3 children; vocab 1000, match probability 0.7."""
    rng = np.random.Generator(np.random.PCG64(seed))
    while True:
        par = [-1, 0, 0, 0]
        dep = [0, 1, 1, 1]
        for i in range(4, 15):
            cand = [j for j in range(1, i) if dep[j] <= 3]
            p = cand[int(rng.integers(len(cand)))]
            par.append(p)
            dep.append(dep[p] + 1)
        if max(dep) == 4:
            break
    return build_workload(CONFIG_NAMES[1], [par], [prefix], 8, 2, 64, "f32", rng,
                          vocab=1000, match_p=0.7, **kw)


def _graft_match_p(b: int, depths: np.ndarray) -> np.ndarray:
    # per-depth acceptance probability decaying linearly 0.8 -> 0.4 over depths 0..9
    return 0.8 - 0.4 * np.minimum(depths, 9) / 9.0


def _cfg2(seed: int, prefix: int = 2048, **kw) -> Workload:
    """Graft-shaped: batch 1, 32 q / 8 kv heads (Qwen3-8B), head_dim 128, bf16,
    prefix 2048, the 60-slot hybrid tree ``GRAFT_TREE_PARENT``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return build_workload(CONFIG_NAMES[2], [list(GRAFT_TREE_PARENT)], [prefix], 32, 8, 128,
                          "bf16", rng, vocab=QWEN3_VOCAB, match_p=_graft_match_p, **kw)


def _cfg3(seed: int, batch: int = 64, prefix_range=(512, 4096), block: int = 16,
          rho: float = 0.5, **kw) -> Workload:
    """D-cut-shaped: ``batch`` requests, each a chain block of D+1 = 16 nodes
    (root + 15 drafted tokens).  Per-position draft confidences ~ Beta(4, 2);
    the score of position k of request i is the prefix product of confidences
    up to k (the root's empty product is 1).  The K = rho * batch * 16 best
    scores over the whole batch are kept (order: score desc, request asc,
    position asc); because scores fall along a block, each request keeps a
    contiguous prefix (D-cut summary, §2 mechanisms and packing).  The target
    agrees with drafted token k+1 at node k with probability equal to its
    confidence.  Prefix lengths uniform over the inclusive range."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lo, hi = prefix_range
    prefix = rng.integers(lo, hi + 1, size=batch).astype(np.int32)
    conf = rng.beta(4.0, 2.0, size=(batch, block - 1))
    score = np.ones((batch, block))
    score[:, 1:] = np.cumprod(conf, axis=1)
    budget = int(round(rho * batch * block))
    order = sorted(((-score[i, k], i, k) for i in range(batch) for k in range(block)))
    keep = np.zeros((batch, block), bool)
    for _, i, k in order[:budget]:
        keep[i, k] = True
    n_keep = keep.sum(axis=1)
    for i in range(batch):  # contiguous prefixes by construction of the scores
        assert keep[i, :n_keep[i]].all() and not keep[i, n_keep[i]:].any()
    trees = [[-1] + list(range(int(n) - 1)) for n in n_keep]

    def match(b, depths):
        p = np.zeros(len(depths))
        p[:-1] = conf[b, :len(depths) - 1]
        return p

    return build_workload(CONFIG_NAMES[3], trees, prefix.tolist(), 32, 8, 128, "bf16", rng,
                          vocab=QWEN3_VOCAB, match_p=match,
                          meta={"rho": rho, "budget": budget, "confidence": conf}, **kw)


def _cfg4(seed: int, batch: int = 8, prefix: int = 32768, **kw) -> Workload:
    """Long-context tree: ``batch`` requests of the 60-node Graft tree over a
    32768-token prefix in 16-token pages from a seeded permutation of the
    pool; 64 q / 8 kv heads (Qwen3-32B-like), head_dim 128, bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kw.setdefault("permute_pages", True)
    return build_workload(CONFIG_NAMES[4], [list(GRAFT_TREE_PARENT)] * batch, [prefix] * batch,
                          64, 8, 128, "bf16", rng, vocab=QWEN3_VOCAB, match_p=_graft_match_p, **kw)


def _cfg5(seed: int, trunk: int = 4096, n_anchors: int = 32, width: int = 16,
          anchor_lo: int = 1024, **kw) -> Workload:
    """SpecOPD proposal tree: causal trunk of 4096 tokens, 32 anchors drawn
    without replacement from [1024, 4096) and sorted, a 16-node chain branch
    per anchor; no separate prefix (prefix_len 0), so all 4608 rows attend
    tree keys only; 32 q / 8 kv heads, head_dim 128, bf16, anchor-form mask.
    Scoring the branches' distributions is the goal there, so no tokens."""
    rng = np.random.Generator(np.random.PCG64(seed))
    anchors = np.sort(rng.choice(np.arange(anchor_lo, trunk), size=n_anchors, replace=False))
    par = trunk_branch_tree(trunk, anchors.tolist(), width)
    return build_workload(CONFIG_NAMES[5], [par], [0], 32, 8, 128, "bf16", rng, tokens=False,
                          mask_kind="anchor", meta={"anchors": anchors, "trunk": trunk,
                                                    "width": width}, **kw)


_MAKERS = {1: _cfg1, 2: _cfg2, 3: _cfg3, 4: _cfg4, 5: _cfg5}


def make(config: int, seed: int | None = None, **overrides) -> Workload:
    """Workload for config 1..5 at full size (seed = config number), or scaled
    down through the config's keyword overrides (e.g. ``prefix=300``)."""
    return _MAKERS[config](config if seed is None else seed, **overrides)
