"""Seeded inputs for stochastic tree verification (sampling at T > 0).

A draft model proposes each node's children by sampling its next-token
distribution without replacement; the target's and the draft's next-token
logits at every node are synthetic: target ~ N(0, spread^2), draft = target +
N(0, noise^2) (a draft that roughly agrees with the target), both rounded to
the working dtype before anything is drawn from them. Uniforms for the
acceptance tests and the bonus draw are drawn here too, so that both the
device path and the oracle get the same numbers. Nothing here verifies
anything.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Sequence

import numpy as np
import torch


@dataclass
class SampledInputs:
    parent: np.ndarray        # int32 [N] request-local
    draft_tok: np.ndarray     # int32 [N]
    cu_nodes: np.ndarray      # int32 [B+1]
    target_logits: np.ndarray  # float32 [N, V] (values of the working dtype)
    draft_logits: np.ndarray   # float32 [N, V]
    u_accept: np.ndarray      # float32 [N] in [0, 1)
    u_bonus: np.ndarray       # float32 [B] in [0, 1)
    max_children: int
    max_depth: int


def _round(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    return torch.from_numpy(x).to(dtype).float().numpy()


def sampled_inputs(rng: np.random.Generator, trees: Sequence[Sequence[int]], vocab: int,
                   dtype: torch.dtype = torch.bfloat16, spread: float = 3.0, noise: float = 1.0,
                   temperature: float = 1.0) -> SampledInputs:
    par, cu = [], [0]
    for t in trees:
        par += list(t)
        cu.append(len(par))
    n = len(par)
    tl = _round(rng.normal(0.0, spread, size=(n, vocab)).astype(np.float32), dtype)
    dl = _round((tl + rng.normal(0.0, noise, size=(n, vocab))).astype(np.float32), dtype)
    tok = np.zeros(n, np.int64)
    max_children, max_depth = 0, 0
    for b, t in enumerate(trees):
        lo = cu[b]
        tok[lo] = int(rng.integers(vocab))          # the current token
        depth = [0] * len(t)
        kids: dict[int, list[int]] = {}
        for i in range(1, len(t)):
            kids.setdefault(t[i], []).append(i)
            depth[i] = depth[t[i]] + 1
        max_depth = max(max_depth, max(depth))
        for u, ch in kids.items():
            max_children = max(max_children, len(ch))
            y = dl[lo + u].astype(np.float64) / temperature
            q = np.exp(y - y.max())
            q /= q.sum()
            k = min(len(ch), int((q > 0).sum()))
            drawn = list(rng.choice(vocab, size=k, replace=False, p=q))
            drawn += [int(rng.integers(vocab)) for _ in range(len(ch) - k)]
            for c, x in zip(ch, drawn):
                tok[lo + c] = int(x)
    return SampledInputs(np.array(par, np.int32), tok.astype(np.int32), np.array(cu, np.int32),
                         tl, dl, rng.random(n).astype(np.float32),
                         rng.random(len(trees)).astype(np.float32), max_children, max_depth)
