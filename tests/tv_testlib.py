"""Shared helpers of the GPU parity tests: upload a workload, run the three
library calls through the binding, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import tree_verification_attention_mask_amd as tv

# Output tolerances (see the test files for where each comes from).
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2      # per element: |g - r| <= atol + rtol |r|
BF16_NERR = 1e-2                       # ||g - r||_2 / ||r||_2
F32_ATOL, F32_RTOL, F32_NERR = 1e-4, 1e-4, 1e-5
LSE_ATOL = 1e-3                        # |lse_g - lse_r|, natural log


class Dev:
    """A workload's arrays on the GPU."""

    def __init__(self, w, device="cuda"):
        self.w = w
        self.parent = torch.from_numpy(w.parent).to(device)
        self.cu = torch.from_numpy(w.cu_nodes).to(device)
        self.prefix = torch.from_numpy(w.prefix_len).to(device)
        self.table = torch.from_numpy(w.block_table).to(device)
        self.q = w.q.to(device)
        self.k = w.k_cache.to(device)
        self.v = w.v_cache.to(device)
        self.draft = torch.from_numpy(w.draft_tok).to(device) if w.draft_tok is not None else None
        self.target = torch.from_numpy(w.target_tok).to(device) if w.target_tok is not None else None

    def mask(self, kind=None, words=None):
        kind = kind or self.w.mask_kind
        return tv.tree_mask_build(self.parent, self.cu, self.w.max_nodes, kind=kind,
                                  words_per_node=words)

    def attn(self, mask=None, **kw):
        m = mask if mask is not None else self.mask()
        return tv.tree_verify_attn(self.q, self.k, self.v, self.table, self.prefix, self.cu, m,
                                   self.w.max_nodes, self.w.max_prefix_len, scale=self.w.scale, **kw)

    def accept(self, max_depth=None):
        md = self.w.max_depth if max_depth is None else max_depth
        return tv.tree_accept(self.parent, self.draft, self.target, self.cu, self.w.max_nodes, md)


def oracle_threads():
    """Host threads for oracle runs: the affinity set, at most 16 (the C
    routine runs outside the interpreter lock, one row range per thread)."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def all_rows(w, nodes=None):
    """(node, q head) rows of the listed global nodes (default: every node)."""
    nodes = np.arange(w.total_nodes) if nodes is None else np.asarray(nodes)
    return np.stack(np.meshgrid(nodes, np.arange(w.num_q_heads), indexing="ij"),
                    -1).reshape(-1, 2).astype(np.int32)


def oracle_attn_threaded(w, rows=None):
    """The oracle over ``rows`` (default: all rows), cut into equal row ranges
    run on host threads; returns (out [R, D], lse [R]) in row order."""
    from concurrent.futures import ThreadPoolExecutor
    rows = all_rows(w) if rows is None else np.asarray(rows, np.int32)
    q = w.q.float().numpy()
    k = w.k_cache.float().numpy()
    v = w.v_cache.float().numpy()
    parts = [c for c in np.array_split(rows, oracle_threads() * 4) if len(c)]

    def run(c):
        return oracle.tree_attn(q, k, v, w.block_table, w.prefix_len, w.cu_nodes, w.parent,
                                w.num_q_heads, w.num_kv_heads, w.scale, rows=c)

    with ThreadPoolExecutor(oracle_threads()) as ex:
        res = list(ex.map(run, parts))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def oracle_attn(w, rows=None, k=None, v=None, q=None):
    return oracle.tree_attn(w.q if q is None else q, w.k_cache if k is None else k,
                            w.v_cache if v is None else v, w.block_table, w.prefix_len,
                            w.cu_nodes, w.parent, w.num_q_heads, w.num_kv_heads, w.scale,
                            rows=rows)


def error_stats(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    nerr = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    return {"max_abs": float(d.max()) if d.size else 0.0, "nerr": nerr,
            "max_rel": float((d / np.maximum(np.abs(ref), 1e-6)).max()) if d.size else 0.0}


def assert_attn_close(got, ref, dtype, got_lse=None, ref_lse=None, what=""):
    got = got.detach().float().cpu().numpy() if isinstance(got, torch.Tensor) else got
    if dtype == "f32":
        atol, rtol, nbar = F32_ATOL, F32_RTOL, F32_NERR
    else:
        atol, rtol, nbar = BF16_ATOL, BF16_RTOL, BF16_NERR
    assert np.isfinite(got).all(), what + ": non-finite output"
    d = np.abs(got - ref)
    bad = d > atol + rtol * np.abs(ref)
    st = error_stats(got, ref)
    assert not bad.any(), "%s: %d elements out of tolerance, %s" % (what, int(bad.sum()), st)
    assert st["nerr"] <= nbar, "%s: normalized error %.3g > %.3g" % (what, st["nerr"], nbar)
    if got_lse is not None:
        gl = got_lse.detach().cpu().numpy() if isinstance(got_lse, torch.Tensor) else got_lse
        dl = np.abs(gl - ref_lse)
        assert dl.max() <= LSE_ATOL, "%s: lse error %.3g" % (what, dl.max())
    return st


def mask_bits_u64(t):
    """int64 tensor of mask words -> uint64 numpy."""
    return t.cpu().numpy().view(np.uint64)
