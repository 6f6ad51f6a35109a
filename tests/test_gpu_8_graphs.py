"""HIP-graph replays of a whole verification step and of the multi-launch entry points (stochastic acceptance,
the Graft update, E2E-TV statistics): every replay, with eager work and
synchronisations between replays, must give the eager result bit for bit
(the library records no memset, and every scratch table is rewritten before
it is read)."""
import numpy as np
import pytest
import torch

import tree_verification_attention_mask_amd as tv
import workloads as W

pytestmark = pytest.mark.gpu


def _replays(capture_fn, read_fn, eager, times=4):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture_fn()
    for i in range(times):
        junk = torch.randn(1 << 20, device="cuda") * i   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = read_fn()
        for a, b in zip(got, eager):
            assert torch.equal(a, b), i
        del junk


def test_sampled_acceptance_graph_replays():
    si = W.sampled_inputs(np.random.default_rng(21), [list(W.GRAFT_TREE_PARENT)] * 2, 50000)
    dev = "cuda"
    args = [torch.from_numpy(x).to(dev) for x in (si.parent, si.draft_tok, si.cu_nodes)]
    tl = torch.from_numpy(si.target_logits).to(torch.bfloat16).to(dev)
    dl = torch.from_numpy(si.draft_logits).to(torch.bfloat16).to(dev)
    ua, ub = torch.from_numpy(si.u_accept).to(dev), torch.from_numpy(si.u_bonus).to(dev)
    n = len(si.parent)
    ws = torch.empty(tv.tree_accept_sampled_workspace_size(n, si.max_children, 50000),
                     dtype=torch.uint8, device=dev)
    out = {"accept_len": torch.empty(2, dtype=torch.int32, device=dev),
           "path": torch.empty((2, si.max_depth + 1), dtype=torch.int32, device=dev),
           "bonus": torch.empty(2, dtype=torch.int32, device=dev)}

    def call():
        tv.tree_accept_sampled(*args, tl, dl, ua, ub, 60, si.max_children, si.max_depth, 1.0,
                               workspace=ws, out=out)
    call()
    torch.cuda.synchronize()
    eager = [out[k].clone() for k in ("accept_len", "path", "bonus")]
    for k in out:
        out[k].fill_(-7)
    _replays(call, lambda: [out[k] for k in ("accept_len", "path", "bonus")], eager)


def test_graft_update_graph_replays():
    rng = np.random.default_rng(22)
    v, k, n = 151936, 8, 60
    dev = "cuda"
    adj0 = torch.from_numpy(rng.integers(0, v, size=(v, k)).astype(np.int32)).to(dev)
    lg = torch.from_numpy(rng.normal(0, 3, size=(n, v)).astype(np.float32)).to(torch.bfloat16).to(dev)
    toks = torch.from_numpy(rng.integers(0, v, size=n).astype(np.int32)).to(dev)
    ws = torch.empty(max(1, tv.graft_update_workspace_size(n, v, k)), dtype=torch.uint8, device=dev)
    adj = adj0.clone()
    tv.graft_update(adj, lg, toks, workspace=ws)
    torch.cuda.synchronize()
    eager = [adj.clone()]
    work = adj0.clone()

    def call():
        tv.graft_update(work, lg, toks, workspace=ws)

    def read():
        return [work]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(4):
        work.copy_(adj0)                                  # eager work: reset the table
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(work, eager[0]), i


def test_e2e_tv_graph_replays():
    g0 = torch.Generator(device="cuda").manual_seed(23)
    n, v = 64, 151936
    t = (torch.randn((n, v), generator=g0, device="cuda") * 3.0).to(torch.bfloat16)
    d = (t.float() + torch.randn((n, v), generator=g0, device="cuda")).to(torch.bfloat16)
    cu = torch.arange(0, n + 1, 16, dtype=torch.int32, device="cuda")
    a, pre, ex = tv.e2e_tv_stats(t, d, cu, 1.0)
    torch.cuda.synchronize()
    eager = [a.clone(), pre.clone(), ex.clone()]
    outs = {}

    def call():
        outs["r"] = tv.e2e_tv_stats(t, d, cu, 1.0)
    _replays(call, lambda: list(outs["r"]), eager)


_STEP_WORKLOADS = {
    "graft-tree-11-splits": lambda: W.make(2),
    "ragged-batch-longest-first": lambda: W.make(3, batch=40, prefix_range=(50, 700)),
    "anchor-trunk-and-branches": lambda: W.make(5, trunk=512, n_anchors=8, anchor_lo=64),
}


@pytest.mark.parametrize("name", sorted(_STEP_WORKLOADS))
def test_verify_step_graph_replays(name):
    """One step (mask build, attention, acceptance) captured in a HIP graph:
    every replay, after its outputs were overwritten and eager work ran, gives
    the eager step's results bit for bit (the split merge, the longest-first
    order and the anchor-form mask included)."""
    from tv_testlib import Dev
    w = _STEP_WORKLOADS[name]()
    d = Dev(w)
    res = {}

    def step():
        m = d.mask()
        out, lse = d.attn(mask=m)
        res.update(out=out, lse=lse, depth=m["depth"], err=m["err"])
        if d.draft is not None:
            al, path, bonus = d.accept()
            res.update(accept_len=al, path=path, bonus=bonus)

    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in res.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        for v in res.values():
            v.fill_(float("nan") if v.is_floating_point() else -7)
        junk = torch.randn(1 << 20, device="cuda") * i   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for k, v in eager.items():
            assert torch.equal(res[k], v), (name, k, i)
        del junk
