"""Thin ctypes binding of ``libtreeverify.so`` (C ABI in ``include/treeverify.h``).

Argument marshalling only: tensors become device pointers, host scalars are
passed through, outputs are allocated with torch when the caller does not
supply them, and every call is enqueued on torch's current HIP stream (or on
the ``stream`` argument: the call then runs with that stream current, so its
temporaries are allocated and freed in that stream's order, after the stream
has been made to wait for the current one).  All computation happens in the
library's kernels.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import functools
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libtreeverify.so")

TV_OK, TV_ERR_INVALID_ARGUMENT, TV_ERR_UNSUPPORTED, TV_ERR_WORKSPACE, TV_ERR_HIP = range(5)
TV_F32, TV_BF16 = 0, 1
TV_MASK_BITS, TV_MASK_ANCHOR = 0, 1
MAX_MASK_WORDS = 16
MAX_ACCEPT_NODES = 8192

# every symbol the header declares
EXPORTS = ("tv_tree_mask_build", "tv_tree_verify_attn_workspace_size", "tv_tree_verify_attn_plan",
           "tv_tree_verify_attn", "tv_tree_verify_attn_noalloc",
           "tv_tree_accept", "tv_dcut_select", "tv_e2e_tv_stats", "tv_graft_retrieve",
           "tv_graft_update_workspace_size", "tv_graft_update",
           "tv_tree_accept_sampled_workspace_size", "tv_tree_accept_sampled", "tv_status_string")
MAX_DCUT_DRAFT_POSITIONS = 32768


class TVError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s failed: status %d (%s)" % (fn, status, msg))
        self.status = status


class AttnPlan(ctypes.Structure):
    _fields_ = [("num_cus", ctypes.c_int32), ("rows_per_block", ctypes.c_int32),
                ("row_blocks", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("keys_per_split", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t)]


class Mask(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("words_per_node", ctypes.c_int32),
                ("bits", ctypes.c_void_p), ("anchor_pos", ctypes.c_void_p),
                ("branch_depth", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libtreeverify.so not found at %s -- build it with "
                          "`python -m tree_verification_attention_mask_amd.build`" % path)
    lib = ctypes.CDLL(path)
    P, I, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.tv_tree_mask_build.argtypes = [P, P, I, I, I, I, I, P, P, P, P, P, P]
    lib.tv_tree_mask_build.restype = ctypes.c_int
    lib.tv_tree_verify_attn_workspace_size.argtypes = [I, I, I, I, I, I, I, I]
    lib.tv_tree_verify_attn_workspace_size.restype = S
    lib.tv_tree_verify_attn_plan.argtypes = [I, I, I, I, I, I, I, I, I, ctypes.POINTER(AttnPlan)]
    lib.tv_tree_verify_attn_plan.restype = ctypes.c_int
    lib.tv_tree_verify_attn.argtypes = [P, P, P, I, P, I, P, P, I, I, I, I, I, I, I, I, I,
                                        ctypes.c_float, ctypes.POINTER(Mask), P, P, P, S, P]
    lib.tv_tree_verify_attn.restype = ctypes.c_int
    lib.tv_tree_verify_attn_noalloc.argtypes = [P, P, P, I, P, I, P, P, I, I, I, I, I, I, I, I, I,
                                                ctypes.c_float, ctypes.POINTER(Mask), P, P, P]
    lib.tv_tree_verify_attn_noalloc.restype = ctypes.c_int
    lib.tv_tree_accept.argtypes = [P, P, P, P, I, I, I, I, P, P, P, P]
    lib.tv_tree_accept.restype = ctypes.c_int
    lib.tv_dcut_select.argtypes = [P, P, I, I, I, P, P, P, P, P]
    lib.tv_dcut_select.restype = ctypes.c_int
    lib.tv_e2e_tv_stats.argtypes = [P, P, I, I, I, ctypes.c_float, P, I, P, P, P, P]
    lib.tv_e2e_tv_stats.restype = ctypes.c_int
    lib.tv_graft_retrieve.argtypes = [P, I, I, P, I, P, P, I, P, P]
    lib.tv_graft_retrieve.restype = ctypes.c_int
    lib.tv_graft_update_workspace_size.argtypes = [I, I, I, I]
    lib.tv_graft_update_workspace_size.restype = S
    lib.tv_graft_update.argtypes = [P, I, I, P, I, I, P, P, S, P]
    lib.tv_graft_update.restype = ctypes.c_int
    lib.tv_tree_accept_sampled_workspace_size.argtypes = [I, I, I]
    lib.tv_tree_accept_sampled_workspace_size.restype = S
    lib.tv_tree_accept_sampled.argtypes = [P, P, P, I, I, I, I, I, P, P, I, I, ctypes.c_float, P, P,
                                           P, P, P, P, S, P]
    lib.tv_tree_accept_sampled.restype = ctypes.c_int
    lib.tv_status_string.argtypes = [ctypes.c_int]
    lib.tv_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != TV_OK:
        raise TVError(fn, status, load_library().tv_status_string(status).decode())


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _dev_i32(x, device):
    if isinstance(x, torch.Tensor):
        assert x.dtype == torch.int32 and x.is_contiguous() and x.device.type == "cuda"
        return x
    return torch.as_tensor(x, dtype=torch.int32, device=device).contiguous()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """Run ``fn`` with its ``stream`` keyword argument as the current stream.

    The stream first waits for the caller's current stream (the inputs were
    made there); temporaries ``fn`` allocates then belong to ``stream``, so
    the caching allocator does not hand their memory out again before the
    kernels enqueued on ``stream`` have run.
    """
    @functools.wraps(fn)
    def run(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, **kw)
        cur = torch.cuda.current_stream(stream.device)
        if stream == cur:
            return fn(*args, **kw)
        stream.wait_stream(cur)
        with torch.cuda.stream(stream):
            return fn(*args, **kw)
    return run


@_on_stream
def tree_mask_build(parent: torch.Tensor, cu_nodes: torch.Tensor, max_nodes: int,
                    kind: str = "bits", words_per_node: int | None = None, out: dict | None = None) -> dict:
    """Depth and ancestor mask of every node (``tv_tree_mask_build``).

    Returns a dict with ``kind``, ``depth``, ``err`` and either ``bits``
    (uint64 as int64 [N, words]) or ``anchor_pos`` / ``branch_depth``.
    """
    lib = load_library()
    dev = parent.device
    batch = cu_nodes.numel() - 1
    n = parent.numel()
    k = TV_MASK_BITS if kind == "bits" else TV_MASK_ANCHOR
    words = words_per_node if words_per_node is not None else max(1, (max_nodes + 63) // 64)
    o = dict(out or {})
    if "depth" not in o:
        o["depth"] = torch.empty(n, dtype=torch.int32, device=dev)
    if "err" not in o:
        o["err"] = torch.empty(batch, dtype=torch.int32, device=dev)
    if k == TV_MASK_BITS:
        if "bits" not in o:
            o["bits"] = torch.empty((n, words), dtype=torch.int64, device=dev)
    else:
        if "anchor_pos" not in o:
            o["anchor_pos"] = torch.empty(n, dtype=torch.int32, device=dev)
        if "branch_depth" not in o:
            o["branch_depth"] = torch.empty(n, dtype=torch.int32, device=dev)
    st = lib.tv_tree_mask_build(_ptr(parent), _ptr(cu_nodes), batch, n, int(max_nodes), k,
                                words if k == TV_MASK_BITS else 0, _ptr(o.get("bits")),
                                _ptr(o.get("anchor_pos")), _ptr(o.get("branch_depth")),
                                _ptr(o["depth"]), _ptr(o["err"]), _stream())
    _check("tv_tree_mask_build", st)
    o["kind"] = kind
    o["words_per_node"] = words if k == TV_MASK_BITS else 0
    return o


def mask_struct(mask: dict) -> Mask:
    if mask["kind"] == "bits":
        return Mask(TV_MASK_BITS, int(mask["words_per_node"]), mask["bits"].data_ptr(), None, None)
    return Mask(TV_MASK_ANCHOR, 0, None, mask["anchor_pos"].data_ptr(),
                mask["branch_depth"].data_ptr())


def verify_attn_workspace_size(batch: int, total_nodes: int, max_nodes: int, max_prefix_len: int,
                               num_q_heads: int, num_kv_heads: int, head_dim: int,
                               dtype: torch.dtype) -> int:
    lib = load_library()
    dt = TV_F32 if dtype == torch.float32 else TV_BF16
    return int(lib.tv_tree_verify_attn_workspace_size(batch, total_nodes, max_nodes, max_prefix_len,
                                                      num_q_heads, num_kv_heads, head_dim, dt))


@_on_stream
def verify_attn_plan(batch: int, total_nodes: int, max_nodes: int, max_prefix_len: int,
                     num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype,
                     num_cus: int = 0) -> dict:
    """Launch plan of ``tv_tree_verify_attn`` for ``num_cus`` compute units
    (0 = the current device's): rows per block, row blocks, key splits, keys
    per split and workspace bytes."""
    lib = load_library()
    dt = TV_F32 if dtype == torch.float32 else TV_BF16
    pl = AttnPlan()
    _check("tv_tree_verify_attn_plan",
           lib.tv_tree_verify_attn_plan(batch, total_nodes, max_nodes, max_prefix_len,
                                        num_q_heads, num_kv_heads, head_dim, dt, num_cus,
                                        ctypes.byref(pl)))
    return {f: getattr(pl, f) for f, _ in AttnPlan._fields_}


@_on_stream
def tree_verify_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     block_table: torch.Tensor, prefix_len: torch.Tensor, cu_nodes: torch.Tensor,
                     mask: dict, max_nodes: int, max_prefix_len: int, scale: float | None = None,
                     out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = True,
                     workspace: torch.Tensor | None = None):
    """One tree-verification attention layer (``tv_tree_verify_attn``).

    ``q`` [N, Hq, D]; ``k_cache`` [pages, Hkv, page, D], ``v_cache`` [pages, Hkv, D, page]
    (bf16 or fp32);
    ``block_table`` int32 [B, max_pages]; returns (out [N, Hq, D], lse [N, Hq] or None).
    """
    lib = load_library()
    n, hq, d = q.shape
    pages, hkv, page, d2 = k_cache.shape
    assert d2 == d and tuple(v_cache.shape) == (pages, hkv, d, page)
    assert q.dtype == k_cache.dtype == v_cache.dtype and q.is_contiguous()
    assert k_cache.is_contiguous() and v_cache.is_contiguous() and block_table.is_contiguous()
    batch = cu_nodes.numel() - 1
    dt = TV_F32 if q.dtype == torch.float32 else TV_BF16
    if out is None:
        out = torch.empty_like(q)
    if lse is True:
        lse = torch.empty((n, hq), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    need = int(lib.tv_tree_verify_attn_workspace_size(batch, n, int(max_nodes), int(max_prefix_len),
                                                      hq, hkv, d, dt))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ms = mask_struct(mask)
    if scale is None:
        scale = d ** -0.5
    st = lib.tv_tree_verify_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), pages, _ptr(block_table),
                                 block_table.shape[1], _ptr(prefix_len), _ptr(cu_nodes), batch, n,
                                 int(max_nodes), int(max_prefix_len), hq, hkv, d, page, dt,
                                 float(scale), ctypes.byref(ms), _ptr(out), _ptr(lse),
                                 _ptr(workspace), ws_bytes, _stream())
    _check("tv_tree_verify_attn", st)
    return out, lse


def tree_verify_attn_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                             block_table: torch.Tensor, prefix_len: torch.Tensor,
                             cu_nodes: torch.Tensor, mask: dict, max_nodes: int,
                             max_prefix_len: int, out: torch.Tensor, lse: torch.Tensor | None,
                             scale: float | None = None, stream=None):
    """``tv_tree_verify_attn_noalloc``: the same layer with the split partials
    in the library's per-device scratch array. Nothing is allocated here
    either: the caller passes ``out`` (and ``lse`` or None); ``stream`` (a
    torch stream, default the current one) is used as given."""
    lib = load_library()
    n, hq, d = q.shape
    pages, hkv, page, d2 = k_cache.shape
    assert d2 == d and tuple(v_cache.shape) == (pages, hkv, d, page)
    assert q.dtype == k_cache.dtype == v_cache.dtype == out.dtype and q.is_contiguous()
    assert k_cache.is_contiguous() and v_cache.is_contiguous() and block_table.is_contiguous()
    assert out.shape == q.shape and out.is_contiguous()
    batch = cu_nodes.numel() - 1
    dt = TV_F32 if q.dtype == torch.float32 else TV_BF16
    ms = mask_struct(mask)
    st = lib.tv_tree_verify_attn_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), pages, _ptr(block_table), block_table.shape[1],
        _ptr(prefix_len), _ptr(cu_nodes), batch, n, int(max_nodes), int(max_prefix_len), hq, hkv,
        d, page, dt, float(d ** -0.5 if scale is None else scale), ctypes.byref(ms), _ptr(out),
        _ptr(lse), _stream(stream))
    _check("tv_tree_verify_attn_noalloc", st)
    return out, lse


@_on_stream
def tree_accept(parent: torch.Tensor, draft_tok: torch.Tensor, target_tok: torch.Tensor,
                cu_nodes: torch.Tensor, max_nodes: int, max_depth: int, out: dict | None = None):
    """Greedy acceptance (``tv_tree_accept``): returns (accept_len [B], path [B, max_depth+1], bonus [B])."""
    lib = load_library()
    dev = parent.device
    batch = cu_nodes.numel() - 1
    o = dict(out or {})
    if "accept_len" not in o:
        o["accept_len"] = torch.empty(batch, dtype=torch.int32, device=dev)
    if "path" not in o:
        o["path"] = torch.empty((batch, max_depth + 1), dtype=torch.int32, device=dev)
    if "bonus" not in o:
        o["bonus"] = torch.empty(batch, dtype=torch.int32, device=dev)
    st = lib.tv_tree_accept(_ptr(parent), _ptr(draft_tok), _ptr(target_tok), _ptr(cu_nodes), batch,
                            parent.numel(), int(max_nodes), int(max_depth), _ptr(o["accept_len"]),
                            _ptr(o["path"]), _ptr(o["bonus"]), _stream())
    _check("tv_tree_accept", st)
    return o["accept_len"], o["path"], o["bonus"]


@_on_stream
def tree_accept_sampled(parent: torch.Tensor, draft_tok: torch.Tensor, cu_nodes: torch.Tensor,
                        target_logits: torch.Tensor, draft_logits: torch.Tensor,
                        u_accept: torch.Tensor, u_bonus: torch.Tensor, max_nodes: int,
                        max_children: int, max_depth: int, temperature: float = 1.0,
                        workspace: torch.Tensor | None = None, out: dict | None = None):
    """Stochastic acceptance (``tv_tree_accept_sampled``): recursive rejection
    sampling over both models' next-token logits [N, V] (bf16 or fp32) with
    the given uniforms (fp32, ``u_accept`` [N], ``u_bonus`` [B]).

    Returns (accept_len [B], path [B, max_depth+1], bonus [B]).
    """
    lib = load_library()
    dev = parent.device
    batch = cu_nodes.numel() - 1
    n = parent.numel()
    assert target_logits.shape == draft_logits.shape and target_logits.dim() == 2
    assert target_logits.shape[0] == n and target_logits.dtype == draft_logits.dtype
    assert target_logits.is_contiguous() and draft_logits.is_contiguous()
    assert u_accept.dtype == torch.float32 and u_bonus.dtype == torch.float32
    assert u_accept.numel() == n and u_bonus.numel() == batch
    dt = TV_F32 if target_logits.dtype == torch.float32 else TV_BF16
    o = dict(out or {})
    if "accept_len" not in o:
        o["accept_len"] = torch.empty(batch, dtype=torch.int32, device=dev)
    if "path" not in o:
        o["path"] = torch.empty((batch, max_depth + 1), dtype=torch.int32, device=dev)
    if "bonus" not in o:
        o["bonus"] = torch.empty(batch, dtype=torch.int32, device=dev)
    need = int(lib.tv_tree_accept_sampled_workspace_size(n, int(max_children),
                                                         target_logits.shape[1]))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.tv_tree_accept_sampled(
        _ptr(parent), _ptr(draft_tok), _ptr(cu_nodes), batch, n, int(max_nodes), int(max_children),
        int(max_depth), _ptr(target_logits), _ptr(draft_logits), dt, target_logits.shape[1],
        float(temperature), _ptr(u_accept), _ptr(u_bonus), _ptr(o["accept_len"]), _ptr(o["path"]),
        _ptr(o["bonus"]), _ptr(workspace), ws_bytes, _stream())
    _check("tv_tree_accept_sampled", st)
    return o["accept_len"], o["path"], o["bonus"]


def tree_accept_sampled_workspace_size(total_nodes: int, max_children: int, vocab: int) -> int:
    """Bytes ``tv_tree_accept_sampled`` needs for these shapes."""
    return int(load_library().tv_tree_accept_sampled_workspace_size(total_nodes, max_children,
                                                                     vocab))


@_on_stream
def dcut_select(conf: torch.Tensor, tokens: torch.Tensor, budget: int, out: dict | None = None):
    """D-cut budget (``tv_dcut_select``): ``conf`` fp32 [B, D], ``tokens`` int32 [B, D+1].

    Returns (n_keep [B], cu_nodes [B+1], parent [budget], packed_tokens [budget]).
    """
    lib = load_library()
    assert conf.dtype == torch.float32 and conf.is_contiguous() and conf.dim() == 2
    batch, d = conf.shape
    assert tokens.dtype == torch.int32 and tokens.is_contiguous()
    assert tuple(tokens.shape) == (batch, d + 1)
    dev = conf.device
    o = dict(out or {})
    if "n_keep" not in o:
        o["n_keep"] = torch.empty(batch, dtype=torch.int32, device=dev)
    if "cu_nodes" not in o:
        o["cu_nodes"] = torch.empty(batch + 1, dtype=torch.int32, device=dev)
    if "parent" not in o:
        o["parent"] = torch.empty(max(int(budget), 1), dtype=torch.int32, device=dev)
    if "packed_tokens" not in o:
        o["packed_tokens"] = torch.empty(max(int(budget), 1), dtype=torch.int32, device=dev)
    st = lib.tv_dcut_select(_ptr(conf), _ptr(tokens), batch, d, int(budget), _ptr(o["n_keep"]),
                            _ptr(o["cu_nodes"]), _ptr(o["parent"]), _ptr(o["packed_tokens"]),
                            _stream())
    _check("tv_dcut_select", st)
    return o["n_keep"], o["cu_nodes"], o["parent"][:budget], o["packed_tokens"][:budget]


@_on_stream
def e2e_tv_stats(target_logits: torch.Tensor, draft_logits: torch.Tensor,
                 cu_branches: torch.Tensor | None, temperature: float = 1.0):
    """SpecOPD E2E-TV statistics (``tv_e2e_tv_stats``): logits [N, V] (bf16 or fp32).

    Returns (alpha [N], prefix_prob [N] or None, expected_len [B] or None), fp32.
    """
    lib = load_library()
    assert target_logits.shape == draft_logits.shape and target_logits.dim() == 2
    assert target_logits.dtype == draft_logits.dtype
    assert target_logits.is_contiguous() and draft_logits.is_contiguous()
    n, v = target_logits.shape
    dt = TV_F32 if target_logits.dtype == torch.float32 else TV_BF16
    dev = target_logits.device
    alpha = torch.empty(n, dtype=torch.float32, device=dev)
    nb = 0 if cu_branches is None else cu_branches.numel() - 1
    prefix = torch.empty(n, dtype=torch.float32, device=dev) if nb else None
    expected = torch.empty(max(nb, 1), dtype=torch.float32, device=dev) if nb else None
    cu = _dev_i32(cu_branches, dev) if nb else None
    st = lib.tv_e2e_tv_stats(_ptr(target_logits), _ptr(draft_logits), dt, n, v,
                             float(temperature), _ptr(cu), nb, _ptr(alpha), _ptr(prefix),
                             _ptr(expected), _stream())
    _check("tv_e2e_tv_stats", st)
    return alpha, prefix, expected


@_on_stream
def graft_retrieve(adj: torch.Tensor, root_tokens: torch.Tensor, tmpl_parent, tmpl_rank,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """Graft retrieval (``tv_graft_retrieve``): ``adj`` int32 [V, k], template as host lists.

    Returns int32 [B, T] retrieved tokens (-1 where there is none).
    """
    lib = load_library()
    assert adj.dtype == torch.int32 and adj.is_contiguous() and adj.dim() == 2
    v, k = adj.shape
    roots = _dev_i32(root_tokens, adj.device)
    par = (ctypes.c_int32 * len(tmpl_parent))(*[int(x) for x in tmpl_parent])
    rank = (ctypes.c_int32 * len(tmpl_rank))(*[int(x) for x in tmpl_rank])
    assert len(tmpl_parent) == len(tmpl_rank)
    if out is None:
        out = torch.empty((roots.numel(), len(tmpl_parent)), dtype=torch.int32, device=adj.device)
    st = lib.tv_graft_retrieve(_ptr(adj), v, k, _ptr(roots), roots.numel(), par, rank,
                               len(tmpl_parent), _ptr(out), _stream())
    _check("tv_graft_retrieve", st)
    return out


def graft_update_workspace_size(num_nodes: int, vocab: int, k: int, dtype=torch.bfloat16) -> int:
    """Bytes ``tv_graft_update`` needs for these shapes (0: none)."""
    dt = TV_F32 if dtype == torch.float32 else TV_BF16
    return int(load_library().tv_graft_update_workspace_size(num_nodes, vocab, k, dt))


@_on_stream
def graft_update(adj: torch.Tensor, target_logits: torch.Tensor, node_tokens: torch.Tensor,
                 workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Graft online update (``tv_graft_update``), in place on ``adj`` int32 [V, k].

    ``workspace`` (uint8, device) is allocated here when absent or too small.
    """
    lib = load_library()
    assert adj.dtype == torch.int32 and adj.is_contiguous() and adj.dim() == 2
    v, k = adj.shape
    assert target_logits.dim() == 2 and target_logits.shape[1] == v
    assert target_logits.is_contiguous()
    dt = TV_F32 if target_logits.dtype == torch.float32 else TV_BF16
    tok = _dev_i32(node_tokens, adj.device)
    n = tok.numel()
    assert n == target_logits.shape[0]
    need = int(lib.tv_graft_update_workspace_size(n, v, k, dt))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=adj.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.tv_graft_update(_ptr(adj), v, k, _ptr(target_logits), dt, n, _ptr(tok),
                             _ptr(workspace), ws_bytes, _stream())
    _check("tv_graft_update", st)
    return adj
