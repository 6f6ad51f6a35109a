"""The C-ABI library loads and exports every symbol ``include/treeverify.h``
declares; host-side argument checks return the documented status codes before
anything is launched (no GPU needed: only early-return paths are called)."""
import ctypes
import os
import re

import numpy as np
import pytest

import tree_verification_attention_mask_amd as tv
from tree_verification_attention_mask_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "treeverify.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below returns before a launch


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tv_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = tv.load_library()
    names = declared_functions()
    assert names == sorted(binding.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    lib = tv.load_library()
    for code, text in [(0, b"ok"), (1, b"invalid argument"), (2, b"unsupported configuration"),
                       (3, b"workspace too small"), (4, b"HIP launch failed"),
                       (99, b"unknown status")]:
        assert lib.tv_status_string(code) == text


def test_workspace_size_is_a_pure_host_query():
    lib = tv.load_library()
    ws = lib.tv_tree_verify_attn_workspace_size
    assert ws(1, 60, 60, 4, 32, 8, 128, 1) == 0            # 64 keys fit one tile: one key split
    big = ws(1, 60, 60, 2048, 32, 8, 128, 1)
    assert big > 0 and big % 256 == 0
    assert ws(1, 60, 60, 2048, 32, 8, 128, 0) == 0         # fp32 path never splits
    assert ws(0, 60, 60, 2048, 32, 8, 128, 1) == 0         # invalid shape -> 0


# (batch, total_nodes, max_nodes, max_prefix_len, hq, hkv) of the measured workloads
PLAN_SHAPES = {"graft-60node-p2048": (1, 60, 60, 2048, 32, 8),
               "dcut-b64-chains": (64, 512, 16, 4096, 32, 8),
               "long-32k-b8-60node": (8, 480, 60, 32768, 64, 8),
               "specopd-trunk4096-32x16": (1, 4608, 4608, 0, 32, 8)}


@pytest.mark.parametrize("cus", [80, 256, 304])
@pytest.mark.parametrize("shape", sorted(PLAN_SHAPES))
def test_attention_plan_follows_the_compute_unit_count(cus, shape):
    """The split count aims at one workgroup per compute unit of the device
    the plan is made for; the splits cover every key; the workspace holds
    the split partials (bf16 o + fp32 m, l per row and split) and is 0
    without splits."""
    batch, total, maxn, maxp, hq, hkv = PLAN_SHAPES[shape]
    pl = tv.verify_attn_plan(batch, total, maxn, maxp, hq, hkv, 128, binding.torch.bfloat16, cus)
    assert pl["num_cus"] == cus
    keys = maxp + maxn
    tiles = -(-keys // 64)
    g = hq // hkv
    assert pl["keys_per_split"] % 64 == 0
    assert pl["splits"] * pl["keys_per_split"] >= keys
    assert (pl["splits"] - 1) * pl["keys_per_split"] < keys       # no empty split
    assert pl["row_blocks"] * pl["rows_per_block"] >= maxn * g
    base = batch * hkv * pl["row_blocks"]
    assert base * pl["splits"] <= max(cus, base), "more workgroups than one pass needs"
    tps = pl["keys_per_split"] // 64
    if base < cus and tps > 1:
        # one tile fewer per split would need more workgroups than one pass
        assert base * -(-tiles // (tps - 1)) > cus
    if pl["splits"] == 1:
        assert pl["workspace_bytes"] == 0
    else:
        rows = total * hq
        o = -(-pl["splits"] * rows * 128 * 2 // 256) * 256
        ml = -(-pl["splits"] * rows * 8 // 256) * 256
        assert pl["workspace_bytes"] >= o + ml
    # the workspace query plans for the current device (no GPU here: 256)
    if cus == 256:
        assert binding.verify_attn_workspace_size(batch, total, maxn, maxp, hq, hkv, 128,
                                                  binding.torch.bfloat16) == pl["workspace_bytes"]


def test_merge_chunk_shapes_reach_every_chunk_size():
    """The GPU test of the merge's chunk sizes (2, 4, 8 and 16 split
    positions loaded at once) uses shapes whose 256-CU plans reach each size."""
    import test_gpu_2_attn as t2
    seen = {}
    for batch, hq, hkv, prefix, nodes in t2._MERGE_CHUNK_SHAPES:
        pl = tv.verify_attn_plan(batch, batch * nodes, nodes, prefix, hq, hkv, 128,
                                 binding.torch.bfloat16, 256)
        s = pl["splits"]
        seen[2 if s <= 2 else 4 if s <= 4 else 8 if s <= 8 else 16] = s
    assert set(seen) == {2, 4, 8, 16}, seen
    assert all(s not in (2, 4, 8, 16) for s in list(seen.values())[1:]), seen  # unused positions


def test_wide_merge_shapes_have_their_split_counts():
    """The GPU test of the merge with 8 elements a lane (16,384 rows or more,
    at most 4 splits) uses shapes whose 256-CU plans give 4, 3 and 2 splits."""
    import test_gpu_2_attn as t2
    for batch, nodes, keys, splits in t2._WIDE_MERGE_SHAPES:
        pl = tv.verify_attn_plan(batch, batch * nodes, nodes, keys, 64, 8, 128,
                                 binding.torch.bfloat16, 256)
        assert (pl["splits"], pl["rows_per_block"]) == (splits, 256)
        assert batch * nodes * 64 >= 16384


def test_attention_plan_splits_are_whole_tiles():
    """Every plan's key splits are whole 64-key tiles and cover the longest
    request's keys once: the kernels mask only keys past a request's end, so
    a split ending inside a tile would also count the next split's keys."""
    rng = np.random.default_rng(8)
    for _ in range(400):
        batch = int(rng.integers(1, 65))
        max_nodes = int(rng.integers(1, 300))
        total = batch * int(rng.integers(1, max_nodes + 1))
        P = int(rng.integers(0, 70000))
        hkv = int(rng.choice([1, 2, 4, 8]))
        hq = hkv * int(rng.choice([1, 2, 4, 8]))
        d = int(rng.choice([64, 128]))
        cus = int(rng.choice([80, 256, 304]))
        pl = tv.verify_attn_plan(batch, total, max_nodes, P, hq, hkv, d, binding.torch.bfloat16, cus)
        kps, splits = pl["keys_per_split"], pl["splits"]
        assert kps % 64 == 0 and kps > 0, pl
        assert (splits - 1) * kps < P + max_nodes <= splits * kps, (P, max_nodes, pl)


def test_attention_plan_splits_grow_with_the_compute_units():
    s = [tv.verify_attn_plan(1, 60, 60, 2048, 32, 8, 128, binding.torch.bfloat16, c)["splits"]
         for c in (80, 256, 304)]
    assert s[0] < s[1] <= s[2]


def _attn(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, pages=10, table=FAKE, maxp=4, prefix=FAKE, cu=FAKE, batch=1,
             total=60, maxn=60, maxP=2048, hq=32, hkv=8, d=128, page=16, dtype=1, scale=0.08,
             out=FAKE, lse=None, ws=None, wsb=0)
    a.update(over)
    m = binding.Mask(0, 1, 0x1000, None, None)
    return lib.tv_tree_verify_attn(a["q"], a["k"], a["v"], a["pages"], a["table"], a["maxp"],
                                   a["prefix"], a["cu"], a["batch"], a["total"], a["maxn"],
                                   a["maxP"], a["hq"], a["hkv"], a["d"], a["page"], a["dtype"],
                                   ctypes.c_float(a["scale"]), ctypes.byref(m), a["out"],
                                   a["lse"], a["ws"], a["wsb"], None)


def test_attn_argument_checks():
    lib = tv.load_library()
    assert _attn(lib, q=None) == 1
    assert _attn(lib, hq=30) == 1            # Hq not a multiple of Hkv
    assert _attn(lib, dtype=7) == 1
    assert _attn(lib, d=96) == 2
    assert _attn(lib, page=6) == 2
    assert _attn(lib, page=48) == 2          # not a power of two
    assert _attn(lib, batch=0) == 1
    assert _attn(lib, maxn=65) == 1          # one mask word cannot hold 65 nodes
    assert _attn(lib) == 3                   # a 2048-key prefix needs split workspace
    assert _attn(lib, ws=FAKE, wsb=16) == 3


def test_mask_and_accept_argument_checks():
    lib = tv.load_library()
    mb = lib.tv_tree_mask_build
    assert mb(None, FAKE, 1, 4, 4, 0, 1, FAKE, None, None, FAKE, FAKE, None) == 1
    assert mb(FAKE, FAKE, 1, 4, 4, 0, 17, FAKE, None, None, FAKE, FAKE, None) == 2
    assert mb(FAKE, FAKE, 1, 2000, 2000, 0, 16, FAKE, None, None, FAKE, FAKE, None) == 2
    assert mb(FAKE, FAKE, 1, 100, 100, 0, 1, FAKE, None, None, FAKE, FAKE, None) == 1
    assert mb(FAKE, FAKE, 1, 4, 4, 1, 0, None, None, None, FAKE, FAKE, None) == 1
    assert mb(FAKE, FAKE, 1, 4, 4, 5, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    ac = lib.tv_tree_accept
    assert ac(None, FAKE, FAKE, FAKE, 1, 4, 4, 3, FAKE, FAKE, None, None) == 1
    assert ac(FAKE, FAKE, FAKE, FAKE, 1, 4, 4, -1, FAKE, FAKE, None, None) == 1
    assert ac(FAKE, FAKE, FAKE, FAKE, 1, 9000, 9000, 3, FAKE, FAKE, None, None) == 2


def test_dcut_argument_checks():
    lib = tv.load_library()
    ds = lib.tv_dcut_select
    assert ds(None, FAKE, 4, 3, 8, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert ds(FAKE, FAKE, 0, 3, 8, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert ds(FAKE, FAKE, 4, 0, 8, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert ds(FAKE, FAKE, 4, 3, 3, FAKE, FAKE, FAKE, FAKE, None) == 1    # budget < batch
    assert ds(FAKE, FAKE, 4, 3, 17, FAKE, FAKE, FAKE, FAKE, None) == 1   # budget > batch*(D+1)
    assert ds(FAKE, FAKE, 4097, 8, 5000, FAKE, FAKE, FAKE, FAKE, None) == 2  # > 32768 positions


def test_e2e_tv_argument_checks():
    lib = tv.load_library()
    f = lib.tv_e2e_tv_stats
    c = ctypes.c_float
    assert f(None, FAKE, 1, 4, 100, c(1.0), FAKE, 1, FAKE, FAKE, FAKE, None) == 1
    assert f(FAKE, FAKE, 1, 0, 100, c(1.0), FAKE, 1, FAKE, FAKE, FAKE, None) == 1
    assert f(FAKE, FAKE, 1, 4, 0, c(1.0), FAKE, 1, FAKE, FAKE, FAKE, None) == 1
    assert f(FAKE, FAKE, 5, 4, 100, c(1.0), FAKE, 1, FAKE, FAKE, FAKE, None) == 1   # dtype
    assert f(FAKE, FAKE, 1, 4, 100, c(0.0), FAKE, 1, FAKE, FAKE, FAKE, None) == 1   # T
    assert f(FAKE, FAKE, 1, 4, 100, c(1.0), None, 1, FAKE, FAKE, FAKE, None) == 1   # branches


def test_graft_argument_checks():
    lib = tv.load_library()
    I3 = ctypes.c_int32 * 3
    par, rank = I3(-1, 0, 1), I3(0, 1, 0)
    r = lib.tv_graft_retrieve
    assert r(None, 10, 4, FAKE, 2, par, rank, 3, FAKE, None) == 1
    assert r(FAKE, 10, 17, FAKE, 2, par, rank, 3, FAKE, None) == 2          # k > 16
    assert r(FAKE, 10, 4, FAKE, 2, I3(-1, 2, 0), rank, 3, FAKE, None) == 1  # not topological
    assert r(FAKE, 10, 1, FAKE, 2, par, rank, 3, FAKE, None) == 1          # rank 1 >= k
    u = lib.tv_graft_update
    assert u(FAKE, 10, 11, FAKE, 1, 4, FAKE, None, 0, None) == 1          # k > vocab
    assert u(FAKE, 100, 17, FAKE, 1, 4, FAKE, None, 0, None) == 2
    assert u(FAKE, 100, 8, FAKE, 3, 4, FAKE, None, 0, None) == 1          # dtype
    assert u(FAKE, (1 << 30) + 1, 8, FAKE, 1, 4, FAKE, None, 0, None) == 2  # vocab
    ws = lib.tv_graft_update_workspace_size
    assert ws(4, 100, 8, 1) == 0                 # one workgroup per row
    need = ws(60, 151936, 8, 1)                  # a row per verified node: split rows
    assert need > 0 and need % 256 == 0
    assert ws(60, 151936, 8, 0) > 0
    assert ws(60, 151936, 8, 3) == 0             # bad dtype: nothing to size
    assert ws(9, 5, 1, 1) == 0 and ws(1, 1, 1, 0) == 0   # below one 16-byte group
    # a workspace below what the call's path needs is refused before anything
    # is launched: 16-byte-aligned bf16 rows take the share kernel (4 shares
    # of k entries of 8 bytes per node here), other rows the one-value shares
    # (9 shares per node here); the query covers both
    assert u(FAKE, 151936, 8, FAKE, 1, 60, FAKE, None, 0, None) == 3
    assert u(FAKE, 151936, 8, FAKE, 1, 60, FAKE, FAKE, 60 * 4 * 8 * 8 - 1, None) == 3
    odd = ctypes.c_void_p(FAKE.value + 2)        # bf16-aligned, not 16-byte aligned
    assert u(FAKE, 151936, 8, odd, 1, 60, FAKE, FAKE, 60 * 9 * 8 * 8 - 1, None) == 3
    assert need >= max(60 * 4 * 8 * 8, 60 * 9 * 8 * 8)


def test_sampled_accept_argument_checks():
    lib = tv.load_library()
    f = lib.tv_tree_accept_sampled
    c = ctypes.c_float
    ok = dict(batch=1, total=4, max_nodes=4, max_children=3, max_depth=3, dtype=1, vocab=10,
              temp=1.0, ws=FAKE, ws_bytes=1 << 20)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(FAKE, FAKE, FAKE, a["batch"], a["total"], a["max_nodes"], a["max_children"],
                 a["max_depth"], FAKE, FAKE, a["dtype"], a["vocab"], c(a["temp"]), FAKE, FAKE,
                 FAKE, FAKE, FAKE, a["ws"], a["ws_bytes"], None)
    assert call(batch=0) == 0                      # nothing to do
    assert call(max_depth=-1) == 1
    assert call(temp=0.0) == 1 and call(temp=float("nan")) == 1 and call(temp=float("inf")) == 1
    assert call(vocab=0) == 1 and call(dtype=2) == 1
    assert call(max_nodes=8193) == 2 and call(max_children=513) == 2
    need = lib.tv_tree_accept_sampled_workspace_size(4, 3, 10)
    assert need > 0 and need % 256 == 0
    assert lib.tv_tree_accept_sampled_workspace_size(0, 3, 10) == 0
    assert lib.tv_tree_accept_sampled_workspace_size(60, 4, 151936) > need
    assert call(ws=None, ws_bytes=0) == 3 and call(ws_bytes=need - 1) == 3
    assert call(ws=ctypes.c_void_p(0x1008)) == 1   # not 256-byte aligned


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "tree_verification_attention_mask_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower().replace("oracle-free", ""), f


def test_noalloc_attention_refuses_plans_beyond_its_scratch_array():
    """tv_tree_verify_attn_noalloc: 8 requests of 60 nodes behind 131,072-key
    prefixes (64 query heads) plan three key splits whose partials (23 MiB)
    exceed the 16 MiB scratch array: TV_ERR_WORKSPACE before anything is
    enqueued; argument errors come first, as in tv_tree_verify_attn."""
    lib = tv.load_library()
    need = lib.tv_tree_verify_attn_workspace_size(8, 480, 60, 131072, 64, 8, 128, 1)
    assert need > 16 << 20
    m = binding.Mask(0, 1, 0x1000, None, None)

    def call(q=FAKE, batch=8, total=480, maxp=131072, hq=64):
        return lib.tv_tree_verify_attn_noalloc(q, FAKE, FAKE, 100000, FAKE, 8193, FAKE, FAKE,
                                               batch, total, 60, maxp, hq, 8, 128, 16, 1,
                                               ctypes.c_float(0.088), ctypes.byref(m), FAKE,
                                               None, None)
    assert call() == 3
    assert call(q=None) == 1
    assert call(hq=60) == 1             # 60 % 8 != 0

