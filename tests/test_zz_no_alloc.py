"""tv_tree_verify_attn_noalloc: the attention call with its split partials in
the library's per-device scratch array instead of a caller workspace. Two
calls in a row (the headline Graft-shaped tree with its 2048-key prefix and
11 key splits, then a smaller one: a 300-key prefix, fewer splits) through the
C ABI give bit for bit the outputs of tv_tree_verify_attn with a workspace on
the same inputs, and both are within the attention tolerance of the oracle."""
import numpy as np
import pytest
import torch

import tree_verification_attention_mask_amd as tv
import workloads as W
from tv_testlib import Dev, all_rows, assert_attn_close, oracle_attn, oracle_attn_threaded

pytestmark = pytest.mark.gpu


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    for prefix in (2048, 300):          # the second call is smaller
        w = W.make(2, prefix=prefix)
        pl = tv.verify_attn_plan(w.batch, w.total_nodes, w.max_nodes, w.max_prefix_len,
                                 w.num_q_heads, w.num_kv_heads, w.head_dim, torch.bfloat16)
        print("prefix", prefix, "plan", pl, flush=True)
        assert pl["splits"] > 1 and pl["workspace_bytes"] > 0      # the scratch array is used
        d = Dev(w)
        m = d.mask()
        ref_out, ref_lse = d.attn(mask=m)
        out = torch.full_like(d.q, float("nan"))
        lse = torch.full((w.total_nodes, w.num_q_heads), float("nan"), device=d.q.device)
        tv.tree_verify_attn_noalloc(d.q, d.k, d.v, d.table, d.prefix, d.cu, m, w.max_nodes,
                                    w.max_prefix_len, out, lse, scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
        ref, rlse = oracle_attn(w)
        print(assert_attn_close(out, ref, "bf16", lse, rlse, what="noalloc P=%d" % prefix))


def test_noalloc_256_row_blocks_with_the_wide_merge():
    """The entry point on the tile-loop kernel's 256-row blocks and the merge
    with 16-byte lanes (8 requests of a 60-node tree over 3000 keys, 64 q / 8
    kv heads: 30,720 rows, 2 splits, 16,220,160 bytes of partials within the
    16 MiB scratch), then a smaller call on the headline tree: both bit for
    bit the workspace entry point's, the first also against the oracle on
    sampled rows."""
    rng = np.random.default_rng(321)
    trees = [W.random_tree(rng, 60) for _ in range(8)]
    big = W.build_workload("noalloc-wide", trees, [3000] * 8, 64, 8, 128, "bf16", rng,
                           permute_pages=True, tokens=False)
    for w in (big, W.make(2, prefix=700)):
        pl = tv.verify_attn_plan(w.batch, w.total_nodes, w.max_nodes, w.max_prefix_len,
                                 w.num_q_heads, w.num_kv_heads, w.head_dim, torch.bfloat16)
        print(w.name, "plan", pl, flush=True)
        assert pl["splits"] > 1 and 0 < pl["workspace_bytes"] <= 16 << 20
        d = Dev(w)
        m = d.mask()
        ref_out, ref_lse = d.attn(mask=m)
        out = torch.full_like(d.q, float("nan"))
        lse = torch.full((w.total_nodes, w.num_q_heads), float("nan"), device=d.q.device)
        tv.tree_verify_attn_noalloc(d.q, d.k, d.v, d.table, d.prefix, d.cu, m, w.max_nodes,
                                    w.max_prefix_len, out, lse, scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
        if w is big:
            assert pl["rows_per_block"] == 256 and w.total_nodes * w.num_q_heads >= 16384
            rows = all_rows(w)
            pick = rows[np.random.default_rng(5).choice(len(rows), 512, replace=False)]
            ref, rlse = oracle_attn_threaded(w, rows=pick)
            got = out[pick[:, 0], pick[:, 1]].float().cpu().numpy()
            gl = lse[pick[:, 0], pick[:, 1]].cpu().numpy()
            print(assert_attn_close(got, ref, "bf16", gl, rlse, what="noalloc wide"))
