"""Parity at the full benchmark sizes (configs 2-5), in the launch
configuration the benchmark times: the whole batch runs on the GPU; the
oracle (on host threads) recomputes every output element of configs 2, 3
and 5, and of config 4 (32K-key prefixes, 8 requests) whole row blocks of the
launch plan -- for the first request, the last one and the one with the most
keys: every (node, query head) row of the first row block, the last one, the
one holding the deepest node and the one with the most visible (row, key)
pairs -- plus a seeded sample of other rows. Masks and acceptance are
compared in full, bit-exactly."""
import numpy as np
import pytest
import torch

import oracle
import tree_verification_attention_mask_amd as tv
import workloads as W
from tv_testlib import Dev, all_rows, assert_attn_close, mask_bits_u64, oracle_attn_threaded

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _whole_blocks(w, depth, rows_per_block, n_rand=48, seed=0):
    """Rows of the chosen row blocks (all query heads of their nodes) plus a
    seeded sample of single rows."""
    g = w.num_q_heads // w.num_kv_heads
    assert rows_per_block % g == 0
    per = rows_per_block // g                      # tree nodes per row block
    keys = w.prefix_len.astype(np.int64) + w.nodes_per_request
    reqs = sorted({0, w.batch - 1, int(np.argmax(keys))})
    nodes = set()
    for b in reqs:
        n0, n1 = int(w.cu_nodes[b]), int(w.cu_nodes[b + 1])
        blocks = [(s, min(s + per, n1)) for s in range(n0, n1, per)]
        dep = [depth[s:e] for s, e in blocks]
        pick = {0, len(blocks) - 1, int(np.argmax([d.max() for d in dep])),
                int(np.argmax([(d.astype(np.int64) + 1).sum() for d in dep]))}
        for k in pick:
            nodes.update(range(*blocks[k]))
    rows = {tuple(r) for r in all_rows(w, sorted(nodes))}
    rng = np.random.default_rng(seed)
    for _ in range(n_rand):
        rows.add((int(rng.integers(w.total_nodes)), int(rng.integers(w.num_q_heads))))
    return np.array(sorted(rows), np.int32), len(nodes)


@pytest.mark.parametrize("config", [2, 3, 4, 5])
def test_full_size_parity(config):
    print("full-size config", config, flush=True)
    w = W.make(config)
    d = Dev(w)
    m = d.mask()
    out, lse = d.attn(mask=m)
    torch.cuda.synchronize()
    if w.mask_kind == "bits":
        bits, depth, err = oracle.mask_bits(w.parent, w.cu_nodes, w.words_per_node)
        np.testing.assert_array_equal(mask_bits_u64(m["bits"]), bits)
    else:
        ap, bd, depth, err = oracle.mask_anchor(w.parent, w.cu_nodes)
        np.testing.assert_array_equal(m["anchor_pos"].cpu().numpy(), ap)
        np.testing.assert_array_equal(m["branch_depth"].cpu().numpy(), bd)
    np.testing.assert_array_equal(m["depth"].cpu().numpy(), depth)
    np.testing.assert_array_equal(m["err"].cpu().numpy(), err)
    pl = tv.verify_attn_plan(w.batch, w.total_nodes, w.max_nodes, w.max_prefix_len,
                             w.num_q_heads, w.num_kv_heads, w.head_dim, torch.bfloat16)
    if config == 4:
        rows, n_nodes = _whole_blocks(w, depth, pl["rows_per_block"], seed=config)
    else:
        rows, n_nodes = all_rows(w), w.total_nodes
    print("plan", pl, "-- oracle over", len(rows), "rows of", n_nodes, "nodes", flush=True)
    ref, rlse = oracle_attn_threaded(w, rows)
    got = out[rows[:, 0], rows[:, 1]].float().cpu().numpy()
    gl = lse[rows[:, 0], rows[:, 1]].cpu().numpy()
    st = assert_attn_close(got, ref, w.dtype, gl, rlse, what="config%d" % config)
    print(st)
    # the whole output is finite
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    if w.draft_tok is not None:
        al, path, bonus = d.accept()
        oal, opath, obonus = oracle.accept(w.parent, w.draft_tok, w.target_tok, w.cu_nodes,
                                           w.max_depth)
        np.testing.assert_array_equal(al.cpu().numpy(), oal)
        np.testing.assert_array_equal(path.cpu().numpy(), opath)
        np.testing.assert_array_equal(bonus.cpu().numpy(), obonus)
