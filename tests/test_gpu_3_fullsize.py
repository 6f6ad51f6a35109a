"""Parity at the full benchmark sizes (configs 2-5), in the launch
configuration the benchmark times: the whole batch runs on the GPU and the
oracle recomputes a seeded sample of (node, head) rows one by one; masks and
acceptance are compared in full, bit-exactly."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tv_testlib import Dev, assert_attn_close, mask_bits_u64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _sample_rows(w, n_rand=48, seed=0):
    rng = np.random.default_rng(seed)
    rows = set()
    for b in (0, w.batch - 1):
        n0, n1 = int(w.cu_nodes[b]), int(w.cu_nodes[b + 1])
        for node in (n0, n1 - 1, (n0 + n1) // 2):
            rows.add((node, 0))
            rows.add((node, w.num_q_heads - 1))
    for _ in range(n_rand):
        rows.add((int(rng.integers(w.total_nodes)), int(rng.integers(w.num_q_heads))))
    return np.array(sorted(rows), np.int32)


@pytest.mark.parametrize("config", [2, 3, 4, 5])
def test_full_size_parity(config):
    print("full-size config", config, flush=True)
    w = W.make(config)
    d = Dev(w)
    m = d.mask()
    out, lse = d.attn(mask=m)
    torch.cuda.synchronize()
    rows = _sample_rows(w, seed=config)
    ref, rlse = oracle.tree_attn(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_len,
                                 w.cu_nodes, w.parent, w.num_q_heads, w.num_kv_heads, w.scale,
                                 rows=rows)
    got = out[rows[:, 0], rows[:, 1]].float().cpu().numpy()
    gl = lse[rows[:, 0], rows[:, 1]].cpu().numpy()
    st = assert_attn_close(got, ref, w.dtype, gl, rlse, what="config%d" % config)
    print(st)
    # the whole output is finite and the mask / acceptance are exact
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    if w.mask_kind == "bits":
        bits, depth, err = oracle.mask_bits(w.parent, w.cu_nodes, w.words_per_node)
        np.testing.assert_array_equal(mask_bits_u64(m["bits"]), bits)
    else:
        ap, bd, depth, err = oracle.mask_anchor(w.parent, w.cu_nodes)
        np.testing.assert_array_equal(m["anchor_pos"].cpu().numpy(), ap)
        np.testing.assert_array_equal(m["branch_depth"].cpu().numpy(), bd)
    np.testing.assert_array_equal(m["depth"].cpu().numpy(), depth)
    np.testing.assert_array_equal(m["err"].cpu().numpy(), err)
    if w.draft_tok is not None:
        al, path, bonus = d.accept()
        oal, opath, obonus = oracle.accept(w.parent, w.draft_tok, w.target_tok, w.cu_nodes,
                                           w.max_depth)
        np.testing.assert_array_equal(al.cpu().numpy(), oal)
        np.testing.assert_array_equal(path.cpu().numpy(), opath)
        np.testing.assert_array_equal(bonus.cpu().numpy(), obonus)
