"""GPU parity of tv_graft_retrieve and tv_graft_update against the oracle:
every token bit-exact (integer lookups and exact comparisons of the input
logits). Covers the full 151,936-token vocabulary, empty and out-of-range
table entries, templates up to 64 nodes, repeated tokens among the verified
nodes, ties, NaN logits, k = 1 / 8 / 16, and update-then-retrieve."""
import numpy as np
import pytest
import torch

import oracle
import tree_verification_attention_mask_amd as tv
import workloads as W

pytestmark = pytest.mark.gpu


def _table(rng, v, k, holes=0.05):
    adj = rng.integers(0, v, size=(v, k)).astype(np.int32)
    adj[rng.random((v, k)) < holes] = -1
    adj[rng.random((v, k)) < holes / 5] = v + 7        # out of range
    return adj


def _template(rng, n, k):
    par = [-1] + [int(rng.integers(-1, j)) for j in range(1, n)]
    rank = [int(rng.integers(0, k)) for _ in range(n)]
    return par, rank


def _retrieve(adj, roots, par, rank):
    a = torch.from_numpy(adj).cuda()
    r = torch.as_tensor(np.asarray(roots, np.int32)).cuda()
    out = tv.graft_retrieve(a, r, par, rank)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("v,k,n,batch", [(151936, 8, 20, 1), (151936, 8, 64, 37), (500, 16, 64, 300),
                                         (50, 1, 10, 5), (1000, 4, 1, 9)])
def test_retrieve_matches_the_oracle(v, k, n, batch):
    rng = np.random.default_rng(v + n + batch)
    adj = _table(rng, v, k)
    par, rank = _template(rng, n, k)
    roots = rng.integers(-2, v + 2, size=batch)
    np.testing.assert_array_equal(_retrieve(adj, roots, par, rank),
                                  oracle.graft_retrieve(adj, roots, par, rank))


def test_retrieve_graft_tree_template():
    """The 20 retrieved slots of the Graft-shaped tree: four successors of the
    graft point; the first heads a chain of four levels keeping three
    successors each, the others keep 2, 1, 1 (its nodes 40..59, re-rooted)."""
    p = W.GRAFT_TREE_PARENT
    graft = p[40]
    local = {graft: -1}
    par, rank, kids = [], [], {}
    for j in range(40, 60):
        local[j] = j - 40
        pp = local[p[j]]
        kids[pp] = kids.get(pp, 0) + 1
        par.append(pp)
        rank.append(kids[pp] - 1)
    rng = np.random.default_rng(60)
    adj = _table(rng, 151936, 8, holes=0.0)
    roots = [17, 151935, 4242]
    np.testing.assert_array_equal(_retrieve(adj, roots, par, rank),
                                  oracle.graft_retrieve(adj, roots, par, rank))


def _update(adj, logits, toks, dtype):
    a = torch.from_numpy(adj.copy()).cuda()
    lg = torch.from_numpy(logits).to(dtype).cuda()
    tv.graft_update(a, lg, torch.as_tensor(np.asarray(toks, np.int32)).cuda())
    torch.cuda.synchronize()
    return a.cpu().numpy(), lg.float().cpu().numpy()


@pytest.mark.parametrize("dtype,k", [(torch.bfloat16, 8), (torch.float32, 16), (torch.bfloat16, 1)])
def test_update_full_vocabulary(dtype, k):
    rng = np.random.default_rng(k)
    v, n = 151936, 60
    adj = _table(rng, v, k)
    logits = rng.normal(0, 3, size=(n, v)).astype(np.float32)
    toks = rng.integers(0, v, size=n)
    toks[10] = toks[3]          # repeated tokens: the later node writes the row
    toks[40] = toks[3]
    toks[5] = -1                # updates nothing
    toks[6] = v
    got, exact = _update(adj, logits, toks, dtype)
    np.testing.assert_array_equal(got, oracle.graft_update(adj, exact, toks))


def test_update_ties_and_nan():
    rng = np.random.default_rng(9)
    v, n, k = 4096, 16, 8
    adj = _table(rng, v, k)
    logits = rng.choice(np.array([0.0, 1.0, 2.0, -1.0], np.float32), size=(n, v))
    logits[rng.random((n, v)) < 0.01] = np.nan
    logits[3, :] = np.nan                   # a row of NaNs: the k smallest ids
    logits[4, :] = 5.0                      # all equal
    toks = rng.integers(0, v, size=n)
    for dtype in (torch.float32, torch.bfloat16):
        got, exact = _update(adj, logits, toks, dtype)
        np.testing.assert_array_equal(got, oracle.graft_update(adj, exact, toks))


@pytest.mark.parametrize("v,k", [(13, 13), (1001, 16), (5, 1), (70, 7), (151937, 8)])
def test_update_small_and_ragged_vocabularies(v, k):
    # vocabularies below one batch of 64 per wave, k == vocab, and sizes that
    # leave a tail after the 16-byte groups (or no groups at all)
    rng = np.random.default_rng(v + k)
    n = 9
    adj = _table(rng, v, k)
    logits = rng.normal(0, 2, size=(n, v)).astype(np.float32)
    logits[2, :] = -np.inf                  # every entry ties at -inf
    logits[4, rng.random(v) < 0.5] = np.nan
    toks = rng.permutation(v)[:n] if v >= n else rng.integers(0, v, size=n)
    for dtype in (torch.float32, torch.bfloat16):
        got, exact = _update(adj, logits, toks, dtype)
        np.testing.assert_array_equal(got, oracle.graft_update(adj, exact, toks))


def test_update_unaligned_rows():
    # a logits view starting one element in: no 16-byte loads
    rng = np.random.default_rng(3)
    v, n, k = 4096, 12, 8
    adj = _table(rng, v, k)
    base = rng.normal(0, 1, size=n * v + 1).astype(np.float32)
    toks = rng.integers(0, v, size=n).astype(np.int32)
    a = torch.from_numpy(adj.copy()).cuda()
    lg = torch.from_numpy(base).cuda()[1:].view(n, v)
    tv.graft_update(a, lg, torch.from_numpy(toks).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a.cpu().numpy(), oracle.graft_update(adj, base[1:].reshape(n, v), toks))


@pytest.mark.parametrize("n,v,k,dtype,offset", [
    (3, 151936, 16, torch.float32, 1),    # one-value loads, 32 shares per row, 512 partials
    (2, 151936, 16, torch.bfloat16, 0),   # 16-byte loads, the most shares per row
    (600, 5000, 8, torch.bfloat16, 0),    # one workgroup per row, many rows
    (257, 70001, 4, torch.float32, 0),    # odd vocabulary, two shares per row
])
def test_update_row_shares(n, v, k, dtype, offset):
    rng = np.random.default_rng(n + k)
    adj = _table(rng, v, k)
    base = rng.normal(0, 2, size=n * v + offset).astype(np.float32)
    toks = rng.integers(0, v, size=n).astype(np.int32)
    toks[-1] = toks[0]                       # the last node writes that row
    a = torch.from_numpy(adj.copy()).cuda()
    lg = torch.from_numpy(base).to(dtype).cuda()[offset:].view(n, v)
    need = tv.graft_update_workspace_size(n, v, k, dtype)
    ws = torch.full((max(need, 1),), 0xAB, dtype=torch.uint8, device="cuda")  # stale contents
    tv.graft_update(a, lg, torch.from_numpy(toks).cuda(), workspace=ws)
    torch.cuda.synchronize()
    exact = lg.float().cpu().numpy()
    np.testing.assert_array_equal(a.cpu().numpy(), oracle.graft_update(adj, exact, toks))


def _threshold_rows(rng, v, k):
    """bf16 rows for the whole-row workgroup's thresholds: each row reaches
    one branch of its bound T (plain bits, flipped bits for negative tops,
    the exact wave lists when T bounds nothing)."""
    rows = []
    rows.append(rng.normal(-12, 3, size=v))                        # log-probabilities: all < 0
    r = np.full(v, -np.inf); r[rng.choice(v, k, replace=False)] = rng.normal(0, 1, k)
    rows.append(r)                                                 # exactly k finite values
    r = np.full(v, -np.inf); r[rng.choice(v, max(k - 1, 0), replace=False)] = 1.5
    rows.append(r)                                                 # fewer than k finite: -inf ties
    r = rng.normal(-5, 1, size=v); at = rng.choice(v, 10, replace=False)
    r[at[:5]] = 0.0; r[at[5:]] = -0.0
    rows.append(r)                                                 # +0 and -0 on top
    r = rng.normal(0, 1, size=v); r[rng.choice(v, 1000, replace=False)] = 7.0
    rows.append(r)                                                 # a plateau of 1000 equal tops
    r = rng.normal(0, 3, size=v); r[rng.random(v) < 0.05] = np.nan
    rows.append(r)                                                 # positive NaNs
    r = rng.normal(0, 3, size=v); r[rng.random(v) < 0.05] = -np.nan
    rows.append(r)                                                 # negative NaNs
    r = rng.normal(0, 1, size=v); r[rng.random(v) < 0.5] = np.inf
    rows.append(r)                                                 # +inf everywhere
    r = rng.normal(0, 1, size=v); r[rng.choice(v, 3, replace=False)] = np.inf
    rows.append(r)                                                 # a few +inf on top
    r = np.full(v, -np.inf); r[rng.choice(v, 5, replace=False)] = np.nan
    rows.append(r)                                                 # -inf and NaN only
    r = rng.normal(0, 3, size=v); top = np.argsort(-r)[:k + 3]; r[top] = r[top[0]]
    rows.append(r)                                                 # k + 3 ties at the maximum
    r = -np.abs(rng.normal(0, 1e-3, size=v)); r[rng.choice(v, 20, replace=False)] = -0.0
    rows.append(r)                                                 # negative tops near -0
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("v,k", [(151936, 8), (151936, 16), (151936, 1), (5000, 8)])
def test_update_whole_row_thresholds(v, k):
    """Rows of one workgroup each (bf16, 16-byte aligned, vocabulary a multiple
    of 8): every table row against the oracle, for rows built to reach each
    way the row's bound T is found or refused."""
    rng = np.random.default_rng(v + 31 * k)
    logits = _threshold_rows(rng, v, k)
    n = logits.shape[0]
    adj = _table(rng, v, k)
    toks = rng.permutation(v)[:n].astype(np.int32)
    lg = torch.from_numpy(logits).to(torch.bfloat16)
    bits = lg.view(torch.int16)                            # NaN bits set from numpy's sign
    nan = np.isnan(logits)
    neg_nan = torch.from_numpy(nan & np.signbit(logits))
    pos_nan = torch.from_numpy(nan & ~np.signbit(logits))
    bits[neg_nan] = np.int16(-64)                          # 0xffc0
    bits[pos_nan] = np.int16(0x7fc0)
    assert int(neg_nan.sum()) > 0 and int(pos_nan.sum()) > 0
    a = torch.from_numpy(adj.copy()).cuda()
    tv.graft_update(a, lg.cuda(), torch.from_numpy(toks).cuda())
    torch.cuda.synchronize()
    exact = lg.float().numpy()
    np.testing.assert_array_equal(a.cpu().numpy(), oracle.graft_update(adj, exact, toks))


def _mixed_row(rng, v):
    kind = rng.integers(0, 6)
    if kind == 0:
        return rng.normal(0, 3, size=v)
    if kind == 1:
        return rng.normal(-20, 2, size=v)                                # all negative
    if kind == 2:
        return np.round(rng.normal(0, 2, size=v))                        # many ties
    if kind == 3:
        r = np.full(v, -np.inf)
        m = int(rng.integers(0, 40))
        r[rng.choice(v, m, replace=False)] = rng.normal(0, 1, m)         # few finite values
        return r
    r = rng.normal(0, 1, size=v)
    r[rng.random(v) < 0.02] = rng.choice([np.nan, np.inf, -np.inf, 0.0, -0.0])
    if kind == 5:
        r[rng.integers(0, v)] = np.inf
    return r


@pytest.mark.parametrize("seed", range(6))
def test_update_share_boundaries_sweep(seed):
    """Seeded sweep of the bf16 share path: vocabularies around multiples of
    one share (40,960 entries), 1 to 8 shares, k in 1..16 within the list
    kernel's 64 entries, rows of mixed kinds (normal, all negative, ties,
    few finite values, scattered NaN / +-inf / +-0), repeated tokens; every
    table row against the oracle."""
    rng = np.random.default_rng(900 + seed)
    share = 40960
    shares = int(rng.integers(1, 9))
    v = 8 * int(rng.integers(max(1, (shares - 1) * share // 8 + 1), shares * share // 8 + 1))
    k = int(rng.integers(1, min(16, 64 // shares) + 1))
    n = int(rng.integers(1, 40))
    logits = np.stack([_mixed_row(rng, v) for _ in range(n)]).astype(np.float32)
    adj = _table(rng, v, k)
    toks = rng.integers(0, v, size=n).astype(np.int32)
    if n > 3:
        toks[n - 1] = toks[1]
    print("sweep", seed, dict(v=v, k=k, n=n, shares=shares), flush=True)
    got, exact = _update(adj, logits, toks, torch.bfloat16)
    np.testing.assert_array_equal(got, oracle.graft_update(adj, exact, toks))


def test_update_many_nodes_one_workgroup_per_row():
    # thousands of verified nodes: one workgroup per row, many repeated tokens
    rng = np.random.default_rng(45)
    v, n, k = 2000, 3000, 16
    adj = _table(rng, v, k)
    logits = rng.normal(0, 2, size=(n, v)).astype(np.float32)
    toks = rng.integers(0, v, size=n).astype(np.int32)
    got, exact = _update(adj, logits, toks, torch.bfloat16)
    np.testing.assert_array_equal(got, oracle.graft_update(adj, exact, toks))


def test_update_then_retrieve_on_device():
    rng = np.random.default_rng(12)
    v, k = 30000, 4
    adj = np.full((v, k), -1, np.int32)
    toks = rng.integers(0, v, size=32)
    logits = rng.normal(0, 1, size=(32, v)).astype(np.float32)
    a = torch.from_numpy(adj).cuda()
    tv.graft_update(a, torch.from_numpy(logits).cuda(), torch.from_numpy(toks.astype(np.int32)).cuda())
    par, rank = [-1, 0, 1, -1, 3], [0, 1, 0, 2, 0]
    out = tv.graft_retrieve(a, torch.from_numpy(toks[:8].astype(np.int32)).cuda(), par, rank)
    torch.cuda.synchronize()
    ref_adj = oracle.graft_update(adj, logits, toks)
    np.testing.assert_array_equal(a.cpu().numpy(), ref_adj)
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.graft_retrieve(ref_adj, toks[:8], par, rank))


def test_bad_templates_are_refused():
    a = torch.zeros((10, 4), dtype=torch.int32, device="cuda")
    r = torch.zeros(2, dtype=torch.int32, device="cuda")
    for par, rank in ([[-1, 1], [0, 0]], [[-1, -2], [0, 0]], [[-1, 0], [0, 4]]):
        with pytest.raises(tv.TVError) as e:
            tv.graft_retrieve(a, r, par, rank)
        assert e.value.status == 1
    with pytest.raises(tv.TVError) as e:
        tv.graft_retrieve(a, r, [-1] * 65, [0] * 65)
    assert e.value.status == 2
