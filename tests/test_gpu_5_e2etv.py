"""GPU parity of tv_e2e_tv_stats against the oracle (float64 numpy).

Tolerance: alpha |g - r| <= 1e-4 + 1e-4 r. The kernel sums up to ~1.5e5
terms per row in fp32 with hardware exp2 / log2 (about 1 ulp each): with
per-thread runs of ~600 terms and a tree over the block the accumulated
error stays near 1e-5 relative; the log-normaliser enters every term's
exponent, adding about the same. Prefix products and their sums (up to 16
factors): |g - r| <= 1e-4 + 5e-4 |r|.
"""
import numpy as np
import pytest
import torch

import oracle
import tree_verification_attention_mask_amd as tv

pytestmark = pytest.mark.gpu


def _logits(rng, n, v, spread=3.0, noise=1.0):
    t = rng.normal(0.0, spread, size=(n, v)).astype(np.float32)
    d = (t + rng.normal(0.0, noise, size=(n, v))).astype(np.float32)
    return t, d


def _check(t, d, cu, temperature=1.0, dtype=torch.bfloat16, offset=0):
    tt = torch.from_numpy(t).to(dtype)
    dd = torch.from_numpy(d).to(dtype)
    if offset:   # rows that do not start on a 16-byte boundary
        n, v = tt.shape
        bt = torch.empty(n * v + offset, dtype=dtype, device="cuda")
        bd = torch.empty(n * v + offset, dtype=dtype, device="cuda")
        bt[offset:] = tt.reshape(-1).cuda()
        bd[offset:] = dd.reshape(-1).cuda()
        gt, gd = bt[offset:].view(n, v), bd[offset:].view(n, v)
    else:
        gt, gd = tt.cuda(), dd.cuda()
    cu_t = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    a, pre, ex = tv.e2e_tv_stats(gt, gd, cu_t, temperature)
    torch.cuda.synchronize()
    ra, rpre, rex = oracle.e2e_tv_stats(tt.float().numpy(), dd.float().numpy(),
                                        cu if cu is not None else [0, t.shape[0]], temperature)
    a = a.cpu().numpy()
    assert np.isfinite(a).all()
    np.testing.assert_array_less(np.abs(a - ra), 1e-4 + 1e-4 * ra)
    if cu is not None:
        np.testing.assert_array_less(np.abs(pre.cpu().numpy() - rpre), 1e-4 + 5e-4 * rpre)
        np.testing.assert_array_less(np.abs(ex.cpu().numpy() - rex), 1e-4 + 5e-4 * rex)
    return a, ra


def test_full_vocabulary_bf16():
    rng = np.random.default_rng(1)
    t, d = _logits(rng, 16, 151936)
    _check(t, d, [0, 8, 16])


@pytest.mark.parametrize("temperature", [0.7, 1.0, 2.0])
def test_fp32_rows_and_temperature(temperature):
    rng = np.random.default_rng(2)
    t, d = _logits(rng, 40, 4096, spread=2.0, noise=0.7)
    _check(t, d, [0, 16, 32, 40], temperature, dtype=torch.float32)


@pytest.mark.parametrize("v,offset,dtype", [(1001, 0, torch.bfloat16), (7, 0, torch.float32),
                                            (1, 0, torch.bfloat16), (4096, 3, torch.bfloat16),
                                            (4096, 1, torch.float32)])
def test_unaligned_and_ragged_vocabularies(v, offset, dtype):
    rng = np.random.default_rng(v + offset)
    t, d = _logits(rng, 12, v)
    _check(t, d, [0, 5, 5, 12], dtype=dtype, offset=offset)     # includes an empty branch


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_masked_vocabulary_entries(dtype):
    # -inf logits (a masked vocabulary) carry no probability: long masked runs,
    # a row masked everywhere but a few tokens, and masks that differ between
    # the target and the draft
    rng = np.random.default_rng(5)
    v = 151936
    t, d = _logits(rng, 6, v)
    t[0, : v // 2] = -np.inf
    d[0, : v // 2] = -np.inf
    t[1, 1000:] = -np.inf
    d[1, 5000:] = -np.inf
    t[2, rng.random(v) < 0.9] = -np.inf
    keep = rng.choice(v, 5, replace=False)
    mask = np.ones(v, bool)
    mask[keep] = False
    t[3, mask] = -np.inf
    d[4, : 3 * v // 4] = -np.inf
    _check(t, d, [0, 6], dtype=dtype)


def test_identical_and_disjoint_distributions():
    rng = np.random.default_rng(4)
    t, _ = _logits(rng, 4, 2048)
    a, _ = _check(t, t.copy(), None)
    assert (np.abs(a - 1.0) < 1e-4).all()
    t2 = np.full((2, 64), -30.0, np.float32)
    d2 = t2.copy()
    t2[:, 0] = 30.0
    d2[:, 1] = 30.0
    a2, _ = _check(t2, d2, None)
    assert (a2 < 1e-4).all()


def test_specopd_shape_sampled_branches():
    """512 branch nodes (32 branches x 16) over the 151,936-token vocabulary;
    four branches are checked against the oracle."""
    g = torch.Generator(device="cuda").manual_seed(5)
    n, v = 512, 151936
    t = (torch.randn((n, v), generator=g, device="cuda") * 3.0).to(torch.bfloat16)
    d = (t.float() + torch.randn((n, v), generator=g, device="cuda")).to(torch.bfloat16)
    cu = torch.arange(0, n + 1, 16, dtype=torch.int32, device="cuda")
    a, pre, ex = tv.e2e_tv_stats(t, d, cu, 1.0)
    torch.cuda.synchronize()
    for br in (0, 7, 19, 31):
        rows = slice(16 * br, 16 * br + 16)
        ra, rpre, rex = oracle.e2e_tv_stats(t[rows].float().cpu().numpy(),
                                            d[rows].float().cpu().numpy(), [0, 16], 1.0)
        ga = a[rows].cpu().numpy()
        np.testing.assert_array_less(np.abs(ga - ra), 1e-4 + 1e-4 * ra)
        np.testing.assert_array_less(np.abs(pre[rows].cpu().numpy() - rpre), 1e-4 + 5e-4 * rpre)
        assert abs(float(ex[br]) - rex[0]) <= 1e-4 + 5e-4 * rex[0]


def test_argument_checks():
    x = torch.zeros((2, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tv.TVError):
        tv.e2e_tv_stats(x, x, None, 0.0)
    with pytest.raises(tv.TVError):
        tv.e2e_tv_stats(x, x, None, float("inf"))
