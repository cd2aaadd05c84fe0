"""CPU checks of the fp8 parity tolerance (fp8_error_model): a float64
computation that rounds every probability to E4M3 the way the fp8 path does
passes it, and the same computation with a systematic slip does not.

The rounded computation here is a model of the fp8 arithmetic for testing the
tolerance, not a second oracle: probabilities P = 2^(s - ref) against a
reference ref at least 3 (base 2) below the row maximum, as the fp8 path keeps
it, rounded to E4M3 by torch's float8_e4m3fn
conversion, with the rounded values feeding both the weighted sum and the row
sum.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_long_rbs_amd import inputs
from oracle import rbs_oracle as orc

import fp8_error_model as M


def _e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def _rounded_attention(q, k, v, block, row_ptr, col_idx, rows, ref_drop, drop_frac=0.0, seed=0):
    """Block-sparse attention with E4M3-rounded probabilities (P = 2^(s - ref)
    in base 2 with ref = the row's largest score minus ref_drop); drop_frac of
    the keys are left out of every row (the planted slip)."""
    S, Hq, D = q.shape
    G = Hq // k.shape[1]
    nb = orc.n_blocks(S, block)
    scale = 1.0 / math.sqrt(D)
    rng = np.random.default_rng(seed)
    out = np.zeros((S, Hq, D))
    for g, i in rows:
        r = g * nb + i
        keys = np.concatenate([np.arange(b * block, min(S, (b + 1) * block))
                               for b in col_idx[row_ptr[r]:row_ptr[r + 1]]])
        t0, t1 = i * block, min(S, (i + 1) * block)
        tok = np.arange(t0, t1)
        qi = q[t0:t1, g * G:(g + 1) * G].transpose(1, 0, 2)
        s = (qi @ k[keys, g].T) * scale
        allowed = (keys[None, :] <= tok[:, None]) & (rng.random(len(keys)) >= drop_frac)[None, :]
        s = np.where(allowed, s, -np.inf)
        ref = s.max(-1, keepdims=True) - ref_drop * math.log(2.0)
        p = _e4m3(np.exp(s - ref))
        o = (p @ v[keys, g]) / p.sum(-1, keepdims=True)
        out[t0:t1, g * G:(g + 1) * G] = o.transpose(1, 0, 2)
    return out


@pytest.fixture(scope="module")
def case():
    w = inputs.mixture_small(S=1500, Hq=8, Hkv=2, rho=0.25, sink=True, seed=11)
    f = inputs.fp8_inputs(w)
    _, sel = None, orc.select(*orc.block_stats(w.q, w.k, 2, w.block),
                              orc.derive_beta(orc.block_stats(w.q, w.k, 2, w.block)[1]),
                              w.keep_ratio_centroid, w.keep_ratio_rescue, w.sink)
    q, k, v = M.decoded(f)
    rows = [(g, i) for g in range(2) for i in range(w.n_blocks)]
    out_o, lse_o = orc.blocksparse_attention(q, k, v, w.block, sel.row_ptr, sel.col_idx)
    sigma = M.rounding_sigma(q, k, v, w.block, sel.row_ptr, sel.col_idx, rows, out_o, lse_o)
    exact = M.exact_slab(out_o, rows, w.block, w.seqlen, w.group)
    return dict(w=w, q=q, k=k, v=v, sel=sel, rows=rows, out_o=out_o, sigma=sigma, exact=exact)


@pytest.mark.parametrize("ref_drop", [3.0, 5.0, 8.0])
def test_e4m3_rounded_probabilities_pass(case, ref_drop):
    c = case
    w = c["w"]
    out = _rounded_attention(c["q"], c["k"], c["v"], w.block, c["sel"].row_ptr,
                             c["sel"].col_idx, c["rows"], ref_drop)
    err = M.exact_slab(out, c["rows"], w.block, w.seqlen, w.group) - c["exact"]
    mean, expected, worst = M.check(err, c["sigma"], c["exact"], f"ref_drop {ref_drop}")
    assert mean >= 0.3 * expected   # the model is not wildly pessimistic either


def test_dropping_three_percent_of_the_keys_fails(case):
    c = case
    w = c["w"]
    out = _rounded_attention(c["q"], c["k"], c["v"], w.block, c["sel"].row_ptr,
                             c["sel"].col_idx, c["rows"], 3.0, drop_frac=0.03, seed=1)
    err = M.exact_slab(out, c["rows"], w.block, w.seqlen, w.group) - c["exact"]
    with pytest.raises(AssertionError):
        M.check(err, c["sigma"], c["exact"], "3% of keys dropped")


def test_sigma_matches_the_variance_by_enumeration():
    """On one tiny row, the closed-form sigma equals the variance summed key
    by key."""
    rng = np.random.default_rng(2)
    S, D, B = 40, 8, 16
    q = rng.standard_normal((S, 1, D))
    k = rng.standard_normal((S, 1, D))
    v = rng.standard_normal((S, 1, D))
    rp, ci = orc.dense_causal_selection(1, orc.n_blocks(S, B))
    out, lse = orc.blocksparse_attention(q, k, v, B, rp, ci)
    sig = M.rounding_sigma(q, k, v, B, rp, ci, [(0, 2)], out, lse).reshape(S - 32, 1, D)
    for t in range(32, S):
        s = (k[:t + 1, 0] @ q[t, 0]) / math.sqrt(D)
        wts = np.exp(s - s.max())
        wts /= wts.sum()
        p = np.exp(s - s.max())
        a = [wts[u] ** 2 if p[u] >= 2.0 ** -9 else (2.0 ** -13 / p.sum()) ** 2 / 2.0 ** -8
             for u in range(t + 1)]
        var = sum(a[u] * (v[u, 0] - out[t, 0]) ** 2 for u in range(t + 1)) * M.SIGMA_REL ** 2
        np.testing.assert_allclose(sig[t - 32, 0], np.sqrt(var), rtol=1e-10)
