"""CPU checks of the fp8 parity tolerance (fp8_error_model): a float64
computation that rounds every probability to E4M3 the way the fp8 path does
passes it, and the same computation with a systematic slip does not.

The rounded computation here is a model of the fp8 arithmetic for testing the
tolerance, not a second oracle: one power of two per (query row, 32-key
block) puts the block's largest probability in (128, 256], the values are
rounded to E4M3 by torch's float8_e4m3fn conversion and the rounded values
feed both the weighted sum and the row sum.
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


def _rounded_attention(q, k, v, block, row_ptr, col_idx, rows, drop_frac=0.0, seed=0):
    """Block-sparse attention with E4M3-rounded probabilities, one power of
    two per (query row, 32-key block) chosen so that the block's largest
    probability lands in (128, 256], the rounded values feeding both the
    weighted sum and the row sum; drop_frac of the keys are left out of every
    row (the planted slip)."""
    S, Hq, D = q.shape
    G = Hq // k.shape[1]
    nb = orc.n_blocks(S, block)
    scale = 1.0 / math.sqrt(D) / math.log(2.0)        # base-2 scores
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
        m = s.max(-1, keepdims=True)
        p = np.zeros_like(s)
        for c0 in range(0, len(keys), 32):
            blk = s[..., c0:c0 + 32]
            x = np.maximum(blk.max(-1, keepdims=True) - m, -118.0)
            e = np.ceil(x) - 8.0
            pe = _e4m3(2.0 ** (blk - m - e))
            assert np.all(np.isfinite(pe)), "a probability overflowed e4m3"
            p[..., c0:c0 + 32] = pe * 2.0 ** e
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


def test_e4m3_rounded_probabilities_pass(case):
    c = case
    w = c["w"]
    out = _rounded_attention(c["q"], c["k"], c["v"], w.block, c["sel"].row_ptr,
                             c["sel"].col_idx, c["rows"])
    err = M.exact_slab(out, c["rows"], w.block, w.seqlen, w.group) - c["exact"]
    mean, expected, worst = M.check(err, c["sigma"], c["exact"], "per-block scaled e4m3")
    assert mean >= 0.3 * expected   # the model is not wildly pessimistic either


def test_one_reference_per_row_loses_a_long_tail():
    """With a single reference per row at its largest score (no per-block
    exponents), probabilities below 2^-10 of it flush to zero: a dominant key
    with a long tail of small ones then breaks the tolerance, which is why the
    fp8 path scales per block."""
    rng = np.random.default_rng(3)
    S, D = 4096, 128
    q = np.zeros((S, 1, D))
    q[:, 0, 0] = 1.0
    k = rng.standard_normal((S, 1, D)) * 0.1
    k[:, 0, 0] = 0.0
    k[5, 0, 0] = 16.0 * math.sqrt(D) * math.log(2.0)   # key 5 sits 2^16 above the rest
    v = rng.standard_normal((S, 1, D))
    rp, ci = orc.dense_causal_selection(1, 32)
    rows = [(0, 31)]
    out_o, lse_o = orc.blocksparse_attention(q, k, v, 128, rp, ci, rows=rows)
    sigma = M.rounding_sigma(q, k, v, 128, rp, ci, rows, out_o, lse_o)
    exact = M.exact_slab(out_o, rows, 128, S, 1)
    good = _rounded_attention(q, k, v, 128, rp, ci, rows)
    M.check(M.exact_slab(good, rows, 128, S, 1) - exact, sigma, exact, "per-block exponents")
    t0, t1 = 31 * 128, 32 * 128
    s = (q[t0:t1, 0] @ k[:t1, 0].T) / math.sqrt(D) / math.log(2.0)
    s = np.where(np.arange(t1)[None, :] <= np.arange(t0, t1)[:, None], s, -np.inf)
    p = _e4m3(2.0 ** (s - s.max(-1, keepdims=True)))
    flat = np.zeros_like(good)
    flat[t0:t1, 0] = (p @ v[:t1, 0]) / p.sum(-1, keepdims=True)
    with pytest.raises(AssertionError):
        M.check(M.exact_slab(flat, rows, 128, S, 1) - exact, sigma, exact, "one reference")


def test_dropping_three_percent_of_the_keys_fails(case):
    c = case
    w = c["w"]
    out = _rounded_attention(c["q"], c["k"], c["v"], w.block, c["sel"].row_ptr,
                             c["sel"].col_idx, c["rows"], drop_frac=0.03, seed=1)
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
        a = [wts[u] ** 2 if p[u] >= 2.0 ** -13 else (2.0 ** -17 / p.sum()) ** 2 / 2.0 ** -8
             for u in range(t + 1)]
        var = sum(a[u] * (v[u, 0] - out[t, 0]) ** 2 for u in range(t + 1)) * M.SIGMA_REL ** 2
        np.testing.assert_allclose(sig[t - 32, 0], np.sqrt(var), rtol=1e-10)
