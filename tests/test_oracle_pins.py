"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these retypes an oracle formula: each checks the oracle against an
independent fact (a hand-worked example, an inequality, a library routine,
a brute-force enumeration, a closed form of RoPE). The planted-mistake tests
at the end show that a plausible slip in the oracle fails at least one pin.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from block_sparse_long_rbs_amd import inputs
from oracle import rbs_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dyadic():
    with open(os.path.join(GOLDEN, "dyadic_rescue.json")) as f:
        d = json.load(f)
    a = lambda x: np.asarray(x, np.float32)  # noqa: E731
    q = a(d["q"])[:, None, :]
    k = a(d["k"])[:, None, :]
    v = a(d["v"])[:, None, :]
    return d, q, k, v


# ---------------------------------------------------------------- worked example

def test_dyadic_worked_example_stats_scores_rows():
    d, q, k, v = _dyadic()
    e = d["expected"]
    c, r, qr, qn = orc.block_stats(q, k, 1, 2)
    assert np.array_equal(c[0], np.asarray(e["centroid"], float))
    assert np.array_equal(r[0], np.asarray(e["radius"], float))
    assert np.array_equal(qr[0], np.asarray(e["q_rep"], float))
    assert np.array_equal(qn[0], np.asarray(e["q_rep_norm"], float))
    assert np.array_equal(orc.derive_beta(r)[0], np.asarray(e["derived_beta"], float))
    ones = np.ones_like(r)
    sc, sr = orc.branch_scores(c, r, qr, qn, ones, 0, 2)
    assert np.array_equal(sc, e["scores_row2_centroid"])
    assert np.array_equal(sr, e["scores_row2_rescue_beta1"])
    sc, sr = orc.branch_scores(c, r, qr, qn, ones, 0, 1)
    assert np.array_equal(sc, e["scores_row1_centroid"])
    assert np.array_equal(sr, e["scores_row1_rescue_beta1"])
    rho = e["keep_ratio"]
    sel = orc.select(c, r, qr, qn, ones, rho, rho, sink=False)
    assert [sel.row(0, i).tolist() for i in range(3)] == e["rows_beta1"]
    sel = orc.select(c, r, qr, qn, orc.derive_beta(r), rho, rho, sink=False)
    assert [sel.row(0, i).tolist() for i in range(3)] == e["rows_derived_beta"]
    out, lse = orc.blocksparse_attention(q, k, v, 2, sel.row_ptr, sel.col_idx, rows=[(0, 0)])
    assert np.array_equal(out[0, 0], e["out_token0"]) and lse[0, 0] == e["lse_token0"]
    assert np.array_equal(out[1, 0], e["out_token1"]) and lse[0, 1] == pytest.approx(math.log(2), abs=1e-15)


# ---------------------------------------------------------------- statistics

def test_stats_closed_form_sphere_blocks():
    """Keys mu +/- R e_d (an axis cross of radius R around mu) have mean mu and
    radius R exactly; queries constant per block have that constant as mean."""
    rng = np.random.default_rng(0)
    D, B, nb, Hkv, G = 8, 16, 5, 2, 3
    k = np.zeros((nb * B, Hkv, D), np.float32)
    q = np.zeros((nb * B, Hkv * G, D), np.float32)
    mus = rng.integers(-4, 5, (Hkv, nb, D)).astype(np.float32)
    Rs = rng.integers(1, 6, (Hkv, nb)).astype(np.float32)
    for g in range(Hkv):
        for b in range(nb):
            for d in range(D):
                k[b * B + 2 * d, g] = mus[g, b]
                k[b * B + 2 * d, g, d] += Rs[g, b]
                k[b * B + 2 * d + 1, g] = mus[g, b]
                k[b * B + 2 * d + 1, g, d] -= Rs[g, b]
            q[b * B:(b + 1) * B, g * G:(g + 1) * G] = mus[g, b][None, None, :] * 0.5
    c, r, qr, qn = orc.block_stats(q, k, Hkv, B)
    np.testing.assert_allclose(c, mus, atol=1e-12)
    np.testing.assert_allclose(r, Rs, atol=1e-12)
    np.testing.assert_allclose(qr, mus * 0.5, atol=1e-12)
    np.testing.assert_allclose(qn, np.linalg.norm(mus * 0.5, axis=-1), atol=1e-12)


def test_stats_ragged_last_block_uses_only_real_tokens():
    w = inputs.random_qkv(100, 2, 1, 4, "f32", seed=3, block=32)
    c, r, qr, qn = orc.block_stats(w.q, w.k, 1, 32)
    assert c.shape == (1, 4, 4)
    np.testing.assert_allclose(c[0, 3], w.k[96:100, 0].astype(float).mean(0), atol=1e-12)
    np.testing.assert_allclose(qr[0, 3], w.q[96:100].astype(float).mean((0, 1)), atol=1e-12)
    d = np.linalg.norm(w.k[96:100, 0] - c[0, 3], axis=-1).max()
    assert r[0, 3] == pytest.approx(d, rel=1e-12)


# ---------------------------------------------------------------- Cauchy-Schwarz

def _cs_check(w, rows=None):
    c, r, qr, qn = orc.block_stats(w.q, w.k, w.n_kv_heads, w.block)
    nb = w.n_blocks
    worst = -np.inf
    for g in range(w.n_kv_heads):
        kk = w.k[:, g].astype(np.float64)
        for i in (range(nb) if rows is None else rows):
            logits = kk[:(i + 1) * w.block] @ qr[g, i]
            for j in range(i + 1):
                bound = qr[g, i] @ c[g, j] + qn[g, i] * r[g, j]
                lj = logits[j * w.block:(j + 1) * w.block]
                worst = max(worst, (lj.max() - bound) / max(1.0, abs(bound)))
    return worst


def test_cauchy_schwarz_bound_exhaustive_tiny():
    """Every key's logit against the representative query stays below the
    centroid score plus ||q|| times the radius (the rescue branch's bound)."""
    assert _cs_check(inputs.tiny_f32_1k()) <= 1e-12


@pytest.mark.slow
def test_cauchy_schwarz_bound_exhaustive_8k():
    assert _cs_check(inputs.needle_bf16_8k()) <= 1e-12


@pytest.mark.slow
@pytest.mark.parametrize("make", [inputs.mixture_bf16_32k, inputs.mixture_bf16_128k],
                         ids=["32k", "128k"])
def test_cauchy_schwarz_bound_sampled_mixtures(make):
    """The same bound on sampled query blocks of the two mixtures (every KV
    head, every key block up to the diagonal), including the last block."""
    w = make()
    rng = np.random.default_rng(0)
    rows = sorted(rng.choice(w.n_blocks - 1, size=5, replace=False).tolist()) + [w.n_blocks - 1]
    assert _cs_check(w, rows) <= 1e-12


def test_cauchy_schwarz_tight_for_aligned_outlier():
    """A block whose farthest key is aligned with q reaches the bound."""
    rng = np.random.default_rng(5)
    D, B = 16, 8
    qdir = rng.standard_normal(D)
    qdir /= np.linalg.norm(qdir)
    k = np.zeros((B, 1, D), np.float32)
    k[0, 0] = 7 * qdir
    k[1:, 0] = -qdir  # collinear: centroid on the q axis
    q = np.tile(qdir.astype(np.float32), (B, 1))[:, None, :]
    c, r, qr, qn = orc.block_stats(q, k, 1, B)
    bound = qr[0, 0] @ c[0, 0] + qn[0, 0] * r[0, 0]
    assert bound == pytest.approx(float(qr[0, 0] @ k[0, 0].astype(float)), rel=1e-6)


# ---------------------------------------------------------------- selection

def test_rescue_never_below_centroid():
    w = inputs.needle_bf16_8k()
    c, r, qr, qn = orc.block_stats(w.q, w.k, w.n_kv_heads, w.block)
    beta = orc.derive_beta(r)
    for g in range(w.n_kv_heads):
        for i in range(0, w.n_blocks, 7):
            sc, sr = orc.branch_scores(c, r, qr, qn, beta, g, i)
            assert np.all(sr >= sc)


def test_beta_one_keeps_every_block_with_a_key_above_threshold():
    """With beta = 1 a block holding a key whose logit exceeds the rescue
    branch's threshold cannot be dropped. Needles of norm 40 (no dilution
    shift) and keep-ratio 0.5 put keys above the threshold, so the check is
    not vacuous."""
    w = inputs.tiny_f32_1k(shift=0.0, needle_norm=40.0)
    c, r, qr, qn = orc.block_stats(w.q, w.k, 1, w.block)
    beta = np.ones_like(r)
    sel = orc.select(c, r, qr, qn, beta, 0.5, 0.5, sink=False)
    kk = w.k[:, 0].astype(np.float64)
    checked = 0
    for i in range(w.n_blocks):
        _, sr = orc.branch_scores(c, r, qr, qn, beta, 0, i)
        n = orc.budget(i + 1, 0.5)
        tau = np.sort(sr)[::-1][n - 1]
        row = set(sel.row(0, i).tolist())
        for j in range(i + 1):
            if (kk[j * w.block:(j + 1) * w.block] @ qr[0, i]).max() > tau:
                assert j in row
                checked += 1
    assert checked > 0


def test_beta_zero_gives_centroid_only():
    w = inputs.needle_bf16_8k()
    c, r, qr, qn = orc.block_stats(w.q, w.k, w.n_kv_heads, w.block)
    zero = np.zeros_like(r)
    sel = orc.select(c, r, qr, qn, zero, 0.1, 0.1, sink=False)
    for g in range(w.n_kv_heads):
        for i in range(w.n_blocks):
            sc = c[g, :i + 1] @ qr[g, i]
            n = orc.budget(i + 1, 0.1)
            best = sorted(range(i + 1), key=lambda j: (-sc[j], j))[:n]
            assert sel.row(g, i).tolist() == sorted(set(best) | {i})


def test_top_n_matches_pairwise_counting_definition():
    """j is kept iff fewer than n entries beat it, where a beats b when its
    score is larger, or equal with a lower index (brute force over pairs)."""
    rng = np.random.default_rng(7)
    for trial in range(200):
        m = int(rng.integers(1, 40))
        s = rng.integers(-3, 4, m).astype(np.float32)  # many ties
        n = int(rng.integers(1, m + 1))
        got = orc.top_n(s, n).tolist()
        want = [j for j in range(m)
                if sum((s[a] > s[j]) or (s[a] == s[j] and a < j) for a in range(m)) < n]
        assert got == want


def test_budget_readings():
    assert orc.budget(10, 0.1) == 1          # 0.1 * 10 is 1 in decimal
    assert orc.budget(11, 0.1) == 2
    assert orc.budget(1, 0.03) == 1          # at least one
    assert orc.budget(100, 0.03) == 3
    assert orc.budget(7, 1.0) == 7           # keep-ratio 1 keeps everything
    # totals per KV head over all query blocks of the named workloads
    assert sum(orc.budget(i + 1, 0.25) for i in range(16)) == 40
    assert sum(orc.budget(i + 1, 0.1) for i in range(64)) == 238
    assert sum(orc.budget(i + 1, 0.05) for i in range(256)) == 1768
    assert sum(orc.budget(i + 1, 0.03) for i in range(1024)) == 16254


def test_beta_properties():
    rng = np.random.default_rng(3)
    r = np.abs(rng.standard_normal((3, 50))) + 1.0
    b = orc.derive_beta(r)
    assert np.all((b >= 0) & (b <= 1))
    for g in range(3):
        assert b[g, r[g].argmax()] == 1.0
        assert np.all(b[g][r[g] <= r[g].mean()] == 0.0)
        o = np.argsort(r[g])
        assert np.all(np.diff(b[g][o]) >= 0)
    assert np.all(orc.derive_beta(np.full((1, 9), 2.5)) == 0.0)   # no spread: no rescue


def test_forced_blocks_and_row_zero():
    w = inputs.mixture_small(S=640, Hq=4, Hkv=2, D=32, B=64, rho=0.1, sink=True, seed=2)
    c, r, qr, qn = orc.block_stats(w.q, w.k, 2, 64)
    sel = orc.select(c, r, qr, qn, orc.derive_beta(r), 0.1, 0.1, sink=True)
    for g in range(2):
        assert sel.row(g, 0).tolist() == [0]
        for i in range(w.n_blocks):
            row = sel.row(g, i).tolist()
            assert row == sorted(set(row)) and row[0] == 0 and row[-1] == i
    assert sel.col_idx.size <= orc.select_capacity(2, w.n_blocks, 0.1, 0.1, True)


# ---------------------------------------------------------------- attention

def _sdpa_causal(q, k, v):
    """Dense causal attention by torch's library routine, float64 on the CPU."""
    S, Hq, D = q.shape
    G = Hq // k.shape[1]
    tq = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k.astype(np.float64)).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v.astype(np.float64)).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    return o[0].permute(1, 0, 2).numpy()


def test_keep_ratio_one_is_dense_causal_attention():
    w = inputs.random_qkv(300, 4, 2, 32, "f32", seed=9, block=64)
    c, r, qr, qn = orc.block_stats(w.q, w.k, 2, 64)
    sel = orc.select(c, r, qr, qn, orc.derive_beta(r), 1.0, 1.0, sink=False)
    rp, ci = orc.dense_causal_selection(2, w.n_blocks)
    assert np.array_equal(sel.row_ptr, rp) and np.array_equal(sel.col_idx, ci)
    out, _ = orc.blocksparse_attention(w.q, w.k, w.v, 64, sel.row_ptr, sel.col_idx)
    np.testing.assert_allclose(out, _sdpa_causal(w.q, w.k, w.v), atol=1e-12, rtol=0)


def test_block_gather_equals_token_level_brute_force():
    w = inputs.mixture_small(S=200, Hq=4, Hkv=2, D=16, B=32, rho=0.3, sink=False, seed=4)
    c, r, qr, qn = orc.block_stats(w.q, w.k, 2, 32)
    sel = orc.select(c, r, qr, qn, orc.derive_beta(r), 0.3, 0.3, sink=False)
    out, lse = orc.blocksparse_attention(w.q, w.k, w.v, 32, sel.row_ptr, sel.col_idx)
    mask = orc.csr_token_mask(sel.row_ptr, sel.col_idx, 2, 200, 32)
    out2, lse2 = orc.masked_attention(w.q, w.k, w.v, mask)
    np.testing.assert_allclose(out, out2, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse2, atol=1e-12, rtol=0)


def test_lse_matches_library_logsumexp():
    from scipy.special import logsumexp
    w = inputs.random_qkv(64, 1, 1, 8, "f32", seed=1, block=64)
    rp, ci = orc.dense_causal_selection(1, 1)
    _, lse = orc.blocksparse_attention(w.q, w.k, w.v, 64, rp, ci)
    t = 40
    logits = (w.k[:t + 1, 0].astype(float) @ w.q[t, 0].astype(float)) / math.sqrt(8)
    assert lse[0, t] == pytest.approx(logsumexp(logits), abs=1e-12)


def test_row_zero_is_causal_attention_inside_block_zero():
    w = inputs.random_qkv(256, 2, 1, 16, "f32", seed=4, block=64)
    rp = np.array([0, 1, 2, 4, 6]); ci = np.array([0, 1, 2, 0, 3, 0])
    out, _ = orc.blocksparse_attention(w.q, w.k, w.v, 64, rp, ci, rows=[(0, 0)])
    ref = _sdpa_causal(w.q[:64], w.k[:64], w.v[:64])
    np.testing.assert_allclose(out[:64], ref, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- per-query-head selection

def test_per_head_reps_average_to_the_group_rep():
    """The mean of a group's per-head representatives is the group's (equal
    token counts per head), ragged last block included."""
    w = inputs.random_qkv(300, 6, 2, 16, "f32", seed=12, block=64)
    _, _, qr, _ = orc.block_stats(w.q, w.k, 2, 64)
    qh, qhn = orc.query_rep_per_head(w.q, 64)
    np.testing.assert_allclose(qh.reshape(2, 3, -1, 16).mean(axis=1), qr, atol=1e-13, rtol=0)
    np.testing.assert_allclose(qhn, np.linalg.norm(qh, axis=-1), atol=1e-13, rtol=0)


def _identical_heads(w, G):
    q = w.q.copy()
    for h in range(q.shape[1]):
        q[:, h] = w.q[:, (h // G) * G]
    return q


def test_per_head_selection_with_identical_heads_is_the_group_selection():
    w = inputs.mixture_small(S=640, Hq=8, Hkv=2, D=32, B=64, rho=0.2, sink=True, seed=6)
    q = _identical_heads(w, 4)
    c, r, qr, qn = orc.block_stats(q, w.k, 2, 64)
    beta = orc.derive_beta(r)
    grp = orc.select(c, r, qr, qn, beta, 0.2, 0.15, sink=True)
    qh, qhn = orc.query_rep_per_head(q, 64)
    per = orc.select_per_head(c, r, qh, qhn, beta, 0.2, 0.15, sink=True)
    nb = w.n_blocks
    for h in range(8):
        for i in range(nb):
            assert per.col_idx[per.row_ptr[h * nb + i]:per.row_ptr[h * nb + i + 1]].tolist() == \
                grp.row(h // 4, i).tolist()


def test_planted_tiled_head_mapping_breaks_identical_heads_pin():
    """Pairing query head h with KV head h % Hkv (tiling instead of repeating
    the KV-head statistics) gives other rows, so the pin above catches it."""
    w = inputs.mixture_small(S=640, Hq=8, Hkv=2, D=32, B=64, rho=0.2, sink=True, seed=6)
    q = _identical_heads(w, 4)
    c, r, qr, qn = orc.block_stats(q, w.k, 2, 64)
    beta = orc.derive_beta(r)
    grp = orc.select(c, r, qr, qn, beta, 0.2, 0.15, sink=True)
    qh, qhn = orc.query_rep_per_head(q, 64)
    tiled = orc.select(np.tile(c, (4, 1, 1)), np.tile(r, (4, 1)), qh, qhn, np.tile(beta, (4, 1)),
                       0.2, 0.15, sink=True)
    nb = w.n_blocks
    assert any(tiled.col_idx[tiled.row_ptr[h * nb + i]:tiled.row_ptr[h * nb + i + 1]].tolist()
               != grp.row(h // 4, i).tolist() for h in range(8) for i in range(nb))


def test_per_head_attention_equals_token_level_brute_force():
    w = inputs.mixture_small(S=200, Hq=4, Hkv=2, D=16, B=32, rho=0.3, sink=False, seed=4)
    c, r, _, _ = orc.block_stats(w.q, w.k, 2, 32)
    qh, qhn = orc.query_rep_per_head(w.q, 32)
    sel = orc.select_per_head(c, r, qh, qhn, orc.derive_beta(r), 0.3, 0.3, sink=False)
    out, lse = orc.blocksparse_attention_per_head(w.q, w.k, w.v, 32, sel.row_ptr, sel.col_idx)
    mask = orc.csr_token_mask(sel.row_ptr, sel.col_idx, 4, 200, 32)   # one mask per query head
    for h in range(4):
        g = h // 2
        o2, l2 = orc.masked_attention(w.q[:, h:h + 1], w.k[:, g:g + 1], w.v[:, g:g + 1], mask[h])
        np.testing.assert_allclose(out[:, h], o2[:, 0], atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse[h], l2[0], atol=1e-12, rtol=0)


def test_per_head_keep_ratio_one_is_dense_causal_attention():
    w = inputs.random_qkv(300, 4, 2, 32, "f32", seed=9, block=64)
    c, r, _, _ = orc.block_stats(w.q, w.k, 2, 64)
    qh, qhn = orc.query_rep_per_head(w.q, 64)
    sel = orc.select_per_head(c, r, qh, qhn, orc.derive_beta(r), 1.0, 1.0, sink=False)
    out, _ = orc.blocksparse_attention_per_head(w.q, w.k, w.v, 64, sel.row_ptr, sel.col_idx)
    np.testing.assert_allclose(out, _sdpa_causal(w.q, w.k, w.v), atol=1e-12, rtol=0)


# ---------------------------------------------------------------- attention mass per block

def test_block_attention_mass_against_library_softmax():
    """Per-block mass with block size 1 is the per-key softmax (scipy),
    averaged over the row's tokens and heads; with any block size it sums to
    1 and equals the per-key masses summed over each block."""
    from scipy.special import softmax
    w = inputs.random_qkv(96, 4, 2, 16, "f32", seed=21, block=32)
    g, i = 1, 2
    m1 = orc.block_attention_mass(w.q, w.k, 1, g, 70)   # one "block" = one token, row t = 70
    ref = np.zeros(71)
    for h in (2, 3):
        ref += softmax(w.k[:71, g].astype(float) @ w.q[70, h].astype(float) / 4.0)
    np.testing.assert_allclose(m1, ref / 2, atol=1e-13, rtol=0)
    m = orc.block_attention_mass(w.q, w.k, 32, g, i)
    assert m.shape == (3,) and abs(m.sum() - 1.0) < 1e-12
    per_tok = np.zeros(96)
    for t in range(64, 96):
        per_tok[:t + 1] += orc.block_attention_mass(w.q, w.k, 1, g, t)[:t + 1] / 32
    np.testing.assert_allclose(m, [per_tok[0:32].sum(), per_tok[32:64].sum(), per_tok[64:96].sum()],
                               atol=1e-12, rtol=0)


# ---------------------------------------------------------------- fp8 (E4M3) inputs

def test_e4m3_decode_matches_torch_on_every_code():
    """The decoder written from the format definition against torch's own
    float8_e4m3fn conversion, all 256 byte values (NaN codes included)."""
    b = np.arange(256, dtype=np.uint8)
    mine = orc.e4m3_decode(b)
    ref = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all(), b[~same]


def test_e4m3_closed_forms():
    d = lambda x: float(orc.e4m3_decode(np.array([x], np.uint8))[0])  # noqa: E731
    assert d(0x38) == 1.0 and d(0xB8) == -1.0          # exponent field 7 = bias
    assert d(0x7E) == 448.0                            # largest finite: 1.75 * 2^8
    assert d(0x08) == 2.0 ** -6                        # smallest normal
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9   # subnormals m/8 * 2^-6
    assert d(0x00) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    pos = orc.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)                    # codes 0..0x7E increase strictly


def _fp8_case(S=200, Hq=4, Hkv=2, D=16, B=32, seed=4):
    w = inputs.mixture_small(S=S, Hq=Hq, Hkv=Hkv, D=D, B=B, rho=0.3, sink=True, seed=seed)
    f = inputs.fp8_inputs(w)
    c, r, qr, qn = orc.block_stats(w.q, w.k, Hkv, B)
    sel = orc.select(c, r, qr, qn, orc.derive_beta(r), 0.3, 0.3, sink=True)
    return w, f, sel


def test_fp8_attention_equals_token_level_brute_force():
    """Decoded-and-scaled inputs through the token-mask attention (a separate
    code path) give the same result."""
    w, f, sel = _fp8_case()
    out, lse = orc.blocksparse_attention_fp8(f.q, f.k, f.v, f.q_descale, f.k_descale,
                                             f.v_descale, 32, sel.row_ptr, sel.col_idx)
    mask = orc.csr_token_mask(sel.row_ptr, sel.col_idx, 2, 200, 32)
    q = orc.e4m3_decode(f.q) * f.q_descale
    k = orc.e4m3_decode(f.k) * f.k_descale
    v = orc.e4m3_decode(f.v) * f.v_descale
    out2, lse2 = orc.masked_attention(q, k, v, mask)
    np.testing.assert_allclose(out, out2, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse2, atol=1e-12, rtol=0)


def test_fp8_descales_act_as_the_definition_says():
    """v_descale scales the output; q_descale and k_descale enter only through
    their product with the softmax scale (a swapped or dropped factor fails)."""
    w, f, sel = _fp8_case()
    base, lse = orc.blocksparse_attention_fp8(f.q, f.k, f.v, 1.0, 1.0, 1.0, 32, sel.row_ptr,
                                              sel.col_idx, scale=0.25)
    o2, l2 = orc.blocksparse_attention_fp8(f.q, f.k, f.v, 1.0, 1.0, 3.0, 32, sel.row_ptr,
                                           sel.col_idx, scale=0.25)
    np.testing.assert_allclose(o2, 3.0 * base, rtol=1e-13, atol=0)
    np.testing.assert_allclose(l2, lse, rtol=0, atol=1e-13)
    o3, l3 = orc.blocksparse_attention_fp8(f.q, f.k, f.v, 2.0, 0.5, 1.0, 32, sel.row_ptr,
                                           sel.col_idx, scale=0.25)
    np.testing.assert_allclose(o3, base, rtol=0, atol=1e-13)
    o4, l4 = orc.blocksparse_attention_fp8(f.q, f.k, f.v, 2.0, 1.0, 1.0, 32, sel.row_ptr,
                                           sel.col_idx, scale=0.125)
    np.testing.assert_allclose(o4, base, rtol=0, atol=1e-13)
    o5, _ = orc.blocksparse_attention_fp8(f.q, f.k, f.v, 2.0, 1.0, 1.0, 32, sel.row_ptr,
                                          sel.col_idx, scale=0.25)
    assert np.abs(o5 - base).max() > 1e-3        # the product really matters


def test_fp8_inputs_round_trip():
    """The generator's quantisation is a rounding: decoded values are within
    half a step (2^-4 relative, 2^-10 absolute below 2^-6) of the scaled input."""
    w = inputs.random_qkv(300, 2, 1, 32, "f32", seed=3, block=64)
    b, d = inputs.to_e4m3(w.q)
    x = w.q.astype(np.float64) / d
    y = orc.e4m3_decode(b)
    assert np.abs(x).max() <= 448.0 * (1 + 1e-6) and np.isfinite(y).all()   # descale is fp32-rounded
    err = np.abs(y - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10) + 1e-12)


# ---------------------------------------------------------------- Block-attention

def test_rope_composition():
    """R(a) R(b) = R(a + b) and R(0) = identity."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 2, 16))
    a, b = np.array([0, 3, 100, 7, 30720]), np.array([5, 0, 9, 1234, 500])
    np.testing.assert_allclose(orc.rope_rotate(orc.rope_rotate(x, a, 5e5), b, 5e5),
                               orc.rope_rotate(x, a + b, 5e5), atol=1e-12)
    np.testing.assert_allclose(orc.rope_rotate(x, np.zeros(5), 5e5), x, atol=0)


def test_rope_relative_position():
    """<R(m) q, R(n) k> depends only on m - n."""
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((1, 1, 32)), rng.standard_normal((1, 1, 32))
    vals = [float(orc.rope_rotate(q, [m], 1e4)[0, 0] @ orc.rope_rotate(k, [m - 17], 1e4)[0, 0])
            for m in (17, 50, 1000, 31000)]
    np.testing.assert_allclose(vals, vals[0], rtol=1e-10)


def test_rope_pairs_rotate_as_complex_numbers():
    """Each pair (x_i, x_{i+D/2}) is multiplied by exp(i * pos * theta^(-2i/D))."""
    rng = np.random.default_rng(2)
    D, theta, pos = 8, 10000.0, 37
    x = rng.standard_normal((1, 1, D))
    y = orc.rope_rotate(x, [pos], theta)[0, 0]
    for i in range(D // 2):
        z = complex(x[0, 0, i], x[0, 0, i + D // 2]) * np.exp(1j * pos * theta ** (-2 * i / D))
        assert y[i] == pytest.approx(z.real, abs=1e-12)
        assert y[i + D // 2] == pytest.approx(z.imag, abs=1e-12)


def _rag_small(seed=3):
    """4 passages of 48 tokens + a final block of 16, with Q and K built from
    raw rows by explicit RoPE: Q at absolute positions, cached passage K at
    local positions, the final block's K at absolute positions."""
    rng = np.random.default_rng(seed)
    P, L, F, Hq, Hkv, D, theta = 4, 48, 16, 4, 2, 16, 5e5
    S = P * L + F
    qr = rng.standard_normal((S, Hq, D)); kr = rng.standard_normal((S, Hkv, D))
    v = rng.standard_normal((S, Hkv, D))
    seg = np.array([p * L for p in range(P + 1)] + [S])
    rer = np.array([p * L for p in range(P)] + [0])
    pos = np.arange(S)
    local = pos - np.where(pos < P * L, (pos // L) * L, 0)
    q = orc.rope_rotate(qr, pos, theta)
    kc = orc.rope_rotate(kr, local, theta)
    return dict(q=q, kc=kc, v=v, qr=qr, kr=kr, seg=seg, rer=rer, theta=theta, S=S, P=P, L=L)


def test_block_attention_passages_equal_independent_attention():
    """A non-final block attends only within itself, so its output equals
    ordinary causal attention over the passage alone at local positions."""
    d = _rag_small()
    out, _ = orc.block_mask_attention(d["q"], d["kc"], d["v"], d["seg"], d["rer"], d["theta"])
    for p in range(d["P"]):
        sl = slice(p * d["L"], (p + 1) * d["L"])
        loc = np.arange(d["L"])
        ql = orc.rope_rotate(d["qr"][sl], loc, d["theta"])
        kl = orc.rope_rotate(d["kr"][sl], loc, d["theta"])
        np.testing.assert_allclose(out[sl], _sdpa_causal(ql, kl, d["v"][sl]), atol=1e-10)


def test_block_attention_final_block_is_dense_causal():
    d = _rag_small()
    out, _ = orc.block_mask_attention(d["q"], d["kc"], d["v"], d["seg"], d["rer"], d["theta"],
                                      q_row_begin=d["P"] * d["L"])
    kabs = orc.rope_rotate(d["kr"], np.arange(d["S"]), d["theta"])
    ref = _sdpa_causal(d["q"], kabs, d["v"])
    fin = slice(d["P"] * d["L"], d["S"])
    np.testing.assert_allclose(out[fin], ref[fin], atol=1e-10)
    assert np.all(np.isnan(out[:d["P"] * d["L"]]))


def test_block_attention_matches_literal_mask():
    d = _rag_small()
    out, lse = orc.block_mask_attention(d["q"], d["kc"], d["v"], d["seg"], d["rer"], d["theta"])
    kabs = orc.reencode_keys(d["kc"], d["seg"], d["rer"], d["theta"])
    mask = orc.block_mask_token_mask(d["seg"], d["S"])
    out2, lse2 = orc.masked_attention(d["q"], kabs, d["v"], mask)
    np.testing.assert_allclose(out, out2, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, atol=1e-12)


def test_attention_pairs_count_dense():
    S, B = 300, 64
    rp, ci = orc.dense_causal_selection(2, orc.n_blocks(S, B))
    assert orc.attention_pairs(rp, ci, S, B, 2, 3) == 2 * 3 * S * (S + 1) // 2


# ---------------------------------------------------------------- planted mistakes

def test_planted_mean_distance_radius_breaks_cauchy_schwarz(monkeypatch):
    """If the radius were the mean (not the largest) key distance, the bound
    check on the needle workload would fail."""
    w = inputs.tiny_f32_1k()
    real = orc.block_stats

    def wrong(q, k, n_kv_heads, block):
        c, r, qr, qn = real(q, k, n_kv_heads, block)
        for b in range(r.shape[1]):
            kb = k[b * block:(b + 1) * block].astype(float)
            r[:, b] = np.sqrt(((kb - c[None, :, b]) ** 2).sum(-1)).mean(0)
        return c, r, qr, qn

    monkeypatch.setattr(orc, "block_stats", wrong)
    assert _cs_check(w) > 1e-3


def test_planted_sign_flip_in_rescue_breaks_invariant():
    w = inputs.tiny_f32_1k()
    c, r, qr, qn = orc.block_stats(w.q, w.k, 1, w.block)
    sc = c[0, :16] @ qr[0, 15]
    wrong = sc - qn[0, 15] * r[0, :16]
    assert not np.all(wrong >= sc)


def test_planted_transposed_gqa_mapping_breaks_dense_pin():
    """Mapping query head h to KV head h % Hkv instead of h // G changes the
    output, so the library-routine pin would catch it."""
    w = inputs.random_qkv(128, 4, 2, 16, "f32", seed=2, block=64)
    rp, ci = orc.dense_causal_selection(2, 2)
    perm = np.array([0, 2, 1, 3])  # h -> h % 2 grouping
    out, _ = orc.blocksparse_attention(w.q[:, perm], w.k, w.v, 64, rp, ci)
    assert np.abs(out[:, np.argsort(perm)] - _sdpa_causal(w.q, w.k, w.v)).max() > 1e-3
