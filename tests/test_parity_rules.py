"""CPU checks of the selection parity rule itself: the oracle's near-tie band
(oracle.near_tie_band) and the comparison the GPU tests apply
(gpu_helpers.compare_selection).

Each branch of the RBS-Attention explainer's "The Fix: A Radius-Adaptive
Rescue Branch" keeps its own top-n blocks, so a lower-precision ranking can
only swap a kept block for a dropped one whose scores are nearly equal. The
band therefore exempts blocks only where it straddles a branch's cut. The
planted selections below (each a slip planted in the oracle's budget or
ranking) must be rejected; the oracle's own selection must be accepted.
"""
import math

import numpy as np
import pytest

from block_sparse_long_rbs_amd import inputs
from oracle import rbs_oracle as orc

import gpu_helpers as H


def _row_stats(scores):
    """One KV head, one query block per entry of `scores`, whose centroid
    scores against every key block are exactly `scores` (q_rep = e_0, norm 1,
    c_j = scores[j] e_0) and whose radii are 0 (rescue = centroid)."""
    nb, D = len(scores), 4
    c = np.zeros((1, nb, D))
    c[0, :, 0] = scores
    qr = np.zeros((1, nb, D))
    qr[0, :, 0] = 1.0
    return c, np.zeros((1, nb)), qr, np.ones((1, nb))


# ------------------------------------------------------------- the band

def test_lone_threshold_block_is_not_exempt():
    # n = 2 of 5: tau = 3 (block 1); nothing else within 1e-4 * 5 of it
    assert orc.near_tie_band(np.array([5.0, 3.0, 1.0, 2.99, 0.0]), 2, floor=5.0) == set()


def test_straddling_near_tie_exempts_both_sides():
    # block 3 sits 1e-4 below tau = 3, inside the band 1e-4 * max(3, 5) = 5e-4
    assert orc.near_tie_band(np.array([5.0, 3.0, 1.0, 2.9999, 0.0]), 2, floor=5.0) == {1, 3}


def test_near_tie_on_the_kept_side_only_is_not_exempt():
    # blocks 0 and 1 are both kept and 1e-5 apart; the first dropped block is far below
    assert orc.near_tie_band(np.array([3.00001, 3.0, 1.0, 0.5]), 2, floor=3.0) == set()


def test_exact_tie_across_the_cut_is_exempt():
    # equal scores: the lower index is kept, the other dropped; rounding may swap them
    assert orc.near_tie_band(np.array([4.0, 2.0, 2.0, 0.0]), 2, floor=4.0) == {1, 2}


def test_band_floor_applies_when_threshold_is_near_zero():
    s = np.array([1.0, 2e-5, -3e-5, -0.5])
    # |tau| = 2e-5 alone would give a band of 2e-9; the floor 1.0 gives 1e-4
    assert orc.near_tie_band(s, 2, floor=1.0) == {1, 2}
    assert orc.near_tie_band(s, 2, floor=1e-3) == set()


def test_every_block_kept_exempts_nothing():
    assert orc.near_tie_band(np.array([1.0, 1.0, 1.0]), 3, floor=1.0) == set()


def test_select_exempt_sets_on_a_hand_built_row():
    # row 4 sees blocks 0..4; keep-ratio 0.4 -> n = 2; block 3 is a near tie of block 1
    c, r, qr, qn = _row_stats([5.0, 3.0, 1.0, 2.9999, 0.0])
    sel = orc.select(c, r, qr, qn, np.zeros_like(r), 0.4, 0.4, sink=False)
    assert sel.row(0, 4).tolist() == [0, 1, 4]
    assert sel.exempt[4] == {1, 3}
    c, r, qr, qn = _row_stats([5.0, 3.0, 1.0, 2.99, 0.0])
    sel = orc.select(c, r, qr, qn, np.zeros_like(r), 0.4, 0.4, sink=False)
    assert sel.exempt[4] == set()


# ------------------------------------------------------------- planted mistakes

def _planted(w, monkeypatch, budget_shift=0, rank_flip=False):
    """The oracle's selection on workload w with a slip planted: budgets moved
    by budget_shift, or the n-th kept block of each branch exchanged for the
    worst-ranked visible block."""
    c, r, qr, qn = orc.block_stats(w.q, w.k, w.n_kv_heads, w.block)
    beta = w.beta.astype(np.float64) if w.beta is not None else orc.derive_beta(r)
    args = (c, r, qr, qn, beta, w.keep_ratio_centroid, w.keep_ratio_rescue, w.sink)
    true_sel = orc.select(*args)
    with monkeypatch.context() as m:
        if budget_shift:
            real = orc.budget
            m.setattr(orc, "budget", lambda nv, rho: max(0, min(nv, real(nv, rho) + budget_shift)))
        if rank_flip:
            real_top = orc.top_n

            def flipped(scores, n):
                order = orc.rank_order(scores)
                if n < 1 or n >= len(order):
                    return real_top(scores, n)
                keep = list(order[:n - 1]) + [order[-1]]
                return np.sort(np.asarray(keep))
            m.setattr(orc, "top_n", flipped)
        bad = orc.select(*args)
    return true_sel, bad.row_ptr, bad.col_idx


WORKLOADS = {
    "tiny_f32_1k": inputs.tiny_f32_1k,
    "mixture_small": lambda: inputs.mixture_small(S=1500, Hq=8, Hkv=2, rho=0.25, sink=True,
                                                  seed=11),
    "needle_bf16_8k": inputs.needle_bf16_8k,
}


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_oracle_selection_is_accepted(name):
    w = WORKLOADS[name]()
    c, r, qr, qn = orc.block_stats(w.q, w.k, w.n_kv_heads, w.block)
    beta = w.beta.astype(np.float64) if w.beta is not None else orc.derive_beta(r)
    sel = orc.select(c, r, qr, qn, beta, w.keep_ratio_centroid, w.keep_ratio_rescue, w.sink)
    diff, total, _ = H.compare_selection(sel, sel.row_ptr, sel.col_idx, w.n_kv_heads,
                                         w.n_blocks, w.sink)
    assert diff == 0 and total == w.n_kv_heads * w.n_blocks


@pytest.mark.parametrize("shift", [-1, +1], ids=["keep_n_minus_1", "keep_n_plus_1"])
@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_planted_budget_slip_is_rejected(name, shift, monkeypatch):
    w = WORKLOADS[name]()
    sel, rp, ci = _planted(w, monkeypatch, budget_shift=shift)
    changed = sum(sel.row(g, i).tolist() != ci[rp[g * w.n_blocks + i]:
                                                rp[g * w.n_blocks + i + 1]].tolist()
                  for g in range(w.n_kv_heads) for i in range(w.n_blocks))
    assert changed > 0   # the slip does change rows, so the check is not vacuous
    with pytest.raises(AssertionError):
        H.compare_selection(sel, rp, ci, w.n_kv_heads, w.n_blocks, w.sink)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_planted_swap_far_from_the_threshold_is_rejected(name, monkeypatch):
    w = WORKLOADS[name]()
    sel, rp, ci = _planted(w, monkeypatch, rank_flip=True)
    with pytest.raises(AssertionError):
        H.compare_selection(sel, rp, ci, w.n_kv_heads, w.n_blocks, w.sink)


def test_swaps_inside_straddling_bands_pass_up_to_the_row_cap():
    """Rows whose near tie is resolved the other way pass; more such rows than
    the cap (1% of the rows, at least one) fail."""
    nb = 300
    scores = np.linspace(10.0, 1.0, nb)
    scores[[1, 2]] = [9.99999, 9.99998]   # near ties of block 0 at the cut (n = 1)
    c, r, qr, qn = _row_stats(scores)
    rho = 1e-9                             # one block per branch
    sel = orc.select(c, r, qr, qn, np.zeros_like(r), rho, rho, sink=False)
    for i in range(3, nb):
        assert sel.row(0, i).tolist() == [0, i] and sel.exempt[i] == {0, 1, 2}

    def with_flips(flip_rows):
        rows = [sel.row(0, i).tolist() for i in range(nb)]
        for i in flip_rows:
            rows[i] = sorted((set(rows[i]) - {0}) | {1})
        rp = np.zeros(nb + 1, np.int64)
        np.cumsum([len(x) for x in rows], out=rp[1:])
        return rp, np.concatenate([np.asarray(x, np.int32) for x in rows])

    diff, _, _ = H.compare_selection(sel, *with_flips([5, 6]), 1, nb, False)
    assert diff == 2
    with pytest.raises(AssertionError, match="rows differ"):
        H.compare_selection(sel, *with_flips(range(5, 15)), 1, nb, False)


# ------------------------------------------------------------- flop count

def test_bench_pair_count_matches_the_oracle_count():
    """The pair count behind every TFLOP/s figure of bench.py equals the
    oracle's enumeration (full blocks below the diagonal, the causal triangle
    on it, a ragged last block) on a random CSR with skipped-free rows."""
    import bench
    rng = np.random.default_rng(4)
    S, B, Hkv, G = 1000, 128, 3, 4
    nb = orc.n_blocks(S, B)
    rows = []
    for _ in range(Hkv):
        for i in range(nb):
            pick = rng.random(i) < 0.4
            rows.append(np.concatenate([np.nonzero(pick)[0], [i]]).astype(np.int32))
    rp = np.zeros(Hkv * nb + 1, np.int64)
    np.cumsum([len(x) for x in rows], out=rp[1:])
    ci = np.concatenate(rows)
    assert bench.selected_pairs(rp, ci, S, B, Hkv) * G == orc.attention_pairs(rp, ci, S, B, Hkv, G)
    rpd, cid = orc.dense_causal_selection(Hkv, nb)
    assert bench.selected_pairs(rpd, cid, S, B, Hkv) == Hkv * S * (S + 1) // 2
    assert math.isclose(bench.selected_pairs(rpd, cid, S, B, Hkv), Hkv * S * (S + 1) / 2)
