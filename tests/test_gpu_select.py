"""GPU parity of rbs_select on its own, on directly drawn block statistics:
both selection paths (register-held rows for up to 1,024 blocks, LDS rows
beyond), derived and given beta, with and without the sink. Sets must equal
the oracle's outside its threshold band; derived beta within 1e-5."""
import numpy as np
import pytest
import torch

import block_sparse_long_rbs_amd as rbs
from block_sparse_long_rbs_amd import inputs
from oracle import rbs_oracle as orc

import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nb,D,rho_c,rho_r,sink,beta_given,seed", [
    (1024, 128, 0.05, 0.05, True, False, 1),    # largest register-path size
    (1032, 64, 0.05, 0.08, True, False, 2),     # just past it: LDS path
    (1500, 128, 0.1, 0.03, False, True, 3),     # LDS path, beta given
    (2100, 128, 0.02, 0.02, True, False, 4),    # long rows
    (300, 64, 0.5, 0.25, False, False, 5),      # short rows, large budgets
])
def test_select_matches_oracle(nb, D, rho_c, rho_r, sink, beta_given, seed):
    Hkv = 2
    cen, rad, qrep, qn, beta = inputs.synthetic_block_stats(Hkv, nb, D, seed, beta_given)
    H.say(f"[select] nb={nb} D={D} rho=({rho_c},{rho_r}) sink={sink} beta_given={beta_given}")
    dev = lambda x: torch.from_numpy(x).cuda()
    rp, ci, beta_out = rbs.rbs_select(dev(cen), dev(rad), dev(qrep), dev(qn), rho_c, rho_r,
                                      sink=sink, beta=dev(beta) if beta is not None else None,
                                      want_beta=True)
    torch.cuda.synchronize()
    rp_h = rp.cpu().numpy().astype(np.int64)
    ci_h = ci.cpu().numpy()[:rp_h[-1]]
    b = beta.astype(np.float64) if beta is not None else orc.derive_beta(rad.astype(np.float64))
    sel = orc.select(cen.astype(np.float64), rad.astype(np.float64), qrep.astype(np.float64),
                     qn.astype(np.float64), b, rho_c, rho_r, sink)
    diff, total, n_ex = H.compare_selection(sel, rp_h, ci_h, Hkv, nb, sink)
    H.say(f"  {diff}/{total} rows differ, all inside near-tie bands ({n_ex} blocks in such bands)")
    np.testing.assert_allclose(beta_out.cpu().numpy(), sel.beta, atol=1e-5)
    assert rp_h[-1] == len(sel.col_idx) or diff > 0


def _patterned_stats(scores, D=64):
    """One KV head whose centroid scores q_rep_i . c_j equal `scores[j]`
    exactly (q_rep = e_0 with norm 1, c_j = scores[j] e_0, radius 0 so the
    rescue branch equals the centroid branch)."""
    nb = len(scores)
    cen = np.zeros((1, nb, D), np.float32)
    cen[0, :, 0] = scores
    rad = np.zeros((1, nb), np.float32)
    qrep = np.zeros((1, nb, D), np.float32)
    qrep[0, :, 0] = 1.0
    qn = np.ones((1, nb), np.float32)
    return cen, rad, qrep, qn


_J = np.arange(1024)
_PATTERNS = {
    "ascending": _J.astype(np.float32),
    "descending": (1024 - _J).astype(np.float32),
    "one_lane_holds_the_top": np.where(_J % 64 == 5, 1000 + _J, _J % 7).astype(np.float32),
    "two_lanes_tied": np.where(_J % 64 < 2, 500, 1).astype(np.float32),
    "three_values": (_J % 3).astype(np.float32),
}


@pytest.mark.parametrize("rho", [0.04, 0.1])
@pytest.mark.parametrize("name", sorted(_PATTERNS))
def test_select_exact_on_integer_scores(name, rho):
    """Integer scores are exact in fp32 and fp64, so every row's set must equal
    the oracle's exactly, ties going to the lower block index. The patterns
    put the top keys in every lane, in one lane, or in long runs of ties, so
    that the budget search meets few, some hundred, or most candidates at or
    above its first bound (budgets up to 41 at rho 0.04, up to 103 at 0.1)."""
    cen, rad, qrep, qn = _patterned_stats(_PATTERNS[name])
    nb = cen.shape[1]
    dev = lambda x: torch.from_numpy(x).cuda()
    rp, ci, _ = rbs.rbs_select(dev(cen), dev(rad), dev(qrep), dev(qn), rho, rho, sink=False)
    torch.cuda.synchronize()
    rp_h = rp.cpu().numpy().astype(np.int64)
    ci_h = ci.cpu().numpy()[:rp_h[-1]]
    sel = orc.select(cen.astype(np.float64), rad.astype(np.float64), qrep.astype(np.float64),
                     qn.astype(np.float64), orc.derive_beta(rad.astype(np.float64)), rho, rho,
                     False)
    for i in range(nb):
        got = ci_h[rp_h[i]:rp_h[i + 1]].tolist()
        want = sel.col_idx[sel.row_ptr[i]:sel.row_ptr[i + 1]].tolist()
        assert got == want, f"{name} rho={rho} row {i}: got {got} want {want}"
