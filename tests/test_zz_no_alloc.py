"""rbs_select_static (the selection entry that allocates nothing and uses the
library's static per-GPU scratch) against rbs_select with a caller workspace,
through the C ABI: the CSR lists and the betas must be identical, on two calls
in a row (the second smaller, on the scratch the first left behind), and a
call that needs more scratch than the static array holds must be refused
before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_long_rbs_amd as rbs
from block_sparse_long_rbs_amd import _lib, inputs
from oracle import rbs_oracle as orc

import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _both(Hkv, nb, D, rho_c, rho_r, sink, beta_given, seed):
    cen, rad, qrep, qn, beta = inputs.synthetic_block_stats(Hkv, nb, D, seed, beta_given)
    args = [_dev(x) for x in (cen, rad, qrep, qn)]
    b = _dev(beta)
    H.say(f"[no-alloc] Hkv={Hkv} nb={nb} D={D} rho=({rho_c},{rho_r}) sink={sink} "
          f"beta_given={beta_given}")
    rp_w, ci_w, be_w = rbs.rbs_select(*args, rho_c, rho_r, sink=sink, beta=b, want_beta=True)
    rp_s, ci_s, be_s = rbs.rbs_select_static(*args, rho_c, rho_r, sink=sink, beta=b,
                                             want_beta=True)
    torch.cuda.synchronize()
    nnz = int(rp_w[-1].item())
    assert torch.equal(rp_s, rp_w), "row_ptr differs"
    assert torch.equal(ci_s[:nnz], ci_w[:nnz]), "col_idx differs"
    assert torch.equal(be_s, be_w), "beta differs"
    # and both against the oracle's selection
    bo = beta.astype(np.float64) if beta is not None else orc.derive_beta(rad.astype(np.float64))
    sel = orc.select(cen.astype(np.float64), rad.astype(np.float64), qrep.astype(np.float64),
                     qn.astype(np.float64), bo, rho_c, rho_r, sink)
    diff, total, _ = H.compare_selection(sel, rp_s.cpu().numpy().astype(np.int64),
                                         ci_s[:nnz].cpu().numpy(), Hkv, nb, sink)
    H.say(f"  identical to the workspace call; {diff}/{total} rows differ from the oracle "
          f"(inside near-tie bands)")
    return nnz


def test_static_scratch_matches_the_workspace_call_twice():
    # 1,024 blocks x 4 KV heads (the 128K layout): about 9.5 MB of scratch
    n1 = _both(4, 1024, 128, 0.03, 0.03, True, False, seed=31)
    # a smaller second call on the scratch the first one left
    n2 = _both(2, 300, 64, 0.1, 0.05, False, True, seed=32)
    assert n2 < n1


def test_static_scratch_refuses_a_call_that_does_not_fit():
    Hkv, nb, D = 32, 1024, 128          # one list per query head at 128K: ~67 MB of scratch
    need = ctypes.c_size_t(0)
    st = _lib.lib().rbs_select(None, None, None, None, None, Hkv, nb, D, 0.03, 0.03, 0, None,
                               None, None, 0, None, ctypes.byref(need), None)
    assert st == _lib.RBS_OK and need.value > _lib.RBS_SELECT_STATIC_SCRATCH_BYTES
    f = dict(device="cuda", dtype=torch.float32)
    cen, qrep = torch.zeros((Hkv, nb, D), **f), torch.zeros((Hkv, nb, D), **f)
    rad, qn = torch.zeros((Hkv, nb), **f), torch.zeros((Hkv, nb), **f)
    with pytest.raises(rbs.RbsError) as e:
        rbs.rbs_select_static(cen, rad, qrep, qn, 0.03, 0.03)
    assert e.value.status == _lib.RBS_E_CAPACITY
