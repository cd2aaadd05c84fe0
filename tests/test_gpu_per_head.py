"""GPU parity of per-query-head selection (one representative query and one
block list per query head) through the C ABI against the float64 oracle:
statistics at 1e-5, sets bit-exact outside the threshold band, attention on
the oracle's per-head CSR within the dtype's tolerance."""
import numpy as np
import pytest
import torch

import block_sparse_long_rbs_amd as rbs
from block_sparse_long_rbs_amd import device, inputs
from oracle import rbs_oracle as orc

import gpu_helpers as H

pytestmark = pytest.mark.gpu


def per_head_case(w, sample_rows=None, seed=0):
    H.say(f"[per-head] {w.name} S={w.seqlen} Hq={w.n_q_heads} Hkv={w.n_kv_heads} "
          f"D={w.head_dim} B={w.block} dtype={w.dtype}")
    t = device.upload(w)
    stats = rbs.rbs_block_stats_per_head(t["q"], t["k"], w.block)
    torch.cuda.synchronize()
    c, r, _, _ = orc.block_stats(w.q, w.k, w.n_kv_heads, w.block)
    qh, qhn = orc.query_rep_per_head(w.q, w.block)
    H.compare_stats([H.to_host(x) for x in stats], (c, r, qh, qhn))
    beta = w.beta.astype(np.float64) if w.beta is not None else orc.derive_beta(r)
    rc, rr = w.keep_ratio_centroid, w.keep_ratio_rescue
    sel = orc.select_per_head(c, r, qh, qhn, beta, rc, rr, w.sink)
    beta_dev = torch.from_numpy(w.beta).cuda() if w.beta is not None else None
    rp, ci, beta_g = rbs.rbs_select_per_head(*stats, rc, rr, sink=w.sink, beta=beta_dev,
                                             want_beta=True)
    torch.cuda.synchronize()
    np.testing.assert_allclose(beta_g.cpu().numpy(), beta, atol=1e-5)
    rp_h = rp.cpu().numpy().astype(np.int64)
    ci_h = ci.cpu().numpy()[:rp_h[-1]]
    nb, Hq = w.n_blocks, w.n_q_heads
    diff, total, n_ex = H.compare_selection(sel, rp_h, ci_h, Hq, nb, w.sink)
    H.say(f"  selection: {diff}/{total} rows differ, all inside near-tie bands "
          f"({n_ex} blocks in such bands)")
    rows = [(h, i) for h in range(Hq) for i in range(nb)]
    if sample_rows is not None and len(rows) > sample_rows:
        rows = H.stratified_rows(Hq, nb, sel.row_ptr, sample_rows, seed)
    rp_o, ci_o = H.csr_to_device(sel.row_ptr, sel.col_idx)
    out_g, lse_g = rbs.blocksparse_attn_fwd_per_head(t["q"], t["k"], t["v"], w.block, rp_o, ci_o,
                                                     want_lse=True)
    out_o, lse_o = orc.blocksparse_attention_per_head(w.q, w.k, w.v, w.block, sel.row_ptr,
                                                      sel.col_idx, rows=rows)
    out_gh, lse_gh = H.to_host(out_g), lse_g.cpu().numpy()
    errs, lerr = [], 0.0
    for h, i in rows:
        t0, t1 = i * w.block, min(w.seqlen, (i + 1) * w.block)
        errs.append(np.abs(out_gh[t0:t1, h] - out_o[t0:t1, h]).reshape(-1))
        lerr = max(lerr, float(np.abs(lse_gh[h, t0:t1] - lse_o[h, t0:t1]).max()))
    e = np.concatenate(errs)
    H.say(f"  attention on oracle per-head CSR: max-abs {e.max():.3e} mean-abs {e.mean():.3e}")
    if w.dtype == "f32":
        assert e.max() <= H.TOL_F32 and lerr <= 1e-5
    else:
        assert e.max() <= H.TOL_BF16_MAX and e.mean() <= H.TOL_BF16_MEAN and lerr <= 2e-2
    # end to end: the GPU's own per-head lists into the GPU's attention, on the
    # sampled rows whose GPU list equals the oracle's
    out_e, _ = rbs.blocksparse_attn_fwd_per_head(t["q"], t["k"], t["v"], w.block, rp, ci)
    out_eh = H.to_host(out_e)
    same = [(h, i) for (h, i) in rows
            if ci_h[rp_h[h * nb + i]:rp_h[h * nb + i + 1]].tolist() ==
            sel.col_idx[sel.row_ptr[h * nb + i]:sel.row_ptr[h * nb + i + 1]].tolist()]
    assert len(same) >= len(rows) // 2, f"only {len(same)} of {len(rows)} sampled rows agree"
    e2 = np.concatenate([np.abs(out_eh[i * w.block:min(w.seqlen, (i + 1) * w.block), h] -
                                out_o[i * w.block:min(w.seqlen, (i + 1) * w.block), h]).reshape(-1)
                         for h, i in same])
    H.say(f"  end to end on {len(same)}/{len(rows)} rows: max-abs {e2.max():.3e} "
          f"mean-abs {e2.mean():.3e}")
    if w.dtype == "f32":
        assert e2.max() <= H.TOL_F32
    else:
        assert e2.max() <= H.TOL_BF16_MAX and e2.mean() <= H.TOL_BF16_MEAN
    return t, stats


def test_per_head_mixture_bf16_ragged():
    per_head_case(inputs.mixture_small(S=1500, Hq=8, Hkv=2, rho=0.25, sink=True, seed=17))


def test_per_head_tiny_f32_given_beta():
    per_head_case(inputs.tiny_f32_1k())


def test_per_head_odd_group_bf16_d64_block64():
    """GQA 3:1 on the vector-ALU path (bf16, head dim 64, block 64)."""
    w = inputs.random_qkv(900, 6, 2, 64, "bf16", seed=19, block=64, name="per_head_g3",
                          keep_ratio_centroid=0.3, keep_ratio_rescue=0.2, sink=True)
    per_head_case(w)


def test_per_head_needle_8k_sampled():
    per_head_case(inputs.needle_bf16_8k(), sample_rows=256)


@pytest.mark.timeout(600)
def test_per_head_mixture_128k_sampled():
    """The benchmarked 128K workload (32/4 heads, keep-ratio 0.03, sink) with
    one list per query head: statistics and every row's set, attention on
    sampled (query head, query block) rows."""
    per_head_case(inputs.mixture_bf16_128k(), sample_rows=256, seed=3)


def test_per_head_reps_average_to_the_group_reps_on_gpu():
    """The GPU's per-head representatives average over each group to the
    GPU's group representative (both from their own single pass)."""
    w = inputs.mixture_small(S=1000, Hq=8, Hkv=2, rho=0.25, sink=False, seed=23)
    t = device.upload(w)
    _, _, qr, _ = rbs.rbs_block_stats(t["q"], t["k"], w.block)
    _, _, qh, _ = rbs.rbs_block_stats_per_head(t["q"], t["k"], w.block)
    torch.cuda.synchronize()
    avg = qh.view(2, 4, w.n_blocks, -1).mean(dim=1)
    assert (avg - qr).abs().max().item() <= 1e-5 * qr.abs().max().item()
