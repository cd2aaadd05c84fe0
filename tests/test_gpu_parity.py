"""GPU parity: the HIP path through the C ABI against the float64 oracle on
the same seeded inputs.

Selection: sets bit-exact except blocks whose oracle score lies in the
threshold band. Attention: run on the oracle's own CSR (so no oracle input
comes from the GPU) within 2e-2 max-abs / 1e-2 mean-abs for bf16 inputs and
1e-5 for fp32; end to end (GPU stats -> GPU select -> GPU attention) on rows
whose GPU block set equals the oracle's.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_rbs_amd as rbs
from block_sparse_long_rbs_amd import device, inputs
from oracle import rbs_oracle as orc

import gpu_helpers as H

pytestmark = pytest.mark.gpu


def test_tiny_f32_1k():
    """1,024 tokens, GQA 2:1, dim 64, block 64, fp32 (needle blocks, beta = 1)."""
    H.pipeline_case(inputs.tiny_f32_1k())


def test_needle_bf16_8k():
    H.pipeline_case(inputs.needle_bf16_8k(), sample_rows=256)


def test_mixture_bf16_ragged_small():
    """12 blocks with a 92-token last block; sink on; several tiles per row."""
    H.pipeline_case(inputs.mixture_small(S=1500, Hq=8, Hkv=2, rho=0.25, sink=True, seed=11))


def test_random_f32_ragged_d128():
    w = inputs.random_qkv(700, 4, 2, 128, "f32", seed=21, block=64, name="random_f32_700",
                          keep_ratio_centroid=0.3, keep_ratio_rescue=0.2)
    H.pipeline_case(w)


def test_random_f32_block128():
    w = inputs.random_qkv(1000, 6, 3, 64, "f32", seed=22, block=128, name="random_f32_1000",
                          keep_ratio_centroid=0.5, keep_ratio_rescue=0.4, sink=True)
    H.pipeline_case(w)


@pytest.mark.parametrize("D,B", [(64, 64), (128, 64), (64, 128)])
def test_bf16_vector_alu_shapes(D, B):
    """bf16 at head dim or block 64 runs on the vector-ALU kernel (fp32
    arithmetic, bf16 output); ragged tail, GQA 4:2."""
    w = inputs.random_qkv(700, 4, 2, D, "bf16", seed=40 + D + B, block=B,
                          name=f"bf16_vec_{D}_{B}", keep_ratio_centroid=0.3,
                          keep_ratio_rescue=0.25, sink=True)
    H.pipeline_case(w)


def test_odd_gqa_ratio_bf16():
    """GQA 3:1 (odd group, single-head workgroups) with a ragged tail."""
    w = inputs.random_qkv(900, 6, 2, 128, "bf16", seed=13, block=128, name="gqa3_bf16_900",
                          keep_ratio_centroid=0.4, keep_ratio_rescue=0.3, sink=True)
    H.pipeline_case(w)


def test_keep_ratio_one_is_dense_bf16():
    w = inputs.random_qkv(640, 8, 1, 128, "bf16", seed=5, block=128, name="dense_bf16_640",
                          keep_ratio_centroid=1.0, keep_ratio_rescue=1.0)
    r = H.pipeline_case(w)
    rp_h = r["rp"].cpu().numpy()
    assert rp_h[-1] == 5 * 6 // 2


def test_single_partial_block_and_tiny_sequences():
    for S in (1, 37, 128):
        w = inputs.random_qkv(S, 2, 1, 128, "bf16", seed=S, block=128, name=f"short_{S}",
                              keep_ratio_centroid=0.5, keep_ratio_rescue=0.5)
        H.pipeline_case(w)


def test_empty_sequence_is_a_noop():
    q = torch.zeros((0, 4, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    cen, rad, qr, qn = rbs.rbs_block_stats(q, k, 128)
    assert cen.shape == (2, 0, 128)
    rp, ci, _ = rbs.rbs_select(cen, rad, qr, qn, 0.1, 0.1)
    assert rp.cpu().tolist() == [0]
    out, _ = rbs.blocksparse_attn_fwd(q, k, k, 128, rp, ci)
    assert out.shape == q.shape


def test_determinism_and_row_permutation():
    w = inputs.mixture_small(S=1024, Hq=8, Hkv=2, rho=0.3, sink=False, seed=3)
    t = device.upload(w)
    res = []
    for _ in range(2):
        st = rbs.rbs_block_stats(t["q"], t["k"], w.block)
        rp, ci, _ = rbs.rbs_select(*st, w.keep_ratio_centroid, w.keep_ratio_rescue)
        out, lse = rbs.blocksparse_attn_fwd(t["q"], t["k"], t["v"], w.block, rp, ci, want_lse=True)
        nnz = int(rp[-1].item())
        res.append((rp.cpu(), ci[:nnz].cpu(), out.cpu(), lse.cpu()))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)
    # reversing every CSR row changes the accumulation order, not the result
    rp_h = res[0][0].numpy()
    ci_h = res[0][1].numpy().copy()
    for r in range(len(rp_h) - 1):
        ci_h[rp_h[r]:rp_h[r + 1]] = ci_h[rp_h[r]:rp_h[r + 1]][::-1]
    rp_d, ci_d = H.csr_to_device(rp_h, ci_h)
    out2, _ = rbs.blocksparse_attn_fwd(t["q"], t["k"], t["v"], w.block, rp_d, ci_d)
    d = (out2.float() - res[0][2].cuda().float()).abs()
    assert d.max().item() <= 2e-2 and d.mean().item() <= 1e-3


def test_csr_entries_outside_the_causal_range_are_skipped():
    w = inputs.random_qkv(512, 4, 1, 128, "bf16", seed=8, block=128, name="skip")
    t = device.upload(w)
    rp, ci = orc.dense_causal_selection(1, 4)
    # add out-of-range entries (> i and negative) to every row
    rows = [list(ci[rp[i]:rp[i + 1]]) + [i + 1, -3, 99] for i in range(4)]
    rp2 = np.zeros(5, np.int64)
    np.cumsum([len(r) for r in rows], out=rp2[1:])
    a, b = H.csr_to_device(rp2, np.concatenate(rows))
    out, _ = rbs.blocksparse_attn_fwd(t["q"], t["k"], t["v"], 128, a, b)
    o, _ = orc.blocksparse_attention(w.q, w.k, w.v, 128, rp, ci)
    d = np.abs(H.to_host(out) - o)
    assert d.max() <= H.TOL_BF16_MAX and d.mean() <= H.TOL_BF16_MEAN


def test_late_dominant_key_raises_the_running_max():
    """A key in block 1 gives the queries of block 3 logits about 70 (base 2)
    above everything in block 0, the first block of their CSR row: the kernel
    must raise its running max and rescale the partial output (its rare path).
    Listing the dominant block first must give the same result."""
    S, Hq, Hkv, D, B = 512, 8, 2, 128, 128
    w = inputs.random_qkv(S, Hq, Hkv, D, "bf16", seed=31, block=B, name="late_max")
    rng = np.random.default_rng(5)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    q = w.q.astype(np.float64)
    q[3 * B:4 * B, 0:Hq // Hkv] += 3.0 * u          # group 0 queries of block 3 lean along u
    k = w.k.astype(np.float64)
    k[200, 0] = 200.0 * u                            # block 1, group 0: dominant key
    w.q = inputs.bf16_round(q.astype(np.float32))
    w.k = inputs.bf16_round(k.astype(np.float32))
    t = device.upload(w)
    rp, ci = orc.dense_causal_selection(Hkv, S // B)
    o, lse_o = orc.blocksparse_attention(w.q, w.k, w.v, B, rp, ci)
    # the logits really do exceed the first block's max by more than 64 (base 2)
    scale_log2 = 1.4426950408889634 / np.sqrt(D)
    qq = w.q[3 * B:4 * B, 0].astype(np.float64)
    first = (qq @ w.k[0:B, 0].astype(np.float64).T).max(axis=1) * scale_log2
    late = (qq @ w.k[200, 0].astype(np.float64)) * scale_log2
    assert (late - first).max() > 64
    for order in ("ascending", "dominant first"):
        ci_o = ci.copy()
        if order != "ascending":
            for r in range(len(rp) - 1):
                row = list(ci_o[rp[r]:rp[r + 1]])
                if 1 in row:
                    row.remove(1)
                    ci_o[rp[r]:rp[r + 1]] = [1] + row
        a, b = H.csr_to_device(rp, ci_o)
        out, lse = rbs.blocksparse_attn_fwd(t["q"], t["k"], t["v"], B, a, b, want_lse=True)
        d = np.abs(H.to_host(out) - o)
        H.say(f"  {order}: max-abs {d.max():.3e} mean-abs {d.mean():.3e}")
        assert d.max() <= H.TOL_BF16_MAX and d.mean() <= H.TOL_BF16_MEAN, order
        dl = np.abs(lse.cpu().numpy() - lse_o)
        assert dl.max() <= 2e-2, (order, dl.max())


@pytest.mark.timeout(300)
def test_rows_longer_than_the_staged_block_list():
    """Dense causal attention at 40,960 tokens (320 blocks per row at the end,
    past the 256 entries the kernel stages in LDS at a time), then one
    hand-built row of 600 entries at 65,536 tokens: every visible block in a
    shuffled order with out-of-range entries spliced in around list positions
    256 and 512. Checked against the oracle on sampled rows, the last row and
    the rows on both sides of 256 entries."""
    S, Hq, Hkv, B = 40960, 2, 1, 128
    w = inputs.random_qkv(S, Hq, Hkv, 128, "bf16", seed=51, block=B, name="dense_40k")
    H.say(f"[case] dense causal S={S} rows up to {S // B} entries")
    t = device.upload(w)
    nb = S // B
    rp, ci = orc.dense_causal_selection(Hkv, nb)
    a, b = H.csr_to_device(rp, ci)
    out, lse = rbs.blocksparse_attn_fwd(t["q"], t["k"], t["v"], B, a, b, want_lse=True)
    rows = [(0, i) for i in (0, 1, 100, 254, 255, 256, 257, 300, nb - 1)]
    o, lo = orc.blocksparse_attention(w.q, w.k, w.v, B, rp, ci, rows=rows)
    mx, mean = H._slab_errors(H.to_host(out), o, rows, w)
    H._assert_attn(w, mx, mean, "dense 40K sampled rows")
    toks = H.row_tokens(rows, B, S)
    assert np.abs(lse.cpu().numpy()[:, toks] - lo[:, toks]).max() <= 2e-2

    S = 65536
    w = inputs.random_qkv(S, Hq, Hkv, 128, "bf16", seed=52, block=B, name="long_row_64k")
    nb = S // B
    (rp, ci), (rpc, cic) = H.long_rows_csr(Hkv, nb, nb - 1, 600, seed=3)
    H.say(f"[case] one row of {rp[nb] - rp[nb - 1]} entries at S={S}")
    t = device.upload(w)
    a, b = H.csr_to_device(rp, ci)
    out, _ = rbs.blocksparse_attn_fwd(t["q"], t["k"], t["v"], B, a, b)
    rows = [(0, 0), (0, 7), (0, nb - 1)]
    o, _ = orc.blocksparse_attention(w.q, w.k, w.v, B, rpc, cic, rows=rows)
    mx, mean = H._slab_errors(H.to_host(out), o, rows, w)
    H._assert_attn(w, mx, mean, "600-entry row")
