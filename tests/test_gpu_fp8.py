"""Parity of the fp8 attention entry (blocksparse_attn_fwd_fp8) with the
oracle: Q, K, V as E4M3 bytes with per-tensor descales on both sides; the
oracle decodes them exactly and runs the float64 block-sparse attention.

Tolerance, from the arithmetic (fp8_error_model): Q.K^T is exact up to fp32
summation (products of two E4M3 values fit in fp32), the softmax is fp32, and
the one coarse step is rounding each probability to E4M3 before it feeds the
P.V product and the row sum. The model gives, per output element, the
standard deviation of that rounding noise from the exact softmax weights; the
mean absolute error must stay within 1.5 times the model's expectation (plus
the bf16 output rounding) and every element within 8 standard deviations
plus half a bf16 unit. A systematic slip of a few percent of the keys' weight
fails the mean. lse is the log of the same rounded row sum (each probability within 2^-4
relative: 0.07 absolute), which keeps (out, lse) pairs consistent when
partial results are merged.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_long_rbs_amd as rbs
from block_sparse_long_rbs_amd import device, inputs
from oracle import rbs_oracle as orc

import fp8_error_model as M
import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _run(f, t, block, row_ptr, col_idx, **kw):
    rp, ci = H.csr_to_device(row_ptr, col_idx)
    out, lse = rbs.blocksparse_attn_fwd_fp8(t["q"], t["k"], t["v"], block, rp, ci, f.q_descale,
                                            f.k_descale, f.v_descale, want_lse=True, **kw)
    torch.cuda.synchronize()
    return H.to_host(out), lse.cpu().numpy().astype(np.float64)


def _compare(w, f, out_g, lse_g, out_o, lse_o, rows, what, row_ptr, col_idx):
    q, k, v = M.decoded(f)
    sigma = M.rounding_sigma(q, k, v, w.block, row_ptr, col_idx, rows, out_o, lse_o)
    exact = M.exact_slab(out_o, rows, w.block, w.seqlen, w.group)
    got = M.exact_slab(out_g, rows, w.block, w.seqlen, w.group)
    err = got - exact
    mean, expected, worst = M.check(err, sigma, exact, what)
    H.say(f"  {what}: {len(rows)} rows, max-abs {np.abs(err).max():.3e}, mean-abs {mean:.3e} "
          f"(rounding model {expected:.3e}, ratio {mean / expected:.2f}), worst element "
          f"{worst:.2f} of its allowance")
    G = w.group
    worst_lse = 0.0
    for g, i in rows:
        t0, t1 = i * w.block, min(w.seqlen, (i + 1) * w.block)
        a, b = lse_g[g * G:(g + 1) * G, t0:t1], lse_o[g * G:(g + 1) * G, t0:t1]
        fin = np.isfinite(b)
        assert np.array_equal(np.isfinite(a), fin), f"{what}: lse row {(g, i)} finiteness"
        if fin.any():
            worst_lse = max(worst_lse, float(np.abs(a[fin] - b[fin]).max()))
    # every probability rounded up by its most would move lse by ln(1 + 2^-4) = 0.061
    assert worst_lse <= 0.07, f"{what}: lse err {worst_lse}"
    H.say(f"  {what}: lse max-abs {worst_lse:.3e}")


def test_fp8_ragged_small_all_rows():
    """1,500 tokens (a ragged last tile), 8/2 heads, the oracle's selection."""
    w = inputs.mixture_small()
    H.say(f"[case] fp8 {w.name} S={w.seqlen}")
    f = inputs.fp8_inputs(w)
    _, sel = H.oracle_selection(w)
    t = device.upload_fp8(f)
    out_g, lse_g = _run(f, t, w.block, sel.row_ptr, sel.col_idx)
    out_o, lse_o = orc.blocksparse_attention_fp8(f.q, f.k, f.v, f.q_descale, f.k_descale,
                                                 f.v_descale, w.block, sel.row_ptr, sel.col_idx)
    rows = [(g, i) for g in range(w.n_kv_heads) for i in range(w.n_blocks)]
    _compare(w, f, out_g, lse_g, out_o, lse_o, rows, "fp8 attention", sel.row_ptr,
             sel.col_idx)


def test_fp8_last_tile_shorter_than_a_half():
    """700 tokens: the last tile holds 60 keys, so its second 64-key half lies
    wholly past the end (every score masked); 4/1 heads, all rows."""
    w = inputs.mixture_small(S=700, Hq=4, Hkv=1, seed=6)
    H.say(f"[case] fp8 short last tile S={w.seqlen}")
    f = inputs.fp8_inputs(w)
    _, sel = H.oracle_selection(w)
    t = device.upload_fp8(f)
    out_g, lse_g = _run(f, t, w.block, sel.row_ptr, sel.col_idx)
    out_o, lse_o = orc.blocksparse_attention_fp8(f.q, f.k, f.v, f.q_descale, f.k_descale,
                                                 f.v_descale, w.block, sel.row_ptr, sel.col_idx)
    rows = [(g, i) for g in range(w.n_kv_heads) for i in range(w.n_blocks)]
    _compare(w, f, out_g, lse_g, out_o, lse_o, rows, "fp8 short last tile", sel.row_ptr,
             sel.col_idx)


def test_fp8_descales_scale_exactly():
    """Doubling v_descale doubles every output bit for bit; moving a factor 2
    from k_descale to q_descale changes nothing."""
    w = inputs.mixture_small(S=700, Hq=4, Hkv=1, seed=5)
    H.say(f"[case] fp8 descales S={w.seqlen}")
    f = inputs.fp8_inputs(w)
    _, sel = H.oracle_selection(w)
    t = device.upload_fp8(f)
    rp, ci = H.csr_to_device(sel.row_ptr, sel.col_idx)
    call = lambda qd, kd, vd: rbs.blocksparse_attn_fwd_fp8(  # noqa: E731
        t["q"], t["k"], t["v"], w.block, rp, ci, qd, kd, vd, want_lse=True)
    o1, l1 = call(f.q_descale, f.k_descale, f.v_descale)
    o2, l2 = call(f.q_descale, f.k_descale, 2 * f.v_descale)
    o3, l3 = call(2 * f.q_descale, f.k_descale / 2, f.v_descale)
    torch.cuda.synchronize()
    assert torch.equal(o2.float(), 2 * o1.float()) and torch.equal(l1, l2)
    assert torch.equal(o3, o1) and torch.equal(l3, l1)


def test_fp8_empty_rows_and_skipped_entries():
    """A row with no usable block gives 0 and lse -inf; entries beyond the
    diagonal are skipped (the oracle reads only blocks <= i as keys)."""
    w = inputs.random_qkv(300, 4, 2, 128, "f32", seed=7, block=128)
    H.say("[case] fp8 empty rows S=300")
    f = inputs.fp8_inputs(w)
    # rows g * 3 + i: (0,0) empty, (0,1) {0,1,2}, (0,2) {2}, (1,0) {0}, (1,1) {1}, (1,2) {0,1,2}
    row_ptr = np.array([0, 0, 3, 4, 5, 6, 9])
    col_idx = np.array([0, 1, 2, 2, 0, 1, 0, 1, 2], np.int32)
    t = device.upload_fp8(f)
    out_g, lse_g = _run(f, t, 128, row_ptr, col_idx)
    assert np.all(out_g[0:128, 0:2] == 0) and np.all(np.isneginf(lse_g[0:2, 0:128]))
    clipped = np.array([0, 0, 2, 3, 4, 5, 8])
    cols = np.array([0, 1, 2, 0, 1, 0, 1, 2], np.int32)   # (0,1) keeps 0, 1
    rows = [(0, 1), (0, 2), (1, 0), (1, 1), (1, 2)]
    out_o, lse_o = orc.blocksparse_attention_fp8(f.q, f.k, f.v, f.q_descale, f.k_descale,
                                                 f.v_descale, 128, clipped, cols, rows=rows)
    _compare(w, f, out_g, lse_g, out_o, lse_o, rows, "fp8 edge rows", clipped, cols)


def test_fp8_late_dominant_key_raises_the_running_max():
    """A key more than 64 (base 2) above the first tile's scores for the
    queries of the last block: the kernel raises its reference by a whole
    number of powers of two and rescales the partial output (its rare path)."""
    w = inputs.random_qkv(512, 2, 1, 128, "f32", seed=8, block=128)
    q = w.q.copy()
    k = w.k.copy()
    k[300, 0] = 5.0 * q[400, 0] / np.linalg.norm(q[400, 0]) * math.sqrt(128)
    w.q, w.k = q, k
    H.say("[case] fp8 late dominant key S=512")
    f = inputs.fp8_inputs(w)
    qd = orc.e4m3_decode(f.q[:, 0]) * f.q_descale
    kd = orc.e4m3_decode(f.k[:, 0]) * f.k_descale
    b = kd @ qd[400] / math.sqrt(128) * math.log2(math.e)
    assert b[300] - b[:64].max() > 64      # the raise path is taken
    row_ptr, col_idx = orc.dense_causal_selection(1, 4)
    t = device.upload_fp8(f)
    out_g, lse_g = _run(f, t, 128, row_ptr, col_idx)
    out_o, lse_o = orc.blocksparse_attention_fp8(f.q, f.k, f.v, f.q_descale, f.k_descale,
                                                 f.v_descale, 128, row_ptr, col_idx)
    _compare(w, f, out_g, lse_g, out_o, lse_o, [(0, i) for i in range(4)], "fp8 late key",
             row_ptr, col_idx)


def test_fp8_raise_in_second_half_lowers_the_first_halfs_exponents():
    """Every query is 4*e0, so a key's base-2 score is b = 4 k0 scale log2(e)
    and is set by its first coordinate alone. Keys default to b = 0, which
    fixes the reference at 0 from the first tile. In tile 2, key 300 (first
    64-key half) sits at b ~ 0.5, so the first half keeps the reference and
    is packed against it. Keys 320..383 (second half) sit at b = 70, more
    than 64 above, so rows that see them raise the reference by 70 in the
    second half: the first half, already packed, only has its block
    exponents lowered by 70 and O is rescaled before the tile's products."""
    w = inputs.random_qkv(512, 2, 1, 128, "f32", seed=11, block=128)
    unit = 1.0 / (4.0 / math.sqrt(128) * math.log2(math.e))  # k0 for b = 1
    q = np.zeros_like(w.q)
    q[:, :, 0] = 4.0
    k = w.k.copy()
    k[:, :, 0] = 0.0
    k[300, 0, 0] = 0.5 * unit
    k[320:384, 0, 0] = 70.0 * unit
    w.q, w.k = q, k
    H.say("[case] fp8 raise in the second half S=512")
    f = inputs.fp8_inputs(w)
    # the construction survives quantisation
    qd = orc.e4m3_decode(f.q[:, 0]) * f.q_descale
    kd = orc.e4m3_decode(f.k[:, 0]) * f.k_descale
    b = kd @ qd[400] / math.sqrt(128) * math.log2(math.e)
    assert np.all(b[:300] == 0) and np.all(b[301:320] == 0) and np.all(b[384:] == 0)
    assert 0.3 < b[300] < 0.7 and np.allclose(b[320:384], 70.0, atol=1e-4)
    row_ptr, col_idx = orc.dense_causal_selection(1, 4)
    t = device.upload_fp8(f)
    out_g, lse_g = _run(f, t, 128, row_ptr, col_idx)
    out_o, lse_o = orc.blocksparse_attention_fp8(f.q, f.k, f.v, f.q_descale, f.k_descale,
                                                 f.v_descale, 128, row_ptr, col_idx)
    _compare(w, f, out_g, lse_g, out_o, lse_o, [(0, i) for i in range(4)],
             "fp8 second-half raise", row_ptr, col_idx)


@pytest.mark.timeout(600)
def test_fp8_32k_64_8_heads_sampled_rows():
    """32,768 tokens, 64/8 heads (the 32K mixture's head layout), the oracle's
    selection, sampled (KV head, query block) rows."""
    w = inputs.mixture_bf16_32k()
    H.say(f"[case] fp8 {w.name} S={w.seqlen}")
    f = inputs.fp8_inputs(w)
    _, sel = H.oracle_selection(w)
    t = device.upload_fp8(f)
    out_g, lse_g = _run(f, t, w.block, sel.row_ptr, sel.col_idx)
    rows = H.stratified_rows(w.n_kv_heads, w.n_blocks, sel.row_ptr, 256, seed=4)
    out_o, lse_o = orc.blocksparse_attention_fp8(f.q, f.k, f.v, f.q_descale, f.k_descale,
                                                 f.v_descale, w.block, sel.row_ptr, sel.col_idx,
                                                 rows=rows)
    _compare(w, f, out_g, lse_g, out_o, lse_o, rows, "fp8 32K sampled rows", sel.row_ptr,
             sel.col_idx)


@pytest.mark.timeout(600)
def test_fp8_128k_sampled_rows():
    """131,072 tokens, 32/4 heads, the 128K key mixture in fp8, seeded block
    lists at about the selection's density (6%), the launch the benchmark times;
    sampled (KV head, query block) rows checked against the oracle."""
    w = inputs.mixture_bf16_128k()
    H.say(f"[case] fp8 {w.name} S={w.seqlen}")
    f = inputs.fp8_inputs(w)
    nb = w.n_blocks
    row_ptr, col_idx = inputs.random_block_csr(w.n_kv_heads, nb, 0.06, seed=9)
    t = device.upload_fp8(f)
    out_g, lse_g = _run(f, t, w.block, row_ptr, col_idx)
    rows = H.stratified_rows(w.n_kv_heads, nb, row_ptr, 256, seed=3)
    out_o, lse_o = orc.blocksparse_attention_fp8(f.q, f.k, f.v, f.q_descale, f.k_descale,
                                                 f.v_descale, w.block, row_ptr, col_idx, rows=rows)
    _compare(w, f, out_g, lse_g, out_o, lse_o, rows, "fp8 128K sampled rows", row_ptr,
             col_idx)


@pytest.mark.timeout(300)
def test_fp8_rows_longer_than_the_staged_block_list():
    """The long-row cases of the bf16 kernel on the fp8 entry: dense causal at
    40,960 tokens (rows of up to 320 entries) and one 600-entry row with
    out-of-range entries around list positions 256 and 512 at 65,536 tokens."""
    for S, seed, hand_built in ((40960, 53, False), (65536, 54, True)):
        w = inputs.random_qkv(S, 2, 1, 128, "f32", seed=seed, block=128, name=f"fp8_long_{S}")
        f = inputs.fp8_inputs(w)
        nb = S // 128
        if hand_built:
            (rp, ci), (rpc, cic) = H.long_rows_csr(1, nb, nb - 1, 600, seed=4)
            rows = [(0, 0), (0, 7), (0, nb - 1)]
        else:
            rp, ci = orc.dense_causal_selection(1, nb)
            rpc, cic = rp, ci
            rows = [(0, i) for i in (0, 1, 100, 254, 255, 256, 257, 300, nb - 1)]
        H.say(f"[case] fp8 S={S} longest row {int(np.diff(rp).max())} entries")
        t = device.upload_fp8(f)
        out_g, lse_g = _run(f, t, 128, rp, ci)
        out_o, lse_o = orc.blocksparse_attention_fp8(f.q, f.k, f.v, f.q_descale, f.k_descale,
                                                     f.v_descale, 128, rpc, cic, rows=rows)
        _compare(w, f, out_g, lse_g, out_o, lse_o, rows, f"fp8 long rows S={S}", rpc, cic)
