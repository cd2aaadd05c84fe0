"""Parity of the fp8 attention entry (blocksparse_attn_fwd_fp8) with the
oracle: Q, K, V as E4M3 bytes with per-tensor descales on both sides; the
oracle decodes them exactly and runs the float64 block-sparse attention.

Tolerance, from the arithmetic. Q.K^T is exact up to fp32 summation (products
of two E4M3 values fit in fp32), the softmax is fp32, and the one coarse step
is rounding each probability p to E4M3 (nearest even: relative error <= 2^-4)
before the P.V product. With weights w_u = p_u / sum p the output error is
sum_u w_u e_u v_u with |e_u| <= 2^-4, so
  max-abs  <= 2^-4 * max|v|  (+ bf16 output rounding, 2^-8 * max|out|),
  mean-abs <= 2^-4 / sqrt(3) * rms(v)   (errors uniform in +-2^-4: their
             rms, times the weighted rms of v, bounds the mean magnitude).
Probabilities below 2^-6 round with absolute error <= 2^-10 instead; they
weigh little and the bounds above hold on these workloads with a margin.
lse: exact up to fp32 rounding of the scores and of the row sum (1e-3).
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_long_rbs_amd as rbs
from block_sparse_long_rbs_amd import device, inputs
from oracle import rbs_oracle as orc

import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _tols(f):
    v = orc.e4m3_decode(f.v) * f.v_descale
    return 2.0 ** -4 * float(np.abs(v).max()), 2.0 ** -4 / math.sqrt(3.0) * float(np.sqrt(np.mean(v * v)))


def _run(f, t, block, row_ptr, col_idx, **kw):
    rp, ci = H.csr_to_device(row_ptr, col_idx)
    out, lse = rbs.blocksparse_attn_fwd_fp8(t["q"], t["k"], t["v"], block, rp, ci, f.q_descale,
                                            f.k_descale, f.v_descale, want_lse=True, **kw)
    torch.cuda.synchronize()
    return H.to_host(out), lse.cpu().numpy().astype(np.float64)


def _compare(w, f, out_g, lse_g, out_o, lse_o, rows, what):
    tmax, tmean = _tols(f)
    mx, mean = H._slab_errors(out_g, out_o, rows, w)
    omax = float(np.nanmax(np.abs(out_o)))
    H.say(f"  {what}: max-abs {mx:.3e} (bound {tmax + 2 ** -8 * omax:.3e}) "
          f"mean-abs {mean:.3e} (bound {tmean:.3e})")
    assert mx <= tmax + 2.0 ** -8 * omax, f"{what}: max-abs {mx}"
    assert mean <= tmean, f"{what}: mean-abs {mean}"
    G = w.group
    for g, i in rows:
        t0, t1 = i * w.block, min(w.seqlen, (i + 1) * w.block)
        d = np.abs(lse_g[g * G:(g + 1) * G, t0:t1] - lse_o[g * G:(g + 1) * G, t0:t1]).max()
        assert d <= 1e-3, f"{what}: lse row {(g, i)} err {d}"


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
    _compare(w, f, out_g, lse_g, out_o, lse_o, rows, "fp8 attention")


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
    _compare(w, f, out_g, lse_g, out_o, lse_o, rows, "fp8 short last tile")


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
    _compare(w, f, out_g, lse_g, out_o, lse_o, rows, "fp8 edge rows")


def test_fp8_late_dominant_key_raises_the_running_max():
    """A key far above the first tile's scores (2^8 past its max) takes the
    rescale path; P stays inside E4M3's range and the result matches."""
    w = inputs.random_qkv(512, 2, 1, 128, "f32", seed=8, block=128)
    q = w.q.copy()
    k = w.k.copy()
    k[300, 0] = 3.0 * q[400, 0] / np.linalg.norm(q[400, 0]) * math.sqrt(128)
    w.q, w.k = q, k
    H.say("[case] fp8 late dominant key S=512")
    f = inputs.fp8_inputs(w)
    row_ptr, col_idx = orc.dense_causal_selection(1, 4)
    t = device.upload_fp8(f)
    out_g, lse_g = _run(f, t, 128, row_ptr, col_idx)
    out_o, lse_o = orc.blocksparse_attention_fp8(f.q, f.k, f.v, f.q_descale, f.k_descale,
                                                 f.v_descale, 128, row_ptr, col_idx)
    _compare(w, f, out_g, lse_g, out_o, lse_o, [(0, i) for i in range(4)], "fp8 late key")


def test_fp8_raise_in_second_half_recomputes_first_half():
    """Every query is 4*e0, so a key's base-2 score is b = 4 k0 scale log2(e)
    and is set by its first coordinate alone. Keys default to b = 0, which
    fixes the running max at 0 from the first tile. In tile 2, key 300 (first
    64-key half) sits at b ~ 3, so the first half keeps the max (a lane's
    share of its row sum is about 8 + 31 < 2^8). Keys 320..383 (second half)
    sit at b = 4, so every lane's share of the second half's row sum is
    32 * 16 > 2^8. Rows that see them therefore raise the max in the second
    half, and the first half's P, already packed, has to be redone from the
    new max. Every kept probability stays in e4m3's normal range."""
    w = inputs.random_qkv(512, 2, 1, 128, "f32", seed=11, block=128)
    unit = 1.0 / (4.0 / math.sqrt(128) * math.log2(math.e))  # k0 for b = 1
    q = np.zeros_like(w.q)
    q[:, :, 0] = 4.0
    k = w.k.copy()
    k[:, :, 0] = 0.0
    k[300, 0, 0] = 3.0 * unit
    k[320:384, 0, 0] = 4.0 * unit
    w.q, w.k = q, k
    H.say("[case] fp8 raise in the second half S=512")
    f = inputs.fp8_inputs(w)
    # the construction survives quantisation
    qd = orc.e4m3_decode(f.q[:, 0]) * f.q_descale
    kd = orc.e4m3_decode(f.k[:, 0]) * f.k_descale
    b = kd @ qd[400] / math.sqrt(128) * math.log2(math.e)
    assert np.all(b[:300] == 0) and np.all(b[301:320] == 0) and np.all(b[384:] == 0)
    assert 2.5 < b[300] < 3.5 and np.allclose(b[320:384], 4.0, atol=1e-6)
    row_ptr, col_idx = orc.dense_causal_selection(1, 4)
    t = device.upload_fp8(f)
    out_g, lse_g = _run(f, t, 128, row_ptr, col_idx)
    out_o, lse_o = orc.blocksparse_attention_fp8(f.q, f.k, f.v, f.q_descale, f.k_descale,
                                                 f.v_descale, 128, row_ptr, col_idx)
    _compare(w, f, out_g, lse_g, out_o, lse_o, [(0, i) for i in range(4)], "fp8 second-half raise")


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
    nb = w.n_blocks
    rng = np.random.default_rng(4)
    allrows = [(g, i) for g in range(w.n_kv_heads) for i in range(nb)]
    pick = rng.choice(len(allrows), size=8, replace=False)
    rows = [allrows[x] for x in sorted(pick)] + [(0, 0), (w.n_kv_heads - 1, nb - 1)]
    out_o, lse_o = orc.blocksparse_attention_fp8(f.q, f.k, f.v, f.q_descale, f.k_descale,
                                                 f.v_descale, w.block, sel.row_ptr, sel.col_idx,
                                                 rows=rows)
    _compare(w, f, out_g, lse_g, out_o, lse_o, rows, "fp8 32K sampled rows")


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
    rng = np.random.default_rng(3)
    allrows = [(g, i) for g in range(w.n_kv_heads) for i in range(nb)]
    pick = rng.choice(len(allrows), size=8, replace=False)
    rows = [allrows[x] for x in sorted(pick)] + [(0, 0), (w.n_kv_heads - 1, nb - 1)]
    out_o, lse_o = orc.blocksparse_attention_fp8(f.q, f.k, f.v, f.q_descale, f.k_descale,
                                                 f.v_descale, w.block, row_ptr, col_idx, rows=rows)
    _compare(w, f, out_g, lse_g, out_o, lse_o, rows, "fp8 128K sampled rows")
