"""GPU parity of Block-attention's RAG mask with RoPE re-encoding of cached
keys (block_mask_attn_fwd) against the float64 oracle."""
import numpy as np
import pytest
import torch

import block_sparse_long_rbs_amd as rbs
from block_sparse_long_rbs_amd import device, inputs
from oracle import rbs_oracle as orc

import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _run(w, q_row_begin=0, tokens=None, workspace=None):
    H.say(f"[case] {w.name} S={w.seqlen} segments={len(w.seg_start) - 1} q_row_begin={q_row_begin}")
    t = device.upload(w)
    k_before = t["k"].clone()
    sentinel = torch.full_like(t["q"], 7.0)
    out, lse = rbs.block_mask_attn_fwd(t["q"], t["k"], t["v"], w.seg_start.tolist(),
                                       w.k_rerotate.tolist(), w.rope_theta,
                                       q_row_begin=q_row_begin, want_lse=True, out=sentinel,
                                       workspace=workspace)
    assert torch.equal(t["k"], k_before), "cached keys were modified"
    out_h = H.to_host(out)
    if tokens is None:
        tokens = np.arange(q_row_begin, w.seqlen)
    o, l = orc.block_mask_attention(w.q, w.k, w.v, w.seg_start, w.k_rerotate, w.rope_theta,
                                    q_row_begin=q_row_begin, rows=tokens)
    d = np.abs(out_h[tokens] - o[tokens])
    H.say(f"  max-abs {d.max():.3e} mean-abs {d.mean():.3e}")
    assert d.max() <= H.TOL_BF16_MAX and d.mean() <= H.TOL_BF16_MEAN
    dl = np.abs(lse.cpu().numpy()[:, tokens] - l[:, tokens]).max()
    assert dl <= 2e-2, f"lse err {dl}"
    if q_row_begin > 0:
        assert np.all(out_h[:q_row_begin] == 7.0), "rows before q_row_begin were written"
    return out_h


def test_rag_small_all_rows_ragged_final_block():
    w = inputs.rag_layout(n_passages=4, passage_len=256, final_len=200, Hq=8, Hkv=2, seed=31,
                          name="rag_small")
    _run(w)


def test_rag_small_final_block_only():
    w = inputs.rag_layout(n_passages=3, passage_len=384, final_len=128, Hq=8, Hkv=4, seed=32,
                          name="rag_small_final")
    _run(w, q_row_begin=int(w.seg_start[-2]))


def test_rag_zero_offsets_is_plain_segment_attention():
    """With every re-rotation offset 0 the keys are used as given."""
    w = inputs.rag_layout(n_passages=2, passage_len=128, final_len=128, Hq=4, Hkv=1, seed=33,
                          name="rag_zero_off")
    w.k_rerotate = np.zeros_like(w.k_rerotate)
    _run(w)


def test_rag_31k_sampled_rows():
    """The 20 x 1,536 + 512 RAG layout, 32/8 heads, theta 5e5: in every
    passage its first two rows, its last row and 12 random rows (300 passage
    rows), and every other row of the final block plus its last (257 rows)."""
    w = inputs.rag_bf16_31k()
    rng = np.random.default_rng(0)
    seg = w.seg_start
    toks = []
    for p in range(len(seg) - 2):
        a, b = int(seg[p]), int(seg[p + 1])
        toks += [a, a + 1, b - 1] + rng.choice(np.arange(a + 2, b - 1), size=12,
                                               replace=False).tolist()
    toks += list(range(int(seg[-2]), w.seqlen, 2)) + [w.seqlen - 1]
    _run(w, tokens=np.unique(np.asarray(toks, np.int64)))


def test_rag_split_final_block_all_final_rows():
    """A final block after 132 key tiles: its rows' key ranges are split into
    chunks run by separate workgroups and merged (every final row checked),
    once with all rows and once with the final block only, starting inside a
    tile."""
    w = inputs.rag_layout(n_passages=11, passage_len=1536, final_len=300, Hq=8, Hkv=2, seed=34,
                          name="rag_split")
    s_last = int(w.seg_start[-2])
    rng = np.random.default_rng(1)
    toks = np.sort(np.concatenate([rng.choice(s_last, size=24, replace=False),
                                   np.arange(s_last, w.seqlen)]))
    # a workspace full of NaN bytes: nothing may depend on its prior contents
    t = device.upload(w)
    nbytes = rbs.block_mask_workspace_bytes(t["q"], t["k"], t["v"], w.seg_start.tolist(),
                                            w.k_rerotate.tolist(), w.rope_theta)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    _run(w, tokens=toks, workspace=ws)
    _run(w, q_row_begin=s_last + 37, tokens=np.arange(s_last + 37, w.seqlen), workspace=ws)


def test_rag_mixed_passage_lengths_from_inside_a_passage():
    """Passages of 128, 512, 384 and 896 tokens and a ragged 300-token final
    block, re-rotation offsets unrelated to the segment starts, theta 1e4;
    every row from inside the second passage (not on a tile boundary) to the
    end, and none before it written."""
    S = 128 + 512 + 384 + 896 + 300
    w = inputs.random_qkv(S, 8, 2, 128, "bf16", seed=35, block=128, name="rag_mixed")
    w.seg_start = np.array([0, 128, 640, 1024, 1920, S], np.int32)
    w.k_rerotate = np.array([0, 50, 700, 12, 0], np.int32)
    w.rope_theta = 1e4
    _run(w, q_row_begin=128 + 77)
