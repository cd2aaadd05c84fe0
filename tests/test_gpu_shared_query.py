"""GPU parity of shared-query execution (blocksparse_attn_fwd_shared_query:
neighbouring query blocks of a head processed together over the union of
their block lists, the QUILT page's idea) with the float64 oracle, whose
definition it must keep, and with blocksparse_attn_fwd, whose output and lse
it must reproduce bit for bit on the same lists (same per-tile arithmetic in
the same order)."""
import numpy as np
import pytest
import torch

import block_sparse_long_rbs_amd as rbs
from block_sparse_long_rbs_amd import device, inputs
from oracle import rbs_oracle as orc

import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _both(t, block, rp, ci):
    o1, l1 = rbs.blocksparse_attn_fwd(t["q"], t["k"], t["v"], block, rp, ci, want_lse=True)
    o2, l2 = rbs.blocksparse_attn_fwd_shared_query(t["q"], t["k"], t["v"], block, rp, ci,
                                                   want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o2, o1), "output differs from blocksparse_attn_fwd"
    assert torch.equal(l2, l1), "lse differs from blocksparse_attn_fwd"
    return o2, l2


def _oracle_rows(w, rows, rp, ci, out):
    o, _ = orc.blocksparse_attention(w.q, w.k, w.v, w.block, rp, ci, rows=rows)
    mx, mean = H._slab_errors(H.to_host(out), o, rows, w)
    H._assert_attn(w, mx, mean, f"shared-query on {len(rows)} rows")


@pytest.mark.parametrize("S", [1400, 1536])
def test_shared_query_small_all_rows(S):
    """11 query blocks (the last pair holds one) and 12 (every pair full), 8/2
    heads, the oracle's selection: every row against the oracle."""
    w = inputs.mixture_small(S=S, Hq=8, Hkv=2, rho=0.25, sink=True, seed=13)
    H.say(f"[shared-query] S={S}")
    t = device.upload(w)
    _, sel = H.oracle_selection(w)
    rp, ci = H.csr_to_device(sel.row_ptr, sel.col_idx)
    out, _ = _both(t, w.block, rp, ci)
    rows = [(g, i) for g in range(w.n_kv_heads) for i in range(w.n_blocks)]
    _oracle_rows(w, rows, sel.row_ptr, sel.col_idx, out)


def test_shared_query_unsorted_rows_skipped_entries_and_empty_rows():
    """Rows listed backwards with entries outside 0..i mixed in (skipped), and
    rows with nothing usable (zero output, lse -inf): the union walk must
    still visit exactly each half's own entries."""
    S, B = 1024, 128
    w = inputs.random_qkv(S, 4, 1, 128, "bf16", seed=17, block=B, name="unsorted")
    t = device.upload(w)
    nb = S // B
    rng = np.random.default_rng(3)
    rows, clean = [], []
    for i in range(nb):
        if i in (2, 5):
            rows.append([i + 1, -4])            # nothing usable
            clean.append([])
            continue
        keep = sorted(set(rng.choice(i + 1, size=max(1, (i + 1) // 2), replace=False).tolist())
                      | {i})
        lst = keep[::-1] + [i + 3, -1]
        rng.shuffle(lst)
        rows.append(lst)
        clean.append(keep)

    def pack(rr):
        rp = np.zeros(len(rr) + 1, np.int64)
        np.cumsum([len(x) for x in rr], out=rp[1:])
        return rp, (np.concatenate([np.asarray(x, np.int32) for x in rr]) if rp[-1] else
                    np.zeros(1, np.int32))
    rp, ci = pack(rows)
    rpc, cic = pack(clean)
    a, b = H.csr_to_device(rp, ci)
    out, lse = _both(t, B, a, b)
    out_h, lse_h = H.to_host(out), lse.cpu().numpy()
    for i in (2, 5):
        assert np.all(out_h[i * B:(i + 1) * B] == 0) and np.all(np.isneginf(lse_h[:, i * B:(i + 1) * B]))
    live = [(0, i) for i in range(nb) if i not in (2, 5)]
    _oracle_rows(w, live, rpc, cic, out)


@pytest.mark.timeout(300)
def test_shared_query_long_rows():
    """Dense causal at 40,960 tokens: both halves' rows pass 256 entries (the
    staged lists reload in step); sampled rows and both sides of 256."""
    S, B = 40960, 128
    w = inputs.random_qkv(S, 2, 1, 128, "bf16", seed=55, block=B, name="dense_40k")
    t = device.upload(w)
    rp, ci = orc.dense_causal_selection(1, S // B)
    a, b = H.csr_to_device(rp, ci)
    out, _ = _both(t, B, a, b)
    _oracle_rows(w, [(0, i) for i in (0, 1, 254, 255, 256, 257, 318, 319)], rp, ci, out)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("make", [inputs.mixture_bf16_32k, inputs.mixture_bf16_128k],
                         ids=["32k", "128k"])
def test_shared_query_full_size(make):
    """The 32K (64/8 heads) and 128K (32/4 heads) mixtures with the GPU's own
    selection: bit-identical to blocksparse_attn_fwd everywhere, and 256
    stratified rows against the oracle on the oracle's selection."""
    w = make()
    H.say(f"[shared-query] {w.name}")
    t = device.upload(w)
    st = rbs.rbs_block_stats(t["q"], t["k"], w.block)
    rp, ci, _ = rbs.rbs_select(*st, w.keep_ratio_centroid, w.keep_ratio_rescue, sink=w.sink)
    _both(t, w.block, rp, ci)
    _, sel = H.oracle_selection(w)
    a, b = H.csr_to_device(sel.row_ptr, sel.col_idx)
    out, _ = _both(t, w.block, a, b)
    rows = H.stratified_rows(w.n_kv_heads, w.n_blocks, sel.row_ptr, 256, seed=5)
    _oracle_rows(w, rows, sel.row_ptr, sel.col_idx, out)
