"""Shared helpers for the GPU parity tests: run the HIP path through the
binding, run the oracle on the same inputs, and compare under the parity
rules (selected sets exact outside the threshold band; attention within the
dtype's tolerance)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import block_sparse_long_rbs_amd as rbs
from block_sparse_long_rbs_amd import device
from oracle import rbs_oracle as orc

# Attention tolerances: bf16 inputs (max-abs, mean-abs) and fp32 inputs.
TOL_BF16_MAX, TOL_BF16_MEAN = 2e-2, 1e-2
TOL_F32 = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_stats(w, t):
    return [x.cpu().numpy().astype(np.float64) for x in rbs.rbs_block_stats(t["q"], t["k"], w.block)]


def gpu_select(w, t, stats_dev):
    cen, rad, qrep, qn = stats_dev
    rp, ci, beta = rbs.rbs_select(cen, rad, qrep, qn, w.keep_ratio_centroid, w.keep_ratio_rescue,
                                  sink=w.sink, beta=t.get("beta"), want_beta=True)
    rp_h = rp.cpu().numpy().astype(np.int64)
    ci_h = ci.cpu().numpy()[:rp_h[-1]]
    return rp, ci, rp_h, ci_h, beta.cpu().numpy()


def oracle_selection(w):
    c, r, qr, qn = orc.block_stats(w.q, w.k, w.n_kv_heads, w.block)
    beta = w.beta.astype(np.float64) if w.beta is not None else orc.derive_beta(r)
    sel = orc.select(c, r, qr, qn, beta, w.keep_ratio_centroid, w.keep_ratio_rescue, w.sink)
    return (c, r, qr, qn), sel


def compare_stats(gpu, ora, rel=1e-5):
    names = ("centroid", "radius", "q_rep", "q_rep_norm")
    for name, g, o in zip(names, gpu, ora):
        scale = np.abs(o).max() if o.size else 1.0
        err = np.abs(g - o).max() if o.size else 0.0
        assert err <= rel * max(scale, 1e-30), f"{name}: max err {err} vs scale {scale}"


# At most this share of rows may differ from the oracle at all (every
# difference must also lie in a near-tie band): float32 scoring should flip
# a near tie only now and then.
MAX_DIFF_ROW_FRAC = 0.01


def compare_selection(sel, rp_h, ci_h, Hkv, nb, sink, max_diff_frac=MAX_DIFF_ROW_FRAC):
    """Sets bit-exact except blocks in a near-tie band of the oracle (a band
    that straddles a branch's cut, see oracle.near_tie_band); the rows that
    differ at all are capped at max_diff_frac of the rows. Returns (rows that
    differ, rows checked, exempt blocks)."""
    differing = 0
    n_exempt = sum(len(e) for e in sel.exempt)
    assert len(rp_h) == Hkv * nb + 1 and rp_h[0] == 0, "row_ptr has the wrong length or start"
    for r in range(Hkv * nb):
        i = r % nb
        got = ci_h[rp_h[r]:rp_h[r + 1]].tolist()
        assert got == sorted(set(got)), f"row {r} not strictly ascending: {got}"
        assert got and got[-1] == i, f"row {r} misses its diagonal block"
        if sink:
            assert got[0] == 0, f"row {r} misses the sink"
        want = set(sel.col_idx[sel.row_ptr[r]:sel.row_ptr[r + 1]].tolist())
        diff = set(got) ^ want
        if diff:
            differing += 1
            assert diff <= sel.exempt[r], (f"row {r}: differs at {sorted(diff)}, "
                                           f"exempt {sorted(sel.exempt[r])}")
    cap = max(1, int(max_diff_frac * Hkv * nb))
    assert differing <= cap, f"{differing} of {Hkv * nb} rows differ (cap {cap})"
    return differing, Hkv * nb, n_exempt


def attn_errors(gpu_out, ora_out, rows_tokens, heads=None):
    g = gpu_out[rows_tokens]
    o = ora_out[rows_tokens]
    if heads is not None:
        g, o = g[:, heads], o[:, heads]
    d = np.abs(g.astype(np.float64) - o)
    return float(d.max()), float(d.mean())


def check_attn(w, gpu_out, ora_out, tokens):
    mx, mean = attn_errors(gpu_out, ora_out, tokens)
    if w.dtype == "f32":
        assert mx <= TOL_F32, f"fp32 attention max-abs {mx}"
    else:
        assert mx <= TOL_BF16_MAX and mean <= TOL_BF16_MEAN, f"bf16 attention max {mx} mean {mean}"
    return mx, mean


def csr_to_device(row_ptr, col_idx, dev="cuda"):
    return (torch.from_numpy(np.asarray(row_ptr, np.int32)).to(dev),
            torch.from_numpy(np.asarray(col_idx, np.int32)).to(dev))


def long_rows_csr(n_kv_heads, nb, long_row, n_entries, seed=0):
    """A CSR whose row `long_row` (of every KV head) lists n_entries entries:
    every visible block 0..long_row in a shuffled order, with out-of-range
    entries (-1, long_row + 1, nb + 7) spliced in around list positions 256 and
    512, where the attention kernels reload their staged block list; every
    other row holds only its diagonal block. Returns (row_ptr, col_idx) as
    listed and the clean (row_ptr, col_idx) the oracle reads (the same rows
    without the out-of-range entries, which attention skips)."""
    rng = np.random.default_rng(seed)
    bad = [-1, long_row + 1, nb + 7]
    rows, clean = [], []
    for _ in range(n_kv_heads):
        for i in range(nb):
            if i != long_row:
                rows.append([i])
                clean.append([i])
                continue
            good = rng.permutation(long_row + 1).tolist()
            n_bad = n_entries - len(good)
            assert n_bad >= 6, "too few entries for the out-of-range splices"
            lst = list(good)
            for pos in (254, 255, 256, 257, 511, 512):
                lst.insert(min(pos, len(lst)), bad[pos % 3])
            while len(lst) < n_entries:
                lst.insert(int(rng.integers(len(lst) + 1)), bad[int(rng.integers(3))])
            rows.append(lst)
            clean.append(sorted(good))

    def pack(rr):
        rp = np.zeros(len(rr) + 1, np.int64)
        np.cumsum([len(x) for x in rr], out=rp[1:])
        return rp, np.concatenate([np.asarray(x, np.int32) for x in rr])
    return pack(rows), pack(clean)


def row_tokens(rows, block, S):
    toks = []
    for (_, i) in rows:
        toks.extend(range(i * block, min(S, (i + 1) * block)))
    return np.unique(np.asarray(toks, np.int64))


def to_host(x: torch.Tensor) -> np.ndarray:
    return x.float().cpu().numpy().astype(np.float64)


def _slab_errors(gpu_out, ora_out, rows, w):
    G = w.group
    errs = []
    for g, i in rows:
        t0, t1 = i * w.block, min(w.seqlen, (i + 1) * w.block)
        a = gpu_out[t0:t1, g * G:(g + 1) * G]
        b = ora_out[t0:t1, g * G:(g + 1) * G]
        errs.append(np.abs(a - b).reshape(-1))
    e = np.concatenate(errs)
    return float(e.max()), float(e.mean())


def _assert_attn(w, mx, mean, what):
    say(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e}")
    if w.dtype == "f32":
        assert mx <= TOL_F32, f"{what}: fp32 max-abs {mx}"
    else:
        assert mx <= TOL_BF16_MAX and mean <= TOL_BF16_MEAN, f"{what}: max {mx} mean {mean}"


def stratified_rows(n_heads, nb, row_ptr, n, seed=0):
    """About n (head, query block) rows for a sampled check: for every head
    its first and last query block and its two longest rows (by the given
    CSR), then random other rows; sorted."""
    lengths = np.diff(np.asarray(row_ptr, np.int64)).reshape(n_heads, nb)
    pick = set()
    for h in range(n_heads):
        pick |= {(h, 0), (h, nb - 1)}
        for i in np.argsort(-lengths[h], kind="stable")[:2]:
            pick.add((h, int(i)))
    rng = np.random.default_rng(seed)
    total = n_heads * nb
    while len(pick) < min(n, total):
        r = int(rng.integers(total))
        pick.add((r // nb, r % nb))
    return sorted(pick)


def pipeline_case(w, sample_rows=None, seed=0):
    """Full parity for one workload; sample_rows bounds the attention oracle."""
    say(f"[case] {w.name} S={w.seqlen} Hq={w.n_q_heads} Hkv={w.n_kv_heads} D={w.head_dim} "
          f"B={w.block} dtype={w.dtype}")
    t = device.upload(w)
    stats_dev = rbs.rbs_block_stats(t["q"], t["k"], w.block)
    torch.cuda.synchronize()
    gstats = [to_host(x) for x in stats_dev]
    ostats, sel = oracle_selection(w)
    compare_stats(gstats, ostats)
    rp, ci, rp_h, ci_h, beta_g = gpu_select(w, t, stats_dev)
    if w.beta is None:
        np.testing.assert_allclose(beta_g, sel.beta, atol=1e-5)
    nb = w.n_blocks
    diff, total, n_ex = compare_selection(sel, rp_h, ci_h, w.n_kv_heads, nb, w.sink)
    say(f"  selection: {diff}/{total} rows differ, all inside near-tie bands "
        f"({n_ex} blocks in such bands)")
    rows = [(g, i) for g in range(w.n_kv_heads) for i in range(nb)]
    if sample_rows is not None and len(rows) > sample_rows:
        rows = stratified_rows(w.n_kv_heads, nb, sel.row_ptr, sample_rows, seed)
    # attention on the oracle's CSR
    rp_o, ci_o = csr_to_device(sel.row_ptr, sel.col_idx)
    out_g, lse_g = rbs.blocksparse_attn_fwd(t["q"], t["k"], t["v"], w.block, rp_o, ci_o,
                                            want_lse=True)
    out_o, lse_o = orc.blocksparse_attention(w.q, w.k, w.v, w.block, sel.row_ptr, sel.col_idx,
                                             rows=rows)
    out_gh = to_host(out_g)
    mx, mean = _slab_errors(out_gh, out_o, rows, w)
    _assert_attn(w, mx, mean, "attention on oracle CSR")
    lse_gh = lse_g.cpu().numpy()
    G = w.group
    for g, i in rows:
        t0, t1 = i * w.block, min(w.seqlen, (i + 1) * w.block)
        d = np.abs(lse_gh[g * G:(g + 1) * G, t0:t1] - lse_o[g * G:(g + 1) * G, t0:t1]).max()
        assert d <= (1e-5 if w.dtype == "f32" else 2e-2), f"lse row {(g, i)} err {d}"
    # end to end on rows whose GPU set equals the oracle's
    out_e, _ = rbs.blocksparse_attn_fwd(t["q"], t["k"], t["v"], w.block, rp, ci)
    out_eh = to_host(out_e)
    same = [(g, i) for (g, i) in rows
            if ci_h[rp_h[g * nb + i]:rp_h[g * nb + i + 1]].tolist() == sel.row(g, i).tolist()]
    if same:
        mx, mean = _slab_errors(out_eh, out_o, same, w)
        _assert_attn(w, mx, mean, f"end to end on {len(same)}/{len(rows)} rows")
    return dict(t=t, sel=sel, rp=rp, ci=ci, out=out_g)


