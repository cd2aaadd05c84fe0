"""Plain float64 CPU oracle for RBS block-sparse prefill attention and for
Block-attention's static RAG mask with RoPE position re-encoding.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. It shares no code with the HIP
library and imports nothing from the product package.

Sources (web pages, cited by title and section):

[RBS]    "RBS-Attention: How a Geometric Rescue Branch Fixes Sparse Prefill for
         Long-Context LLMs" (techfordev.netlify.app/articles/4709260).
[RBS-ID] "RBS-Attention Bikin Prefill LLM Gede 20x Lebih Cepat, Tanpa Training
         Lagi?" (news.captivela.com), section "Dual-Branch Selection: Centroid
         Base + Rescue Branch".
[BA]     "Block-Attention for Efficient Prefilling" (paperlayer.ai/abs/2409.15355v5).

Where the pages leave a step open the oracle takes one stated reading; each
is marked READING in the function that takes it. Parity unpinned (the pages
fix nothing, so oracle and GPU can only agree with each other): the value of
the derived rescue coefficient beta (``derive_beta``), the pooling of the
representative query over heads and tokens (``block_stats``; per query head
in ``query_rep_per_head``), the rounding of
the per-branch budget (``budget``), the tie-break (``top_n``) and the RoPE
pairing style (``rope_rotate``).

Everything is computed in float64 from the given (float32-held) inputs,
selection decisions included: scores are ranked as float64 numbers.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterable, Optional

import numpy as np

F64 = np.float64


def n_blocks(seqlen: int, block: int) -> int:
    """Number of key (and query) blocks; the last one may be partial."""
    return -(-seqlen // block)


def _block_range(b: int, block: int, seqlen: int):
    return b * block, min(seqlen, (b + 1) * block)


# ---------------------------------------------------------------------------
# Block statistics
# ---------------------------------------------------------------------------

def block_stats(q: np.ndarray, k: np.ndarray, n_kv_heads: int, block: int):
    """Per (KV head g, key block b): centroid and radius; per (g, query block i):
    representative query and its Euclidean norm.

    [RBS] "The Standard Approach and Its Blind Spot": a key block is summarised
    by its centroid, the average of its key vectors; its radius is the largest
    distance from any key of the block to that centroid (Euclidean, matching the
    2-norm of q in the bound of "The Fix").

    READING (representative query): one vector per (KV head, query block), the
    mean over the group's query heads and the block's tokens; its norm is the
    ||q||_2 of the rescue score. (Parity unpinned.)

    q: [S, Hq, D], k: [S, Hkv, D]. Returns float64 arrays
    centroid [Hkv, nb, D], radius [Hkv, nb], q_rep [Hkv, nb, D], q_rep_norm [Hkv, nb].
    """
    S, Hq, D = q.shape
    assert k.shape == (S, n_kv_heads, D)
    G = Hq // n_kv_heads
    nb = n_blocks(S, block)
    centroid = np.zeros((n_kv_heads, nb, D), F64)
    radius = np.zeros((n_kv_heads, nb), F64)
    q_rep = np.zeros((n_kv_heads, nb, D), F64)
    for b in range(nb):
        t0, t1 = _block_range(b, block, S)
        kb = k[t0:t1].astype(F64)                       # [L, Hkv, D]
        cb = kb.mean(axis=0)                            # [Hkv, D]
        dist = np.sqrt(((kb - cb[None]) ** 2).sum(axis=-1))   # [L, Hkv]
        centroid[:, b] = cb
        radius[:, b] = dist.max(axis=0)
        qb = q[t0:t1].astype(F64).reshape(t1 - t0, n_kv_heads, G, D)
        q_rep[:, b] = qb.mean(axis=(0, 2))
    q_rep_norm = np.sqrt((q_rep ** 2).sum(axis=-1))
    return centroid, radius, q_rep, q_rep_norm


def query_rep_per_head(q: np.ndarray, block: int):
    """Per (query head h, query block i): the mean of head h's queries over the
    block's tokens, and its Euclidean norm.

    READING (per-query-head selection): the other reading of the "q" in [RBS]
    "The Fix" -- one representative per query head instead of one per GQA
    group; each query head then ranks its KV head's key blocks on its own.
    (Parity unpinned, like the group reading.)

    q: [S, Hq, D]. Returns q_rep_head [Hq, nb, D], q_rep_head_norm [Hq, nb].
    """
    S, Hq, D = q.shape
    nb = n_blocks(S, block)
    rep = np.zeros((Hq, nb, D), F64)
    for b in range(nb):
        t0, t1 = _block_range(b, block, S)
        rep[:, b] = q[t0:t1].astype(F64).mean(axis=0)
    return rep, np.sqrt((rep ** 2).sum(axis=-1))


# ---------------------------------------------------------------------------
# Rescue coefficient
# ---------------------------------------------------------------------------

def derive_beta(radius: np.ndarray) -> np.ndarray:
    """Radius-adaptive rescue coefficient in [0, 1], per KV head.

    [RBS] "The Fix: A Radius-Adaptive Rescue Branch" gives beta_b as clamped to
    [0, 1] and derived from the distribution of block radii; [RBS-ID] adds that
    it uses the largest key-block radius and its per-prompt, per-layer, per-head
    distribution. No formula is printed.

    READING: for each KV head of one call, with mu the mean and M the maximum
    radius over all its blocks, beta_b = clamp((r_b - mu) / (M - mu), 0, 1);
    every beta is 0 when M - mu <= 1e-6 * M. The largest-radius block gets the
    full Cauchy-Schwarz margin, blocks at or below the mean get none.
    (Parity of the value unpinned; its range, monotonicity and end points are
    pinned as properties.)
    """
    r = radius.astype(F64)
    mu = r.mean(axis=1, keepdims=True)
    mx = r.max(axis=1, keepdims=True)
    spread = mx - mu
    ok = spread > 1e-6 * mx
    beta = np.clip((r - mu) / np.where(ok, spread, 1.0), 0.0, 1.0)
    return np.where(ok, beta, 0.0)


# ---------------------------------------------------------------------------
# Selection
# ---------------------------------------------------------------------------

def budget(n_visible: int, keep_ratio: float) -> int:
    """Blocks one branch keeps for a query block that sees n_visible key blocks.

    READING: the keep-ratio is a fraction of the causally visible blocks,
    rounded up, at least one; 1e-6 is subtracted before the ceiling so that a
    product that is an integer in decimal (0.1 * 10) is not pushed up by binary
    rounding. Computed in float64. (Parity unpinned.)
    """
    return min(n_visible, max(1, math.ceil(float(keep_ratio) * n_visible - 1e-6)))


def rank_order(scores: np.ndarray) -> np.ndarray:
    """Entry indices from best to worst: larger float64 score first, equal
    scores by lower index (READING: the pages give no tie rule)."""
    idx = np.arange(scores.shape[0])
    return np.lexsort((idx, -np.asarray(scores, F64)))


def top_n(scores: np.ndarray, n: int) -> np.ndarray:
    """Indices of the n best entries (see :func:`rank_order`), ascending."""
    return np.sort(rank_order(scores)[:n])


def near_tie_band(scores: np.ndarray, n: int, floor: float, band_rel: float = 1e-4) -> set:
    """Entries whose membership in one branch's top-n is decided by rounding.

    tau is the n-th best float64 score and the band is every entry within
    band_rel * max(|tau|, floor) of it (READING: the relative 1e-4 of the
    parity rule, with floor the natural size of the branch's score terms so
    that a threshold near zero still has a band). A computation carried out in
    lower precision can exchange a kept entry for a dropped one only when both
    lie in the band, so the band counts only when it holds entries on both
    sides of the cut (at least one kept and one dropped); otherwise it is
    empty and the n-th entry itself is decided exactly.
    """
    s = np.asarray(scores, F64)
    order = rank_order(s)
    tau = s[order[n - 1]]
    near = np.abs(s - tau) <= band_rel * max(abs(tau), floor)
    kept = np.zeros(s.shape[0], bool)
    kept[order[:n]] = True
    if not (near & ~kept).any():
        return set()
    return set(np.nonzero(near)[0].tolist())


@dataclasses.dataclass
class Selection:
    """CSR block lists for rows r = g * nb + i, plus per-row diagnostics."""
    row_ptr: np.ndarray          # [Hkv*nb + 1] int64
    col_idx: np.ndarray          # [nnz] int32, ascending within a row
    n_blocks: int
    # Per row: blocks whose float64 score lies inside the tolerance band of a
    # branch's threshold (either set membership is acceptable there).
    exempt: list
    beta: np.ndarray             # [Hkv, nb] float64 as used

    def row(self, g: int, i: int) -> np.ndarray:
        r = g * self.n_blocks + i
        return self.col_idx[self.row_ptr[r]:self.row_ptr[r + 1]]


def branch_scores(centroid, radius, q_rep, q_rep_norm, beta, g, i):
    """Both branch scores for query block i of KV head g over key blocks 0..i.

    [RBS] "The Fix": centroid branch q^T c_b; rescue branch
    q^T c_b + ||q||_2 * r_b * beta_b. No softmax scale is applied: a common
    positive factor changes neither ranking.
    """
    sc = centroid[g, :i + 1] @ q_rep[g, i]
    sr = sc + q_rep_norm[g, i] * radius[g, :i + 1] * beta[g, :i + 1]
    return sc, sr


def select(centroid, radius, q_rep, q_rep_norm, beta, keep_ratio_centroid: float,
           keep_ratio_rescue: float, sink: bool, band_rel: float = 1e-4) -> Selection:
    """Dual-branch key-block selection, emitted as CSR block lists.

    [RBS] "The Fix": the two branches are thresholded independently and their
    masks combined; [RBS-ID] "Dual-Branch Selection" says the same. Here each
    branch keeps its top budget(i+1, keep_ratio) blocks among 0..i (causal),
    the two sets are OR-ed, the diagonal block i is always added and block 0
    too when ``sink`` is set (READING: forced blocks do not use a branch's
    budget). Rows are sorted ascending.

    beta: [Hkv, nb] array (given or from :func:`derive_beta`).

    ``exempt`` marks, per row, the non-forced blocks of each branch's
    :func:`near_tie_band`, with floor ||q|| * max_j ||c_j|| for the centroid
    branch and ||q|| * max_j (||c_j|| + r_j * beta_j) for the rescue branch:
    the only blocks whose membership a lower-precision ranking may decide
    differently. A branch whose budget-th block has no rival across the cut
    inside the band exempts nothing.
    """
    Hkv, nb, D = centroid.shape
    beta = np.asarray(beta, F64)
    cnorm = np.sqrt((centroid.astype(F64) ** 2).sum(-1))
    rows, exempt = [], []
    for g in range(Hkv):
        for i in range(nb):
            sc, sr = branch_scores(centroid, radius, q_rep, q_rep_norm, beta, g, i)
            nc = budget(i + 1, keep_ratio_centroid)
            nr = budget(i + 1, keep_ratio_rescue)
            keep = set(top_n(sc, nc).tolist())
            keep |= set(top_n(sr, nr).tolist())
            forced = {i} | ({0} if sink else set())
            keep |= forced
            rows.append(np.array(sorted(keep), dtype=np.int32))
            floor_c = q_rep_norm[g, i] * cnorm[g, :i + 1].max()
            floor_r = q_rep_norm[g, i] * (cnorm[g, :i + 1] +
                                          radius[g, :i + 1] * beta[g, :i + 1]).max()
            ex = near_tie_band(sc, nc, floor_c, band_rel) | near_tie_band(sr, nr, floor_r, band_rel)
            exempt.append(ex - forced)
    counts = np.array([len(r) for r in rows], dtype=np.int64)
    row_ptr = np.zeros(Hkv * nb + 1, np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    col_idx = np.concatenate(rows) if rows else np.zeros(0, np.int32)
    return Selection(row_ptr=row_ptr, col_idx=col_idx.astype(np.int32), n_blocks=nb,
                     exempt=exempt, beta=beta)


def select_per_head(centroid, radius, q_rep_head, q_rep_head_norm, beta,
                    keep_ratio_centroid: float, keep_ratio_rescue: float, sink: bool,
                    band_rel: float = 1e-4) -> Selection:
    """Per-query-head selection: row r = h * nb + i holds query head h's blocks,
    ranked with h's own representative query against the centroids, radii and
    beta of its KV head g = h // G (contiguous groups), with the same branches,
    budgets, forced blocks and ties as :func:`select`. ``beta`` is per KV head
    [Hkv, nb]; the returned Selection keeps it that way."""
    Hkv = centroid.shape[0]
    Hq = q_rep_head.shape[0]
    G = Hq // Hkv
    per_head = lambda x: np.repeat(np.asarray(x, F64), G, axis=0)
    sel = select(per_head(centroid), per_head(radius), q_rep_head, q_rep_head_norm,
                 per_head(beta), keep_ratio_centroid, keep_ratio_rescue, sink, band_rel)
    sel.beta = np.asarray(beta, F64)
    return sel


def select_capacity(n_kv_heads: int, nb: int, keep_ratio_centroid: float,
                    keep_ratio_rescue: float, sink: bool) -> int:
    """Largest possible number of CSR entries: per row, both budgets, the
    diagonal and the sink, capped by the i+1 visible blocks."""
    per_g = sum(min(i + 1, budget(i + 1, keep_ratio_centroid) + budget(i + 1, keep_ratio_rescue)
                    + 1 + (1 if sink else 0)) for i in range(nb))
    return n_kv_heads * per_g


def dense_causal_selection(n_kv_heads: int, nb: int) -> tuple:
    """CSR with every causally visible block (keep-ratio 1)."""
    rows = [np.arange(i + 1, dtype=np.int32) for _ in range(n_kv_heads) for i in range(nb)]
    counts = np.array([len(r) for r in rows], np.int64)
    row_ptr = np.zeros(len(rows) + 1, np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    return row_ptr, np.concatenate(rows)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def softmax_attend(logits: np.ndarray, allowed: np.ndarray, v: np.ndarray):
    """Masked softmax attention, two passes (row max, then exponentials).

    logits [H, L, U] float64, allowed [L, U] or [H, L, U] bool, v [U, D].
    Returns out [H, L, D] and the natural-log sum-exp lse [H, L]; a row with no
    allowed key gives out 0 and lse -inf.
    """
    masked = np.where(allowed, logits, -np.inf)
    m = masked.max(axis=-1, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.where(allowed, np.exp(masked - m_safe), 0.0)
    s = e.sum(axis=-1, keepdims=True)
    out = (e @ v.astype(F64)) / np.where(s > 0, s, 1.0)
    lse = np.where(s[..., 0] > 0, m_safe[..., 0] + np.log(np.where(s[..., 0] > 0, s[..., 0], 1.0)),
                   -np.inf)
    return out, lse


def blocksparse_attention(q, k, v, block: int, row_ptr, col_idx, scale: Optional[float] = None,
                          rows: Optional[Iterable] = None):
    """Causal GQA attention restricted to the selected key blocks.

    [RBS] "The Fix" and [RBS-ID] "Dual-Branch Selection": the combined mask
    runs through a standard block-sparse attention. For query token t in block
    i of head h (KV head g = h // G), the allowed keys are the tokens u <= t of
    the blocks listed in row g * nb + i; o = sum_u softmax_u(q.k_u * scale) v_u.
    READING: scale defaults to 1/sqrt(D).

    rows: optional iterable of (g, i) to evaluate; other outputs stay NaN.
    Returns out [S, Hq, D] float64 and lse [Hq, S] float64.
    """
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    nb = n_blocks(S, block)
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    out = np.full((S, Hq, D), np.nan, F64)
    lse = np.full((Hq, S), np.nan, F64)
    if rows is None:
        rows = [(g, i) for g in range(Hkv) for i in range(nb)]
    for g, i in rows:
        r = g * nb + i
        blocks = np.asarray(col_idx[row_ptr[r]:row_ptr[r + 1]])
        keys = np.concatenate([np.arange(*_block_range(int(b), block, S)) for b in blocks]) \
            if len(blocks) else np.zeros(0, np.int64)
        t0, t1 = _block_range(i, block, S)
        tok = np.arange(t0, t1)
        qi = q[t0:t1, g * G:(g + 1) * G].astype(F64).transpose(1, 0, 2)   # [G, L, D]
        kk = k[keys, g].astype(F64)                                         # [U, D]
        logits = (qi @ kk.T) * scale                                        # [G, L, U]
        allowed = keys[None, :] <= tok[:, None]
        o, l = softmax_attend(logits, allowed, v[keys, g])
        out[t0:t1, g * G:(g + 1) * G] = o.transpose(1, 0, 2)
        lse[g * G:(g + 1) * G, t0:t1] = l
    return out, lse


def e4m3_decode(b) -> np.ndarray:
    """Real values of fp8 E4M3 bytes, float64, exact.

    Format definition: the OCP 8-bit floating point specification's E4M3
    (not from the pages; [RBS] "Integration with vLLM and Benchmark Results"
    only says the evaluated model is an FP8 checkpoint). Bit 7 is the sign,
    bits 6..3 the exponent e with bias 7, bits 2..0 the mantissa m: e > 0
    gives (1 + m/8) * 2^(e - 7), e = 0 the subnormal (m/8) * 2^-6; the two
    codes with every exponent and mantissa bit set (0x7F, 0xFF) are NaN and
    there is no infinity, so the largest finite value is 448 (0x7E).
    """
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(F64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(F64) - 7.0))
    return np.where((b & 0x7F) == 0x7F, np.nan, sign * mag)


def blocksparse_attention_fp8(q8, k8, v8, q_descale: float, k_descale: float, v_descale: float,
                              block: int, row_ptr, col_idx, scale: Optional[float] = None,
                              rows: Optional[Iterable] = None):
    """blocksparse_attention on fp8 inputs: the real inputs are the decoded
    E4M3 bytes times one dequantisation factor per tensor (q_descale * q,
    k_descale * k, v_descale * v); everything after that is
    blocksparse_attention's definition, in float64.

    q8, k8, v8: uint8 arrays of E4M3 bytes, [S, Hq, D] and [S, Hkv, D].
    """
    lut = e4m3_decode(np.arange(256))   # every code once; indexing applies it elementwise
    q = lut[np.asarray(q8, np.uint8)]
    q *= float(q_descale)
    k = lut[np.asarray(k8, np.uint8)] * float(k_descale)
    v = lut[np.asarray(v8, np.uint8)] * float(v_descale)
    return blocksparse_attention(q, k, v, block, row_ptr, col_idx, scale, rows)


def block_attention_mass(q, k, block: int, g: int, i: int, scale: Optional[float] = None):
    """Dense causal attention mass per key block for one (KV head g, query
    block i) row: for every query token t of block i and query head h of
    group g, p_u = softmax_u(scale * q[t][h] . k[u][g]) over the keys u <= t;
    the mass of key block j is the sum of p_u over its tokens, averaged over
    the row's tokens and heads. Returns float64 [i + 1] (sums to 1).

    [RBS] "The Standard Approach and Its Blind Spot": a block's importance is
    the attention it actually receives; the selectors only estimate it.
    READING: scale defaults to 1/sqrt(D).
    """
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    t0, t1 = _block_range(i, block, S)
    qi = q[t0:t1, g * G:(g + 1) * G].astype(F64).transpose(1, 0, 2)   # [G, L, D]
    kk = k[:t1, g].astype(F64)                                          # [t1, D]
    logits = (qi @ kk.T) * scale                                        # [G, L, t1]
    tok = np.arange(t0, t1)
    logits[:, np.arange(t1)[None, :] > tok[:, None]] = -np.inf
    logits -= logits.max(axis=-1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=-1, keepdims=True)
    per_key = p.mean(axis=(0, 1))                                       # [t1]
    edges = np.arange(0, t1, block)
    return np.add.reduceat(per_key, edges)


def blocksparse_attention_per_head(q, k, v, block: int, row_ptr, col_idx,
                                   scale: Optional[float] = None, rows: Optional[Iterable] = None):
    """Causal GQA attention over per-query-head block lists: query token t in
    block i of head h sees the tokens u <= t of the blocks in row h * nb + i
    (keys and values of KV head h // G). Same softmax as
    :func:`blocksparse_attention`.

    rows: optional iterable of (h, i); other outputs stay NaN.
    Returns out [S, Hq, D] and lse [Hq, S], float64.
    """
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    nb = n_blocks(S, block)
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    out = np.full((S, Hq, D), np.nan, F64)
    lse = np.full((Hq, S), np.nan, F64)
    if rows is None:
        rows = [(h, i) for h in range(Hq) for i in range(nb)]
    for h, i in rows:
        g = h // G
        r = h * nb + i
        blocks = np.asarray(col_idx[row_ptr[r]:row_ptr[r + 1]])
        keys = np.concatenate([np.arange(*_block_range(int(b), block, S)) for b in blocks]) \
            if len(blocks) else np.zeros(0, np.int64)
        t0, t1 = _block_range(i, block, S)
        tok = np.arange(t0, t1)
        logits = (q[t0:t1, h].astype(F64) @ k[keys, g].astype(F64).T) * scale   # [L, U]
        allowed = keys[None, :] <= tok[:, None]
        o, l = softmax_attend(logits[None], allowed, v[keys, g])
        out[t0:t1, h] = o[0]
        lse[h, t0:t1] = l[0]
    return out, lse


def masked_attention(q, k, v, mask, scale: Optional[float] = None):
    """Literal token-level attention: mask [Hkv, S, Sk] (or [S, Sk]) boolean,
    True = key allowed. Used as the brute-force form on tiny inputs."""
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    mask = np.asarray(mask, bool)
    if mask.ndim == 2:
        mask = np.broadcast_to(mask, (Hkv,) + mask.shape)
    out = np.zeros((S, Hq, D), F64)
    lse = np.zeros((Hq, S), F64)
    for h in range(Hq):
        g = h // G
        logits = (q[:, h].astype(F64) @ k[:, g].astype(F64).T) * scale    # [S, Sk]
        o, l = softmax_attend(logits[None], mask[g][None], v[:, g])
        out[:, h] = o[0]
        lse[h] = l[0]
    return out, lse


def csr_token_mask(row_ptr, col_idx, n_kv_heads: int, seqlen: int, block: int) -> np.ndarray:
    """Token-level mask [Hkv, S, S] of a CSR block selection with the causal
    rule u <= t."""
    nb = n_blocks(seqlen, block)
    tb = np.arange(seqlen) // block
    mask = np.zeros((n_kv_heads, seqlen, seqlen), bool)
    for g in range(n_kv_heads):
        for i in range(nb):
            r = g * nb + i
            sel = np.zeros(nb, bool)
            sel[np.asarray(col_idx[row_ptr[r]:row_ptr[r + 1]])] = True
            t0, t1 = _block_range(i, block, seqlen)
            mask[g, t0:t1] = sel[tb][None, :]
    return mask & np.tril(np.ones((seqlen, seqlen), bool))[None]


# ---------------------------------------------------------------------------
# Block-attention: RoPE re-encoding and the RAG mask
# ---------------------------------------------------------------------------

def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """omega_i = theta^(-2i/D), i < D/2, float64."""
    return float(theta) ** (-2.0 * np.arange(head_dim // 2, dtype=F64) / head_dim)


def rope_rotate(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotary position encoding of rows x [S, H, D] at integer positions [S].

    READING (the pages name RoPE but not its pairing): rotate-half pairs
    (x_i, x_{i+D/2}) turned by angle pos * omega_i; angles formed in float64.
    """
    S, H, D = x.shape
    ang = np.asarray(positions, F64)[:, None] * rope_inv_freq(D, theta)[None, :]   # [S, D/2]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x = x.astype(F64)
    x1, x2 = x[..., :D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def segment_of(seg_start: np.ndarray, seqlen: int) -> np.ndarray:
    """Segment index of every token."""
    return np.searchsorted(np.asarray(seg_start), np.arange(seqlen), side="right") - 1


def reencode_keys(k_cached, seg_start, k_rerotate, theta):
    """[BA] section 2.3 "Position Re-encoding": a cached block's keys, encoded
    from position 0, are rotated on to their new prompt position. Here every
    key of segment p is rotated by k_rerotate[p] positions."""
    seg = segment_of(seg_start, k_cached.shape[0])
    return rope_rotate(k_cached, np.asarray(k_rerotate)[seg], theta)


def block_mask_attention(q, k_cached, v, seg_start, k_rerotate, theta: float,
                         q_row_begin: int = 0, scale: Optional[float] = None,
                         rows: Optional[Iterable] = None):
    """Block-attention prefill with re-encoded cached keys.

    [BA] section 1 and 2.1 "Main Idea": blocks compute their key/value states
    independently and the final block attends to all preceding blocks; section
    2.4 "Block Fine-tune": a non-final block attends only within itself; section
    2.5 "Inference": cached blocks are re-encoded, then the final block is
    computed. So a query t of non-final segment p sees keys [s_p, t], a query of
    the final segment sees [0, t], after every cached key has been rotated to its
    position (``reencode_keys``). READING: Q is given at absolute positions;
    rows before q_row_begin are not computed; scale defaults to 1/sqrt(D).

    rows: optional iterable of token indices to evaluate (others NaN).
    Returns out [S, Hq, D] and lse [Hq, S] (float64).
    """
    S, Hq, D = q.shape
    Hkv = k_cached.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    seg_start = np.asarray(seg_start)
    n_seg = len(seg_start) - 1
    k_abs = reencode_keys(k_cached, seg_start, k_rerotate, theta)
    seg = segment_of(seg_start, S)
    out = np.full((S, Hq, D), np.nan, F64)
    lse = np.full((Hq, S), np.nan, F64)
    tok_all = np.arange(S)
    if rows is None:
        rows = tok_all[q_row_begin:]
    rows = np.asarray(sorted(set(int(t) for t in rows if t >= q_row_begin)), np.int64)
    for p in range(n_seg):
        tok = rows[seg[rows] == p]
        if tok.size == 0:
            continue
        lo = 0 if p == n_seg - 1 else int(seg_start[p])
        hi = int(tok.max()) + 1
        keys = np.arange(lo, hi)
        allowed = keys[None, :] <= tok[:, None]
        for g in range(Hkv):
            qi = q[tok, g * G:(g + 1) * G].astype(F64).transpose(1, 0, 2)
            logits = (qi @ k_abs[lo:hi, g].T) * scale
            o, l = softmax_attend(logits, allowed, v[lo:hi, g])
            out[tok, g * G:(g + 1) * G] = o.transpose(1, 0, 2)
            lse[g * G:(g + 1) * G, tok] = l
    return out, lse


def block_mask_token_mask(seg_start, seqlen: int) -> np.ndarray:
    """Literal [S, S] Block-attention mask (True = allowed)."""
    seg_start = np.asarray(seg_start)
    n_seg = len(seg_start) - 1
    seg = segment_of(seg_start, seqlen)
    t = np.arange(seqlen)
    lo = np.where(seg == n_seg - 1, 0, seg_start[seg])
    return (t[None, :] >= lo[:, None]) & (t[None, :] <= t[:, None])


# ---------------------------------------------------------------------------
# Work counts
# ---------------------------------------------------------------------------

def attention_pairs(row_ptr, col_idx, seqlen: int, block: int, n_kv_heads: int, group: int) -> int:
    """Number of (query, key) pairs the selection admits, summed over query
    heads (each pair costs 4*D flops: q.k and p*v)."""
    nb = n_blocks(seqlen, block)
    total = 0
    for g in range(n_kv_heads):
        for i in range(nb):
            r = g * nb + i
            t0, t1 = _block_range(i, block, seqlen)
            for b in col_idx[row_ptr[r]:row_ptr[r + 1]]:
                u0, u1 = _block_range(int(b), block, seqlen)
                if b < i:
                    total += (t1 - t0) * (u1 - u0)
                else:  # diagonal: pairs u <= t
                    L = t1 - t0
                    total += L * (L + 1) // 2
    return total * group
