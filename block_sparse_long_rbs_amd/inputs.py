"""Seeded synthetic workloads for RBS block-sparse prefill attention and
Block-attention.

This module only draws random arrays (NumPy PCG64, float32 standard normals)
and plants structure into them; it computes no step of the method. Both the
HIP library (through the binding) and the CPU oracle are fed from the arrays
it returns, so a mistake here cannot cancel between the two sides.

Every array is returned as float32 holding values exactly representable in
the workload's dtype (bf16 values are rounded to nearest-even on the host).
``to_bf16_bits`` gives the raw 16-bit patterns for upload.

Workload recipes (named by what they are):

* ``tiny_f32_1k``   1,024 tokens, 2 query heads / 1 KV head, head dim 64,
  block 64, fp32; four "needle" blocks whose single aligned key sits among
  keys pushed away from the needle direction (high radius, low centroid
  score). This is the mean-dilution case of the RBS-Attention explainer
  (section "The Standard Approach and Its Blind Spot").
* ``needle_bf16_8k``    8,192 tokens, 32/4 heads, dim 128, block 128, bf16;
  5% of key blocks per KV head hold one needle of norm 6 among N(0,1) keys.
* ``mixture_bf16_32k``  32,768 tokens, 64/8 heads; key blocks are 80% compact
  (spread 0.3 around a random block mean) and 20% high-radius (spread 1.5 plus
  one outlier aligned with a later query block).
* ``mixture_bf16_128k`` 131,072 tokens, 32/4 heads, the same key mixture.
* ``rag_bf16_31k``      Block-attention RAG layout: 20 passages of 1,536
  tokens plus a 512-token final block, 32/8 heads, dim 128, RoPE theta 5e5.

``fp8_inputs`` turns any workload into fp8 (E4M3) Q, K, V with one
dequantisation factor per tensor, the way an fp8 checkpoint stores them.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass
class Fp8Inputs:
    """fp8 copies of a workload's Q, K, V as an fp8 checkpoint stores them:
    OCP E4M3 bytes (uint8, same shapes) and one dequantisation factor per
    tensor (real value = descale * decoded byte)."""

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_descale: float
    k_descale: float
    v_descale: float


def to_e4m3(x: np.ndarray):
    """Per-tensor fp8 quantisation: scale so that the largest magnitude maps
    to 448 (E4M3's largest finite value), round to nearest even with torch's
    float8_e4m3fn conversion. Returns (uint8 bytes, float32 descale)."""
    import torch  # host-side conversion only

    x = np.ascontiguousarray(x, np.float32)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    descale = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    scaled = torch.from_numpy(x / descale)
    return scaled.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy(), float(descale)


def fp8_inputs(w: "Workload") -> Fp8Inputs:
    """E4M3 copies of w.q, w.k, w.v with per-tensor descales."""
    q, qd = to_e4m3(w.q)
    k, kd = to_e4m3(w.k)
    v, vd = to_e4m3(w.v)
    return Fp8Inputs(q, k, v, qd, kd, vd)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.
    Inputs must be finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Raw bfloat16 bit patterns (uint16) of float32 values already rounded
    with :func:`bf16_round`."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


@dataclasses.dataclass
class Workload:
    """One synthetic prefill-attention layer input (batch = one sequence).

    Layouts are token-major: q is [S, Hq, D], k and v are [S, Hkv, D].
    Query head h reads KV head h // (Hq // Hkv).
    """

    name: str
    dtype: str  # "bf16" or "f32"
    seqlen: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    keep_ratio_centroid: float = 1.0
    keep_ratio_rescue: float = 1.0
    sink: bool = False
    beta: Optional[np.ndarray] = None  # [Hkv, nb] fixed rescue coefficients, or None (derive)
    # Block-attention fields (RAG layout): segment starts (n_seg + 1 entries,
    # last == seqlen), re-rotation offsets per segment, RoPE base.
    seg_start: Optional[np.ndarray] = None
    k_rerotate: Optional[np.ndarray] = None
    rope_theta: float = 0.0
    seed: int = 0
    recipe: dict = dataclasses.field(default_factory=dict)

    @property
    def n_blocks(self) -> int:
        return -(-self.seqlen // self.block)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def _unit_mean_direction(qblock: np.ndarray) -> np.ndarray:
    """Unit vector along the sum of a slab of query rows [tokens, heads, D]
    (the direction a needle key is planted along)."""
    s = qblock.astype(np.float64).sum(axis=(0, 1))
    return s / np.linalg.norm(s)


def random_qkv(seqlen, n_q_heads, n_kv_heads, head_dim, dtype, seed, block=64,
               name="random", **kw) -> Workload:
    """Plain N(0,1) Q, K, V; drawn in the order Q, K, V."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _round(rng.standard_normal((seqlen, n_q_heads, head_dim), dtype=np.float32), dtype)
    k = _round(rng.standard_normal((seqlen, n_kv_heads, head_dim), dtype=np.float32), dtype)
    v = _round(rng.standard_normal((seqlen, n_kv_heads, head_dim), dtype=np.float32), dtype)
    return Workload(name=name, dtype=dtype, seqlen=seqlen, n_q_heads=n_q_heads,
                    n_kv_heads=n_kv_heads, head_dim=head_dim, block=block,
                    q=q, k=k, v=v, seed=seed, **kw)


def tiny_f32_1k(seed: int = 1, shift: float = 8.0, needle_norm: float = 4.0) -> Workload:
    """1,024 tokens, GQA 2:1, dim 64, block 64, fp32, keep-ratio 0.25 per
    branch, beta = 1 for every block, no sink.

    The last query block (15) is the chosen one; q_hat is the unit mean
    direction of its queries over both heads. Four distinct key blocks in
    0..14 each get one key set to needle_norm * q_hat at a random token; their
    other 63 keys become z - shift * q_hat.
    """
    S, Hq, Hkv, D, B = 1024, 2, 1, 64, 64
    nb = S // B
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((S, Hq, D), dtype=np.float32)
    k = rng.standard_normal((S, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((S, Hkv, D), dtype=np.float32)
    istar = nb - 1
    qhat = _unit_mean_direction(q[istar * B:(istar + 1) * B, 0:Hq])
    needle_blocks = np.sort(rng.choice(istar, size=4, replace=False))
    needle_tok = rng.integers(0, B, size=4)
    for b, t in zip(needle_blocks, needle_tok):
        sl = k[b * B:(b + 1) * B, 0]
        sl[:] = (sl.astype(np.float64) - shift * qhat).astype(np.float32)
        sl[t] = (needle_norm * qhat).astype(np.float32)
    beta = np.ones((Hkv, nb), dtype=np.float32)
    return Workload(name="tiny_f32_1k", dtype="f32", seqlen=S, n_q_heads=Hq, n_kv_heads=Hkv,
                    head_dim=D, block=B, q=q, k=k, v=v, keep_ratio_centroid=0.25,
                    keep_ratio_rescue=0.25, sink=False, beta=beta, seed=seed,
                    recipe=dict(query_block=int(istar), needle_blocks=needle_blocks.tolist(),
                                needle_tokens=needle_tok.tolist(), shift=shift,
                                needle_norm=needle_norm))


def needle_bf16_8k(seed: int = 2, needle_norm: float = 6.0, frac: float = 0.05) -> Workload:
    """8,192 tokens, 32/4 heads, dim 128, block 128, bf16, keep-ratio 0.1 per
    branch, beta derived from the radii, no sink.

    Per KV head, round(frac * nb) distinct key blocks b in 0..nb-2 get one key
    set to needle_norm * q_hat(g, i*), i* uniform in b+1..nb-1, where q_hat is
    the unit mean direction of block i*'s queries over the group's heads.
    """
    S, Hq, Hkv, D, B = 8192, 32, 4, 128, 128
    nb = S // B
    G = Hq // Hkv
    rng = np.random.Generator(np.random.PCG64(seed))
    q = bf16_round(rng.standard_normal((S, Hq, D), dtype=np.float32))
    k = rng.standard_normal((S, Hkv, D), dtype=np.float32)
    v = bf16_round(rng.standard_normal((S, Hkv, D), dtype=np.float32))
    n_needle = int(round(frac * nb))
    planted = []
    for g in range(Hkv):
        blocks = np.sort(rng.choice(nb - 1, size=n_needle, replace=False))
        istars = rng.integers(blocks + 1, nb)
        toks = rng.integers(0, B, size=n_needle)
        for b, i_s, t in zip(blocks, istars, toks):
            qhat = _unit_mean_direction(q[i_s * B:(i_s + 1) * B, g * G:(g + 1) * G])
            k[b * B + t, g] = (needle_norm * qhat).astype(np.float32)
            planted.append((g, int(b), int(i_s), int(t)))
    k = bf16_round(k)
    return Workload(name="needle_bf16_8k", dtype="bf16", seqlen=S, n_q_heads=Hq, n_kv_heads=Hkv,
                    head_dim=D, block=B, q=q, k=k, v=v, keep_ratio_centroid=0.1,
                    keep_ratio_rescue=0.1, sink=False, beta=None, seed=seed,
                    recipe=dict(needles=planted, needle_norm=needle_norm))


def _mixture(name, S, Hq, Hkv, D, B, rho, sink, seed, frac_high=0.2, sigma_c=0.3,
             sigma_h=1.5, outlier_scale=2.0) -> Workload:
    """Key mixture: per (KV head, block) a mean mu ~ N(0, I); round(frac_high*nb)
    blocks per head (random permutation) are high-radius with spread sigma_h
    and one outlier mu + a * q_hat(g, i*) (a = outlier_scale * sigma_h * sqrt(D),
    i* uniform in b..nb-1); the rest are compact with spread sigma_c.
    Q and V are N(0,1). Draw order: Q, K noise, V, then structure."""
    nb = -(-S // B)
    G = Hq // Hkv
    rng = np.random.Generator(np.random.PCG64(seed))
    q = bf16_round(rng.standard_normal((S, Hq, D), dtype=np.float32))
    z = rng.standard_normal((S, Hkv, D), dtype=np.float32)
    v = bf16_round(rng.standard_normal((S, Hkv, D), dtype=np.float32))
    mu = rng.standard_normal((Hkv, nb, D), dtype=np.float32)
    n_high = int(round(frac_high * nb))
    a = outlier_scale * sigma_h * np.sqrt(D)
    k = np.empty_like(z)
    outliers = []
    for g in range(Hkv):
        high = np.zeros(nb, dtype=bool)
        hb = rng.permutation(nb)[:n_high]
        high[hb] = True
        hb = np.sort(hb)
        toks = rng.integers(0, B, size=n_high)
        istars = rng.integers(hb, nb)
        sig = np.where(high, sigma_h, sigma_c).astype(np.float32)
        for b in range(nb):
            t0, t1 = b * B, min(S, (b + 1) * B)
            k[t0:t1, g] = mu[g, b][None, :] + sig[b] * z[t0:t1, g]
        for b, t, i_s in zip(hb, toks, istars):
            if b * B + t >= S:
                continue
            qhat = _unit_mean_direction(q[i_s * B:min(S, (i_s + 1) * B), g * G:(g + 1) * G])
            k[b * B + t, g] = (mu[g, b].astype(np.float64) + a * qhat).astype(np.float32)
            outliers.append((g, int(b), int(i_s), int(t)))
    k = bf16_round(k)
    return Workload(name=name, dtype="bf16", seqlen=S, n_q_heads=Hq, n_kv_heads=Hkv,
                    head_dim=D, block=B, q=q, k=k, v=v, keep_ratio_centroid=rho,
                    keep_ratio_rescue=rho, sink=sink, beta=None, seed=seed,
                    recipe=dict(frac_high=frac_high, sigma_compact=sigma_c, sigma_high=sigma_h,
                                outlier_norm=float(a), n_outliers=len(outliers)))


def mixture_bf16_32k(seed: int = 3) -> Workload:
    """32,768 tokens, 64/8 heads (dense-32B-like layer), dim 128, block 128,
    keep-ratio 0.05 per branch, beta derived, no sink."""
    return _mixture("mixture_bf16_32k", 32768, 64, 8, 128, 128, 0.05, False, seed)


def mixture_bf16_128k(seed: int = 4) -> Workload:
    """131,072 tokens, 32/4 heads (30B-A3B-like layer), dim 128, block 128,
    keep-ratio 0.03 per branch, beta derived, first key block kept as sink."""
    return _mixture("mixture_bf16_128k", 131072, 32, 4, 128, 128, 0.03, True, seed)


def mixture_small(S=1500, Hq=8, Hkv=2, D=128, B=128, rho=0.25, sink=True, seed=11) -> Workload:
    """A few-tile version of the key mixture with a ragged last block, for
    parity runs the oracle finishes in seconds."""
    return _mixture(f"mixture_bf16_{S}", S, Hq, Hkv, D, B, rho, sink, seed)


def rag_layout(n_passages=20, passage_len=1536, final_len=512, Hq=32, Hkv=8, D=128,
               theta=5e5, dtype="bf16", seed: int = 5, name="rag_bf16_31k") -> Workload:
    """Block-attention RAG layout: n_passages passages then one final block.

    Passage p occupies [s_p, s_p + passage_len). Its cached keys were encoded
    at local positions 0..passage_len-1 and must be re-rotated by s_p; the
    final block's keys are already at absolute positions (offset 0).

    RoPE applied to i.i.d. N(0, I) rows leaves them i.i.d. N(0, I), so the
    already-rotated Q and cached K are drawn directly as N(0,1); only the
    positions (segment starts and offsets) carry the layout.
    """
    S = n_passages * passage_len + final_len
    w = random_qkv(S, Hq, Hkv, D, dtype, seed, block=128, name=name)
    seg = np.array([p * passage_len for p in range(n_passages + 1)] + [S], dtype=np.int32)
    rer = np.array([p * passage_len for p in range(n_passages)] + [0], dtype=np.int32)
    w.seg_start, w.k_rerotate, w.rope_theta = seg, rer, float(theta)
    w.recipe = dict(n_passages=n_passages, passage_len=passage_len, final_len=final_len)
    return w


def rag_bf16_31k(seed: int = 5) -> Workload:
    return rag_layout(seed=seed)



def synthetic_block_stats(n_kv_heads: int, n_blocks: int, head_dim: int, seed: int = 0,
                          beta_given: bool = False):
    """Block statistics drawn directly (for testing the selection on its own at
    sizes the attention workloads do not reach, e.g. more than 1,024 blocks).

    Centroids are a per-block random mean scaled by a lognormal factor, the
    representative queries N(0, I), their norms the float32 Euclidean norms,
    radii positive with a heavy upper tail. Returns float32 arrays
    (centroid, radius, q_rep, q_rep_norm, beta or None)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (n_kv_heads, n_blocks, head_dim)
    scale = np.exp(0.3 * rng.standard_normal((n_kv_heads, n_blocks, 1))).astype(np.float32)
    cen = (rng.standard_normal(shape, dtype=np.float32) * scale).astype(np.float32)
    qrep = rng.standard_normal(shape, dtype=np.float32)
    qn = np.sqrt((qrep.astype(np.float64) ** 2).sum(-1)).astype(np.float32)
    rad = (1.0 + np.abs(rng.standard_normal((n_kv_heads, n_blocks), dtype=np.float32)) * 2.0
           + (rng.random((n_kv_heads, n_blocks)) < 0.1) * 6.0).astype(np.float32)
    beta = rng.random((n_kv_heads, n_blocks)).astype(np.float32) if beta_given else None
    return cen, rad, qrep, qn, beta

WORKLOADS = {
    "tiny_f32_1k": tiny_f32_1k,
    "needle_bf16_8k": needle_bf16_8k,
    "mixture_bf16_32k": mixture_bf16_32k,
    "mixture_bf16_128k": mixture_bf16_128k,
    "rag_bf16_31k": rag_bf16_31k,
}


def random_block_csr(n_kv_heads: int, n_blocks: int, density: float, seed: int = 0,
                     sink: bool = True):
    """Seeded block lists in rbs_select's CSR form (row g * nb + i, ascending
    block indices in 0..i, the diagonal always present, block 0 too when
    sink): each earlier block is drawn with probability `density`. A stand-in
    selection for attention-only tests; it computes nothing of the method.
    Returns (row_ptr int64 [Hkv*nb+1], col_idx int32)."""
    rng = np.random.default_rng(seed)
    rows = []
    for _ in range(n_kv_heads):
        for i in range(n_blocks):
            pick = np.flatnonzero(rng.random(i) < density) if i else np.zeros(0, np.int64)
            blocks = set(pick.tolist()) | {i}
            if sink:
                blocks.add(0)
            rows.append(sorted(blocks))
    row_ptr = np.zeros(len(rows) + 1, np.int64)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col_idx = np.fromiter((b for r in rows for b in r), np.int32, count=int(row_ptr[-1]))
    return row_ptr, col_idx
