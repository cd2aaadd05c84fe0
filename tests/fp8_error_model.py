"""Expected output error of fp8 block-sparse attention from rounding the
probabilities to E4M3, used as the parity tolerance of the fp8 entry.

The only coarse step of the fp8 path is rounding each probability P to E4M3
(round to nearest even, 3 mantissa bits): in the normal range the rounding
error is at most half a unit in the last place, 2^-4 of the value, and across
many keys it behaves as independent noise with standard deviation at most
2^-4 / sqrt(3) of P. When the same rounded values feed both P.V and the row
sum, the output is sum_u w'_u v_u with w'_u = round(P_u) / sum round(P), so to
first order

    out - exact = sum_u w_u e_u (v_u - exact),   e_u the relative rounding error,

with w_u the exact softmax weights. Values below 2^-6 (E4M3 subnormals)
round to multiples of 2^-9 instead, an absolute error of at most 2^-10. The
fp8 path scales each 32-key block of a query row by its own power of two so
that the block's largest probability lands in (128, 256]; with p_u =
exp(s_u - M), M the row's largest logit (so every block maximum is <= 1),
and L = sum_u p_u, a probability can be subnormal only when p_u < 2^-13,
and its error is then at most 2^-17 in units of p. The variance per output
element is at most
    sigma^2 = 1/3 * sum_u a_u (v_u - exact)^2,
    a_u = (2^-4 w_u)^2 if p_u >= 2^-13, else (2^-17 / L)^2,
and a Gaussian's mean absolute value is sqrt(2/pi) sigma. The bf16 output
rounding adds at most 2^-9 |out| on average (half a unit in the last place of
an 8-bit significand, averaged).

A systematic slip (keys dropped, a row sum that does not match the weights,
a scale off by a percent) moves the error mean by far more than these
random-rounding figures on rows of many keys, which is what the tolerance is
for.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import rbs_oracle as orc

SIGMA_REL = 2.0 ** -4 / math.sqrt(3.0)


def decoded(f):
    """Real Q, K, V of an fp8 input set (decoded bytes times descales)."""
    lut = orc.e4m3_decode(np.arange(256))
    return (lut[np.asarray(f.q, np.uint8)] * f.q_descale,
            lut[np.asarray(f.k, np.uint8)] * f.k_descale,
            lut[np.asarray(f.v, np.uint8)] * f.v_descale)


def rounding_sigma(q, k, v, block, row_ptr, col_idx, rows, out_exact, lse_exact, scale=None):
    """Per output element of the given (KV head, query block) rows, the
    standard deviation of the P-rounding error, in the order
    [row][token][query head of the group][head dim] flattened (the order the
    parity tests flatten their errors in)."""
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    nb = orc.n_blocks(S, block)
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    parts = []
    for g, i in rows:
        r = g * nb + i
        blocks = [int(b) for b in col_idx[row_ptr[r]:row_ptr[r + 1]] if 0 <= b <= i]
        t0, t1 = i * block, min(S, (i + 1) * block)
        if not blocks:
            parts.append(np.zeros((t1 - t0) * G * D))
            continue
        keys = np.concatenate([np.arange(b * block, min(S, (b + 1) * block)) for b in blocks])
        tok = np.arange(t0, t1)
        qi = q[t0:t1, g * G:(g + 1) * G].astype(np.float64).transpose(1, 0, 2)   # [G, L, D]
        logits = (qi @ k[keys, g].astype(np.float64).T) * scale                  # [G, L, U]
        allowed = keys[None, :] <= tok[:, None]
        lse = lse_exact[g * G:(g + 1) * G, t0:t1]                                # [G, L]
        w = np.where(allowed, np.exp(np.where(allowed, logits, 0.0) - lse[..., None]), 0.0)
        mx = np.where(allowed, logits, -np.inf).max(-1, keepdims=True)          # [G, L, 1]
        mass = np.exp(lse[..., None] - mx)                                       # L = sum_u p_u
        normal = w * mass >= 2.0 ** -13                                          # p_u >= 2^-13
        a = np.where(allowed, np.where(normal, w * w, 2.0 ** -26 / (mass * mass)), 0.0)
        vv = v[keys, g].astype(np.float64)                                        # [U, D]
        o = out_exact[t0:t1, g * G:(g + 1) * G].transpose(1, 0, 2)               # [G, L, D]
        var = (a @ (vv * vv) - 2.0 * o * (a @ vv) + o * o * a.sum(-1, keepdims=True))
        sig = SIGMA_REL * np.sqrt(np.maximum(var, 0.0))
        parts.append(sig.transpose(1, 0, 2).reshape(-1))
    return np.concatenate(parts)


def exact_slab(out_exact, rows, block, S, G):
    """The exact outputs of the given rows in the same flattened order."""
    return np.concatenate([out_exact[i * block:min(S, (i + 1) * block), g * G:(g + 1) * G]
                           .reshape(-1) for g, i in rows])


def check(err, sigma, exact, what, mean_margin=1.5, max_sigmas=8.0):
    """The fp8 parity rule: the mean absolute error within mean_margin times
    the model's expectation plus the bf16 output rounding, and every element
    within max_sigmas standard deviations plus one bf16 half-unit of its
    value. Returns (mean, expected mean, worst element ratio)."""
    err = np.abs(err)
    expected = math.sqrt(2.0 / math.pi) * float(sigma.mean()) + 2.0 ** -9 * float(np.abs(exact).mean())
    mean = float(err.mean())
    allow = max_sigmas * sigma + 2.0 ** -8 * np.abs(exact) + 1e-6
    worst = float((err / allow).max())
    assert mean <= mean_margin * expected, (f"{what}: mean-abs {mean:.3e} above {mean_margin} x "
                                            f"the rounding model's {expected:.3e}")
    if worst > 1.0:
        top = np.argsort(-(err / allow))[:5]
        detail = "; ".join(f"#{k}: err {err[k]:.3e} sigma {sigma[k]:.3e} exact {exact[k]:.3e}"
                           for k in top)
        raise AssertionError(f"{what}: an element is {worst:.2f} x its allowance ({detail})")
    return mean, expected, worst
