"""The row ops written out from their definitions, in float64.

TEST INFRASTRUCTURE (see the package docstring).  Plain and slow: one row at a
time, ``math.fsum`` for every sum of squares, float64 everywhere except at the
rounding points the pages fix.

Sources (cited by page and section):

* TensorFold PR #1260, the commit adding the unit-sphere row kernels for the
  looped nGPT model: ``l2_rows`` computes y = bf16(s / sqrt(sum(s^2) + eps))
  with s = x, or s = bf16(x + r) when a residual is given; ``slerp_rows``
  computes h = bf16(l2(a + |alpha| (b - a))) with a = bf16(l2(res)),
  b = bf16(l2(out)) and the lerp done in fp32 steps.  Its rounding points are
  the sum before the norm, the slerp's a and b, and each output.  eps is added
  to the sum of squares (same PR, the q/k row kernel's "eps on the sum").
* DragonScale README, "What DragonScale changes": W_eff = diag(g) r W / ||W||_row,
  one gain per row, r the row radius (1 for linears and convs, sqrt(dim) for
  embeddings).  The formula has no eps.

Readings where the pages leave a step open:

* bf16 rounding is to nearest, ties to even.
* eps arrives as an fp32 value, so the oracle uses float64(float32(eps)).
* The lerp's "fp32 steps" are three separately rounded binary32 operations in
  the written order: d = b - a, t = |alpha| * d, u = a + t (no fused
  multiply-add).  u itself is not rounded to bf16.  numpy's float32 arithmetic
  is IEEE binary32 with round-to-nearest-even, which is what these steps are.
* A weight row of length zero scales by 0 (W_eff = bf16(w * 0)).
* Non-finite inputs follow IEEE float64 semantics.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

from .bf16 import bf16_rne, bf16_value

__all__ = ["eps_as_passed", "l2_rows", "slerp_rows", "slerp_rows_detail",
           "weight_rownorm_gain", "sum_sq", "l2_backward_values", "l2_rows_backward",
           "rownorm_backward_values", "weight_rownorm_gain_backward",
           "gate_gated_row", "gate_l2_rows", "swiglu_product_row", "swiglu_l2_rows",
           "rope_angles", "qk_rotated_heads", "qk_rows_l2",
           "rescale_project_values", "rescale_project", "rescale_after_step",
           "rms_rows", "rms_backward_values", "rms_rows_backward",
           "gains_of", "column_block_rows", "to_column_block", "scalar_gain_gradient",
           "weight_rownorm_scalar_gain_backward"]


def eps_as_passed(eps: float) -> float:
    """eps as the kernels receive it: rounded to fp32, held in float64."""
    return float(np.float32(eps))


def sum_sq(row: np.ndarray) -> float:
    """Correctly rounded float64 sum of squares of one row.

    Squares of bf16 and fp32 values are exact in float64 (at most 48
    significant bits), so ``math.fsum`` returns the exact sum, rounded once.
    """
    with np.errstate(all="ignore"):
        sq = np.asarray(row, dtype=np.float64) ** 2
    if np.isnan(sq).any():
        return math.nan
    if np.isinf(sq).any():
        return math.inf
    return math.fsum(sq)


def _l2_of_values(s: np.ndarray, eps64: float) -> np.ndarray:
    """Row-wise s / sqrt(sum(s^2) + eps) in float64 (not yet rounded)."""
    out = np.empty_like(s)
    with np.errstate(all="ignore"):
        for i in range(s.shape[0]):
            d = math.sqrt(sum_sq(s[i]) + eps64)
            out[i] = s[i] / d
    return out


def l2_rows(x_bits: np.ndarray, r_bits: Optional[np.ndarray] = None,
            eps: float = 1e-6) -> np.ndarray:
    """y = bf16(s / sqrt(sum(s^2) + eps)), s = x or bf16(x + r); bf16 bits in/out.

    TensorFold PR #1260, the l2 row kernel.  The sum x + r of two bf16 values
    is formed in float64 and rounded once to bf16 (the first rounding point).
    """
    x = bf16_value(np.atleast_2d(x_bits))
    if r_bits is not None:
        with np.errstate(all="ignore"):
            s = bf16_value(bf16_rne(x + bf16_value(np.atleast_2d(r_bits))))
    else:
        s = x
    y = _l2_of_values(s, eps_as_passed(eps))
    return bf16_rne(y).reshape(np.shape(x_bits))


def slerp_rows_detail(res_bits: np.ndarray, out_bits: np.ndarray,
                      alpha: np.ndarray, eps: float = 1e-6
                      ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """slerp_rows with its intermediates: returns (a_bits, b_bits, u_f32, h_bits).

    TensorFold PR #1260, the slerp row kernel (the nGPT residual update):
    a = bf16(l2(res)), b = bf16(l2(out)), u = a + |alpha| (b - a) in fp32
    steps, h = bf16(l2(u)).  alpha is one fp32 value per column.
    """
    eps64 = eps_as_passed(eps)
    res = bf16_value(np.atleast_2d(res_bits))
    out = bf16_value(np.atleast_2d(out_bits))
    a_bits = bf16_rne(_l2_of_values(res, eps64))
    b_bits = bf16_rne(_l2_of_values(out, eps64))
    a32 = bf16_value(a_bits).astype(np.float32)
    b32 = bf16_value(b_bits).astype(np.float32)
    abs_alpha = np.abs(np.asarray(alpha, dtype=np.float32))
    with np.errstate(all="ignore"):
        d = b32 - a32                 # fp32 step 1
        t = abs_alpha * d             # fp32 step 2
        u = a32 + t                   # fp32 step 3
    h = _l2_of_values(u.astype(np.float64), eps64)
    return a_bits, b_bits, u, bf16_rne(h)


def slerp_rows(res_bits: np.ndarray, out_bits: np.ndarray, alpha: np.ndarray,
               eps: float = 1e-6) -> np.ndarray:
    """h bits of :func:`slerp_rows_detail`."""
    return slerp_rows_detail(res_bits, out_bits, alpha, eps)[3].reshape(np.shape(res_bits))


def weight_rownorm_gain(w: Sequence[np.ndarray], gain: Sequence[np.ndarray],
                        radius: Sequence[float]
                        ) -> Tuple[list, list]:
    """Per matrix m and row i: n_i = ||W_i||, W_eff_i = bf16(g_i rho W_i / n_i).

    DragonScale README, "What DragonScale changes".  Returns, per matrix, the
    fp32 row lengths (the float64 length rounded to fp32) and the bf16 bits of
    W_eff.  A zero-length row scales by 0.  A matrix's gain is [rows], one
    value for every row (a scalar gain) or None (unit rows: g = 1).
    """
    norms, weffs = [], []
    for wm, gm, rho in zip(w, gain, radius):
        w64 = np.asarray(wm, dtype=np.float64)
        g64 = gains_of(gm, w64.shape[0])
        rho64 = float(np.float32(rho))
        n = np.empty(w64.shape[0])
        weff = np.empty_like(w64)
        with np.errstate(all="ignore"):
            for i in range(w64.shape[0]):
                ss = sum_sq(w64[i])
                n[i] = math.sqrt(ss)
                if n[i] == 0.0:
                    weff[i] = w64[i] * 0.0
                else:
                    weff[i] = (g64[i] * rho64 * w64[i]) / n[i]
        norms.append(n.astype(np.float32))
        weffs.append(bf16_rne(weff))
    return norms, weffs


# ------------------------------------------------------------------ backward
#
# Readings: the gradient is that of the unrounded forward function at the
# forward's inputs; a rounding to bf16 passes the gradient through unchanged
# (so x and r of l2_rows receive the same gradient ds).  A zero weight row,
# which the forward scales by 0, receives zero gradients.

def l2_backward_values(s: np.ndarray, dy: np.ndarray, eps64: float) -> np.ndarray:
    """ds = (dy - yhat <yhat, dy>) / D per row, yhat = s / D, D = sqrt(sum s^2 + eps).

    The Jacobian of s -> s / D is (I - yhat yhat^T) / D, applied to dy.
    Products of two bf16 values are exact in float64, so the sums are the
    correctly rounded float64 sums of the exact products.
    """
    out = np.empty_like(s)
    with np.errstate(all="ignore"):
        for i in range(s.shape[0]):
            d2 = sum_sq(s[i]) + eps64
            p = math.fsum(s[i] * dy[i])
            out[i] = (dy[i] - s[i] * (p / d2)) / math.sqrt(d2)
    return out


def l2_rows_backward(x_bits: np.ndarray, r_bits: Optional[np.ndarray], dy_bits: np.ndarray,
                     eps: float = 1e-6) -> np.ndarray:
    """bf16 bits of ds, the gradient of l2_rows with respect to s (and to x, r)."""
    x = bf16_value(np.atleast_2d(x_bits))
    if r_bits is not None:
        with np.errstate(all="ignore"):
            s = bf16_value(bf16_rne(x + bf16_value(np.atleast_2d(r_bits))))
    else:
        s = x
    dy = bf16_value(np.atleast_2d(dy_bits))
    return bf16_rne(l2_backward_values(s, dy, eps_as_passed(eps))).reshape(np.shape(x_bits))


def rownorm_backward_values(w64: np.ndarray, g64: np.ndarray, rho64: float, dwe: np.ndarray):
    """Per row: dW = (g rho / n) (dWe - w <w, dWe> / n^2), dg = rho <w, dWe> / n.

    DragonScale README, "What DragonScale changes": the gradient reaching W is
    (g r / ||W||) (I - w_hat w_hat^T) dL/dW_eff, tangent to the row; dg follows
    from W_eff = g r w_hat by the chain rule.  n = 0 gives zeros.
    """
    dw = np.zeros_like(w64)
    dg = np.zeros(w64.shape[0])
    with np.errstate(all="ignore"):
        for i in range(w64.shape[0]):
            ss = sum_sq(w64[i])
            n = math.sqrt(ss)
            if n == 0.0:
                continue
            p = math.fsum(w64[i] * dwe[i])
            dg[i] = rho64 * p / n
            dw[i] = (g64[i] * rho64 / n) * (dwe[i] - w64[i] * (p / ss))
    return dw, dg


def weight_rownorm_gain_backward(w: Sequence[np.ndarray], gain: Sequence[np.ndarray],
                                 radius: Sequence[float], dweff_bits: Sequence[np.ndarray]):
    """Per matrix: (dW fp32, dg fp32) from bf16 dL/dW_eff; the float64 values rounded once."""
    dws, dgs = [], []
    for wm, gm, rho, de in zip(w, gain, radius, dweff_bits):
        w64 = np.asarray(wm, np.float64)
        dw, dg = rownorm_backward_values(w64, gains_of(gm, w64.shape[0]),
                                         float(np.float32(rho)), bf16_value(de))
        with np.errstate(over="ignore"):          # beyond fp32's range: +-inf
            dws.append(dw.astype(np.float32))
            dgs.append(dg.astype(np.float32))
    return dws, dgs


# ------------------------------------------------------- activation rows
#
# TensorFold PR #1260, the commit adding two activation rows for Dory:
#   gate_l2_rows    out = bf16(l2(bf16(o * sigmoid(g * sg))))   over the whole row
#   swiglu_l2_rows  out = bf16(l2(bf16(silu(bf16(g * sug)) * bf16(u * suu))))
# with sigmoid(x) = 1 / (1 + exp(-x)) and silu(x) = x / (1 + exp(-x)), and fp32
# scale vectors (one value per column) formed by the caller.
#
# Readings: a product of a bf16 row by an fp32 scale vector is one IEEE fp32
# multiply (the form torch computes bf16 * fp32 in), rounded to bf16 where
# the formula names bf16; the oracle does that multiply in numpy float32.
# Everything after it up to the next bf16 rounding is float64 (exp from the
# float64 library, one rounding per operation).

def _sigmoid64(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def _f32_scale(v_bits: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """fp32(bf16 value * fp32 scale), the product rounded once in binary32."""
    with np.errstate(all="ignore"):
        return (bf16_value(v_bits).astype(np.float32)
                * np.asarray(scale, dtype=np.float32)).astype(np.float64)


def gate_gated_row(o_bits: np.ndarray, g_bits: np.ndarray, sg: np.ndarray) -> np.ndarray:
    """bf16 bits of the gated row t = bf16(o * sigmoid(fp32(g * sg)))."""
    o = bf16_value(np.atleast_2d(o_bits))
    x = _f32_scale(np.atleast_2d(g_bits), sg)
    with np.errstate(all="ignore"):
        return bf16_rne(o * _sigmoid64(x))


def gate_l2_rows(o_bits: np.ndarray, g_bits: np.ndarray, sg: np.ndarray,
                 eps: float = 1e-6) -> np.ndarray:
    """bf16 bits of l2 over each gated row (all heads of the row at once)."""
    t = bf16_value(gate_gated_row(o_bits, g_bits, sg))
    return bf16_rne(_l2_of_values(t, eps_as_passed(eps))).reshape(np.shape(o_bits))


def swiglu_product_row(g_bits: np.ndarray, u_bits: np.ndarray, sug: np.ndarray,
                       suu: np.ndarray) -> np.ndarray:
    """bf16 bits of p = bf16(silu(a) * b), a = bf16(fp32(g * sug)), b = bf16(fp32(u * suu))."""
    a = bf16_value(bf16_rne(_f32_scale(np.atleast_2d(g_bits), sug)))
    b = bf16_value(bf16_rne(_f32_scale(np.atleast_2d(u_bits), suu)))
    with np.errstate(all="ignore"):
        silu = a * _sigmoid64(a)
        return bf16_rne(silu * b)


def swiglu_l2_rows(g_bits: np.ndarray, u_bits: np.ndarray, sug: np.ndarray, suu: np.ndarray,
                   eps: float = 1e-6) -> np.ndarray:
    """bf16 bits of l2 over each SwiGLU product row."""
    p = bf16_value(swiglu_product_row(g_bits, u_bits, sug, suu))
    return bf16_rne(_l2_of_values(p, eps_as_passed(eps))).reshape(np.shape(g_bits))


# ------------------------------------------------------------------ q/k rows
#
# TensorFold PR #1260, the q/k commit (dory.py's order): rotate-half RoPE on
# the projection's bf16 rows with the fp32 angle pos * inv, rounded to bf16
# (the rotated head); then each head's L2 norm with eps on the sum, rounded to
# bf16 (the normalized head); then q times an fp32 scale vector; k is its
# normalized head.  For a head x = [x1, x2] (halves of head_dim / 2) and
# frequency i:  rot_i = x1_i cos(t_i) - x2_i sin(t_i),
#               rot_{i + hd/2} = x2_i cos(t_i) + x1_i sin(t_i).
#
# Readings: the angle is the fp32 product fp32(pos) * inv_freq_i (IEEE, as
# torch forms it; numpy float32 here); cos and sin of that fp32 value are
# float64.  The scale product is one fp32 multiply rounded to bf16, the form
# of the other scaled rows.  The scale vector covers the whole q row
# (n_q_heads * head_dim values).

def rope_angles(positions: np.ndarray, inv_freq: np.ndarray) -> np.ndarray:
    """float64 values of the fp32 angles fp32(pos) * inv_freq, [rows, hd/2]."""
    p = np.asarray(positions).astype(np.float32)[:, None]
    with np.errstate(all="ignore"):
        return (p * np.asarray(inv_freq, np.float32)[None, :]).astype(np.float64)


def qk_rotated_heads(x_bits: np.ndarray, theta: np.ndarray, head_dim: int) -> np.ndarray:
    """bf16 bits of every head rotated (rounding point 1), same layout as x."""
    x = bf16_value(np.atleast_2d(x_bits))
    rows, width = x.shape
    h2 = head_dim // 2
    xh = x.reshape(rows, width // head_dim, head_dim)
    x1, x2 = xh[..., :h2], xh[..., h2:]
    c = np.cos(theta)[:, None, :]
    s = np.sin(theta)[:, None, :]
    with np.errstate(all="ignore"):
        rot = np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
    return bf16_rne(rot.reshape(rows, width))


def _l2_heads(r_bits: np.ndarray, head_dim: int, eps: float) -> np.ndarray:
    rows, width = r_bits.shape
    r = bf16_value(r_bits).reshape(rows * (width // head_dim), head_dim)
    return bf16_rne(_l2_of_values(r, eps_as_passed(eps))).reshape(rows, width)


def qk_rows_l2(q_bits: np.ndarray, k_bits: Optional[np.ndarray], positions: np.ndarray,
               inv_freq: np.ndarray, q_scale: np.ndarray, head_dim: int, eps: float = 1e-6):
    """(q_out bits, k_out bits or None): RoPE, per-head L2, q scaled."""
    theta = rope_angles(positions, inv_freq)
    nq = _l2_heads(qk_rotated_heads(q_bits, theta, head_dim), head_dim, eps)
    with np.errstate(all="ignore"):
        q_out = bf16_rne((bf16_value(nq).astype(np.float32)
                          * np.asarray(q_scale, np.float32)[None, :]).astype(np.float64))
    k_out = None
    if k_bits is not None and np.size(k_bits):
        k_out = _l2_heads(qk_rotated_heads(k_bits, theta, head_dim), head_dim, eps)
    return q_out, k_out


# ------------------------------------------------------------ rescale method
#
# DragonScale README, "Optimizer" (and the `method` option of "Patching
# options": raw rows, rescaled by the optimizer after each step).  Per row of
# a raw weight w, with w_hat = w / ||w||:
#   before the step: g <- g - w_hat <w_hat, g>       (the gradient's radial part)
#   after the step:  m <- m - w_hat <w_hat, m>       (the momentum's, same part)
#                    w <- radius * w_hat             (back to its radius)
# Readings: after the step the direction is the stepped row's (rescaling
# does not change it); a zero row has no direction and is left as it is.

def rescale_project_values(w64: np.ndarray, v64: np.ndarray) -> np.ndarray:
    """v - w <w, v> / ||w||^2 per row (float64); rows with ||w|| = 0 unchanged."""
    out = np.array(v64, dtype=np.float64, copy=True)
    with np.errstate(all="ignore"):
        for i in range(w64.shape[0]):
            ss = sum_sq(w64[i])
            if ss == 0.0:
                continue
            p = math.fsum(w64[i] * v64[i])
            out[i] = v64[i] - w64[i] * (p / ss)
    return out


def rescale_project(w: Sequence[np.ndarray], v: Sequence[np.ndarray]):
    """Per matrix: fp32 v with its radial part removed (products of two fp32
    values are exact in float64, so each sum is the correctly rounded one)."""
    return [rescale_project_values(np.asarray(wm, np.float64), np.asarray(vm, np.float64))
            .astype(np.float32) for wm, vm in zip(w, v)]


def rescale_after_step(w: Sequence[np.ndarray], m: Sequence[Optional[np.ndarray]],
                       radius: Sequence[float]):
    """Per matrix: (fp32 w rescaled to its radius, fp32 m projected or None)."""
    ws, ms = [], []
    for wm, mm, rho in zip(w, m, radius):
        w64 = np.asarray(wm, np.float64)
        ms.append(None if mm is None else
                  rescale_project_values(w64, np.asarray(mm, np.float64)).astype(np.float32))
        out = np.array(w64, copy=True)
        r64 = float(np.float32(rho))
        with np.errstate(all="ignore"):
            for i in range(w64.shape[0]):
                n = math.sqrt(sum_sq(w64[i]))
                if n != 0.0:
                    out[i] = w64[i] * (r64 / n)
        ws.append(out.astype(np.float32))
    return ws, ms


# ------------------------------------------------------------------ RMSNorm
#
# The parameter-free RMSNorm of the ternary/8-bit GPT model page (its
# `rms_norm`: torch's rms_norm over the last dimension, eps 1e-6):
#   y = bf16(s / sqrt(mean(s^2) + eps)),   mean(s^2) = sum(s^2) / n
# over a row of n values, with s = x, or s = bf16(x + r) given a residual, as
# for l2_rows.  Readings: the mean divides the sum by the row's length; eps is
# added to the mean, not to the sum; the output is rounded once to bf16.
# Algebraically y = sqrt(n) * s / sqrt(sum(s^2) + n eps): l2_rows with eps
# scaled by n, times sqrt(n).

def _s_values(x_bits, r_bits):
    x = bf16_value(np.atleast_2d(x_bits))
    if r_bits is None:
        return x
    with np.errstate(all="ignore"):
        return bf16_value(bf16_rne(x + bf16_value(np.atleast_2d(r_bits))))


def _rms_of_values(s: np.ndarray, eps64: float) -> np.ndarray:
    """Row-wise s / sqrt(sum(s^2) / n + eps) in float64 (not yet rounded)."""
    out = np.empty_like(s)
    n = s.shape[1]
    with np.errstate(all="ignore"):
        for i in range(s.shape[0]):
            d = math.sqrt(sum_sq(s[i]) / n + eps64)
            out[i] = s[i] / d
    return out


def rms_rows(x_bits: np.ndarray, r_bits: Optional[np.ndarray] = None,
             eps: float = 1e-6) -> np.ndarray:
    """y = bf16(s / sqrt(mean(s^2) + eps)), s = x or bf16(x + r); bf16 bits in/out."""
    y = _rms_of_values(_s_values(x_bits, r_bits), eps_as_passed(eps))
    return bf16_rne(y).reshape(np.shape(x_bits))


def rms_backward_values(s: np.ndarray, dy: np.ndarray, eps64: float) -> np.ndarray:
    """ds = (dy - s <s, dy> / (n D^2)) / D per row, D = sqrt(sum(s^2) / n + eps).

    y = s / D with dD/ds_j = s_j / (n D), so the Jacobian is
    (I - s s^T / (n D^2)) / D, symmetric, applied to dy.
    """
    out = np.empty_like(s)
    n = s.shape[1]
    with np.errstate(all="ignore"):
        for i in range(s.shape[0]):
            d2 = sum_sq(s[i]) / n + eps64
            p = math.fsum(s[i] * dy[i])
            out[i] = (dy[i] - s[i] * (p / (n * d2))) / math.sqrt(d2)
    return out


def rms_rows_backward(x_bits: np.ndarray, r_bits: Optional[np.ndarray], dy_bits: np.ndarray,
                      eps: float = 1e-6) -> np.ndarray:
    """bf16 bits of ds, the gradient of rms_rows with respect to s (and to x, r)."""
    s = _s_values(x_bits, r_bits)
    dy = bf16_value(np.atleast_2d(dy_bits))
    return bf16_rne(rms_backward_values(s, dy, eps_as_passed(eps))).reshape(np.shape(x_bits))


# ---------------------------------------------- gain modes and weight layouts
#
# DragonScale README, "Patching options" and "Supported layers": the gain is
# one per row ("channel") or one for the whole layer ("scalar"), and mode
# "unit" keeps unit rows with no gain; the patched layers are Linear,
# Conv1d/2d/3d, ConvTranspose1d/2d/3d, Embedding and GPT-2's Conv1D.
# Readings:
# * a scalar gain is one value that every row of the matrix uses; "unit" is
#   a gain of 1 (W_eff = r W / ||W||);
# * a scalar gain's gradient is the sum over the rows of what each row's own
#   gain would receive (the chain rule: every row shares the one value);
# * a row is everything that feeds one output unit.  Linear, Conv and
#   Embedding store it contiguously (W[o, ...]); GPT-2's Conv1D stores its
#   weight as [in, out], so row o is the column W[:, o]; ConvTranspose stores
#   [in, out / groups, k...], so row o of a group is W[:, o, ...] over the
#   group's input channels: `in` segments of prod(k) contiguous values, one
#   per stored row.  Both are "column-block" layouts: a weight stored as
#   A rows of ld values whose unit u owns the seg values at u * seg of every
#   stored row (Conv1D: A = in, seg = 1, ld = out; ConvTranspose, one group:
#   A = in / groups, seg = prod(k), ld = (out / groups) * prod(k)).

def gains_of(gain: Optional[np.ndarray], rows: int) -> np.ndarray:
    """The per-row gains a gain mode stands for (float64): a [rows] array as
    given, a one-element array for every row, None for 1 (mode "unit")."""
    if gain is None:
        return np.ones(rows)
    g = np.asarray(gain, dtype=np.float64).reshape(-1)
    return np.full(rows, g[0]) if g.size == 1 else g


def column_block_rows(stored: np.ndarray, units: int, seg: int) -> np.ndarray:
    """The unit rows [units, A * seg] of a column-block weight stored [A, ld]:
    row u, element a * seg + b, is stored[a, u * seg + b]."""
    a = np.asarray(stored)
    out = np.empty((units, a.shape[0] * seg), dtype=a.dtype)
    for u in range(units):
        out[u] = a[:, u * seg:(u + 1) * seg].reshape(-1)
    return out


def to_column_block(rows: np.ndarray, stored_shape, seg: int, fill=0) -> np.ndarray:
    """Inverse of column_block_rows: an array of stored_shape [A, ld] holding
    each unit row in its columns, `fill` elsewhere."""
    units = rows.shape[0]
    out = np.full(stored_shape, fill, dtype=rows.dtype)
    for u in range(units):
        out[:, u * seg:(u + 1) * seg] = rows[u].reshape(stored_shape[0], seg)
    return out


def scalar_gain_gradient(dg_rows64: np.ndarray) -> np.float32:
    """dL/dg of a scalar gain from the per-row values rho <w, dW_eff> / ||w||
    (float64): their exact sum, rounded once to fp32."""
    with np.errstate(over="ignore"):
        return np.float32(math.fsum(np.asarray(dg_rows64, dtype=np.float64)))


def weight_rownorm_scalar_gain_backward(w: np.ndarray, gain: Optional[np.ndarray], radius: float,
                                        dweff_bits: np.ndarray):
    """One matrix with a scalar gain (one value) or none: (dW fp32, dL/dg fp32).

    dW is the per-row formula with g_i = g; dL/dg sums rho <w_i, dW_eff_i> /
    ||w_i|| over the rows (float64, rounded once).  With no gain there is
    nothing to differentiate and dL/dg is returned as None.
    """
    w64 = np.asarray(w, np.float64)
    dw, dg = rownorm_backward_values(w64, gains_of(gain, w64.shape[0]), float(np.float32(radius)),
                                     bf16_value(dweff_bits))
    with np.errstate(over="ignore"):
        dw32 = dw.astype(np.float32)
    return dw32, (None if gain is None else scalar_gain_gradient(dg))
