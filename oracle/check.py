"""Tolerance checks of a result against the oracle.

TEST INFRASTRUCTURE (see the package docstring).

Two checks:

1. **Contract**: every bf16 output within one bf16 ulp (the spacing at the
   oracle value's binade) of the oracle's value, with NaN where the oracle has
   NaN, the same infinities, and the same sign on zeros; every fp32 row length
   within 2e-6 relative of the float64 length.

2. **Admissible set** (the method of TensorFold PR #1260's kernel-contract
   check: each output compared with float64's value at the bf16 rounding
   points "as a range over the fp32 run's spread").  For every element the
   float64 value of what an fp32 run may compute is bounded above and below,
   and the admissible outputs are the bf16 values from bf16(lo) to bf16(hi):
   one value, or two at a near-tie.  The fp32 run modelled here:

   * a sum of squares of exactly representable terms accumulated by any tree
     whose deepest path has at most ``depth`` additions, each rounded once
     (relative error at most (1 + u)**depth - 1 for nonnegative terms,
     u = 2**-24), with the sum kept free of overflow and of underflow loss by
     power-of-two scaling;
   * one rounding each for adding eps, the square root and the reciprocal;
   * one rounding for each product, plus 2**-149 absolute for results in the
     subnormal range;
   * for slerp, the lerp's three fp32 steps exactly as the oracle does them,
     over every admissible choice of a and b.

   An interval that spans more than two bf16 values means the bound is too
   loose for the check to be sharp; it is reported, not hidden.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from .bf16 import bf16_rne, bf16_ulp, bf16_value
from .rows import eps_as_passed, sum_sq

U = 2.0 ** -24
ETA = 2.0 ** -149          # least fp32 subnormal step
F64_WIDEN = 2.0 ** -46     # covers float64 rounding inside the bound arithmetic

__all__ = ["contract_bf16", "contract_rel", "Report", "admissible_l2_rows",
           "admissible_slerp_rows", "admissible_rownorm", "default_depth",
           "ordered", "slerp_unique_mask", "GRAD_SLACK", "l2_grad_terms",
           "rownorm_grad_terms", "contract_grad", "admissible_l2_backward",
           "admissible_rownorm_backward", "EXPF_ULPS", "gate_candidates", "swiglu_candidates",
           "admissible_act_rows", "act_unique_mask", "COSF_ULPS", "admissible_qk_rows",
           "rescale_terms", "admissible_rescale"]


def default_depth(cols: int) -> int:
    """A bound on the additions along any path of a row's fp32 sum tree."""
    return cols // 64 + 32


# ----------------------------------------------------------------- contract

def contract_bf16(got_bits, want_bits, zero_sign: bool = True) -> np.ndarray:
    """Boolean mask of elements that MEET the 1-ulp contract."""
    g = bf16_value(got_bits)
    w = bf16_value(want_bits)
    gn, wn = np.isnan(g), np.isnan(w)
    with np.errstate(all="ignore"):
        near = np.abs(g - w) <= bf16_ulp(w)
    inf = np.isinf(g) | np.isinf(w)
    ok = np.where(inf, g == w, near)
    ok = np.where(gn | wn, gn & wn, ok)
    if zero_sign:
        both0 = (g == 0) & (w == 0)
        ok &= ~both0 | (np.signbit(g) == np.signbit(w))
    return ok


def contract_rel(got, want, rel: float = 2e-6) -> np.ndarray:
    """Boolean mask of fp32 values within ``rel`` of the float64/fp32 reference."""
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    gn, wn = np.isnan(g), np.isnan(w)
    with np.errstate(all="ignore"):
        ok = np.abs(g - w) <= rel * np.abs(w)
        ok |= (g == w)
    return np.where(gn | wn, gn & wn, ok)


# ------------------------------------------------------------ admissible set

def ordered(bits) -> np.ndarray:
    """bf16 bits -> integers in value order (+0 and -0 both map to 0)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


@dataclass
class Report:
    """Outcome of an admissible-set check over many elements."""
    n: int = 0
    outside: int = 0          # result not in its admissible set
    two: int = 0              # elements whose set has two values (near-ties)
    loose: int = 0            # sets wider than two values (bound too loose)
    wide: int = 0             # gradient sets wider than two values (cancellation)
    first_bad: list = field(default_factory=list)

    @property
    def ok(self) -> bool:
        return self.outside == 0 and self.loose == 0

    def merge(self, other: "Report") -> "Report":
        self.n += other.n
        self.outside += other.outside
        self.two += other.two
        self.loose += other.loose
        self.wide += other.wide
        self.first_bad = (self.first_bad + other.first_bad)[:20]
        return self

    def __str__(self) -> str:
        return (f"n={self.n} outside={self.outside} two={self.two} "
                f"loose={self.loose} wide={self.wide} first_bad={self.first_bad[:5]}")


def _sum_bounds(sq_lo: np.ndarray, sq_hi: np.ndarray, depth: int):
    """Bounds of an fp32 sum of nonnegative terms lying in [sq_lo, sq_hi]."""
    lo = math.fsum(sq_lo)
    hi = math.fsum(sq_hi)
    k = depth + 1
    return lo * (1 - U) ** k * (1 - F64_WIDEN), hi * (1 + U) ** k * (1 + F64_WIDEN)


def _inv_bounds(s_lo: float, s_hi: float, eps64: float):
    """Bounds of fl(1 / fl(sqrt(fl(S + eps)))) for S in [s_lo, s_hi]."""
    t_lo = (s_lo + eps64) * (1 - 2 * U)
    t_hi = (s_hi + eps64) * (1 + 2 * U)
    r_lo = math.sqrt(t_lo) * (1 - U)
    r_hi = math.sqrt(t_hi) * (1 + U)
    with np.errstate(all="ignore"):
        inv_lo = (1.0 / r_hi) * (1 - U) * (1 - F64_WIDEN) if r_hi > 0 else math.inf
        inv_hi = (1.0 / r_lo) * (1 + U) * (1 + F64_WIDEN) if r_lo > 0 else math.inf
    return inv_lo, inv_hi


def _product_bounds(v_lo, v_hi, c_lo, c_hi):
    """Bounds of fl(v * c) for v in [v_lo, v_hi] (arrays), c in [c_lo, c_hi] > 0."""
    with np.errstate(all="ignore"):
        cands = np.stack([v_lo * c_lo, v_lo * c_hi, v_hi * c_lo, v_hi * c_hi])
    lo = cands.min(axis=0)
    hi = cands.max(axis=0)
    lo = np.where(lo >= 0, lo * (1 - U), lo * (1 + U)) * (1 + np.sign(-lo) * F64_WIDEN) - 2 * ETA
    hi = np.where(hi >= 0, hi * (1 + U), hi * (1 - U)) * (1 + np.sign(hi) * F64_WIDEN) + 2 * ETA
    return lo, hi


def _judge(got_bits, lo, hi, exact_bits, exact_mask, zero_any_sign,
           base_index, report: Report, wide_ok: bool = False):
    """Compare one row: interval elements and exactly-determined elements."""
    lo_b = bf16_rne(lo)
    hi_b = bf16_rne(hi)
    g = ordered(got_bits)
    ol, oh = ordered(lo_b), ordered(hi_b)
    width = oh - ol + 1
    inside = (g >= ol) & (g <= oh)
    # Exactly-determined elements: zeros from zero inputs, non-finite rows.
    if exact_mask is not None and exact_mask.any():
        gv = bf16_value(got_bits[exact_mask])
        ev = bf16_value(exact_bits[exact_mask])
        same = (np.isnan(gv) & np.isnan(ev)) | (gv == ev)
        if not zero_any_sign:
            z = (gv == 0) & (ev == 0)
            same &= ~z | (np.signbit(gv) == np.signbit(ev))
        inside[exact_mask] = same
        width[exact_mask] = 1
    n = got_bits.size
    bad = np.nonzero(~inside)[0]
    report.n += n
    report.outside += bad.size
    report.two += int((width == 2).sum())
    if wide_ok:
        report.wide += int((width > 2).sum())
    else:
        report.loose += int((width > 2).sum())
    for j in bad[: max(0, 20 - len(report.first_bad))]:
        report.first_bad.append(int(base_index + j))


def _mean_bounds(s_lo: float, s_hi: float, n: int):
    """Bounds of fl(S / n) for S in [s_lo, s_hi] >= 0 (one rounding).

    Relative error only, like the sum bounds: a row whose S / n + eps falls
    below 2^-96 is summed again scaled by a power of two (the kernels'
    rescue), so the quotient that decides the result is a normal fp32 value;
    where eps keeps S / n + eps above 2^-96 without a rescue, an absolute
    subnormal error in S / n is far below the 2u the inverse allows for.
    """
    return s_lo / n * (1 - U) * (1 - F64_WIDEN), s_hi / n * (1 + U) * (1 + F64_WIDEN)


def _row_inv(s_row: np.ndarray, eps64: float, depth: int, mean: bool = False):
    sq = s_row.astype(np.float64) ** 2
    s_lo, s_hi = _sum_bounds(sq, sq, depth)
    if mean:
        s_lo, s_hi = _mean_bounds(s_lo, s_hi, s_row.size)
    return _inv_bounds(s_lo, s_hi, eps64)


def _l2_value_bounds(s_row: np.ndarray, eps64: float, depth: int, mean: bool = False):
    inv_lo, inv_hi = _row_inv(s_row, eps64, depth, mean)
    return _product_bounds(s_row, s_row, inv_lo, inv_hi)


def admissible_l2_rows(got_bits, x_bits, r_bits=None, eps: float = 1e-6,
                       depth: Optional[int] = None, row_ids=None, mean: bool = False) -> Report:
    """Strict check of l2_rows outputs ``got_bits`` for the given input rows.

    ``mean=True`` checks rms_rows instead: the fp32 sum is divided by the
    row's length (one more rounding) before eps is added.
    """
    from .rows import l2_rows, rms_rows
    l2_ref = rms_rows if mean else l2_rows
    x = bf16_value(np.atleast_2d(x_bits))
    if r_bits is not None:
        with np.errstate(all="ignore"):
            s = bf16_value(bf16_rne(x + bf16_value(np.atleast_2d(r_bits))))
    else:
        s = x
    got = np.atleast_2d(got_bits)
    cols = s.shape[1]
    depth = default_depth(cols) if depth is None else depth
    eps64 = eps_as_passed(eps)
    rep = Report()
    for i in range(s.shape[0]):
        row = s[i]
        base = (row_ids[i] if row_ids is not None else i) * cols
        if not np.isfinite(row).all() or (eps64 == 0 and not row.any()):
            exact = l2_ref(x_bits[i:i + 1] if x_bits.ndim == 2 else x_bits,
                           None if r_bits is None else r_bits[i:i + 1], eps)[0]
            _judge(got[i], row, row, exact, np.ones(cols, bool), False, base, rep)
            continue
        lo, hi = _l2_value_bounds(row, eps64, depth, mean)
        zero = row == 0
        exact = np.where(np.signbit(row), np.uint16(0x8000), np.uint16(0)).astype(np.uint16)
        _judge(got[i], lo, hi, exact, zero, False, base, rep)
    return rep


def _f32_lerp(a32, b32, abs_alpha):
    with np.errstate(all="ignore"):
        d = b32 - a32
        t = abs_alpha * d
        return a32 + t


def admissible_slerp_rows(got_bits, res_bits, out_bits, alpha, eps: float = 1e-6,
                          depth: Optional[int] = None, row_ids=None) -> Report:
    """Strict check of slerp_rows outputs over every admissible a and b."""
    from .rows import slerp_rows as slerp_ref
    res = bf16_value(np.atleast_2d(res_bits))
    out = bf16_value(np.atleast_2d(out_bits))
    got = np.atleast_2d(got_bits)
    cols = res.shape[1]
    depth = default_depth(cols) if depth is None else depth
    eps64 = eps_as_passed(eps)
    abs_alpha = np.abs(np.asarray(alpha, dtype=np.float32))
    rep = Report()
    for i in range(res.shape[0]):
        base = (row_ids[i] if row_ids is not None else i) * cols
        if not (np.isfinite(res[i]).all() and np.isfinite(out[i]).all()
                and np.isfinite(abs_alpha).all()):
            exact = slerp_ref(np.atleast_2d(res_bits)[i:i + 1],
                              np.atleast_2d(out_bits)[i:i + 1], alpha, eps)[0]
            _judge(got[i], res[i], res[i], exact, np.ones(cols, bool), False, base, rep)
            continue
        cand = []
        for v in (res[i], out[i]):
            lo, hi = _l2_value_bounds(v, eps64, depth)
            lo_b, hi_b = bf16_rne(lo), bf16_rne(hi)
            if (ordered(hi_b) - ordered(lo_b) > 1).any():
                rep.loose += int((ordered(hi_b) - ordered(lo_b) > 1).sum())
            cand.append((bf16_value(lo_b).astype(np.float32),
                         bf16_value(hi_b).astype(np.float32)))
        (a_lo, a_hi), (b_lo, b_hi) = cand
        us = np.stack([_f32_lerp(a, b, abs_alpha)
                       for a in (a_lo, a_hi) for b in (b_lo, b_hi)]).astype(np.float64)
        sq = us ** 2
        s_lo, s_hi = _sum_bounds(sq.min(axis=0), sq.max(axis=0), depth)
        inv_lo, inv_hi = _inv_bounds(s_lo, s_hi, eps64)
        # admissible: the union over the choices of (a, b) of each choice's set
        g = ordered(got[i])
        inside = np.zeros(cols, bool)
        width = np.zeros(cols, np.int64)
        for u in us:
            lo, hi = _product_bounds(u, u, inv_lo, inv_hi)
            ol, oh = ordered(bf16_rne(lo)), ordered(bf16_rne(hi))
            zero = u == 0
            # a zero u gives a zero h of the same sign
            zs = np.where(np.signbit(u), -1, 1)
            ok = np.where(zero, (g == 0) & (np.where(np.signbit(bf16_value(got[i])), -1, 1) == zs),
                          (g >= ol) & (g <= oh))
            inside |= ok
            width = np.maximum(width, np.where(zero, 1, oh - ol + 1))
        bad = np.nonzero(~inside)[0]
        rep.n += cols
        rep.outside += bad.size
        rep.two += int((width == 2).sum())
        rep.loose += int((width > 2).sum())
        for j in bad[: max(0, 20 - len(rep.first_bad))]:
            rep.first_bad.append(int(base + j))
    return rep


def slerp_unique_mask(res_bits, out_bits, eps: float = 1e-6,
                      depth: Optional[int] = None) -> np.ndarray:
    """Elements whose a and b each have exactly one admissible bf16 value.

    Where a_j or b_j lies so near a bf16 midpoint that an fp32 run may round
    it either way, both choices are correct, and the lerp can amplify the
    one-ulp difference (b - a cancels): h_j is then not unique, and only the
    admissible-set check applies.  Elsewhere the 1-ulp contract applies.
    """
    res = bf16_value(np.atleast_2d(res_bits))
    out = bf16_value(np.atleast_2d(out_bits))
    cols = res.shape[1]
    depth = default_depth(cols) if depth is None else depth
    eps64 = eps_as_passed(eps)
    mask = np.ones(res.shape, bool)
    for i in range(res.shape[0]):
        for v in (res[i], out[i]):
            if not np.isfinite(v).all():
                continue
            lo, hi = _l2_value_bounds(v, eps64, depth)
            mask[i] &= ordered(bf16_rne(lo)) == ordered(bf16_rne(hi))
    return mask


def admissible_rownorm(got_norm, got_weff_bits, w, g, rho: float = 1.0,
                       depth: Optional[int] = None, row_offset: int = 0):
    """Strict check of one matrix: (norm Report, W_eff Report).

    The row length must lie in [fl(sqrt(S_lo)), fl(sqrt(S_hi))]; W_eff in the
    admissible set of fl(w * fl(fl(g * rho) / norm)).
    """
    w64 = np.asarray(w, dtype=np.float64)
    g64 = np.asarray(g, dtype=np.float64)
    rho64 = float(np.float32(rho))
    rows, cols = w64.shape
    depth = default_depth(cols) if depth is None else depth
    got_w = np.atleast_2d(got_weff_bits)
    got_n = np.asarray(got_norm, dtype=np.float64)
    rn, rw = Report(), Report()
    for i in range(rows):
        base = (row_offset + i) * cols
        row = w64[i]
        if not np.isfinite(row).all() or not np.isfinite(g64[i]):
            from .rows import weight_rownorm_gain as ref
            n_ref, w_ref = ref([w[i:i + 1]], [g[i:i + 1]], [rho])
            rn.n += 1
            same = (np.isnan(got_n[i]) and np.isnan(n_ref[0][0])) or got_n[i] == n_ref[0][0]
            rn.outside += 0 if same else 1
            _judge(got_w[i], row, row, w_ref[0][0], np.ones(cols, bool), True, base, rw)
            continue
        s_lo, s_hi = _sum_bounds(row ** 2, row ** 2, depth)
        n_lo = math.sqrt(s_lo) * (1 - U) * (1 - F64_WIDEN) - ETA
        n_hi = math.sqrt(s_hi) * (1 + U) * (1 + F64_WIDEN) + ETA
        rn.n += 1
        if not (n_lo <= got_n[i] <= n_hi):
            rn.outside += 1
            if len(rn.first_bad) < 20:
                rn.first_bad.append(row_offset + i)
        if s_hi == 0:
            exact = np.zeros(cols, np.uint16)
            _judge(got_w[i], row, row, exact, np.ones(cols, bool), True, base, rw)
            continue
        gr = g64[i] * rho64
        gr_lo, gr_hi = sorted((gr * (1 - U), gr * (1 + U)))
        if rho64 == 1.0:
            gr_lo = gr_hi = gr
        r_lo = max(math.sqrt(s_lo) * (1 - U), 0.0)
        r_hi = math.sqrt(s_hi) * (1 + U)
        with np.errstate(all="ignore"):
            cs = [gr_lo / r_lo, gr_lo / r_hi, gr_hi / r_lo, gr_hi / r_hi]
        c_lo = min(cs)
        c_hi = max(cs)
        c_lo = c_lo * (1 - U) if c_lo >= 0 else c_lo * (1 + U)
        c_hi = c_hi * (1 + U) if c_hi >= 0 else c_hi * (1 - U)
        with np.errstate(all="ignore"):
            cands = np.stack([row * c_lo, row * c_hi])
        lo = cands.min(axis=0)
        hi = cands.max(axis=0)
        lo = np.where(lo >= 0, lo * (1 - U), lo * (1 + U)) * (1 - np.sign(lo) * F64_WIDEN) - 2 * ETA
        hi = np.where(hi >= 0, hi * (1 + U), hi * (1 - U)) * (1 + np.sign(hi) * F64_WIDEN) + 2 * ETA
        zero = row == 0
        _judge(got_w[i], lo, hi, np.zeros(cols, np.uint16), zero, True, base, rw)
    return rn, rw


# ------------------------------------------------------------------ backward
#
# A gradient element is a difference of two terms (dy_j and s_j <s,dy>/D^2
# for l2_rows; dWe_j and w_j <w,dWe>/||w||^2 for the weights) that may cancel,
# so an fp32 run's error is a few fp32 units of the larger term, not of the
# result.  The contract therefore allows, beyond the output format's own
# rounding (one bf16 ulp, or 2e-6 relative for fp32), GRAD_SLACK times the
# size of those terms: 2**-16 = 256 fp32 units, enough for fp32 sums whose
# tree is up to ~250 additions deep (a kernel reducing a row of 65,536 columns
# over 1,024 lanes needs about 100).

GRAD_SLACK = 2.0 ** -16


def l2_grad_terms(s: np.ndarray, dy: np.ndarray, eps64: float, mean: bool = False) -> np.ndarray:
    """Per element (|dy_j| + |s_j| sum|s dy| / D^2) / D: the size of ds_j's terms.

    With mean=True (the rms_rows gradient) D^2 = sum s^2 / n + eps and the
    second term is |s_j| sum|s dy| / (n D^2).
    """
    out = np.empty(s.shape)
    n = s.shape[1] if mean else 1
    with np.errstate(all="ignore"):
        for i in range(s.shape[0]):
            d2 = sum_sq(s[i]) / n + eps64
            a = math.fsum(np.abs(s[i] * dy[i]))
            out[i] = (np.abs(dy[i]) + np.abs(s[i]) * (a / (n * d2))) / math.sqrt(d2)
    return out


def rownorm_grad_terms(w: np.ndarray, g: np.ndarray, rho: float, dwe: np.ndarray):
    """(per element |g rho| / n (|dWe_j| + |w_j| sum|w dWe| / n^2), per row |rho| sum|w dWe| / n)."""
    tw = np.zeros(w.shape)
    tg = np.zeros(w.shape[0])
    with np.errstate(all="ignore"):
        for i in range(w.shape[0]):
            ss = sum_sq(w[i])
            n = math.sqrt(ss)
            if n == 0.0:
                continue
            a = math.fsum(np.abs(w[i] * dwe[i]))
            tw[i] = abs(g[i] * rho) / n * (np.abs(dwe[i]) + np.abs(w[i]) * (a / ss))
            tg[i] = abs(rho) * a / n
    return tw, tg


def contract_grad(got, want, terms, fmt: str = "bf16") -> np.ndarray:
    """Boolean mask of gradient elements that MEET the contract.

    ``got``/``want`` are bf16 bits (fmt "bf16") or fp32/float64 values (fmt
    "f32"); ``terms`` from l2_grad_terms / rownorm_grad_terms.  NaN must match
    NaN and infinities must match; the sign of a zero is not compared (a
    cancelling difference may give either).
    """
    if fmt == "bf16":
        g, w = bf16_value(got), bf16_value(want)
        with np.errstate(all="ignore"):
            tol = bf16_ulp(w) + GRAD_SLACK * terms
    else:
        g = np.asarray(got, np.float64)
        w = np.asarray(want, np.float64)
        with np.errstate(all="ignore"):
            tol = 2e-6 * np.abs(w) + GRAD_SLACK * terms
    gn, wn = np.isnan(g), np.isnan(w)
    with np.errstate(all="ignore"):
        near = np.abs(g - w) <= tol
    inf = np.isinf(g) | np.isinf(w)
    ok = np.where(inf, g == w, near)
    return np.where(gn | wn, gn & wn, ok)


def _mixed_sum_bounds(terms: np.ndarray, depth: int):
    """Bounds of an fp32 sum of float64-exact terms of any sign.

    Each term may be rounded once to fp32 (a product) and every leaf passes
    through at most ``depth`` rounded additions, so the error is at most
    ((1 + u)^(depth + 1) - 1) sum|t|, plus 2**-149 per term for products in
    fp32's subnormal range.
    """
    p = math.fsum(terms)
    a = math.fsum(np.abs(terms))
    err = (((1 + U) ** (depth + 1) - 1) * a + terms.size * ETA) * (1 + F64_WIDEN) \
        + abs(p) * 2.0 ** -52
    return p - err, p + err


def _corner_bounds(a_lo, a_hi, b_lo, b_hi):
    """Bounds of fl(a * b) for a, b in intervals of any sign (arrays broadcast)."""
    return _product_bounds(np.asarray(a_lo, np.float64), np.asarray(a_hi, np.float64),
                           b_lo, b_hi)


def _diff_bounds(a, m_lo, m_hi):
    """Bounds of fl(a - m) for exact a and m in [m_lo, m_hi] (one rounding)."""
    lo = a - m_hi
    hi = a - m_lo
    lo = np.where(lo >= 0, lo * (1 - U), lo * (1 + U)) * (1 + np.sign(-lo) * F64_WIDEN)
    hi = np.where(hi >= 0, hi * (1 + U), hi * (1 - U)) * (1 + np.sign(hi) * F64_WIDEN)
    return lo, hi


def _tangent_bounds(v, d, k_lo, k_hi, c_lo, c_hi):
    """Bounds of fl(c * fl(d - fl(v * k))) per element (v, d exact arrays)."""
    with np.errstate(all="ignore"):
        m = np.stack([v * k_lo, v * k_hi])
    m_lo, m_hi = m.min(axis=0), m.max(axis=0)
    m_lo = np.where(m_lo >= 0, m_lo * (1 - U), m_lo * (1 + U)) * (1 - np.sign(m_lo) * F64_WIDEN) - ETA
    m_hi = np.where(m_hi >= 0, m_hi * (1 + U), m_hi * (1 - U)) * (1 + np.sign(m_hi) * F64_WIDEN) + ETA
    t_lo, t_hi = _diff_bounds(d, m_lo, m_hi)
    return _corner_bounds(t_lo, t_hi, c_lo, c_hi)


F32_OVERFLOW = (2.0 - 2.0 ** -24) * 2.0 ** 127    # fp32 rounding sends |v| >= this to inf


def _f32_inside(got, lo, hi):
    """fp32 results inside [lo, hi]; an infinity is inside when the interval
    reaches the overflow threshold on its side."""
    got = np.asarray(got, np.float64)
    with np.errstate(invalid="ignore"):
        ok = (got >= lo) & (got <= hi)
    ok |= (got == np.inf) & (hi >= F32_OVERFLOW)
    ok |= (got == -np.inf) & (lo <= -F32_OVERFLOW)
    return ok


def _scalar(lo_hi):
    lo, hi = lo_hi
    return float(np.min(lo)), float(np.max(hi))


def admissible_l2_backward(got_bits, x_bits, r_bits, dy_bits, eps: float = 1e-6,
                           depth: Optional[int] = None, row_ids=None,
                           mean: bool = False) -> Report:
    """Strict check of l2_rows gradients ``got_bits`` (bf16 bits).

    The fp32 run modelled: S and P = <s, dy> summed as above (depth
    additions); inv = 1/sqrt(S + eps) as in the forward; k = fl(fl(P inv) inv);
    ds_j = fl(fl(dy_j - fl(s_j k)) inv), or any fusing of those steps.  A set
    of more than two bf16 values is counted in ``wide`` (cancellation makes
    it legitimate), not as a failure.  ``mean=True`` checks the rms_rows
    gradient: S and P are each divided by the row's length (one rounding
    each) before inv and k are formed.
    """
    from .rows import l2_rows_backward, rms_rows_backward
    ref = rms_rows_backward if mean else l2_rows_backward
    x = bf16_value(np.atleast_2d(x_bits))
    if r_bits is not None:
        with np.errstate(all="ignore"):
            s = bf16_value(bf16_rne(x + bf16_value(np.atleast_2d(r_bits))))
    else:
        s = x
    dy = bf16_value(np.atleast_2d(dy_bits))
    got = np.atleast_2d(got_bits)
    cols = s.shape[1]
    depth = default_depth(cols) if depth is None else depth
    eps64 = eps_as_passed(eps)
    rep = Report()
    for i in range(s.shape[0]):
        base = (row_ids[i] if row_ids is not None else i) * cols
        row, d = s[i], dy[i]
        if not (np.isfinite(row).all() and np.isfinite(d).all()) or (eps64 == 0 and not row.any()):
            exact = ref(np.atleast_2d(x_bits)[i:i + 1],
                        None if r_bits is None else np.atleast_2d(r_bits)[i:i + 1],
                        np.atleast_2d(dy_bits)[i:i + 1], eps)[0]
            _judge(got[i], row, row, exact, np.ones(cols, bool), True, base, rep)
            continue
        sq = row ** 2
        s_lo, s_hi = _sum_bounds(sq, sq, depth)
        p_lo, p_hi = _mixed_sum_bounds(row * d, depth)
        if mean:
            s_lo, s_hi = _mean_bounds(s_lo, s_hi, cols)
            p_lo, p_hi = _scalar(_corner_bounds([p_lo], [p_hi], 1.0 / cols, 1.0 / cols))
        inv_lo, inv_hi = _inv_bounds(s_lo, s_hi, eps64)
        q = _scalar(_corner_bounds([p_lo], [p_hi], inv_lo, inv_hi))
        k_lo, k_hi = _scalar(_corner_bounds([q[0]], [q[1]], inv_lo, inv_hi))
        lo, hi = _tangent_bounds(row, d, k_lo, k_hi, inv_lo, inv_hi)
        _judge(got[i], lo, hi, None, None, True, base, rep, wide_ok=True)
    return rep


def admissible_rownorm_backward(got_dw, got_dg, w, g, rho, dweff_bits,
                                depth: Optional[int] = None, row_offset: int = 0):
    """Strict check of one matrix's weight gradients: (dW Report, dg Report).

    fp32 outputs must lie inside the interval itself.  The fp32 run
    modelled: S = sum w^2 and P = <w, dWe> as above; inv = 1/sqrt(S) with at
    most three roundings; dg = fl(fl(rho P) inv); c = fl(fl(g rho) inv);
    k = fl(fl(P inv) inv); dW_j = fl(c fl(dWe_j - fl(w_j k))), or any fusing
    of those steps.  A zero row must give exact zeros.
    """
    from .rows import rownorm_backward_values as ref
    w64 = np.asarray(w, dtype=np.float64)
    g64 = np.asarray(g, dtype=np.float64)
    rho64 = float(np.float32(rho))
    de = bf16_value(np.asarray(dweff_bits))
    rows, cols = w64.shape
    depth = default_depth(cols) if depth is None else depth
    gw = np.atleast_2d(np.asarray(got_dw, np.float64))
    gg = np.asarray(got_dg, np.float64)
    rw, rg = Report(), Report()

    def mark(rep, bad, base):
        rep.n += bad.size
        idx = np.nonzero(bad)[0]
        rep.outside += idx.size
        for j in idx[: max(0, 20 - len(rep.first_bad))]:
            rep.first_bad.append(int(base + j))

    for i in range(rows):
        row, d = w64[i], de[i]
        base = (row_offset + i) * cols
        if not (np.isfinite(row).all() and np.isfinite(d).all() and np.isfinite(g64[i])):
            dw_ref, dg_ref = ref(row[None], g64[i:i + 1], rho64, d[None])
            want = dw_ref[0].astype(np.float32).astype(np.float64)
            mark(rw, ~((gw[i] == want) | (np.isnan(gw[i]) & np.isnan(want))), base)
            wg = float(np.float32(dg_ref[0]))
            mark(rg, np.array([not (gg[i] == wg or (np.isnan(gg[i]) and np.isnan(wg)))]),
                 row_offset + i)
            continue
        sq = row ** 2
        s_lo, s_hi = _sum_bounds(sq, sq, depth)
        if s_hi == 0:
            mark(rw, gw[i] != 0, base)
            mark(rg, np.array([gg[i] != 0]), row_offset + i)
            continue
        inv_lo, inv_hi = _inv_bounds(s_lo, s_hi, 0.0)
        p_lo, p_hi = _mixed_sum_bounds(row * d, depth)
        rp = _scalar(_corner_bounds([p_lo], [p_hi], rho64, rho64))
        if rho64 == 1.0:
            rp = (p_lo, p_hi)
        dg_lo, dg_hi = _scalar(_corner_bounds([rp[0]], [rp[1]], inv_lo, inv_hi))
        mark(rg, ~_f32_inside(np.array([gg[i]]), dg_lo, dg_hi), row_offset + i)
        gr = g64[i] * rho64
        gr_lo, gr_hi = (gr, gr) if rho64 == 1.0 else _scalar(_corner_bounds([gr], [gr], 1.0, 1.0))
        c_lo, c_hi = _scalar(_corner_bounds([gr_lo], [gr_hi], inv_lo, inv_hi))
        q = _scalar(_corner_bounds([p_lo], [p_hi], inv_lo, inv_hi))
        k_lo, k_hi = _scalar(_corner_bounds([q[0]], [q[1]], inv_lo, inv_hi))
        lo, hi = _tangent_bounds(row, d, k_lo, k_hi, c_lo, c_hi)
        mark(rw, ~_f32_inside(gw[i], lo, hi), base)
    return rw, rg


# ---------------------------------------------------------- activation rows
#
# The fp32 run modelled for gate_l2_rows and swiglu_l2_rows: the products by
# the fp32 scale vectors are IEEE multiplies (deterministic, as the oracle
# does them); exp is within EXPF_ULPS units in the last place of exp where
# the result is a normal fp32 number, anywhere in [0, 2**-126] below that,
# and may return +inf where exp exceeds fp32's largest value; 1 + e, the IEEE
# division and the product by o (or b) round once each.  That bounds the pre-norm value of each element;
# its admissible bf16 values run from bf16(lo) to bf16(hi), and the output
# is checked over every such choice as slerp's is over a and b.

# EXPF_ULPS: the error the page's check allows for exp is "expf's ulps"
# (TensorFold PR #1260, the activation-row commit): the fp32 expf of the
# CUDA toolchain those kernels were built with, whose published maximum error
# is 2 units in the last place over its full range (the CUDA C++ Programming
# Guide's table of single-precision mathematical functions).  The bound is
# the page's, not a measurement of the kernels checked here (gfx950's exp
# measured within 1.22 ulp, inside it).
EXPF_ULPS = 2.0
F32_MAX = float(np.finfo(np.float32).max)


def _expf_bounds(v):
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(v)
        rel = EXPF_ULPS * 2.0 ** -23
        lo = np.maximum(e * (1 - rel) - EXPF_ULPS * ETA, 0.0)
        hi = e * (1 + rel) + EXPF_ULPS * ETA
        tiny = e < 2.0 ** -126
        lo = np.where(tiny, 0.0, lo)
        hi = np.where(tiny, 2.0 ** -126, hi)
    return lo, np.where(hi >= F32_MAX, np.inf, hi)


def _one_plus_bounds(e_lo, e_hi):
    """Bounds of fl(1 + e), e >= 0."""
    return (1 + e_lo) * (1 - U), (1 + e_hi) * (1 + U)


def _outward(lo, hi):
    lo = np.where(lo >= 0, lo * (1 - U), lo * (1 + U)) * (1 + np.sign(-lo) * F64_WIDEN) - ETA
    hi = np.where(hi >= 0, hi * (1 + U), hi * (1 - U)) * (1 + np.sign(hi) * F64_WIDEN) + ETA
    return lo, hi


def gate_candidates(o_bits, g_bits, sg):
    """Float64 values of the lowest and highest admissible gated-row bf16 value."""
    from .rows import _f32_scale
    o = bf16_value(np.atleast_2d(o_bits))
    x = _f32_scale(np.atleast_2d(g_bits), sg)
    e_lo, e_hi = _expf_bounds(-x)
    d_lo, d_hi = _one_plus_bounds(e_lo, e_hi)
    with np.errstate(all="ignore"):
        r_lo, r_hi = _outward(1.0 / d_hi, 1.0 / d_lo)
    r_lo = np.maximum(r_lo, 0.0)
    lo, hi = _product_bounds(o, o, r_lo, r_hi)
    return bf16_value(bf16_rne(lo)), bf16_value(bf16_rne(hi))


def swiglu_candidates(g_bits, u_bits, sug, suu):
    """Float64 values of the lowest and highest admissible SwiGLU product bf16 value."""
    from .rows import _f32_scale
    a = bf16_value(bf16_rne(_f32_scale(np.atleast_2d(g_bits), sug)))
    b = bf16_value(bf16_rne(_f32_scale(np.atleast_2d(u_bits), suu)))
    e_lo, e_hi = _expf_bounds(-a)
    d_lo, d_hi = _one_plus_bounds(e_lo, e_hi)
    with np.errstate(all="ignore"):
        q1, q2 = a / d_hi, a / d_lo
        s_lo, s_hi = _outward(np.minimum(q1, q2), np.maximum(q1, q2))
        s_lo = np.where(a == 0, 0.0, s_lo)
        s_hi = np.where(a == 0, 0.0, s_hi)
    lo, hi = _product_bounds(s_lo, s_hi, b, b)
    return bf16_value(bf16_rne(lo)), bf16_value(bf16_rne(hi))


def act_unique_mask(c_lo, c_hi) -> np.ndarray:
    """Elements whose pre-norm value has exactly one admissible bf16 value."""
    return ordered(bf16_rne(c_lo)) == ordered(bf16_rne(c_hi))


def admissible_act_rows(got_bits, c_lo, c_hi, exact_bits=None, finite_rows=None,
                        eps: float = 1e-6, depth: Optional[int] = None) -> Report:
    """Strict check of l2 over rows whose elements lie in [c_lo, c_hi] (bf16 values).

    Rows flagged False in ``finite_rows`` are compared with ``exact_bits``
    (NaN by position, values exactly).
    """
    got = np.atleast_2d(got_bits)
    c_lo = np.atleast_2d(c_lo)
    c_hi = np.atleast_2d(c_hi)
    cols = got.shape[1]
    depth = default_depth(cols) if depth is None else depth
    eps64 = eps_as_passed(eps)
    rep = Report()
    for i in range(got.shape[0]):
        base = i * cols
        fin = np.isfinite(c_lo[i]).all() and np.isfinite(c_hi[i]).all()
        if finite_rows is not None:
            fin = fin and bool(finite_rows[i])
        lo_i, hi_i = c_lo[i], c_hi[i]
        if not fin or (eps64 == 0 and not (lo_i.any() or hi_i.any())):
            _judge(got[i], lo_i, lo_i, exact_bits[i], np.ones(cols, bool), False, base, rep)
            continue
        sq_a, sq_b = lo_i ** 2, hi_i ** 2
        sq_lo = np.where((lo_i <= 0) & (hi_i >= 0), 0.0, np.minimum(sq_a, sq_b))
        s_lo, s_hi = _sum_bounds(sq_lo, np.maximum(sq_a, sq_b), depth)
        inv_lo, inv_hi = _inv_bounds(s_lo, s_hi, eps64)
        g = ordered(got[i])
        outs = []
        width = np.zeros(cols, np.int64)
        for c in (lo_i, hi_i):
            lo, hi = _product_bounds(c, c, inv_lo, inv_hi)
            ol, oh = ordered(bf16_rne(lo)), ordered(bf16_rne(hi))
            outs.append((ol, oh))
            width = np.maximum(width, oh - ol + 1)
        hull_lo = np.minimum(outs[0][0], outs[1][0])
        hull_hi = np.maximum(outs[0][1], outs[1][1])
        inside = (g >= hull_lo) & (g <= hull_hi)
        many = ordered(bf16_rne(hi_i)) - ordered(bf16_rne(lo_i)) > 1
        bad = np.nonzero(~inside)[0]
        rep.n += cols
        rep.outside += bad.size
        rep.two += int(((hull_hi - hull_lo) == 1).sum())
        rep.loose += int((width > 2).sum())
        rep.wide += int(many.sum())
        for j in bad[: max(0, 20 - len(rep.first_bad))]:
            rep.first_bad.append(int(base + j))
    return rep


# ------------------------------------------------------------------ q/k rows
#
# The fp32 run modelled for qk_rows_l2: the angle is the IEEE product (as the
# oracle forms it); cos and sin are within COSF_ULPS units in the last place
# of the float64 values of the fp32 angle; each of the four products and the
# two sums of the rotation rounds once; then the head's l2 over every
# admissible rotated value (as for the activation rows); then q's scale is
# one fp32 product rounded to bf16 -- a monotone map of the normalized value,
# so the admissible q outputs are the images of the admissible n range.

# COSF_ULPS: "cosf's ulps on the fp32 angle pos * inv" (TensorFold PR
# #1260, the q/k commit): the published maximum error of CUDA's fp32 cosf and
# sinf (and sincosf), 2 units in the last place over the full range (the same
# table).  gfx950's device library sincosf measured within 1.57 ulp, inside it.
COSF_ULPS = 2.0


def _trig_bounds(v):
    a = np.abs(v)
    ulp = np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 23)
    d = COSF_ULPS * ulp + ETA
    return v - d, v + d


def _mul_iv(x, lo, hi):
    """Bounds of fl(x * c) for exact x and c in [lo, hi]."""
    with np.errstate(all="ignore"):
        a, b = x * lo, x * hi
    return _outward(np.minimum(a, b), np.maximum(a, b))


def _l2_range(c_lo, c_hi, eps64, depth):
    """Ordered bf16 bounds of bf16(l2) over heads whose values lie in [c_lo, c_hi]."""
    sq_a, sq_b = c_lo ** 2, c_hi ** 2
    sq_lo = np.where((c_lo <= 0) & (c_hi >= 0), 0.0, np.minimum(sq_a, sq_b))
    s_lo, s_hi = _sum_bounds(sq_lo, np.maximum(sq_a, sq_b), depth)
    inv_lo, inv_hi = _inv_bounds(s_lo, s_hi, eps64)
    outs = []
    for c in (c_lo, c_hi):
        lo, hi = _product_bounds(c, c, inv_lo, inv_hi)
        outs.append((ordered(bf16_rne(lo)), ordered(bf16_rne(hi))))
    return np.minimum(outs[0][0], outs[1][0]), np.maximum(outs[0][1], outs[1][1])


def _ordered_to_bits(o):
    o = np.asarray(o, np.int64)
    return np.where(o < 0, 0x8000 | (-o), o).astype(np.uint16)


def admissible_qk_rows(got_q, got_k, q_bits, k_bits, positions, inv_freq, q_scale, head_dim,
                       eps: float = 1e-6, depth: Optional[int] = None):
    """Strict check of qk_rows_l2: (q Report, k Report, q unique mask, k unique mask).

    A unique element is one whose admissible output is a single bf16 value.
    Heads holding a non-finite input are compared with the oracle exactly.
    """
    from .rows import qk_rows_l2 as ref
    from .rows import rope_angles
    hd, h2 = head_dim, head_dim // 2
    depth = default_depth(hd) if depth is None else depth
    eps64 = eps_as_passed(eps)
    theta = rope_angles(positions, inv_freq)
    c_lo, c_hi = _trig_bounds(np.cos(theta))
    s_lo, s_hi = _trig_bounds(np.sin(theta))
    reps, masks = [], []
    for which, (got, x_bits) in enumerate(((got_q, q_bits), (got_k, k_bits))):
        rep = Report()
        if x_bits is None or not np.size(x_bits):
            reps.append(rep)
            masks.append(None)
            continue
        got = np.atleast_2d(got)
        x = bf16_value(np.atleast_2d(x_bits))
        rows, width = x.shape
        uniq = np.zeros((rows, width), bool)
        want_q, want_k = ref(q_bits, k_bits, positions, inv_freq, q_scale, hd, eps)
        want = want_q if which == 0 else want_k
        for i in range(rows):
            for h in range(width // hd):
                sl = slice(h * hd, (h + 1) * hd)
                base = i * width + h * hd
                xh = x[i, sl]
                if not np.isfinite(xh).all():
                    _judge(got[i, sl], xh, xh, want[i, sl], np.ones(hd, bool), True, base, rep)
                    continue
                x1, x2 = xh[:h2], xh[h2:]
                a1, b1 = _mul_iv(x1, c_lo[i], c_hi[i])
                a2, b2 = _mul_iv(x2, s_lo[i], s_hi[i])
                lo1, hi1 = _outward(a1 - b2, b1 - a2)              # x1 c - x2 s
                a3, b3 = _mul_iv(x2, c_lo[i], c_hi[i])
                a4, b4 = _mul_iv(x1, s_lo[i], s_hi[i])
                lo2, hi2 = _outward(a3 + a4, b3 + b4)              # x2 c + x1 s
                r_lo = bf16_value(bf16_rne(np.concatenate([lo1, lo2])))
                r_hi = bf16_value(bf16_rne(np.concatenate([hi1, hi2])))
                ol, oh = _l2_range(r_lo, r_hi, eps64, depth)
                if which == 0:
                    sc = np.asarray(q_scale, np.float32)[sl]
                    f = []
                    for o in (ol, oh):
                        nv = bf16_value(_ordered_to_bits(o)).astype(np.float32)
                        with np.errstate(all="ignore"):
                            f.append(ordered(bf16_rne((nv * sc).astype(np.float64))))
                    ol, oh = np.minimum(f[0], f[1]), np.maximum(f[0], f[1])
                g = ordered(got[i, sl])
                inside = (g >= ol) & (g <= oh)
                uniq[i, sl] = ol == oh
                bad = np.nonzero(~inside)[0]
                rep.n += hd
                rep.outside += bad.size
                rep.two += int(((oh - ol) == 1).sum())
                rep.wide += int(((oh - ol) > 1).sum())
                for j in bad[: max(0, 20 - len(rep.first_bad))]:
                    rep.first_bad.append(int(base + j))
        reps.append(rep)
        masks.append(uniq)
    return reps[0], reps[1], masks[0], masks[1]


# ------------------------------------------------------------ rescale method
#
# The projection v - w <w, v> / ||w||^2 cancels like a gradient (contract:
# 2e-6 relative plus GRAD_SLACK of its terms |v_j| + |w_j| sum|w v| / ||w||^2);
# the rescaled row w rho / ||w|| is within 2e-6 relative.  The fp32 run
# modelled: S, P as for the gradients; inv = 1/sqrt(S) (three roundings);
# k = fl(fl(P inv) inv); v_j = fl(v_j - fl(w_j k)); w_j = fl(w_j fl(rho inv)).

def rescale_terms(w: np.ndarray, v: np.ndarray) -> np.ndarray:
    out = np.zeros(w.shape)
    with np.errstate(all="ignore"):
        for i in range(w.shape[0]):
            ss = sum_sq(w[i])
            if ss == 0.0:
                continue
            a = math.fsum(np.abs(w[i] * v[i]))
            out[i] = np.abs(v[i]) + np.abs(w[i]) * (a / ss)
    return out


def admissible_rescale(got_w, got_v, w, v, rho: float = 1.0, after_step: bool = True,
                       depth: Optional[int] = None):
    """Strict check of one matrix: (w Report, v Report)."""
    from .rows import rescale_after_step as ref
    w64 = np.asarray(w, dtype=np.float64)
    v64 = None if v is None else np.asarray(v, dtype=np.float64)
    rho64 = float(np.float32(rho))
    rows, cols = w64.shape
    depth = default_depth(cols) if depth is None else depth
    gw = np.atleast_2d(np.asarray(got_w, np.float64))
    gv = None if got_v is None else np.atleast_2d(np.asarray(got_v, np.float64))
    rw, rv = Report(), Report()

    def mark(rep, bad, base):
        rep.n += bad.size
        idx = np.nonzero(bad)[0]
        rep.outside += idx.size
        for j in idx[: max(0, 20 - len(rep.first_bad))]:
            rep.first_bad.append(int(base + j))

    for i in range(rows):
        row = w64[i]
        base = i * cols
        vr = None if v64 is None else v64[i]
        if not (np.isfinite(row).all() and (vr is None or np.isfinite(vr).all())):
            ws, ms = ref([w[i:i + 1]], [None if v is None else v[i:i + 1]], [rho])
            exact_w = ws[0][0].astype(np.float64) if after_step else row
            if after_step:
                mark(rw, ~((gw[i] == exact_w) | (np.isnan(gw[i]) & np.isnan(exact_w))), base)
            if vr is not None:
                ev = ms[0][0].astype(np.float64)
                mark(rv, ~((gv[i] == ev) | (np.isnan(gv[i]) & np.isnan(ev))), base)
            continue
        sq = row ** 2
        s_lo, s_hi = _sum_bounds(sq, sq, depth)
        if s_hi == 0:                                   # a zero row stays as it is
            if after_step:
                mark(rw, gw[i] != row, base)
            if vr is not None:
                mark(rv, gv[i] != vr, base)
            continue
        inv_lo, inv_hi = _inv_bounds(s_lo, s_hi, 0.0)
        if after_step:
            c_lo, c_hi = _scalar(_corner_bounds([rho64], [rho64], inv_lo, inv_hi))
            lo, hi = _corner_bounds(row, row, c_lo, c_hi)
            mark(rw, ~_f32_inside(gw[i], lo, hi), base)
        if vr is not None:
            p_lo, p_hi = _mixed_sum_bounds(row * vr, depth)
            q = _scalar(_corner_bounds([p_lo], [p_hi], inv_lo, inv_hi))
            k_lo, k_hi = _scalar(_corner_bounds([q[0]], [q[1]], inv_lo, inv_hi))
            lo, hi = _tangent_bounds(row, vr, k_lo, k_hi, 1.0, 1.0)
            mark(rv, ~_f32_inside(gv[i], lo, hi), base)
    return rw, rv
