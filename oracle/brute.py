"""Exact-arithmetic versions of the row ops, for tiny rows.

TEST INFRASTRUCTURE (see the package docstring).  Independent of
:mod:`oracle.rows` and :mod:`oracle.bf16`: inputs become exact rationals
(``fractions.Fraction``), sums of squares are exact, square roots and
quotients are carried in 60-digit ``decimal`` arithmetic, and rounding to
bf16 / fp32 is done on the exact rational by integer arithmetic.  Each result
comes with a flag that marks values lying so close to a rounding midpoint that
60 digits, or float64's rounding in the fast oracle, could decide either way.

Definitions followed: TensorFold PR #1260 (the l2 and slerp row kernels; the
lerp in fp32 steps) and the DragonScale README's W_eff formula ("What
DragonScale changes").
"""
from __future__ import annotations

import struct
from decimal import Decimal, localcontext
from fractions import Fraction
from typing import List, Optional, Sequence, Tuple

__all__ = ["bits_to_fraction", "round_fraction", "bf16_of", "fp32_of",
           "l2_row", "slerp_row", "rownorm_row", "l2_backward_row", "rownorm_backward_row",
           "gate_row", "swiglu_row", "qk_head", "rescale_row", "rms_row", "rms_backward_row",
           "NEAR_TIE_REL"]

PREC = 60
NEAR_TIE_REL = Fraction(1, 10 ** 12)     # flag values this close to a midpoint


def bits_to_fraction(bits: int, width: int = 16) -> Optional[Fraction]:
    """Exact value of a bf16 (width 16) or fp32 (width 32) bit pattern."""
    if width == 16:
        bits = bits << 16
    sign = -1 if bits >> 31 else 1
    exp = (bits >> 23) & 0xFF
    man = bits & 0x7FFFFF
    if exp == 0xFF:
        return None                                  # inf / nan: not used here
    if exp == 0:
        return sign * Fraction(man, 1 << 149)
    return sign * Fraction((1 << 23) | man, 1) * Fraction(2) ** (exp - 150)


def f32_to_fraction(x: float) -> Fraction:
    (b,) = struct.unpack("<I", struct.pack("<f", x))
    return bits_to_fraction(b, 32)


def _binade(a: Fraction) -> int:
    """floor(log2(a)) for a > 0, by integer arithmetic."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if a < Fraction(2) ** e:
        e -= 1
    return e


def round_fraction(v: Fraction, sig_bits: int, emin: int, emax: int
                   ) -> Tuple[Fraction, bool]:
    """Round exact v to a binary format (nearest, ties to even).

    sig_bits counts the leading bit; emin is the smallest normal exponent.
    Returns (rounded value or +-inf as None-free Fraction sentinel, near_tie),
    where near_tie says v is within NEAR_TIE_REL (relative) of a midpoint.
    Overflow returns Fraction(+-2**(emax+1)) so callers can test for it.
    """
    if v == 0:
        return Fraction(0), False
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = max(_binade(a), emin)
    q = Fraction(2) ** (e - sig_bits + 1)
    m = a / q
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    near = abs(rem - Fraction(1, 2)) * q <= NEAR_TIE_REL * a
    r = fl * q
    if r >= Fraction(2) ** (emax + 1):
        r = Fraction(2) ** (emax + 1)               # overflow marker
    return sign * r, near


def bf16_of(v: Fraction) -> Tuple[Fraction, bool]:
    return round_fraction(v, 8, -126, 127)


def fp32_of(v: Fraction) -> Tuple[Fraction, bool]:
    return round_fraction(v, 24, -126, 127)


def _dec(f: Fraction) -> Decimal:
    return Decimal(f.numerator) / Decimal(f.denominator)


def _l2_exact(s: Sequence[Fraction], eps: Fraction) -> Tuple[List[Fraction], List[bool]]:
    """bf16(s_j / sqrt(sum s^2 + eps)) for every j, with near-tie flags."""
    with localcontext() as ctx:
        ctx.prec = PREC
        total = sum((x * x for x in s), Fraction(0)) + eps
        root = _dec(total).sqrt()
        out, near = [], []
        for x in s:
            q = Fraction(_dec(x) / root)
            r, n = bf16_of(q)
            out.append(r)
            near.append(n)
    return out, near


def l2_row(x_bits: Sequence[int], r_bits: Optional[Sequence[int]], eps32: float
           ) -> Tuple[List[Fraction], List[bool]]:
    """One row of l2_rows, exactly: s = x or bf16(x + r), then the normalised row."""
    x = [bits_to_fraction(int(b)) for b in x_bits]
    if r_bits is not None:
        # x + r is exact here, so its rounding is exact too (a tie is a tie)
        s = [bf16_of(xj + bits_to_fraction(int(rb)))[0] for xj, rb in zip(x, r_bits)]
    else:
        s = x
    return _l2_exact(s, f32_to_fraction(eps32))


def slerp_row(res_bits: Sequence[int], out_bits: Sequence[int],
              alpha: Sequence[float], eps32: float) -> Tuple[List[Fraction], bool]:
    """One row of slerp_rows, exactly; the flag covers the whole row.

    a, b are exact bf16 roundings of the exact l2 rows; the lerp is three
    binary32 roundings (b - a, |alpha| * that, a + that); h is the exact bf16
    rounding of the exact l2 of u.  The lerp's operands are exact, so its
    roundings are exact; a near-tie in a, b or h (values carried through a
    60-digit square root) flags the row.
    """
    eps = f32_to_fraction(eps32)
    res = [bits_to_fraction(int(b)) for b in res_bits]
    out = [bits_to_fraction(int(b)) for b in out_bits]
    a, na = _l2_exact(res, eps)
    b, nb = _l2_exact(out, eps)
    u = []
    near = any(na) or any(nb)
    for aj, bj, al in zip(a, b, alpha):
        d = fp32_of(bj - aj)[0]
        t = fp32_of(abs(f32_to_fraction(float(al))) * d)[0]
        u.append(fp32_of(aj + t)[0])
    h, nh = _l2_exact(u, eps)
    return h, near or any(nh)


def rownorm_row(w: Sequence[float], g: float, rho: float
                ) -> Tuple[Fraction, List[Fraction], bool]:
    """One weight row exactly: fp32(||w||) and bf16(g rho w / ||w||), with a flag."""
    wf = [f32_to_fraction(x) for x in w]
    gf = f32_to_fraction(g) * f32_to_fraction(rho)
    with localcontext() as ctx:
        ctx.prec = PREC
        total = sum((x * x for x in wf), Fraction(0))
        if total == 0:
            return Fraction(0), [Fraction(0)] * len(wf), False
        root = _dec(total).sqrt()
        n32, near = fp32_of(Fraction(root))
        out = []
        for x in wf:
            r, n = bf16_of(Fraction(_dec(gf * x) / root))
            out.append(r)
            near = near or n
    return n32, out, near


# The float64 oracle forms each gradient element as a difference of two terms
# that may cancel; its error is then a few float64 units of the terms, not of
# the result.  An element is flagged when rounding cannot be decided within
# SLACK_REL times the size of those terms.
SLACK_REL = Fraction(1, 2 ** 48)


def _round_with_slack(v: Fraction, slack: Fraction, fmt) -> Tuple[Fraction, bool]:
    r, near = fmt(v)
    if slack > 0 and (fmt(v - slack)[0] != r or fmt(v + slack)[0] != r):
        near = True
    return r, near


def l2_backward_row(x_bits: Sequence[int], r_bits: Optional[Sequence[int]],
                    dy_bits: Sequence[int], eps32: float) -> Tuple[List[Fraction], List[bool]]:
    """One row of the l2_rows gradient, exactly: bf16((dy - s <s, dy> / D^2) / D)."""
    x = [bits_to_fraction(int(b)) for b in x_bits]
    if r_bits is not None:
        s = [bf16_of(xj + bits_to_fraction(int(rb)))[0] for xj, rb in zip(x, r_bits)]
    else:
        s = x
    dy = [bits_to_fraction(int(b)) for b in dy_bits]
    eps = f32_to_fraction(eps32)
    with localcontext() as ctx:
        ctx.prec = PREC
        d2 = sum((v * v for v in s), Fraction(0)) + eps
        p = sum((a * b for a, b in zip(s, dy)), Fraction(0))
        pa = sum((abs(a * b) for a, b in zip(s, dy)), Fraction(0))
        root = _dec(d2).sqrt()
        out, near = [], []
        for sj, gj in zip(s, dy):
            num = gj - sj * p / d2                  # exact
            terms = abs(gj) + abs(sj) * pa / d2
            v, n = _round_with_slack(Fraction(_dec(num) / root),
                                     SLACK_REL * Fraction(_dec(terms) / root), bf16_of)
            out.append(v)
            near.append(n)
    return out, near


def rownorm_backward_row(w: Sequence[float], g: float, rho: float, dwe_bits: Sequence[int]
                         ) -> Tuple[List[Fraction], Fraction, List[bool], bool]:
    """One weight row's gradients exactly: fp32(dW) with per-element flags, fp32(dg), flag."""
    wf = [f32_to_fraction(float(x)) for x in w]
    de = [bits_to_fraction(int(b)) for b in dwe_bits]
    grho = f32_to_fraction(g) * f32_to_fraction(rho)
    rho_f = f32_to_fraction(rho)
    with localcontext() as ctx:
        ctx.prec = PREC
        ss = sum((v * v for v in wf), Fraction(0))
        if ss == 0:
            return [Fraction(0)] * len(wf), Fraction(0), [False] * len(wf), False
        p = sum((a * b for a, b in zip(wf, de)), Fraction(0))
        pa = sum((abs(a * b) for a, b in zip(wf, de)), Fraction(0))
        root = _dec(ss).sqrt()
        dg, near_g = fp32_of(Fraction(_dec(rho_f * p) / root))
        out, near = [], []
        for wj, ej in zip(wf, de):
            num = grho * (ej - wj * p / ss)          # exact
            terms = abs(grho) * (abs(ej) + abs(wj) * pa / ss)
            v, n = _round_with_slack(Fraction(_dec(num) / root),
                                     SLACK_REL * Fraction(_dec(terms) / root), fp32_of)
            out.append(v)
            near.append(n)
    return out, dg, near, near_g


# ------------------------------------------------------- activation rows

def _sigmoid_exact(x: Fraction) -> Fraction:
    """1 / (1 + exp(-x)) at PREC digits (exp from the decimal module)."""
    with localcontext() as ctx:
        ctx.prec = PREC
        return Fraction(Decimal(1) / (Decimal(1) + (-_dec(x)).exp()))


def _fp32_product(v_bits: int, scale: float) -> Fraction:
    """The IEEE fp32 product of a bf16 value and an fp32 scale, exactly."""
    return fp32_of(bits_to_fraction(int(v_bits)) * f32_to_fraction(float(scale)))[0]


def gate_row(o_bits: Sequence[int], g_bits: Sequence[int], sg: Sequence[float], eps32: float
             ) -> Tuple[List[Fraction], List[bool]]:
    """bf16(l2(bf16(o * sigmoid(fp32(g * sg))))) exactly, with near-tie flags."""
    t, near_t = [], []
    for ob, gb, sc in zip(o_bits, g_bits, sg):
        x = _fp32_product(gb, sc)
        v, n = bf16_of(bits_to_fraction(int(ob)) * _sigmoid_exact(x))
        t.append(v)
        near_t.append(n)
    y, near = _l2_exact(t, f32_to_fraction(eps32))
    return y, [a or any(near_t) for a in near]


def swiglu_row(g_bits: Sequence[int], u_bits: Sequence[int], sug: Sequence[float],
               suu: Sequence[float], eps32: float) -> Tuple[List[Fraction], List[bool]]:
    """bf16(l2(bf16(silu(a) * b))), a = bf16(fp32(g sug)), b = bf16(fp32(u suu)), exactly."""
    p, near_p = [], []
    for gb, ub, s1, s2 in zip(g_bits, u_bits, sug, suu):
        a = bf16_of(_fp32_product(gb, s1))[0]
        b = bf16_of(_fp32_product(ub, s2))[0]
        v, n = bf16_of(a * _sigmoid_exact(a) * b)
        p.append(v)
        near_p.append(n)
    y, near = _l2_exact(p, f32_to_fraction(eps32))
    return y, [a or any(near_p) for a in near]


# ------------------------------------------------------------------ q/k rows

def qk_head(x_bits: Sequence[int], pos: int, inv_freq: Sequence[float], scale: Sequence[float],
            eps32: float) -> Tuple[List[Fraction], List[Fraction], bool]:
    """One head exactly: (normalized head n, bf16(fp32(n * scale)), near-tie flag).

    The angle is the IEEE fp32 product fp32(pos) * inv_i; cos and sin of it at
    50 digits (mpmath); rotation, sum and quotient exact or at 60 digits.
    """
    import mpmath
    hd = len(x_bits)
    h2 = hd // 2
    x = [bits_to_fraction(int(b)) for b in x_bits]
    p32 = fp32_of(Fraction(int(pos)))[0]
    near = False
    r = [Fraction(0)] * hd
    with mpmath.workdps(50):
        for i in range(h2):
            th = fp32_of(p32 * f32_to_fraction(float(inv_freq[i])))[0]
            t = mpmath.mpf(th.numerator) / th.denominator
            c = Fraction(mpmath.nstr(mpmath.cos(t), 48, min_fixed=-1, max_fixed=1))
            s = Fraction(mpmath.nstr(mpmath.sin(t), 48, min_fixed=-1, max_fixed=1))
            v1, n1 = bf16_of(x[i] * c - x[i + h2] * s)
            v2, n2 = bf16_of(x[i + h2] * c + x[i] * s)
            r[i], r[i + h2] = v1, v2
            near = near or n1 or n2
    n, nn = _l2_exact(r, f32_to_fraction(eps32))
    near = near or any(nn)
    out = []
    for v, sc in zip(n, scale):
        o, f = bf16_of(fp32_of(v * f32_to_fraction(float(sc)))[0])
        out.append(o)
        near = near or f
    return n, out, near


# ------------------------------------------------------------ rescale method

def rescale_row(w: Sequence[float], v: Optional[Sequence[float]], rho: float
                ) -> Tuple[List[Fraction], Optional[List[Fraction]], List[bool]]:
    """One row exactly: (fp32(rho w/||w||), fp32(v - w <w,v>/||w||^2) or None, flags).

    Flags mark elements whose projection float64 cannot round within
    SLACK_REL of its cancelling terms, or whose rescaled value is near a tie.
    """
    wf = [f32_to_fraction(float(x)) for x in w]
    ss = sum((x * x for x in wf), Fraction(0))
    if ss == 0:
        return wf, None if v is None else [f32_to_fraction(float(x)) for x in v], [False] * len(wf)
    near = [False] * len(wf)
    with localcontext() as ctx:
        ctx.prec = PREC
        root = _dec(ss).sqrt()
        rf = f32_to_fraction(float(rho))
        w_out = []
        for j, x in enumerate(wf):
            r, n = fp32_of(Fraction(_dec(rf * x) / root))
            w_out.append(r)
            near[j] = near[j] or n
    v_out = None
    if v is not None:
        vf = [f32_to_fraction(float(x)) for x in v]
        p = sum((a * b for a, b in zip(wf, vf)), Fraction(0))
        pa = sum((abs(a * b) for a, b in zip(wf, vf)), Fraction(0))
        v_out = []
        for j, (x, y) in enumerate(zip(wf, vf)):
            r, n = _round_with_slack(y - x * p / ss, SLACK_REL * (abs(y) + abs(x) * pa / ss), fp32_of)
            v_out.append(r)
            near[j] = near[j] or n
    return w_out, v_out, near


# ------------------------------------------------------------------ RMSNorm
# The ternary/8-bit GPT model page's parameter-free rms_norm: y = s / sqrt(
# sum(s^2) / n + eps), n the row's length, rounded once to bf16.

def _s_exact(x_bits, r_bits):
    x = [bits_to_fraction(int(b)) for b in x_bits]
    if r_bits is None:
        return x
    return [bf16_of(xj + bits_to_fraction(int(rb)))[0] for xj, rb in zip(x, r_bits)]


def rms_row(x_bits: Sequence[int], r_bits: Optional[Sequence[int]], eps32: float
            ) -> Tuple[List[Fraction], List[bool]]:
    """One row of rms_rows, exactly, with near-tie flags."""
    s = _s_exact(x_bits, r_bits)
    n = len(s)
    eps = f32_to_fraction(eps32)
    with localcontext() as ctx:
        ctx.prec = PREC
        ms = sum((v * v for v in s), Fraction(0)) / n + eps
        root = _dec(ms).sqrt()
        out, near = [], []
        for v in s:
            r, fl = bf16_of(Fraction(_dec(v) / root))
            out.append(r)
            near.append(fl)
    return out, near


def rms_backward_row(x_bits: Sequence[int], r_bits: Optional[Sequence[int]],
                     dy_bits: Sequence[int], eps32: float) -> Tuple[List[Fraction], List[bool]]:
    """One row of the rms_rows gradient, exactly: bf16((dy - s <s,dy> / (n D^2)) / D)."""
    s = _s_exact(x_bits, r_bits)
    n = len(s)
    dy = [bits_to_fraction(int(b)) for b in dy_bits]
    eps = f32_to_fraction(eps32)
    with localcontext() as ctx:
        ctx.prec = PREC
        nd2 = sum((v * v for v in s), Fraction(0)) + n * eps        # n D^2, exact
        p = sum((a * b for a, b in zip(s, dy)), Fraction(0))
        pa = sum((abs(a * b) for a, b in zip(s, dy)), Fraction(0))
        root = _dec(nd2 / n).sqrt()
        out, near = [], []
        for sj, gj in zip(s, dy):
            num = gj - sj * p / nd2
            terms = abs(gj) + abs(sj) * pa / nd2
            v, fl = _round_with_slack(Fraction(_dec(num) / root),
                                      SLACK_REL * Fraction(_dec(terms) / root), bf16_of)
            out.append(v)
            near.append(fl)
    return out, near
