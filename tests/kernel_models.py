"""numpy float32 models of an fp32 row kernel, for testing the strict checker.

These emulate what an fp32 GPU run computes (fp32 sums of squares in a
64-lane layout, fp32 square root and reciprocal, bf16 rounding at the named
points).  The faithful model must pass the admissible-set check; each control
drops one rounding point or narrows the accumulator and must fail it --
TensorFold PR #1260's mutation controls (the sum before the norm, the slerp's
a, its b) and its fp16-sum control on integer rows.  Test code only.
"""
import numpy as np

from oracle.bf16 import bf16_rne, bf16_value


def bf16_of_f32(v32):
    return bf16_value(bf16_rne(np.asarray(v32, np.float32).astype(np.float64))).astype(np.float32)


def lane_sum_sq(s32, acc="f32"):
    """Row sums of squares: 64 lane accumulators, then a pairwise tree."""
    return lane_sum((s32 * s32).astype(np.float32), acc)


def lane_sum(sq, acc="f32"):
    """Row sums of fp32 terms: 64 lane accumulators, then a pairwise tree."""
    rows, cols = sq.shape
    pad = (-cols) % 64
    sq = np.concatenate([sq.astype(np.float32), np.zeros((rows, pad), np.float32)], axis=1)
    if acc == "f16":
        a = np.zeros((rows, 64), np.float16)
        with np.errstate(over="ignore"):
            for c in range(0, sq.shape[1], 64):
                a = (a + sq[:, c:c + 64].astype(np.float16)).astype(np.float16)
            while a.shape[1] > 1:
                a = (a[:, 0::2] + a[:, 1::2]).astype(np.float16)
        return a[:, 0].astype(np.float32)
    a = np.zeros((rows, 64), np.float32)
    for c in range(0, sq.shape[1], 64):
        a = a + sq[:, c:c + 64]
        if acc == "bf16":
            a = bf16_of_f32(a)
    while a.shape[1] > 1:
        a = a[:, 0::2] + a[:, 1::2]
        if acc == "bf16":
            a = bf16_of_f32(a)
    return a[:, 0]


def inv_norm(S32, eps):
    with np.errstate(all="ignore"):
        return np.float32(1.0) / np.sqrt((S32 + np.float32(eps)).astype(np.float32))


def l2_model(x_bits, r_bits=None, eps=1e-6, round_s=True, acc="f32", mean=False,
             eps_on_sum=False):
    """l2_rows, or rms_rows with mean=True (S / n in fp32 before eps); the
    eps_on_sum control adds eps to the sum before dividing by n."""
    x = bf16_value(x_bits).astype(np.float32)
    s = x if r_bits is None else x + bf16_value(r_bits).astype(np.float32)
    if r_bits is not None and round_s:
        s = bf16_of_f32(s)
    S = lane_sum_sq(s, acc)
    if mean:
        n = np.float32(s.shape[1])
        if eps_on_sum:
            S, eps = (S + np.float32(eps)).astype(np.float32) / n, 0.0
        else:
            S = (S / n).astype(np.float32)
    inv = inv_norm(S, eps)
    return bf16_rne((s * inv[:, None]).astype(np.float64))


def slerp_model(res_bits, out_bits, alpha, eps=1e-6, round_a=True, round_b=True):
    res = bf16_value(res_bits).astype(np.float32)
    out = bf16_value(out_bits).astype(np.float32)
    a = res * inv_norm(lane_sum_sq(res), eps)[:, None]
    b = out * inv_norm(lane_sum_sq(out), eps)[:, None]
    if round_a:
        a = bf16_of_f32(a)
    if round_b:
        b = bf16_of_f32(b)
    d = b - a
    t = np.abs(alpha.astype(np.float32)) * d
    u = a + t
    inv = inv_norm(lane_sum_sq(u), eps)
    return bf16_rne((u * inv[:, None]).astype(np.float64))


def rownorm_model(w, g, rho=1.0):
    w32 = np.asarray(w, np.float32)
    S = lane_sum_sq(w32)
    n = np.sqrt(S).astype(np.float32)
    with np.errstate(all="ignore"):
        c = np.where(n > 0, (np.asarray(g, np.float32) * np.float32(rho)) / n, np.float32(0))
    return n, bf16_rne((w32 * c[:, None].astype(np.float32)).astype(np.float64))


# ------------------------------------------------------------------ backward

def l2_backward_model(x_bits, r_bits, dy_bits, eps=1e-6, round_s=True, acc="f32",
                      proj="s", use_eps=True, mean=False, k_mean=True):
    """ds = (dy - s k) inv, k = P inv inv; controls: an unrounded s, a narrow
    accumulator, the projection taken on the rounded output y (proj="y"),
    eps left out.  mean=True models the rms_rows gradient (S / n and P / n in
    fp32); its control k_mean=False leaves P undivided."""
    x = bf16_value(x_bits).astype(np.float32)
    s = x if r_bits is None else x + bf16_value(r_bits).astype(np.float32)
    if r_bits is not None and round_s:
        s = bf16_of_f32(s)
    dy = bf16_value(dy_bits).astype(np.float32)
    n = np.float32(s.shape[1])
    S = lane_sum_sq(s, acc)
    if mean:
        S = (S / n).astype(np.float32)
    inv = inv_norm(S, eps if use_eps else 0.0)[:, None]
    with np.errstate(all="ignore"):
        if proj == "y":
            y = bf16_of_f32(s * inv)
            py = lane_sum((y * dy).astype(np.float32), acc)[:, None]
            ds = (dy - y * py) * inv
        else:
            p = lane_sum((s * dy).astype(np.float32), acc)[:, None]
            if mean and k_mean:
                p = (p / n).astype(np.float32)
            k = (p * inv) * inv
            ds = (dy - s * k) * inv
    return bf16_rne(ds.astype(np.float32).astype(np.float64))


def rownorm_backward_model(w, g, rho, dwe_bits, acc="f32", proj="w"):
    """dW = c (dWe - w k), c = g rho inv, dg = rho P inv; controls: a narrow
    accumulator, the projection taken on bf16(W_eff / (g rho)) (proj="weff")."""
    w32 = np.asarray(w, np.float32)
    de = bf16_value(dwe_bits).astype(np.float32)
    g32 = np.asarray(g, np.float32)[:, None]
    r32 = np.float32(rho)
    with np.errstate(all="ignore"):
        inv = (np.float32(1) / np.sqrt(lane_sum_sq(w32, acc)))[:, None]
        if proj == "weff":
            wh = bf16_of_f32(w32 * inv)
            pw = lane_sum((wh * de).astype(np.float32), acc)[:, None]
            dg = r32 * pw
            dw = (g32 * r32) * inv * (de - wh * pw)
        else:
            p = lane_sum((w32 * de).astype(np.float32), acc)[:, None]
            dg = (r32 * p) * inv
            k = (p * inv) * inv
            dw = ((g32 * r32) * inv) * (de - w32 * k)
    zero = ~w32.any(axis=1)
    dw[zero] = 0
    dg[zero] = 0
    return dw.astype(np.float32), dg[:, 0].astype(np.float32)


# ------------------------------------------------------------ activation rows

def _l2_of_f32_rows(t32, eps, acc="f32"):
    with np.errstate(all="ignore"):
        inv = inv_norm(lane_sum_sq(t32, acc), eps)
        return bf16_rne((t32 * inv[:, None]).astype(np.float64))


def gate_model(o_bits, g_bits, sg, eps=1e-6, round_t=True, acc="f32"):
    """fp32 steps of the gate row; the control leaves the gated row unrounded
    (or, with acc="f16", sums its squares in fp16)."""
    o = bf16_value(o_bits).astype(np.float32)
    g = bf16_value(g_bits).astype(np.float32)
    with np.errstate(all="ignore"):
        x = g * np.asarray(sg, np.float32)
        sig = np.float32(1) / (np.float32(1) + np.exp(-x))
        t = o * sig
    if round_t:
        t = bf16_of_f32(t)
    return _l2_of_f32_rows(t.astype(np.float32), eps, acc)


def swiglu_model(g_bits, u_bits, sug, suu, eps=1e-6, round_a=True, round_b=True, round_p=True,
                 acc="f32"):
    """fp32 steps of the SwiGLU row; each control leaves one rounding point out
    (or, with acc="f16", sums the squares in fp16)."""
    g = bf16_value(g_bits).astype(np.float32)
    u = bf16_value(u_bits).astype(np.float32)
    with np.errstate(all="ignore"):
        a = g * np.asarray(sug, np.float32)
        b = u * np.asarray(suu, np.float32)
        if round_a:
            a = bf16_of_f32(a)
        if round_b:
            b = bf16_of_f32(b)
        silu = a / (np.float32(1) + np.exp(-a))
        p = silu * b
    if round_p:
        p = bf16_of_f32(p)
    return _l2_of_f32_rows(p.astype(np.float32), eps, acc)


# ------------------------------------------------------------------ q/k rows

def qk_model(q_bits, k_bits, positions, inv_freq, q_scale, hd, eps=1e-6,
             round_r=True, round_n=True, acc="f32"):
    """fp32 steps of qk_rows_l2; the controls leave the rotated head or the
    normalized head unrounded, or (acc="f16") sum each head's squares in fp16."""
    th = (np.asarray(positions).astype(np.float32)[:, None]
          * np.asarray(inv_freq, np.float32)[None, :]).astype(np.float32)
    c, s = np.cos(th)[:, None, :], np.sin(th)[:, None, :]

    def heads(x_bits):
        x = bf16_value(x_bits).astype(np.float32)
        rows, width = x.shape
        xh = x.reshape(rows, width // hd, hd)
        x1, x2 = xh[..., :hd // 2], xh[..., hd // 2:]
        rot = np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1).astype(np.float32)
        r = bf16_of_f32(rot) if round_r else rot
        r2 = r.reshape(-1, hd)
        with np.errstate(all="ignore"):
            inv = inv_norm(lane_sum_sq(r2, acc), eps)
            n = (r2 * inv[:, None]).astype(np.float32)
        if round_n:
            n = bf16_of_f32(n)
        return n.reshape(rows, width)

    nq = heads(q_bits)
    q_out = bf16_rne((nq * np.asarray(q_scale, np.float32)).astype(np.float32).astype(np.float64))
    k_out = bf16_rne(heads(k_bits).astype(np.float64)) if k_bits is not None else None
    return q_out, k_out


# ------------------------------------------------------------ rescale method

def rescale_model(w, v, rho=1.0, after_step=True, k_over_norm=False, project=True):
    """fp32 steps of the rescale row ops; controls: k = P/||w|| instead of
    P/||w||^2, and no projection at all."""
    w32 = np.asarray(w, np.float32)
    v32 = None if v is None else np.asarray(v, np.float32)
    with np.errstate(all="ignore"):
        S = lane_sum_sq(w32)
        inv = (np.float32(1) / np.sqrt(S)).astype(np.float32)[:, None]
        zero = (S == 0)[:, None]
        v_out = None
        if v32 is not None:
            P = lane_sum((w32 * v32).astype(np.float32))[:, None]
            k = (P * inv) if k_over_norm else (P * inv) * inv
            v_out = np.where(zero | (not project), v32, v32 - w32 * k).astype(np.float32)
        w_out = np.where(zero, w32, w32 * (np.float32(rho) * inv)).astype(np.float32) if after_step else w32
    return w_out, v_out
