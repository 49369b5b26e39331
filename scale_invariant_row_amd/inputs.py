"""Seeded synthetic workloads for the row ops.

This module draws random numbers and lays out the workloads; it holds none of
the row ops' arithmetic.  Every value is fixed here once, as bit patterns
(bf16 activations as ``uint16``, fp32 weights/gains/scales as ``float32``), and
the same arrays feed the CPU oracle and the GPU library.

Recipe (shared by every workload):

* ``numpy.random.Generator(PCG64(SeedSequence(seed)))``; one child stream per
  tensor, spawned in a fixed order (``SeedSequence.spawn``).
* Activations: float64 samples, cast to float32 by numpy, then to bf16 by
  torch's own round-to-nearest-even conversion.  The cast only decides what the
  input values are.
* Weights and gains: float64 samples cast to float32 by numpy (round to
  nearest even).

Workloads (widths follow the pages: activation rows 1,024-8,192 wide and the
7,168-wide MLP row of the looped nGPT model in the TensorFold Dory PR; weights
are the linears of a 12-layer pre-norm transformer, d=768, d_ff=3072, as in the
DragonScale README's unit-row op):

========================  =======================================================
name                      contents
========================  =======================================================
l2_rows_64x1024           x ~ N(0,1), no residual, eps 1e-6
l2_rows_res_8192x4096     x, r ~ N(0,1) independent, eps 1e-6
slerp_rows_8192x7168      res ~ N(0,1), out ~ N(0, sd 2), alpha ~ U(-0.2, 0.2)
rownorm_gain_12x4_d768    12 x {qkv 2304x768, o 768x768, up 3072x768,
                          down 768x3072}; W ~ N(0, sd 0.02); g ~ U(0.5, 2); rho 1
l2_rows_res_stress        32768x8192: x ~ N(0,1), 1% of entries x1000; 327 rows
                          all-zero in x and r; 327 rows of integers in [-64, 64]
                          with r = 0; r ~ N(0,1) elsewhere
slerp_rows_8192x4096      as slerp_rows_8192x7168 at width 4096
l2_rows_res_bwd_8192x4096 x, r as l2_rows_res_8192x4096; upstream dy ~ N(0,1)
rownorm_gain_bwd_12x4     rownorm_gain_12x4_d768's matrices; dL/dW_eff ~ N(0,1)
rownorm_gain_bwd_11008x   one 11008x4096 matrix (the DragonScale README's
4096                      kernel-speed shape), W ~ N(0, sd 0.02), g ~ U(0.5, 2),
                          dL/dW_eff ~ N(0,1)
qk_rows_l2_8192_h16x4     8192 token rows, head_dim 256, 16 q heads, 4 kv heads:
_d256                     q, k ~ N(0,1) bf16; positions 0.. for two thirds of
                          the rows and 199,800.. for the last third; inv_freq =
                          10000^(-2i/256) in fp32; q_scale ~ U(0.5, 2) fp32
gate_l2_rows_8192x4096    o, g ~ N(0,1) bf16; sg ~ U(0.5, 2) fp32 per column
swiglu_l2_rows_8192x7168  g, u ~ N(0,1) bf16; sug, suu ~ U(0.5, 2) fp32 per column
rescale_12x4_d768         the 48 linears of rownorm_gain_12x4_d768 as raw rows,
                          W ~ N(0, sd 0.02) fp32, gradients / momenta
                          ~ N(0, sd 1e-3) fp32, radius 1
rownorm_gain_resnet50     ResNet-50's 53 convolutions and classifier as unit rows
                          (out channels x in * kh * kw; the stem's 147 is not
                          a multiple of 4); W ~ N(0, sd 0.02); g ~ U(0.5, 2)
rownorm_gain_bwd_resnet50 the same matrices; dL/dW_eff ~ N(0,1)
rownorm_gain_embedding    a 50304 x 768 vocabulary embedding, radius sqrt(768)
_50304x768                (the DragonScale README's radius for embeddings)
rownorm_gain_gpt2_conv1d  GPT-2 small's 48 Conv1D weights stored [in, out]
                          (c_attn 768x2304, c_proj 768x768, c_fc 768x3072,
                          mlp c_proj 3072x768), units = columns; W ~ N(0, sd
                          0.02), g ~ U(0.5, 2) per unit, dL/dW_eff ~ N(0,1)
rms_rows_bwd_16384x768    RMSNorm rows of the GPT model page's 100m size
                          (d_model 768) over 8 sequences of 2,048 tokens:
                          x ~ N(0,1), no residual; upstream dy ~ N(0,1)
========================  =======================================================

Upstream gradients (dy, dL/dW_eff) are bf16 values drawn like activations.
The activation rows' widths are the Dory rows the TensorFold PR names (4,096
over all heads, 7,168 for the MLP).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

__all__ = [
    "L2Case", "SlerpCase", "RownormCase",
    "to_bf16_bits", "l2_case", "slerp_case", "rownorm_case",
    "transformer_linears", "stress_l2_case", "WORKLOADS", "make",
    "L2GradCase", "RownormGradCase", "grad_bits", "l2_grad_case", "rownorm_grad_case",
    "ActCase", "gate_case", "swiglu_case", "QkCase", "qk_case", "rope_inv_freq",
    "RescaleCase", "rescale_case", "resnet50_convs", "gpt2_conv1d", "colblock_grad_case",
]


@dataclass
class L2Case:
    """Inputs of ``l2_rows``: ``x`` and optional residual ``r`` as bf16 bits."""
    name: str
    x: np.ndarray                     # uint16 [rows, cols]
    r: Optional[np.ndarray]           # uint16 [rows, cols] or None
    eps: float = 1e-6
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.x.shape[0]

    @property
    def cols(self) -> int:
        return self.x.shape[1]


@dataclass
class SlerpCase:
    """Inputs of ``slerp_rows``: ``res``, ``out`` (bf16 bits), ``alpha`` (fp32)."""
    name: str
    res: np.ndarray                   # uint16 [rows, cols]
    out: np.ndarray                   # uint16 [rows, cols]
    alpha: np.ndarray                 # float32 [cols]
    eps: float = 1e-6

    @property
    def rows(self) -> int:
        return self.res.shape[0]

    @property
    def cols(self) -> int:
        return self.res.shape[1]


@dataclass
class RownormCase:
    """Inputs of ``weight_rownorm_gain``: a ragged list of fp32 matrices."""
    name: str
    w: List[np.ndarray]               # float32 [rows_m, cols_m] each
    gain: List[np.ndarray]            # float32 [rows_m] each
    radius: List[float]

    @property
    def total_rows(self) -> int:
        return sum(m.shape[0] for m in self.w)

    @property
    def total_elems(self) -> int:
        return sum(m.size for m in self.w)


@dataclass
class L2GradCase:
    """Inputs of the l2_rows gradient: the forward's x, r and the upstream dy."""
    name: str
    x: np.ndarray                     # uint16 [rows, cols]
    r: Optional[np.ndarray]
    dy: np.ndarray                    # uint16 [rows, cols]
    eps: float = 1e-6
    meta: dict = field(default_factory=dict)


@dataclass
class RownormGradCase:
    """Inputs of the weight gradient: the forward's matrices and dL/dW_eff."""
    name: str
    w: List[np.ndarray]
    gain: List[np.ndarray]
    radius: List[float]
    dwe: List[np.ndarray]             # uint16 bf16 bits, shaped like w

    @property
    def total_rows(self) -> int:
        return sum(m.shape[0] for m in self.w)

    @property
    def total_elems(self) -> int:
        return sum(m.size for m in self.w)


@dataclass
class ActCase:
    """Inputs of an activation row: two bf16 rows and one or two fp32 column scales
    (gate: a = o, b = g, s0 = sg; SwiGLU: a = g, b = u, s0 = sug, s1 = suu)."""
    name: str
    a: np.ndarray
    b: np.ndarray
    s0: np.ndarray
    s1: Optional[np.ndarray]
    eps: float = 1e-6


@dataclass
class QkCase:
    """Inputs of qk_rows_l2: q and k rows (heads concatenated), positions,
    the fp32 inverse frequencies and q's fp32 scale vector."""
    name: str
    q: np.ndarray                     # uint16 [rows, nq * hd]
    k: Optional[np.ndarray]           # uint16 [rows, nk * hd]
    pos: np.ndarray                   # int32 [rows]
    inv_freq: np.ndarray              # float32 [hd / 2]
    q_scale: np.ndarray               # float32 [nq * hd]
    head_dim: int
    eps: float = 1e-6


@dataclass
class RescaleCase:
    """Inputs of the rescale method's row ops: raw rows and, per matrix, a
    gradient or momentum of the same shape."""
    name: str
    w: List[np.ndarray]
    v: List[np.ndarray]
    radius: List[float]


def _streams(seed: int, n: int) -> List[np.random.Generator]:
    children = np.random.SeedSequence(seed).spawn(n)
    return [np.random.Generator(np.random.PCG64(c)) for c in children]


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float64/float32 samples -> bf16 bit patterns (uint16), via torch's cast."""
    import torch
    f32 = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    t = torch.from_numpy(f32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def l2_case(rows: int, cols: int, seed: int, residual: bool = True,
            eps: float = 1e-6, name: Optional[str] = None) -> L2Case:
    gx, gr = _streams(seed, 2)
    x = to_bf16_bits(gx.standard_normal((rows, cols)))
    r = to_bf16_bits(gr.standard_normal((rows, cols))) if residual else None
    return L2Case(name or f"l2_rows{'_res' if residual else ''}_{rows}x{cols}", x, r, eps)


def slerp_case(rows: int, cols: int, seed: int, eps: float = 1e-6,
               out_sd: float = 2.0, alpha_lim: float = 0.2,
               name: Optional[str] = None) -> SlerpCase:
    gres, gout, galpha = _streams(seed, 3)
    res = to_bf16_bits(gres.standard_normal((rows, cols)))
    out = to_bf16_bits(out_sd * gout.standard_normal((rows, cols)))
    alpha = galpha.uniform(-alpha_lim, alpha_lim, cols).astype(np.float32)
    return SlerpCase(name or f"slerp_rows_{rows}x{cols}", res, out, alpha, eps)


def transformer_linears(layers: int = 12, d: int = 768, d_ff: int = 3072):
    """(rows, cols) of each linear, layer-major: qkv, o, up, down."""
    shapes = []
    for _ in range(layers):
        shapes += [(3 * d, d), (d, d), (d_ff, d), (d, d_ff)]
    return shapes


def resnet50_convs():
    """(out channels, in * kh * kw) of ResNet-50's 53 convolutions, then its
    1000 x 2048 classifier: the rows of a convolutional network's weights
    (the stem's 3 x 7 x 7 = 147 is a width that is not a multiple of 4)."""
    shapes = [(64, 3 * 49)]
    cin = 64
    for blocks, width in ((3, 64), (4, 128), (6, 256), (3, 512)):
        out = 4 * width
        for b in range(blocks):
            shapes += [(width, cin), (width, width * 9), (out, width)]
            if b == 0:
                shapes.append((out, cin))                 # the projection shortcut
            cin = out
    shapes.append((1000, 2048))
    return shapes


def gpt2_conv1d(layers: int = 12, d: int = 768):
    """Stored shapes [in, out] of GPT-2's Conv1D weights, layer-major: c_attn,
    attn c_proj, mlp c_fc, mlp c_proj.  Each output unit is a column."""
    shapes = []
    for _ in range(layers):
        shapes += [(d, 3 * d), (d, d), (d, 4 * d), (4 * d, d)]
    return shapes


def colblock_grad_case(stored_shapes, seg: int, seed: int, w_sd: float = 0.02,
                       g_lo: float = 0.5, g_hi: float = 2.0, radius: float = 1.0,
                       name: Optional[str] = None) -> "RownormGradCase":
    """Weights stored as column blocks ([A, ld], units = ld // seg): fp32 W, one
    gain per unit, a bf16 dL/dW_eff of the stored shape."""
    gens = _streams(seed, 3 * len(stored_shapes))
    ws, gs, des = [], [], []
    for i, (a, ld) in enumerate(stored_shapes):
        ws.append((w_sd * gens[3 * i].standard_normal((a, ld))).astype(np.float32))
        gs.append(gens[3 * i + 1].uniform(g_lo, g_hi, ld // seg).astype(np.float32))
        des.append(to_bf16_bits(gens[3 * i + 2].standard_normal((a, ld))))
    return RownormGradCase(name or f"colblock_{len(stored_shapes)}", ws, gs,
                           [float(radius)] * len(stored_shapes), des)


def rownorm_case(shapes, seed: int, w_sd: float = 0.02, g_lo: float = 0.5,
                 g_hi: float = 2.0, radius: float = 1.0,
                 name: Optional[str] = None) -> RownormCase:
    gens = _streams(seed, 2 * len(shapes))
    ws, gs = [], []
    for i, (rows, cols) in enumerate(shapes):
        gw, gg = gens[2 * i], gens[2 * i + 1]
        ws.append((w_sd * gw.standard_normal((rows, cols))).astype(np.float32))
        gs.append(gg.uniform(g_lo, g_hi, rows).astype(np.float32))
    return RownormCase(name or f"rownorm_gain_{len(shapes)}", ws, gs,
                       [float(radius)] * len(shapes))


def stress_l2_case(rows: int = 32768, cols: int = 8192, seed: int = 1005,
                   residual: bool = True, eps: float = 1e-6,
                   outlier_p: float = 0.01, outlier_scale: float = 1000.0,
                   int_lim: int = 64, name: Optional[str] = None) -> L2Case:
    """Outlier entries, all-zero rows and small-integer rows (see module doc).

    The integer rows keep r = 0 so that s stays an integer row, and their
    sums of squares stay below 2**24 so that every fp32 partial sum is an
    exact integer.
    """
    gx, gr, gmask, gperm, gint = _streams(seed, 5)
    x = gx.standard_normal((rows, cols))
    mask = gmask.random((rows, cols)) < outlier_p
    x[mask] *= outlier_scale
    r = gr.standard_normal((rows, cols))
    n_special = int(rows * 0.01)
    perm = gperm.permutation(rows)
    zero_rows = np.sort(perm[:n_special])
    int_rows = np.sort(perm[n_special:2 * n_special])
    x[zero_rows] = 0.0
    r[zero_rows] = 0.0
    ints = gint.integers(-int_lim, int_lim + 1, (len(int_rows), cols))
    assert (ints.astype(np.int64) ** 2).sum(axis=1).max() < 2 ** 24
    x[int_rows] = ints
    r[int_rows] = 0.0
    xb = to_bf16_bits(x)
    rb = to_bf16_bits(r) if residual else None
    meta = {"zero_rows": zero_rows, "int_rows": int_rows}
    return L2Case(name or f"l2_rows{'_res' if residual else ''}_stress_{rows}x{cols}",
                  xb, rb, eps, meta)


def grad_bits(shape, seed: int, sd: float = 1.0) -> np.ndarray:
    """An upstream gradient: N(0, sd) samples as bf16 bits."""
    (g,) = _streams(seed, 1)
    return to_bf16_bits(sd * g.standard_normal(shape))


def l2_grad_case(rows: int, cols: int, seed: int, residual: bool = True,
                 eps: float = 1e-6, name: Optional[str] = None) -> L2GradCase:
    """x, r drawn as l2_case(rows, cols, seed) does, dy from the stream after them."""
    fwd = l2_case(rows, cols, seed, residual, eps)
    dy = grad_bits((rows, cols), seed + 7919)
    return L2GradCase(name or f"l2_rows{'_res' if residual else ''}_bwd_{rows}x{cols}",
                      fwd.x, fwd.r, dy, eps)


def rownorm_grad_case(shapes, seed: int, radius: float = 1.0,
                      name: Optional[str] = None) -> RownormGradCase:
    fwd = rownorm_case(shapes, seed, radius=radius)
    dwe = [grad_bits(w.shape, seed + 7919 + i) for i, w in enumerate(fwd.w)]
    return RownormGradCase(name or f"rownorm_gain_bwd_{len(shapes)}", fwd.w, fwd.gain,
                           fwd.radius, dwe)


def gate_case(rows: int, cols: int, seed: int, g_sd: float = 1.0,
              name: Optional[str] = None) -> ActCase:
    go, gg, gs = _streams(seed, 3)
    o = to_bf16_bits(go.standard_normal((rows, cols)))
    g = to_bf16_bits(g_sd * gg.standard_normal((rows, cols)))
    sg = gs.uniform(0.5, 2.0, cols).astype(np.float32)
    return ActCase(name or f"gate_l2_rows_{rows}x{cols}", o, g, sg, None)


def swiglu_case(rows: int, cols: int, seed: int, name: Optional[str] = None) -> ActCase:
    gg, gu, s1, s2 = _streams(seed, 4)
    g = to_bf16_bits(gg.standard_normal((rows, cols)))
    u = to_bf16_bits(gu.standard_normal((rows, cols)))
    sug = s1.uniform(0.5, 2.0, cols).astype(np.float32)
    suu = s2.uniform(0.5, 2.0, cols).astype(np.float32)
    return ActCase(name or f"swiglu_l2_rows_{rows}x{cols}", g, u, sug, suu)


def rope_inv_freq(head_dim: int, theta: float = 10000.0) -> np.ndarray:
    """theta^(-2i/head_dim), i < head_dim/2, in float64, rounded to fp32."""
    return (theta ** (-np.arange(0, head_dim, 2, dtype=np.float64) / head_dim)).astype(np.float32)


def qk_case(rows: int, nq: int, nk: int, head_dim: int, seed: int, far: float = 1 / 3,
            far_start: int = 199_800, name: Optional[str] = None) -> QkCase:
    """Rows at positions 0, 1, ... and, for the last `far` of them, far_start, ..."""
    gq, gk, gs = _streams(seed, 3)
    q = to_bf16_bits(gq.standard_normal((rows, nq * head_dim)))
    k = to_bf16_bits(gk.standard_normal((rows, nk * head_dim))) if nk else None
    n_far = int(rows * far)
    pos = np.concatenate([np.arange(rows - n_far), far_start + np.arange(n_far)]).astype(np.int32)
    sc = gs.uniform(0.5, 2.0, nq * head_dim).astype(np.float32)
    return QkCase(name or f"qk_rows_l2_{rows}_h{nq}x{nk}_d{head_dim}", q, k, pos,
                  rope_inv_freq(head_dim), sc, head_dim)


def rescale_case(shapes, seed: int, w_sd: float = 0.02, v_sd: float = 1e-3,
                 radius: float = 1.0, name: Optional[str] = None) -> RescaleCase:
    gens = _streams(seed, 2 * len(shapes))
    ws, vs = [], []
    for i, (rows, cols) in enumerate(shapes):
        ws.append((w_sd * gens[2 * i].standard_normal((rows, cols))).astype(np.float32))
        vs.append((v_sd * gens[2 * i + 1].standard_normal((rows, cols))).astype(np.float32))
    return RescaleCase(name or f"rescale_{len(shapes)}", ws, vs, [float(radius)] * len(shapes))


# name -> (description, builder, seed).  Seeds are 1000 + a fixed number.
WORKLOADS = {
    "l2_rows_64x1024": (
        "l2_rows, no residual, 64 x 1024 bf16, x ~ N(0,1), eps 1e-6",
        lambda: l2_case(64, 1024, 1001, residual=False, name="l2_rows_64x1024")),
    "l2_rows_res_8192x4096": (
        "l2_rows with fused residual, 8192 x 4096 bf16, x, r ~ N(0,1), eps 1e-6",
        lambda: l2_case(8192, 4096, 1002, residual=True, name="l2_rows_res_8192x4096")),
    "slerp_rows_8192x7168": (
        "slerp_rows, 8192 x 7168 bf16, res ~ N(0,1), out ~ N(0, sd 2), "
        "alpha ~ U(-0.2, 0.2) fp32, eps 1e-6",
        lambda: slerp_case(8192, 7168, 1003, name="slerp_rows_8192x7168")),
    "rownorm_gain_12x4_d768": (
        "weight rownorm + gain over 12 pre-norm layers' linears (d 768, d_ff 3072), "
        "W ~ N(0, sd 0.02) fp32, g ~ U(0.5, 2) fp32, rho 1",
        lambda: rownorm_case(transformer_linears(), 1004, name="rownorm_gain_12x4_d768")),
    "l2_rows_res_stress_32768x8192": (
        "l2_rows with residual, 32768 x 8192 bf16: 1% outliers x1000, 1% zero rows, "
        "1% integer rows in [-64, 64], eps 1e-6",
        lambda: stress_l2_case(name="l2_rows_res_stress_32768x8192")),
    "slerp_rows_8192x4096": (
        "slerp_rows, 8192 x 4096 bf16, res ~ N(0,1), out ~ N(0, sd 2), "
        "alpha ~ U(-0.2, 0.2) fp32, eps 1e-6",
        lambda: slerp_case(8192, 4096, 1006, name="slerp_rows_8192x4096")),
    "l2_rows_res_bwd_8192x4096": (
        "l2_rows gradient with residual, 8192 x 4096 bf16: x, r, dy ~ N(0,1), eps 1e-6",
        lambda: l2_grad_case(8192, 4096, 1007, name="l2_rows_res_bwd_8192x4096")),
    "rownorm_gain_bwd_12x4_d768": (
        "weight rownorm + gain gradient over 12 pre-norm layers' linears (d 768, d_ff 3072): "
        "W ~ N(0, sd 0.02), g ~ U(0.5, 2), rho 1, dL/dW_eff ~ N(0,1) bf16",
        lambda: rownorm_grad_case(transformer_linears(), 1008,
                                  name="rownorm_gain_bwd_12x4_d768")),
    "rownorm_gain_bwd_11008x4096": (
        "weight rownorm + gain gradient, one 11008 x 4096 matrix: W ~ N(0, sd 0.02), "
        "g ~ U(0.5, 2), rho 1, dL/dW_eff ~ N(0,1) bf16",
        lambda: rownorm_grad_case([(11008, 4096)], 1009, name="rownorm_gain_bwd_11008x4096")),
    "gate_l2_rows_8192x4096": (
        "gate_l2_rows, 8192 x 4096 bf16 (all heads of a row): o, g ~ N(0,1), "
        "sg ~ U(0.5, 2) fp32, eps 1e-6",
        lambda: gate_case(8192, 4096, 1010, name="gate_l2_rows_8192x4096")),
    "swiglu_l2_rows_8192x7168": (
        "swiglu_l2_rows, 8192 x 7168 bf16 (the MLP width): g, u ~ N(0,1), "
        "sug, suu ~ U(0.5, 2) fp32, eps 1e-6",
        lambda: swiglu_case(8192, 7168, 1011, name="swiglu_l2_rows_8192x7168")),
    "qk_rows_l2_8192_h16x4_d256": (
        "qk_rows_l2, 8192 token rows, head_dim 256, 16 q heads over 4 kv heads, a third "
        "of the rows past position 199,800, inv_freq 10000^(-2i/256), q_scale ~ U(0.5, 2)",
        lambda: qk_case(8192, 16, 4, 256, 1012, name="qk_rows_l2_8192_h16x4_d256")),
    "rescale_12x4_d768": (
        "rescale method over 12 pre-norm layers' linears (d 768, d_ff 3072): raw rows "
        "W ~ N(0, sd 0.02) fp32, gradients / momenta ~ N(0, sd 1e-3) fp32, radius 1",
        lambda: rescale_case(transformer_linears(), 1013, name="rescale_12x4_d768")),
    "rownorm_gain_resnet50": (
        "weight rownorm + gain over ResNet-50's 53 convolutions (rows = output channels, "
        "in * kh * kw values each; the stem's 147 takes single elements) and classifier: "
        "W ~ N(0, sd 0.02) fp32, g ~ U(0.5, 2), rho 1",
        lambda: rownorm_case(resnet50_convs(), 1015, name="rownorm_gain_resnet50")),
    "rownorm_gain_bwd_resnet50": (
        "the gradient of rownorm_gain_resnet50: dL/dW_eff ~ N(0,1) bf16",
        lambda: rownorm_grad_case(resnet50_convs(), 1016, name="rownorm_gain_bwd_resnet50")),
    "rownorm_gain_embedding_50304x768": (
        "a GPT vocabulary embedding, 50304 x 768 fp32, radius sqrt(768) (rows of unit RMS): "
        "W ~ N(0, sd 0.02), g ~ U(0.5, 2)",
        lambda: rownorm_case([(50304, 768)], 1017, radius=float(np.sqrt(np.float32(768))),
                             name="rownorm_gain_embedding_50304x768")),
    "rownorm_gain_gpt2_conv1d": (
        "weight rownorm + gain over GPT-2 small's 48 Conv1D weights, stored [in, out] (each "
        "output unit a column): W ~ N(0, sd 0.02) fp32, g ~ U(0.5, 2) per unit, "
        "dL/dW_eff ~ N(0,1) bf16 (same layout)",
        lambda: colblock_grad_case(gpt2_conv1d(), 1, 1018, name="rownorm_gain_gpt2_conv1d")),
    "rms_rows_bwd_16384x768": (
        "rms_rows and its gradient, 16384 x 768 bf16 (d_model 768, 8 x 2048 tokens): "
        "x ~ N(0,1), no residual, dy ~ N(0,1), eps 1e-6",
        lambda: l2_grad_case(16384, 768, 1014, residual=False, name="rms_rows_bwd_16384x768")),
}


def make(name: str):
    """Build a named workload (deterministic)."""
    return WORKLOADS[name][1]()
