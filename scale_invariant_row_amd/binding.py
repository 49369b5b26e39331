"""ctypes binding of libdsrows.so (include/ds_rows.h): argument marshalling only.

Every computation runs in the library's HIP kernels.  The functions take
torch tensors on a HIP device, check dtype/shape/contiguity/device, pass raw
pointers and the current stream, and raise ``RuntimeError`` with the
library's status string on a nonzero status.  Loading fails loudly if the
library has not been built (``python -m scale_invariant_row_amd.build``).

bf16 tensors may be ``torch.bfloat16`` or ``torch.int16``/``torch.uint16``
holding the bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import List, Optional, Sequence, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
# DS_ROWS_LIB may name another build of the same library (the tests'
# AddressSanitizer build of the host code); there is no fallback either way
LIB_PATH = os.environ.get("DS_ROWS_LIB") or os.path.join(PKG, "_lib", "libdsrows.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "ds_rows.h")

DS_OK = 0
DS_ERR_NULL = -1
DS_ERR_SHAPE = -2
DS_ERR_ALIGN = -3
DS_ERR_ARG = -4
DS_ERR_ALLOC = -5
DS_ERR_LAUNCH = -6
DS_ERR_DEVICE = -7
DS_ERR_CAPTURE = -8
DS_ERR_SCRATCH = -9
DS_SCRATCH_FLOATS = 1 << 20


class RownormDesc(ctypes.Structure):
    """ds_rownorm_desc."""
    _fields_ = [
        ("w", ctypes.c_void_p),
        ("gain", ctypes.c_void_p),
        ("radius", ctypes.c_float),
        ("norm_out", ctypes.c_void_p),
        ("w_eff", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("gain_mode", ctypes.c_int32),
        ("seg", ctypes.c_int32),
        ("ld", ctypes.c_int64),
    ]


class RownormGradDesc(ctypes.Structure):
    """ds_rownorm_grad_desc."""
    _fields_ = [
        ("w", ctypes.c_void_p),
        ("gain", ctypes.c_void_p),
        ("radius", ctypes.c_float),
        ("dw_eff", ctypes.c_void_p),
        ("dw", ctypes.c_void_p),
        ("dgain", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("gain_mode", ctypes.c_int32),
        ("dgain_total", ctypes.c_void_p),
        ("seg", ctypes.c_int32),
        ("ld", ctypes.c_int64),
    ]


class RescaleDesc(ctypes.Structure):
    """ds_rescale_desc."""
    _fields_ = [
        ("w", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("radius", ctypes.c_float),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("seg", ctypes.c_int32),
        ("ld", ctypes.c_int64),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m scale_invariant_row_amd.build` (there is no fallback)")
        # torch first: it maps its own HIP runtime (same soname), and the
        # library then binds to that one, so the kernels, the tensors' memory
        # and the streams all live in one HIP runtime.  Loaded the other way
        # round, the process would hold two runtimes and the library's own
        # would not share torch's device state.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
        for name in ("ds_l2_rows", "ds_rms_rows"):
            getattr(L, name).argtypes = [vp, vp, vp, i64, i64, f32, vp]
            getattr(L, name).restype = ctypes.c_int
        L.ds_slerp_rows.argtypes = [vp, vp, vp, vp, i64, i64, f32, vp]
        L.ds_slerp_rows.restype = ctypes.c_int
        L.ds_weight_rownorm_gain.argtypes = [ctypes.POINTER(RownormDesc), ctypes.c_int32, vp]
        L.ds_weight_rownorm_gain.restype = ctypes.c_int
        L.ds_gate_l2_rows.argtypes = [vp, vp, vp, vp, i64, i64, f32, vp]
        L.ds_gate_l2_rows.restype = ctypes.c_int
        L.ds_swiglu_l2_rows.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, vp]
        L.ds_swiglu_l2_rows.restype = ctypes.c_int
        i32 = ctypes.c_int32
        L.ds_qk_rows_l2.argtypes = [vp, i64, vp, i64, vp, vp, vp, vp, i64, vp, i64, i64,
                                    i32, i32, i32, f32, vp]
        L.ds_qk_rows_l2.restype = ctypes.c_int
        for name in ("ds_rescale_project", "ds_rescale_after_step"):
            getattr(L, name).argtypes = [ctypes.POINTER(RescaleDesc), ctypes.c_int32, vp]
            getattr(L, name).restype = ctypes.c_int
        for name in ("ds_l2_rows_backward", "ds_rms_rows_backward"):
            getattr(L, name).argtypes = [vp, vp, vp, vp, i64, i64, f32, vp]
            getattr(L, name).restype = ctypes.c_int
        for name in ("ds_weight_rownorm_gain_backward", "ds_weight_rownorm_gain_backward_noalloc"):
            getattr(L, name).argtypes = [ctypes.POINTER(RownormGradDesc), ctypes.c_int32, vp]
            getattr(L, name).restype = ctypes.c_int
        L.ds_status_string.argtypes = [ctypes.c_int]
        L.ds_status_string.restype = ctypes.c_char_p
        L.ds_version.argtypes = []
        L.ds_version.restype = ctypes.c_int
        _lib = L
    return _lib


def header_functions() -> List[str]:
    """Names of the functions include/ds_rows.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ds_\w+)\s*\(", text, re.M)))


def ds_status_string(status: int) -> str:
    return lib().ds_status_string(int(status)).decode()


def ds_version() -> int:
    return lib().ds_version()


def _check(status: int, what: str) -> None:
    if status != DS_OK:
        raise RuntimeError(f"{what}: {ds_status_string(status)}")


# --------------------------------------------------------------- tensors

def _torch():
    import torch
    return torch


def _bf16_2d(t, name, device: bool = True):
    """A bf16 [rows, cols] contiguous tensor (and, unless the caller checks
    devices itself afterwards, on a HIP device)."""
    torch = _torch()
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name}: expected bf16 data (bfloat16 or 16-bit int bits), got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name}: expected a 2-D [rows, cols] tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if device and t.device.type != "cuda":
        raise ValueError(f"{name}: must be on a HIP device")


def _same(a, b, name):
    if b.shape != a.shape or b.device != a.device:
        raise ValueError(f"{name}: shape/device mismatch {tuple(b.shape)} vs {tuple(a.shape)}")


def _stream_of(t, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _torch_stream(t, stream):
    """The torch stream object for ``stream`` (None: t's current stream; a raw
    handle is wrapped without taking ownership)."""
    torch = _torch()
    if t is None:
        return None
    if stream is None:
        return torch.cuda.current_stream(t.device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.ExternalStream(handle, device=t.device)


def _norm_rows(name, x, r, eps, out, stream):
    torch = _torch()
    _bf16_2d(x, "x")
    if r is not None:
        _bf16_2d(r, "r")
        _same(x, r, "r")
    if out is None:
        out = torch.empty_like(x)
    _bf16_2d(out, "out")
    _same(x, out, "out")
    with torch.cuda.device(x.device):
        st = getattr(lib(), name)(x.data_ptr(), None if r is None else r.data_ptr(),
                                  out.data_ptr(), x.shape[0], x.shape[1], float(eps),
                                  _stream_of(x, stream))
    _check(st, name)
    return out


def ds_rms_rows(x, r=None, eps: float = 1e-6, out=None, stream=None):
    """y = bf16(s / sqrt(sum(s^2) / cols + eps)) per row, s = x or bf16(x + r).

    Returns ``out`` (allocated like ``x`` when not given; may be ``x`` or ``r``).
    """
    return _norm_rows("ds_rms_rows", x, r, eps, out, stream)


def ds_rms_rows_backward(x, r, dy, eps: float = 1e-6, out=None, stream=None):
    """dx = bf16((dy - s <s,dy>/(cols D^2)) / D), D^2 = sum(s^2)/cols + eps: the
    gradient of ds_rms_rows(x, r, eps) with respect to x (and r).  Returns
    ``out`` (allocated like ``dy`` when not given; may be ``x``, ``r`` or ``dy``)."""
    return _norm_rows_backward("ds_rms_rows_backward", x, r, dy, eps, out, stream)


def ds_l2_rows(x, r=None, eps: float = 1e-6, out=None, stream=None):
    """y = bf16(s / sqrt(sum(s^2) + eps)) per row, s = x or bf16(x + r).

    Returns ``out`` (allocated like ``x`` when not given; may be ``x`` or ``r``).
    """
    return _norm_rows("ds_l2_rows", x, r, eps, out, stream)


def ds_slerp_rows(res, out_rows, alpha, eps: float = 1e-6, h=None, stream=None):
    """h = bf16(l2(a + |alpha| (b - a))), a = bf16(l2(res)), b = bf16(l2(out_rows))."""
    torch = _torch()
    _bf16_2d(res, "res")
    _bf16_2d(out_rows, "out")
    _same(res, out_rows, "out")
    if alpha.dtype != torch.float32 or alpha.dim() != 1 or alpha.shape[0] != res.shape[1] \
            or not alpha.is_contiguous() or alpha.device != res.device:
        raise ValueError("alpha: expected a contiguous fp32 [cols] tensor on the rows' device")
    if h is None:
        h = torch.empty_like(res)
    _bf16_2d(h, "h")
    _same(res, h, "h")
    with torch.cuda.device(res.device):
        st = lib().ds_slerp_rows(res.data_ptr(), out_rows.data_ptr(), alpha.data_ptr(),
                                 h.data_ptr(), res.shape[0], res.shape[1], float(eps),
                                 _stream_of(res, stream))
    _check(st, "ds_slerp_rows")
    return h


DS_GAIN_ROW, DS_GAIN_SCALAR, DS_GAIN_NONE = 0, 1, 2


def _layout(w, seg):
    """(rows, cols, seg, ld) of a stored 2-D weight.  seg None or 0: its rows
    are the unit rows.  seg > 0: a column block (GPT-2's Conv1D [in, out] with
    seg 1; one ConvTranspose group [in, out * k] with seg k): unit u owns the
    seg values at u * seg of every stored row."""
    if not seg:
        return w.shape[0], w.shape[1], 0, 0
    if w.shape[1] % seg != 0:
        raise ValueError(f"a column block of seg {seg} needs a multiple of {seg} stored columns")
    return w.shape[1] // seg, w.shape[0] * seg, int(seg), w.shape[1]


def _gain_mode(g, rows: int, name: str) -> int:
    """A gain tensor's mode: None (no gain), a 0-dim or one-element tensor for
    rows != 1 (one gain for the matrix), or a [rows] tensor (a gain per row)."""
    torch = _torch()
    if g is None:
        return DS_GAIN_NONE
    if g.dtype != torch.float32 or not g.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous fp32 tensor")
    if g.dim() == 0 or (g.numel() == 1 and rows != 1):
        return DS_GAIN_SCALAR
    if g.shape != (rows,):
        raise ValueError(f"{name}: expected fp32 [rows], one value, or None")
    return DS_GAIN_ROW


def ds_weight_rownorm_gain(ws: Sequence, gains: Sequence, radius: Optional[Sequence[float]] = None,
                           norm_out: Optional[Sequence] = None, w_eff: Optional[Sequence] = None,
                           stream=None, segs: Optional[Sequence] = None) -> Tuple[list, list]:
    """Per matrix: ||W_i|| (fp32) and bf16(W_i * g_i * radius / ||W_i||), in one call.

    ``ws``: fp32 2-D tensors; ``gains``: per matrix an fp32 [rows] tensor (a
    gain per row), a single value (one gain for the matrix) or None (no gain);
    ``segs``: per matrix None (the stored rows are the unit rows) or the seg
    of a column block (see ``_layout``).  Returns (norms, w_effs); w_effs are
    bfloat16 tensors shaped like ws unless given.
    """
    torch = _torch()
    n = len(ws)
    if len(gains) != n:
        raise ValueError("one gain entry per matrix")
    radius = [1.0] * n if radius is None else list(radius)
    lay = [_layout(w, None if segs is None else segs[i]) for i, w in enumerate(ws)]
    if norm_out is None:
        norm_out = [torch.empty(lay[i][0], dtype=torch.float32, device=w.device)
                    for i, w in enumerate(ws)]
    if w_eff is None:
        w_eff = [torch.empty(w.shape, dtype=torch.bfloat16, device=w.device) for w in ws]
    descs = (RownormDesc * max(n, 1))()
    dev = None
    for i, (w, g) in enumerate(zip(ws, gains)):
        if w.dtype != torch.float32 or w.dim() != 2 or not w.is_contiguous():
            raise ValueError(f"ws[{i}]: expected a contiguous fp32 [rows, cols] tensor")
        rows, cols, seg, ld = lay[i]
        mode = _gain_mode(g, rows, f"gains[{i}]")
        _bf16_2d(w_eff[i], f"w_eff[{i}]", device=False)
        if tuple(w_eff[i].shape) != tuple(w.shape):
            raise ValueError(f"w_eff[{i}]: shape mismatch")
        if norm_out[i] is not None and (norm_out[i].dtype != torch.float32
                                        or norm_out[i].shape != (rows,)
                                        or not norm_out[i].is_contiguous()):
            raise ValueError(f"norm_out[{i}]: expected a contiguous fp32 [rows] tensor")
        for t in (w, g, w_eff[i], norm_out[i]):
            if t is None:
                continue
            if t.device.type != "cuda" or (dev is not None and t.device != dev):
                raise ValueError("all tensors must be on one HIP device")
            dev = t.device
        descs[i] = RownormDesc(w.data_ptr(), None if g is None else g.data_ptr(), float(radius[i]),
                               None if norm_out[i] is None else norm_out[i].data_ptr(),
                               w_eff[i].data_ptr(), rows, cols, mode, seg, ld)
    if n == 0:
        return [], []
    with torch.cuda.device(dev):
        st = lib().ds_weight_rownorm_gain(descs, n, _stream_of(ws[0], stream))
    _check(st, "ds_weight_rownorm_gain")
    return list(norm_out), list(w_eff)


def _norm_rows_backward(name, x, r, dy, eps, out, stream):
    torch = _torch()
    _bf16_2d(x, "x")
    _bf16_2d(dy, "dy")
    _same(x, dy, "dy")
    if r is not None:
        _bf16_2d(r, "r")
        _same(x, r, "r")
    if out is None:
        out = torch.empty_like(dy)
    _bf16_2d(out, "out")
    _same(x, out, "out")
    with torch.cuda.device(x.device):
        st = getattr(lib(), name)(x.data_ptr(), None if r is None else r.data_ptr(),
                                  dy.data_ptr(), out.data_ptr(), x.shape[0], x.shape[1],
                                  float(eps), _stream_of(x, stream))
    _check(st, name)
    return out


def ds_l2_rows_backward(x, r, dy, eps: float = 1e-6, out=None, stream=None):
    """dx = bf16((dy - s <s,dy>/D^2) / D), the gradient of ds_l2_rows(x, r, eps)
    with respect to x (and to r when given).  Returns ``out`` (allocated like
    ``dy`` when not given; may be ``x``, ``r`` or ``dy``)."""
    return _norm_rows_backward("ds_l2_rows_backward", x, r, dy, eps, out, stream)


def ds_weight_rownorm_gain_backward(ws: Sequence, gains: Sequence, dw_effs: Sequence,
                                    radius: Optional[Sequence[float]] = None,
                                    dw: Optional[Sequence] = None,
                                    dgain: Optional[Sequence] = None,
                                    want_dgain: bool = True, stream=None,
                                    segs: Optional[Sequence] = None,
                                    _noalloc: bool = False) -> Tuple[list, list]:
    """Per matrix: dL/dW (fp32) and dL/dg (fp32) from dL/dW_eff (bf16), in one call.

    ``gains`` and ``segs`` as for ds_weight_rownorm_gain.  Returns (dws, dgains): dL/dg is
    an fp32 [rows] tensor for a gain per row, a 0-dim fp32 tensor for one gain
    per matrix (the library sums the rows' shares, kept in a [rows] buffer),
    and None with no gain or when ``want_dgain`` is false and none was given.
    """
    torch = _torch()
    n = len(ws)
    if len(gains) != n or len(dw_effs) != n:
        raise ValueError("one gain entry and one dW_eff per matrix")
    radius = [1.0] * n if radius is None else list(radius)
    if dw is None:
        dw = [torch.empty(w.shape, dtype=torch.float32, device=w.device) for w in ws]
    lay = [_layout(w, None if segs is None else segs[i]) for i, w in enumerate(ws)]
    modes = [_gain_mode(g, lay[i][0], f"gains[{i}]") for i, g in enumerate(gains)]
    if dgain is None:
        dgain = [torch.empty(lay[i][0] if m == DS_GAIN_ROW else (), dtype=torch.float32,
                             device=w.device) if want_dgain and m != DS_GAIN_NONE else None
                 for i, (w, m) in enumerate(zip(ws, modes))]
    dev = None
    for i, (w, g, de) in enumerate(zip(ws, gains, dw_effs)):
        if w.dtype != torch.float32 or w.dim() != 2 or not w.is_contiguous():
            raise ValueError(f"ws[{i}]: expected a contiguous fp32 [rows, cols] tensor")
        _bf16_2d(de, f"dw_effs[{i}]", device=False)
        if tuple(de.shape) != tuple(w.shape):
            raise ValueError(f"dw_effs[{i}]: shape mismatch")
        if dw[i].dtype != torch.float32 or tuple(dw[i].shape) != tuple(w.shape) \
                or not dw[i].is_contiguous():
            raise ValueError(f"dw[{i}]: expected a contiguous fp32 tensor shaped like ws[{i}]")
        want = (lay[i][0],) if modes[i] == DS_GAIN_ROW else ()
        if dgain[i] is not None and (dgain[i].dtype != torch.float32 or dgain[i].shape != want
                                     or not dgain[i].is_contiguous()):
            raise ValueError(f"dgain[{i}]: expected a contiguous fp32 tensor of shape {want}")
        for t in (w, g, de, dw[i], dgain[i]):
            if t is None:
                continue
            if t.device.type != "cuda" or (dev is not None and t.device != dev):
                raise ValueError("all tensors must be on one HIP device")
            dev = t.device
    if n == 0:
        return [], []
    # A scalar gain's per-row shares: a temporary the kernels write and read
    # on the launch stream.  It is allocated on that stream, so when it is
    # dropped below, the caching allocator hands its block only to work
    # ordered after those kernels.  (The allocation-free entry point keeps
    # them in the library's own scratch instead.)
    with torch.cuda.device(dev), torch.cuda.stream(_torch_stream(ws[0], stream)):
        shares = [torch.empty(lay[i][0], dtype=torch.float32, device=dev)
                  if m == DS_GAIN_SCALAR and dgain[i] is not None and not _noalloc else None
                  for i, m in enumerate(modes)]
    descs = (RownormGradDesc * n)()
    for i, (w, g, de) in enumerate(zip(ws, gains, dw_effs)):
        rows, cols, seg, ld = lay[i]
        per_row = dgain[i] if modes[i] == DS_GAIN_ROW else shares[i]
        total = dgain[i] if modes[i] == DS_GAIN_SCALAR else None
        descs[i] = RownormGradDesc(w.data_ptr(), None if g is None else g.data_ptr(),
                                   float(radius[i]), de.data_ptr(), dw[i].data_ptr(),
                                   None if per_row is None else per_row.data_ptr(),
                                   rows, cols, modes[i],
                                   None if total is None else total.data_ptr(), seg, ld)
    name = "ds_weight_rownorm_gain_backward" + ("_noalloc" if _noalloc else "")
    with torch.cuda.device(dev):
        st = getattr(lib(), name)(descs, n, _stream_of(ws[0], stream))
    _check(st, name)
    return list(dw), list(dgain)


def ds_weight_rownorm_gain_backward_noalloc(ws: Sequence, gains: Sequence, dw_effs: Sequence,
                                            radius: Optional[Sequence[float]] = None,
                                            dw: Optional[Sequence] = None,
                                            dgain: Optional[Sequence] = None,
                                            want_dgain: bool = True, stream=None,
                                            segs: Optional[Sequence] = None
                                            ) -> Tuple[list, list]:
    """ds_weight_rownorm_gain_backward through the allocation-free entry point:
    the library allocates nothing (a scalar gain's row shares live in its fixed
    per-GPU scratch).  Pass ``dw`` and ``dgain`` to keep this wrapper from
    allocating its outputs through torch."""
    return ds_weight_rownorm_gain_backward(ws, gains, dw_effs, radius, dw, dgain, want_dgain,
                                           stream, segs, _noalloc=True)


def _col_vector(v, cols, like, name):
    torch = _torch()
    if v.dtype != torch.float32 or v.dim() != 1 or v.shape[0] != cols \
            or not v.is_contiguous() or v.device != like.device:
        raise ValueError(f"{name}: expected a contiguous fp32 [cols] tensor on the rows' device")


def ds_gate_l2_rows(o, g, sg, eps: float = 1e-6, out=None, stream=None):
    """y = bf16(l2(bf16(o * sigmoid(g * sg)))) per row (sg: fp32 [cols])."""
    torch = _torch()
    _bf16_2d(o, "o")
    _bf16_2d(g, "g")
    _same(o, g, "g")
    _col_vector(sg, o.shape[1], o, "sg")
    if out is None:
        out = torch.empty_like(o)
    _bf16_2d(out, "out")
    _same(o, out, "out")
    with torch.cuda.device(o.device):
        st = lib().ds_gate_l2_rows(o.data_ptr(), g.data_ptr(), sg.data_ptr(), out.data_ptr(),
                                   o.shape[0], o.shape[1], float(eps), _stream_of(o, stream))
    _check(st, "ds_gate_l2_rows")
    return out


def ds_swiglu_l2_rows(g, u, sug, suu, eps: float = 1e-6, out=None, stream=None):
    """y = bf16(l2(bf16(silu(bf16(g * sug)) * bf16(u * suu)))) per row."""
    torch = _torch()
    _bf16_2d(g, "g")
    _bf16_2d(u, "u")
    _same(g, u, "u")
    _col_vector(sug, g.shape[1], g, "sug")
    _col_vector(suu, g.shape[1], g, "suu")
    if out is None:
        out = torch.empty_like(g)
    _bf16_2d(out, "out")
    _same(g, out, "out")
    with torch.cuda.device(g.device):
        st = lib().ds_swiglu_l2_rows(g.data_ptr(), u.data_ptr(), sug.data_ptr(), suu.data_ptr(),
                                     out.data_ptr(), g.shape[0], g.shape[1], float(eps),
                                     _stream_of(g, stream))
    _check(st, "ds_swiglu_l2_rows")
    return out


def ds_qk_rows_l2(q, k, positions, inv_freq, q_scale, head_dim: int, eps: float = 1e-6,
                  q_out=None, k_out=None, stream=None):
    """RoPE, per-head L2 and q's scale on q [rows, >= nq*hd] and k [rows, >= nk*hd].

    ``q``/``k`` may be strided row views (a fused projection's slices); the
    number of heads is the used width / head_dim, given by ``q_scale``'s
    length for q and by k's width for k.  Returns (q_out, k_out).

    Every argument is checked (dtype, shape, row count, unit column stride,
    contiguity of the vectors, one HIP device for all) before anything is
    launched; a bad one raises ValueError naming it.
    """
    torch = _torch()
    bf16 = (torch.bfloat16, torch.int16, torch.uint16)
    head_dim = int(head_dim)
    if head_dim <= 0:
        raise ValueError("head_dim: must be positive")

    def rows_tensor(t, name):
        if t.dtype not in bf16 or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name}: expected a bf16 [rows, cols] tensor with unit column stride")

    def vector(t, name, dtype, n=None):
        if t.dtype != dtype or t.dim() != 1 or not t.is_contiguous() \
                or (n is not None and t.shape[0] != n):
            want = f"[{n}]" if n is not None else "[n]"
            raise ValueError(f"{name}: expected a contiguous {dtype} {want} tensor")

    rows_tensor(q, "q")
    rows = q.shape[0]
    vector(q_scale, "q_scale", torch.float32)
    if q_scale.shape[0] == 0 or q_scale.shape[0] % head_dim:
        raise ValueError("q_scale: its length must be n_q_heads * head_dim")
    nq = q_scale.shape[0] // head_dim
    if q.shape[1] < nq * head_dim:
        raise ValueError("q: must hold n_q_heads * head_dim columns")
    nk = 0
    if k is not None:
        rows_tensor(k, "k")
        if k.shape[0] != rows:
            raise ValueError(f"k: expected {rows} rows like q, got {k.shape[0]}")
        if k.shape[1] % head_dim:
            raise ValueError("k: its width must be a whole number of heads")
        nk = k.shape[1] // head_dim
    elif k_out is not None:
        raise ValueError("k_out: given without k")
    vector(positions, "positions", torch.int32, rows)
    vector(inv_freq, "inv_freq", torch.float32, head_dim // 2)
    if q_out is not None:
        rows_tensor(q_out, "q_out")
        if q_out.shape[0] != rows or q_out.shape[1] < nq * head_dim:
            raise ValueError(f"q_out: expected [{rows}, >= {nq * head_dim}]")
    if k_out is not None:
        rows_tensor(k_out, "k_out")
        if k_out.shape[0] != rows or k_out.shape[1] < nk * head_dim:
            raise ValueError(f"k_out: expected [{rows}, >= {nk * head_dim}]")
    tensors = [("q", q), ("k", k), ("positions", positions), ("inv_freq", inv_freq),
               ("q_scale", q_scale), ("q_out", q_out), ("k_out", k_out)]
    for name, t in tensors:
        if t is not None and (t.device.type != "cuda" or t.device != q.device):
            raise ValueError(f"{name}: must be on the HIP device of q")
    if q_out is None:
        q_out = torch.empty(rows, nq * head_dim, dtype=q.dtype, device=q.device)
    if k is not None and k_out is None:
        k_out = torch.empty(rows, nk * head_dim, dtype=k.dtype, device=k.device)
    with torch.cuda.device(q.device):
        st = lib().ds_qk_rows_l2(
            q.data_ptr(), q.stride(0), None if k is None else k.data_ptr(),
            0 if k is None else k.stride(0), positions.data_ptr(), inv_freq.data_ptr(),
            q_scale.data_ptr(), q_out.data_ptr(), q_out.stride(0),
            None if k_out is None else k_out.data_ptr(), 0 if k_out is None else k_out.stride(0),
            rows, nq, nk, head_dim, float(eps), _stream_of(q, stream))
    _check(st, "ds_qk_rows_l2")
    return q_out, k_out


def _rescale(ws, vs, radius, after_step, stream, segs=None):
    torch = _torch()
    n = len(ws)
    vs = [None] * n if vs is None else list(vs)
    radius = [1.0] * n if radius is None else list(radius)
    descs = (RescaleDesc * max(n, 1))()
    dev = None
    for i, w in enumerate(ws):
        for t, name in ((w, "w"), (vs[i], "v")):
            if t is None:
                continue
            if t.dtype != torch.float32 or t.dim() != 2 or not t.is_contiguous() \
                    or t.shape != w.shape or t.device.type != "cuda" \
                    or (dev is not None and t.device != dev):
                raise ValueError(f"{name}[{i}]: expected a contiguous fp32 HIP tensor shaped like w")
            dev = t.device
        rows, cols, seg, ld = _layout(w, None if segs is None else segs[i])
        descs[i] = RescaleDesc(w.data_ptr(), None if vs[i] is None else vs[i].data_ptr(),
                               float(radius[i]), rows, cols, seg, ld)
    if n == 0:
        return
    with torch.cuda.device(dev):
        fn = lib().ds_rescale_after_step if after_step else lib().ds_rescale_project
        st = fn(descs, n, _stream_of(ws[0], stream))
    _check(st, "ds_rescale_after_step" if after_step else "ds_rescale_project")


def ds_rescale_project(ws: Sequence, grads: Sequence, stream=None,
                       segs: Optional[Sequence] = None) -> None:
    """In place, per matrix: grad <- grad - w <w, grad> / ||w||^2 per unit row
    (``segs`` as for ds_weight_rownorm_gain)."""
    if len(grads) != len(ws):
        raise ValueError("one gradient per matrix")
    _rescale(ws, grads, None, False, stream, segs)


def ds_rescale_after_step(ws: Sequence, moms: Optional[Sequence] = None,
                          radius: Optional[Sequence[float]] = None, stream=None,
                          segs: Optional[Sequence] = None) -> None:
    """In place, per matrix: project the momentum (if given), then w <- radius w/||w||."""
    _rescale(ws, moms, radius, True, stream, segs)
