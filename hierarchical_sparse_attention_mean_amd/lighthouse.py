"""ctypes binding of liblighthouse.so (the C ABI in include/lighthouse.h).

The ``lh_*`` functions take the same arguments as their C counterparts, with
torch tensors in place of device pointers; they only marshal arguments and
return what the C call returns.  torch is used for device memory and the
current stream, nothing else: every step of the layer runs in the library's
HIP kernels.  The library must have been built (``build.py``); importing this
module raises if it is missing.

Convenience wrappers (``forward``, ``backward``, ``LighthouseAttention``)
allocate the caller-owned buffers with torch and call the entry points.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch  # noqa: F401  (must load torch's HIP runtime before the library)

_HERE = os.path.dirname(os.path.abspath(__file__))
# LH_LIBRARY names another build of the same library (e.g. a host-side
# sanitizer build for the host-only tests); default: the in-tree build
LIB_PATH = os.environ.get("LH_LIBRARY") or os.path.join(_HERE, "liblighthouse.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "lighthouse.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m hierarchical_sparse_attention_mean_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

LH_F32, LH_BF16 = 0, 1
STATUS = {0: "LH_OK", 1: "LH_EINVAL", 2: "LH_EDIVIS", 3: "LH_EUNSUPPORTED", 4: "LH_EWORKSPACE", 5: "LH_EHIP"}


class LighthouseError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}: {lh_last_error()}")


class SavedLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("scores", "flags", "slot", "coords", "qt", "kt", "vt", "ot", "lse", "total")] + \
               [(n, ctypes.c_int64) for n in ("P", "E", "Bsel", "S", "Sv")]


class LayerLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("q", "k", "v", "o", "inner", "inner_bytes", "total")]


_i, _i64, _sz, _vp = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
_P = ctypes.POINTER
_lib.lh_query.argtypes = [_i, _i, _i64, _i, _i, _i, _i64, _i, _P(_i64), _P(_sz), _P(_sz), _P(_sz)]
_lib.lh_query.restype = _i
_lib.lh_saved_layout.argtypes = [_i, _i, _i64, _i, _i, _i, _i64, _i, _P(SavedLayout)]
_lib.lh_saved_layout.restype = _i
_lib.lh_forward.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i64, _i, _i, _i, _i64, _i, _vp, _sz, _vp, _sz, _vp]
_lib.lh_forward.restype = _i
_lib.lh_backward.argtypes = [_vp, _vp, _vp, _vp, _i, _vp, _sz, _vp, _vp, _vp, _i,
                             _i, _i, _i64, _i, _i, _i, _i64, _i, _vp, _sz, _vp]
_lib.lh_backward.restype = _i
_lib.lh_attention_forward.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i64, _i, _i, _vp]
_lib.lh_attention_forward.restype = _i
_lib.lh_attention_backward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i64, _i, _i, _vp, _sz, _vp]
_lib.lh_attention_backward.restype = _i
_lib.lh_attention_backward_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i64, _i, _i, _vp]
_lib.lh_attention_backward_noalloc.restype = _i
_lib.lh_layer_query.argtypes = [_i, _i, _i64, _i, _i, _i, _i, _i64, _i, _P(_i64), _P(_sz), _P(_sz), _P(_sz)]
_lib.lh_layer_query.restype = _i
_lib.lh_layer_saved_layout.argtypes = [_i, _i, _i64, _i, _i, _i, _i, _i64, _i, _P(LayerLayout)]
_lib.lh_layer_saved_layout.restype = _i
_lib.lh_layer_forward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i64, _i, _i, _i, _i, _i64, _i,
                                  _vp, _sz, _vp, _sz, _vp]
_lib.lh_layer_forward.restype = _i
_lib.lh_layer_backward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _i, _vp, _vp, _vp, _vp,
                                   _i, _i, _i64, _i, _i, _i, _i, _i64, _i, _vp, _sz, _vp]
_lib.lh_layer_backward.restype = _i
_lib.lh_status_string.argtypes = [_i]
_lib.lh_status_string.restype = ctypes.c_char_p
_lib.lh_last_error.argtypes = []
_lib.lh_last_error.restype = ctypes.c_char_p
_lib.lh_stage_name.argtypes = [_i]
_lib.lh_stage_name.restype = ctypes.c_char_p
_lib.lh_timing_begin.argtypes = []
_lib.lh_timing_begin.restype = _i
_lib.lh_timing_end.argtypes = [_P(ctypes.c_double), _P(_i), _i]
_lib.lh_timing_end.restype = _i
STAGE_COUNT = 13   # LH_STAGE_COUNT


def library():
    """The loaded ctypes library (for symbol checks)."""
    return _lib


def declared_symbols() -> list[str]:
    """Names of the functions include/lighthouse.h declares."""
    with open(HEADER) as f:
        txt = f.read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(lh_[a-z_]+)\s*\(", txt)))


def dtype_code(dt) -> int:
    if dt in (torch.float32, "f32", LH_F32):
        return LH_F32
    if dt in (torch.bfloat16, "bf16", LH_BF16):
        return LH_BF16
    raise ValueError(f"unsupported dtype {dt}")


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        if not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------------------
# entry points, same names and arguments as the C ABI
# ---------------------------------------------------------------------------
def lh_status_string(status: int) -> str:
    return _lib.lh_status_string(status).decode()


def lh_last_error() -> str:
    return _lib.lh_last_error().decode()


def lh_stage_name(stage: int) -> str:
    return _lib.lh_stage_name(stage).decode()


def lh_timing_begin() -> int:
    return _lib.lh_timing_begin()


def lh_timing_end():
    """Returns (status, {stage name: (summed ms, spans)}) for every stage."""
    ms = (ctypes.c_double * STAGE_COUNT)()
    spans = (_i * STAGE_COUNT)()
    st = _lib.lh_timing_end(ms, spans, STAGE_COUNT)
    return st, {lh_stage_name(i): (ms[i], spans[i]) for i in range(STAGE_COUNT)}


def lh_query(B, H, N, d, L, p, topk, io):
    """Returns (status, S, saved_bytes, fwd_ws_bytes, bwd_ws_bytes)."""
    S, a, b, c = _i64(), _sz(), _sz(), _sz()
    st = _lib.lh_query(B, H, N, d, L, p, topk, dtype_code(io), ctypes.byref(S), ctypes.byref(a),
                       ctypes.byref(b), ctypes.byref(c))
    return st, S.value, a.value, b.value, c.value


def lh_saved_layout(B, H, N, d, L, p, topk, io):
    """Returns (status, dict of byte offsets and sizes)."""
    out = SavedLayout()
    st = _lib.lh_saved_layout(B, H, N, d, L, p, topk, dtype_code(io), ctypes.byref(out))
    return st, {n: getattr(out, n) for n, _ in SavedLayout._fields_}


def lh_forward(q, k, v, o, o_dtype, B, H, N, d, L, p, topk, io, saved, saved_bytes, ws, ws_bytes, stream=None):
    return _lib.lh_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), dtype_code(o_dtype), B, H, N, d, L, p, topk,
                           dtype_code(io), _ptr(saved), saved_bytes, _ptr(ws), ws_bytes, _stream(stream))


def lh_backward(q, k, v, dout, dout_dtype, saved, saved_bytes, dq, dk, dv, grad_dtype, B, H, N, d, L, p, topk, io,
                ws, ws_bytes, stream=None):
    return _lib.lh_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), dtype_code(dout_dtype), _ptr(saved),
                            saved_bytes, _ptr(dq), _ptr(dk), _ptr(dv), dtype_code(grad_dtype), B, H, N, d, L, p,
                            topk, dtype_code(io), _ptr(ws), ws_bytes, _stream(stream))


def lh_attention_forward(q, k, v, o, lse, BH, S, d, io, stream=None):
    return _lib.lh_attention_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), BH, S, d, dtype_code(io),
                                     _stream(stream))


def lh_attention_backward(q, k, v, o, lse, dout, dq, dk, dv, BH, S, d, io, ws, ws_bytes, stream=None):
    return _lib.lh_attention_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                      _ptr(dk), _ptr(dv), BH, S, d, dtype_code(io), _ptr(ws), ws_bytes,
                                      _stream(stream))


def lh_attention_backward_noalloc(q, k, v, o, lse, dout, dq, dk, dv, BH, S, d, io, stream=None):
    return _lib.lh_attention_backward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                              _ptr(dk), _ptr(dv), BH, S, d, dtype_code(io), _stream(stream))


def lh_layer_query(B, H, N, d_model, d, L, p, topk, io):
    """Returns (status, S, saved_bytes, fwd_ws_bytes, bwd_ws_bytes)."""
    S, a, b, c = _i64(), _sz(), _sz(), _sz()
    st = _lib.lh_layer_query(B, H, N, d_model, d, L, p, topk, dtype_code(io), ctypes.byref(S), ctypes.byref(a),
                             ctypes.byref(b), ctypes.byref(c))
    return st, S.value, a.value, b.value, c.value


def lh_layer_saved_layout(B, H, N, d_model, d, L, p, topk, io):
    """Returns (status, dict of byte offsets and sizes)."""
    out = LayerLayout()
    st = _lib.lh_layer_saved_layout(B, H, N, d_model, d, L, p, topk, dtype_code(io), ctypes.byref(out))
    return st, {n: getattr(out, n) for n, _ in LayerLayout._fields_}


def lh_layer_forward(x, wq, wk, wv, wo, y, y_dtype, B, H, N, d_model, d, L, p, topk, io, saved, saved_bytes, ws,
                     ws_bytes, stream=None):
    return _lib.lh_layer_forward(_ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), _ptr(y), dtype_code(y_dtype), B, H,
                                 N, d_model, d, L, p, topk, dtype_code(io), _ptr(saved), saved_bytes, _ptr(ws),
                                 ws_bytes, _stream(stream))


def lh_layer_backward(x, wq, wk, wv, wo, dy, saved, saved_bytes, dx, dx_dtype, dwq, dwk, dwv, dwo, B, H, N, d_model,
                      d, L, p, topk, io, ws, ws_bytes, stream=None):
    return _lib.lh_layer_backward(_ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), _ptr(dy), _ptr(saved),
                                  saved_bytes, _ptr(dx), dtype_code(dx_dtype), _ptr(dwq), _ptr(dwk), _ptr(dwv),
                                  _ptr(dwo), B, H, N, d_model, d, L, p, topk, dtype_code(io), _ptr(ws), ws_bytes,
                                  _stream(stream))


def attention_backward_ws_bytes(BH, S, io) -> int:
    """Workspace lh_attention_backward needs (see lighthouse.h)."""
    return (8 if dtype_code(io) == LH_BF16 else 4) * BH * S


# ---------------------------------------------------------------------------
# convenience: torch-allocated buffers around the entry points
# ---------------------------------------------------------------------------
def _check(st, where):
    if st != 0:
        raise LighthouseError(st, where)


def _require(name, t, shape=None, dtype=None, device=None):
    """Refuse, before anything reaches the library, a buffer its kernels would
    misread or fault on: not a device tensor, on another device, of another
    shape or dtype, or not contiguous."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (HIP) tensor, got one on {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _require_bytes(name, t, device):
    if t is not None:
        _require(name, t, dtype=torch.uint8, device=device)


def _shape(q, k, v):
    """[B, H, N, d] of q, with k and v required to match it."""
    _require("q", q)
    if q.dim() != 4:
        raise ValueError(f"q must be a [B, H, N, d] tensor, got shape {tuple(q.shape)}")
    for name, t in (("k", k), ("v", v)):
        _require(name, t, q.shape, q.dtype, q.device)
    return q.shape


def _same_problem(plan, B, H, N, d, io):
    got = (plan.B, plan.H, plan.N, plan.d, plan.io)
    if got != (B, H, N, d, dtype_code(io)):
        raise ValueError(f"plan was made for (B, H, N, d, io) = {got}, not for these inputs")


class Plan:
    """Sizes and layouts for one (B, H, N, d, L, p, topk, io) problem."""

    def __init__(self, B, H, N, d, L, p, topk, io):
        self.B, self.H, self.N, self.d, self.L, self.p, self.topk = B, H, N, d, L, p, topk
        self.io = dtype_code(io)
        st, self.S, self.saved_bytes, self.fwd_ws_bytes, self.bwd_ws_bytes = lh_query(B, H, N, d, L, p, topk,
                                                                                      self.io)
        _check(st, "lh_query")
        st, self.layout = lh_saved_layout(B, H, N, d, L, p, topk, self.io)
        _check(st, "lh_saved_layout")

    def args(self):
        return (self.B, self.H, self.N, self.d, self.L, self.p, self.topk, self.io)


def forward(q, k, v, L, p, topk, out_dtype=None, saved=None, ws=None, plan=None):
    """O = Lighthouse(q, k, v).  Returns (o, saved, plan); `saved` feeds backward."""
    B, H, N, d = _shape(q, k, v)
    dev = q.device
    _require_bytes("saved", saved, dev)
    _require_bytes("ws", ws, dev)
    plan = plan or Plan(B, H, N, d, L, p, topk, q.dtype)
    _same_problem(plan, B, H, N, d, q.dtype)
    out_dtype = out_dtype or q.dtype
    o = torch.empty((B, H, N, d), dtype=out_dtype, device=dev)
    if saved is None:
        saved = torch.empty(plan.saved_bytes, dtype=torch.uint8, device=dev)
    if ws is None:
        ws = torch.empty(plan.fwd_ws_bytes, dtype=torch.uint8, device=dev)
    st = lh_forward(q, k, v, o, dtype_code(out_dtype), *plan.args()[:7], plan.io, saved, saved.numel(), ws,
                    ws.numel())
    _check(st, "lh_forward")
    return o, saved, plan


def backward(q, k, v, dout, saved, plan, grad_dtype=None, ws=None):
    """(dq, dk, dv) with the forward's selection frozen."""
    B, H, N, d = _shape(q, k, v)
    dev = q.device
    dout = dout.contiguous()
    _require("dout", dout, q.shape, device=dev)
    _require_bytes("saved", saved, dev)
    _require_bytes("ws", ws, dev)
    _same_problem(plan, B, H, N, d, q.dtype)
    grad_dtype = grad_dtype or q.dtype
    dq = torch.empty((B, H, N, d), dtype=grad_dtype, device=dev)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    if ws is None:
        ws = torch.empty(plan.bwd_ws_bytes, dtype=torch.uint8, device=dev)
    st = lh_backward(q, k, v, dout, dtype_code(dout.dtype), saved, saved.numel(), dq, dk, dv,
                     dtype_code(grad_dtype), *plan.args()[:7], plan.io, ws, ws.numel())
    _check(st, "lh_backward")
    return dq, dk, dv


def saved_view(saved, plan, name):
    """Typed view of one array inside the saved buffer (see lighthouse.h)."""
    lay = plan.layout
    BH, P, S, d = plan.B * plan.H, lay["P"], lay["S"], plan.d
    io = torch.bfloat16 if plan.io == LH_BF16 else torch.float32
    spec = {
        "scores": (torch.float32, (BH, 2, P)), "flags": (torch.uint8, (BH, P)), "slot": (torch.int32, (BH, P)),
        "coords": (torch.int32, (BH, S)), "qt": (io, (BH, lay["Sv"], d)), "kt": (io, (BH, lay["Sv"], d)),
        "vt": (io, (BH, lay["Sv"], d)),
        "ot": (torch.float32, (BH, S, d)), "lse": (torch.float32, (BH, S)),
    }[name]
    dt, shape = spec
    n = 1
    for x in shape:
        n *= x
    nbytes = n * torch.tensor([], dtype=dt).element_size()
    off = lay[name]
    return saved[off:off + nbytes].view(dt).view(shape)


class LighthouseAttention(torch.autograd.Function):
    """autograd wrapper: forward and backward both run in liblighthouse.

    q, k, v may be any strided [B, H, N, d] views (e.g. [B, N, H, d] tensors
    transposed): the library is given contiguous copies, and those copies (the
    inputs themselves when already contiguous) are what the backward receives,
    so it sees exactly the operands the forward ran on.  The gradients come
    back contiguous in the [B, H, N, d] shape of the inputs."""

    @staticmethod
    def forward(ctx, q, k, v, L, p, topk):
        qc, kc, vc = q.contiguous(), k.contiguous(), v.contiguous()
        o, saved, plan = forward(qc, kc, vc, L, p, topk)
        ctx.save_for_backward(qc, kc, vc, saved)
        ctx.plan = plan
        return o

    @staticmethod
    def backward(ctx, do):
        qc, kc, vc, saved = ctx.saved_tensors
        dq, dk, dv = backward(qc, kc, vc, do.contiguous(), saved, ctx.plan)
        return dq, dk, dv, None, None, None


# ---------------------------------------------------------------------------
# projection-inclusive layer
# ---------------------------------------------------------------------------
class LayerPlan:
    """Sizes and layouts for one (B, H, N, d_model, d, L, p, topk, io) layer."""

    def __init__(self, B, H, N, d_model, d, L, p, topk, io):
        self.B, self.H, self.N, self.d_model, self.d = B, H, N, d_model, d
        self.L, self.p, self.topk, self.io = L, p, topk, dtype_code(io)
        st, self.S, self.saved_bytes, self.fwd_ws_bytes, self.bwd_ws_bytes = lh_layer_query(*self.args())
        _check(st, "lh_layer_query")
        st, self.layout = lh_layer_saved_layout(*self.args())
        _check(st, "lh_layer_saved_layout")
        self.inner = Plan(B, H, N, d, L, p, topk, self.io)

    def args(self):
        return (self.B, self.H, self.N, self.d_model, self.d, self.L, self.p, self.topk, self.io)

    def view(self, saved, name):
        """q, k, v, o [B, H, N, d] (io dtype) inside the layer's saved buffer, or
        the Lighthouse saved buffer itself ('inner')."""
        if name == "inner":
            off = self.layout["inner"]
            return saved[off:off + self.layout["inner_bytes"]]
        io = torch.bfloat16 if self.io == LH_BF16 else torch.float32
        n = self.B * self.H * self.N * self.d
        off = self.layout[name]
        return saved[off:off + n * (2 if self.io == LH_BF16 else 4)].view(io).view(self.B, self.H, self.N, self.d)


def _layer_shape(x, wq, wk, wv, wo, H):
    """(B, N, d_model, d) of the layer, with every operand checked against x."""
    _require("x", x)
    if x.dim() != 3:
        raise ValueError(f"x must be a [B, N, d_model] tensor, got shape {tuple(x.shape)}")
    B, N, dm = x.shape
    if wq.dim() != 2 or wq.shape[1] % H:
        raise ValueError(f"wq must be [d_model, H d] with H = {H}, got shape {tuple(wq.shape)}")
    d = wq.shape[1] // H
    for name, w, shape in (("wq", wq, (dm, H * d)), ("wk", wk, (dm, H * d)), ("wv", wv, (dm, H * d)),
                           ("wo", wo, (H * d, dm))):
        _require(name, w, shape, x.dtype, x.device)
    return B, N, dm, d


def _same_layer(plan, B, H, N, dm, d, io):
    got = (plan.B, plan.H, plan.N, plan.d_model, plan.d, plan.io)
    if got != (B, H, N, dm, d, dtype_code(io)):
        raise ValueError(f"plan was made for (B, H, N, d_model, d, io) = {got}, not for these inputs")


def layer_forward(x, wq, wk, wv, wo, H, L, p, topk, y_dtype=None, plan=None, saved=None, ws=None):
    """Y of the layer for x [B, N, d_model].  Returns (y, saved, plan)."""
    B, N, dm, d = _layer_shape(x, wq, wk, wv, wo, H)
    _require_bytes("saved", saved, x.device)
    _require_bytes("ws", ws, x.device)
    plan = plan or LayerPlan(B, H, N, dm, d, L, p, topk, x.dtype)
    _same_layer(plan, B, H, N, dm, d, x.dtype)
    y_dtype = y_dtype or x.dtype
    y = torch.empty((B, N, dm), dtype=y_dtype, device=x.device)
    if saved is None:
        saved = torch.empty(plan.saved_bytes, dtype=torch.uint8, device=x.device)
    if ws is None:
        ws = torch.empty(plan.fwd_ws_bytes, dtype=torch.uint8, device=x.device)
    st = lh_layer_forward(x, wq, wk, wv, wo, y, y_dtype, *plan.args(), saved, saved.numel(), ws, ws.numel())
    _check(st, "lh_layer_forward")
    return y, saved, plan


def layer_backward(x, wq, wk, wv, wo, dy, saved, plan, dx_dtype=None, ws=None):
    """(dx, dwq, dwk, dwv, dwo) with the forward's selection frozen."""
    B, N, dm, d = _layer_shape(x, wq, wk, wv, wo, plan.H)
    dy = dy.contiguous()
    _require("dy", dy, x.shape, x.dtype, x.device)
    _require_bytes("saved", saved, x.device)
    _require_bytes("ws", ws, x.device)
    _same_layer(plan, B, plan.H, N, dm, d, x.dtype)
    dx_dtype = dx_dtype or x.dtype
    dev = x.device
    dx = torch.empty(x.shape, dtype=dx_dtype, device=dev)
    dws = [torch.empty(w.shape, dtype=torch.float32, device=dev) for w in (wq, wk, wv, wo)]
    if ws is None:
        ws = torch.empty(plan.bwd_ws_bytes, dtype=torch.uint8, device=dev)
    st = lh_layer_backward(x, wq, wk, wv, wo, dy, saved, saved.numel(), dx, dx_dtype, *dws,
                           *plan.args(), ws, ws.numel())
    _check(st, "lh_layer_backward")
    return (dx, *dws)
