"""Python binding of libgconv.so, the MI355X FP32 NCHW convolution library.

Argument marshalling only: every function here forwards to the C entry
point of the same name declared in include/gconv.h, passing device pointers
taken from torch tensors (or raw integers) and the current HIP stream.
Every step of the computation runs in the library's HIP kernels; there is
no CPU or PyTorch fallback, and importing this package fails when the
library has not been built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# GCONV_SANITIZED=1 loads the build whose host code carries AddressSanitizer
# and UndefinedBehaviorSanitizer (build.py --sanitize; the process must
# preload clang's ASan runtime, as tests/sanitize_host.py does)
LIB_PATH = os.path.join(_HERE, "libgconv_san.so" if os.environ.get("GCONV_SANITIZED") == "1" else "libgconv.so")

GCONV_OK = 0
GCONV_ERR_INVALID_ARG = 1
GCONV_ERR_WORKSPACE = 2
GCONV_ERR_UNSUPPORTED = 3
GCONV_ERR_LAUNCH = 4
GCONV_ERR_SCRATCH_LIMIT = 5

ALGO_AUTO = 0
ALGO_DIRECT = 1
ALGO_GROUPED3X3 = 2
ALGO_IGEMM = 3
ALGO_DEPTHWISE = 4
ALGO_NAMES = {ALGO_AUTO: "auto", ALGO_DIRECT: "direct", ALGO_GROUPED3X3: "grouped3x3", ALGO_IGEMM: "igemm",
              ALGO_DEPTHWISE: "depthwise"}

FUSED_AUTO = 0
FUSED_STORE = 1
FUSED_RECOMPUTE = 2
FUSED_ONEPASS = 3
FUSED_NAMES = {FUSED_AUTO: "auto", FUSED_STORE: "store", FUSED_RECOMPUTE: "recompute", FUSED_ONEPASS: "onepass"}

EXPORTED = (
    "conv_desc_create", "conv_desc_create_2d", "conv_desc_destroy", "conv_desc_get_output_dims", "conv_desc_set_algo",
    "conv_desc_get_algo", "conv_desc_set_fused_variant", "conv_desc_get_fused_variant", "conv_desc_set_fused_wait",
    "conv_fwd",
    "conv_fused_gn_workspace_size", "conv_fused_gn_fwd", "conv_fused_gn_fwd_noalloc", "gconv_time_graph",
    "gconv_probe_peaks", "gconv_probe_vector_peaks", "gconv_probe_copy", "conv_fused_gn_noalloc_limit", "gconv_status_string", "gconv_last_launch_error",
)

if not os.path.exists(LIB_PATH):
    raise ImportError("libgconv.so is not built; run `python grouped_convolution_conv_amd/build.py` "
                      "(or __graft_entry__.build())")

# One HIP runtime per process: torch ships its own libamdhip64 (soname
# libamdhip64.so.7, loaded under the file name libamdhip64.so).  Importing
# torch first makes libgconv.so's libamdhip64.so.7 dependency resolve to that
# already-loaded runtime; loading libgconv.so first would pull in a second
# runtime from /opt/rocm, and the two do not share devices or streams.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)
_i, _p, _sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
_lib.conv_desc_create.argtypes = [ctypes.POINTER(_p)] + [_i] * 11
_lib.conv_desc_create_2d.argtypes = [ctypes.POINTER(_p)] + [_i] * 14
_lib.conv_desc_destroy.argtypes = [_p]
_lib.conv_desc_get_output_dims.argtypes = [_p, ctypes.POINTER(_i), ctypes.POINTER(_i)]
_lib.conv_desc_set_algo.argtypes = [_p, _i]
_lib.conv_desc_get_algo.argtypes = [_p, ctypes.POINTER(_i)]
_lib.conv_desc_set_fused_variant.argtypes = [_p, _i]
_lib.conv_desc_get_fused_variant.argtypes = [_p, _i, ctypes.POINTER(_i)]
_lib.conv_desc_set_fused_wait.argtypes = [_p, _i]
_lib.conv_fwd.argtypes = [_p, _p, _p, _p, _p, _p]
_lib.conv_fused_gn_workspace_size.argtypes = [_p, _i, ctypes.POINTER(_sz)]
_lib.conv_fused_gn_fwd.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i, ctypes.c_float, _p, _p, _sz, _p]
_lib.conv_fused_gn_fwd_noalloc.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i, ctypes.c_float, _p, _p]
_lib.conv_fused_gn_noalloc_limit.argtypes = []
_lib.gconv_time_graph.argtypes = [_p, _i, ctypes.POINTER(_p), ctypes.POINTER(_p), _i, _p, _p, _p, _p, _p, _i,
                                  ctypes.c_float, _p, _sz, _i, _i, ctypes.POINTER(ctypes.c_float), _p]
_lib.gconv_probe_peaks.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float), _p, _p]
_lib.gconv_probe_vector_peaks.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float), _p, _p]
_lib.gconv_probe_copy.argtypes = [ctypes.POINTER(ctypes.c_float), _p, _p, _sz, _p]
_lib.gconv_status_string.argtypes = [_i]
_lib.gconv_status_string.restype = ctypes.c_char_p
_lib.gconv_last_launch_error.argtypes = []
_lib.gconv_last_launch_error.restype = ctypes.c_char_p
for _name in EXPORTED[:-2]:
    getattr(_lib, _name).restype = _i
_lib.conv_fused_gn_noalloc_limit.restype = _sz


class GconvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = "%s: %s (status %d)" % (fn, gconv_status_string(status), status)
        if status == GCONV_ERR_LAUNCH:
            msg += ": " + gconv_last_launch_error()
        super().__init__(msg)
        self.status = status


def gconv_last_launch_error() -> str:
    return _lib.gconv_last_launch_error().decode()


def gconv_status_string(status: int) -> str:
    return _lib.gconv_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != GCONV_OK:
        raise GconvError(fn, status)


class ConvDesc:
    """Owns a gconv_desc_t; released on close() or garbage collection."""

    def __init__(self, handle: int, geom: tuple):
        self._h = ctypes.c_void_p(handle)
        self.geom = geom  # (N, C, H, W, K, R, S, stride, pad, dilation, groups)
        ho, wo = _i(), _i()
        _check("conv_desc_get_output_dims", _lib.conv_desc_get_output_dims(self._h, ctypes.byref(ho),
                                                                           ctypes.byref(wo)))
        N, C, H, W, K, R, S = geom[:7]
        # element counts of x, w, y and a per-channel vector, checked against
        # tensor arguments before every call
        self.sizes = dict(x=N * C * H * W, w=K * (C // geom[10]) * R * S, y=N * K * ho.value * wo.value, vec=K)

    @property
    def handle(self):
        return self._h

    def close(self):
        if self._h is not None and self._h.value:
            _lib.conv_desc_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def conv_desc_create(N, C, H, W, K, R, S, stride=1, pad=0, dilation=1, groups=1) -> ConvDesc:
    """Descriptor with symmetric stride, padding and dilation; any of them
    given as an (h, w) pair goes to conv_desc_create_2d."""
    if any(isinstance(v, (tuple, list)) for v in (stride, pad, dilation)):
        pair = lambda v: tuple(v) if isinstance(v, (tuple, list)) else (v, v)
        return conv_desc_create_2d(N, C, H, W, K, R, S, pair(stride), pair(pad), pair(dilation), groups)
    h = ctypes.c_void_p()
    _check("conv_desc_create", _lib.conv_desc_create(ctypes.byref(h), N, C, H, W, K, R, S, stride, pad,
                                                     dilation, groups))
    return ConvDesc(h.value, (N, C, H, W, K, R, S, stride, pad, dilation, groups))


def conv_desc_create_2d(N, C, H, W, K, R, S, stride=(1, 1), pad=(0, 0), dilation=(1, 1), groups=1) -> ConvDesc:
    """Descriptor with per-axis stride, padding and dilation, each an (h, w) pair."""
    (sh, sw), (ph, pw), (dh, dw) = stride, pad, dilation
    h = ctypes.c_void_p()
    _check("conv_desc_create_2d", _lib.conv_desc_create_2d(ctypes.byref(h), N, C, H, W, K, R, S, sh, sw, ph, pw,
                                                           dh, dw, groups))
    return ConvDesc(h.value, (N, C, H, W, K, R, S, (sh, sw), (ph, pw), (dh, dw), groups))


def conv_desc_destroy(desc: ConvDesc) -> None:
    desc.close()


def conv_desc_get_output_dims(desc: ConvDesc):
    ho, wo = _i(), _i()
    _check("conv_desc_get_output_dims", _lib.conv_desc_get_output_dims(desc.handle, ctypes.byref(ho),
                                                                       ctypes.byref(wo)))
    return ho.value, wo.value


def conv_desc_set_algo(desc: ConvDesc, algo: int) -> None:
    _check("conv_desc_set_algo", _lib.conv_desc_set_algo(desc.handle, algo))


def conv_desc_get_algo(desc: ConvDesc) -> int:
    a = _i()
    _check("conv_desc_get_algo", _lib.conv_desc_get_algo(desc.handle, ctypes.byref(a)))
    return a.value


def conv_desc_set_fused_variant(desc: ConvDesc, variant: int) -> None:
    _check("conv_desc_set_fused_variant", _lib.conv_desc_set_fused_variant(desc.handle, variant))


def conv_desc_set_fused_wait(desc: ConvDesc, wait_us: int) -> None:
    _check("conv_desc_set_fused_wait", _lib.conv_desc_set_fused_wait(desc.handle, wait_us))


def conv_desc_get_fused_variant(desc: ConvDesc, gn_groups: int) -> int:
    v = _i()
    _check("conv_desc_get_fused_variant", _lib.conv_desc_get_fused_variant(desc.handle, gn_groups, ctypes.byref(v)))
    return v.value


def _ptr(t, numel=None, name="tensor"):
    """Device address of a torch tensor (checked: cuda, float32, contiguous,
    and `numel` elements when given) or a raw int, which is passed as is."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    import torch
    if not t.is_cuda:
        raise ValueError("%s must live on the GPU" % name)
    if t.dtype != torch.float32:
        raise ValueError("%s must be float32, got %s" % (name, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if numel is not None and t.numel() != numel:
        raise ValueError("%s has %d elements; the descriptor needs %d" % (name, t.numel(), numel))
    return t.data_ptr()


def _workspace_ptr(ws):
    if ws is None or isinstance(ws, int):
        return ws
    if not ws.is_cuda:
        raise ValueError("workspace must live on the GPU")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return ws.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def conv_fwd(desc: ConvDesc, x, w, bias, y, stream=None) -> None:
    """y = conv(x, w) [+ bias] on `stream` (default: torch's current stream)."""
    n = desc.sizes
    _check("conv_fwd", _lib.conv_fwd(desc.handle, _ptr(x, n["x"], "x"), _ptr(w, n["w"], "w"),
                                     _ptr(bias, n["vec"], "bias"), _ptr(y, n["y"], "y"), _stream(stream)))


def conv_fused_gn_workspace_size(desc: ConvDesc, gn_groups: int) -> int:
    n = _sz()
    _check("conv_fused_gn_workspace_size", _lib.conv_fused_gn_workspace_size(desc.handle, gn_groups,
                                                                             ctypes.byref(n)))
    return n.value


def conv_fused_gn_fwd(desc: ConvDesc, x, w, bias, scale, gamma, beta, gn_groups: int, eps: float, y,
                      workspace, workspace_bytes: int = None, stream=None) -> None:
    """conv -> +bias -> *scale -> sigmoid -> GroupNorm(gn_groups, eps, gamma, beta) into y."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    n = desc.sizes
    v = n["vec"]
    _check("conv_fused_gn_fwd", _lib.conv_fused_gn_fwd(desc.handle, _ptr(x, n["x"], "x"), _ptr(w, n["w"], "w"),
                                                       _ptr(bias, v, "bias"), _ptr(scale, v, "scale"),
                                                       _ptr(gamma, v, "gamma"), _ptr(beta, v, "beta"), gn_groups,
                                                       float(eps), _ptr(y, n["y"], "y"), _workspace_ptr(workspace),
                                                       workspace_bytes, _stream(stream)))


def conv_fused_gn_fwd_noalloc(desc: ConvDesc, x, w, bias, scale, gamma, beta, gn_groups: int, eps: float, y,
                              stream=None) -> None:
    """The fused chain without a caller workspace: the library's static
    scratch array (conv_fused_gn_noalloc_limit() bytes per GPU) holds the
    GroupNorm statistics.  Calls that overlap on one GPU race."""
    n = desc.sizes
    v = n["vec"]
    _check("conv_fused_gn_fwd_noalloc",
           _lib.conv_fused_gn_fwd_noalloc(desc.handle, _ptr(x, n["x"], "x"), _ptr(w, n["w"], "w"),
                                          _ptr(bias, v, "bias"), _ptr(scale, v, "scale"), _ptr(gamma, v, "gamma"),
                                          _ptr(beta, v, "beta"), gn_groups, float(eps), _ptr(y, n["y"], "y"),
                                          _stream(stream)))


def conv_fused_gn_noalloc_limit() -> int:
    """Bytes of the static scratch array behind conv_fused_gn_fwd_noalloc."""
    return int(_lib.conv_fused_gn_noalloc_limit())


def gconv_time_graph(desc: ConvDesc, xs, ys, w, bias=None, launches: int = 1, replays: int = 1, fused=None,
                     stream=None):
    """Per-launch milliseconds of `replays` replays of a graph of `launches` calls.

    xs, ys: sequences of input / output tensors (or raw pointers) rotated over
    the launches.  fused: None for conv_fwd, else a dict with scale, gamma,
    beta, gn_groups, eps and workspace for conv_fused_gn_fwd.  Returns a
    list of `replays` floats."""
    if len(xs) != len(ys) or not xs:
        raise ValueError("xs and ys must be non-empty sequences of the same length")
    n = len(xs)
    sz = desc.sizes
    xa = (_p * n)(*[_ptr(t, sz["x"], "x") for t in xs])
    ya = (_p * n)(*[_ptr(t, sz["y"], "y") for t in ys])
    out = (ctypes.c_float * replays)()
    if fused is None:
        args = (0, None, None, None, 0, 0.0, None, 0)
    else:
        ws = fused.get("workspace")
        wsb = fused.get("workspace_bytes")
        if wsb is None:
            wsb = ws.numel() * ws.element_size() if ws is not None else 0
        v = sz["vec"]
        args = (1, _ptr(fused["scale"], v, "scale"), _ptr(fused.get("gamma"), v, "gamma"),
                _ptr(fused.get("beta"), v, "beta"), int(fused["gn_groups"]), float(fused["eps"]), _workspace_ptr(ws),
                wsb)
    fl, sc, ga, be, gg, eps, wsp, wsb = args
    _check("gconv_time_graph", _lib.gconv_time_graph(desc.handle, fl, xa, ya, n, _ptr(w, sz["w"], "w"),
                                                     _ptr(bias, sz["vec"], "bias"), sc, ga, be, gg,
                                                     eps, wsp, wsb, launches, replays, out, _stream(stream)))
    return list(out)


def gconv_probe_peaks(sink, stream=None):
    """Measured (FP32 MFMA, non-packed FP32 FMA) peaks of the current GPU in
    TFLOP/s.  sink: a device tensor (or raw pointer) of at least 4 bytes."""
    m, f = ctypes.c_float(), ctypes.c_float()
    _check("gconv_probe_peaks", _lib.gconv_probe_peaks(ctypes.byref(m), ctypes.byref(f), _ptr(sink), _stream(stream)))
    return float(m.value), float(f.value)


def gconv_probe_vector_peaks(sink, stream=None):
    """Measured (non-packed FP32 FMA, FP64 FMA) rates of the current GPU in
    TFLOP/s.  sink: a device tensor (or raw pointer) of at least 4 bytes."""
    a, b = ctypes.c_float(), ctypes.c_float()
    _check("gconv_probe_vector_peaks",
           _lib.gconv_probe_vector_peaks(ctypes.byref(a), ctypes.byref(b), _ptr(sink), _stream(stream)))
    return float(a.value), float(b.value)


def gconv_probe_copy(dst, src, nbytes: int = None, stream=None) -> float:
    """Streaming copy rate (bytes read + written per second, in GB/s) of the
    library's own copy kernel over `nbytes` (default: all of src)."""
    if nbytes is None:
        nbytes = src.numel() * src.element_size()
    g = ctypes.c_float()
    _check("gconv_probe_copy", _lib.gconv_probe_copy(ctypes.byref(g), _ptr(dst), _ptr(src), int(nbytes),
                                                     _stream(stream)))
    return float(g.value)


def library():
    """The loaded ctypes library (for symbol checks)."""
    return _lib
