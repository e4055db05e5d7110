"""Thin ctypes binding over libssm_scan.so (argument marshalling only).

Every step of the selective scan runs in the library's HIP kernels; this
module checks tensor dtypes, shapes, devices and contiguity, allocates outputs
with torch (device memory and streams are the only things torch provides), and
passes raw pointers and the current HIP stream through the C ABI declared in
include/ssm_scan.h.  There is no fallback: if the library is missing the
import fails with an error that says how to build it.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssm_scan.so")

SSM_F32 = 0
SSM_BF16 = 1
SSM_OK = 0

# ssm_disc_t: how B is discretized by the _ex entry points.
DISC_CODES = {"delta_b": 0, "zoh": 1}

STATUS_NAMES = {
    0: "SSM_OK",
    1: "SSM_ERR_NULL",
    2: "SSM_ERR_SHAPE",
    3: "SSM_ERR_DSTATE_UNSUPPORTED",
    4: "SSM_ERR_DTYPE",
    5: "SSM_ERR_ALIGN",
    6: "SSM_ERR_ALIAS",
    7: "SSM_ERR_HIP",
    8: "SSM_ERR_UNSUPPORTED",
}

# Every symbol the header declares, with its ctypes signature.
_I64 = ctypes.c_int64
_P = ctypes.c_void_p
_I = ctypes.c_int
SIGNATURES = {
    "ssm_scan_fwd": (_I, [_I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P]),
    "ssm_state_update": (_I, [_I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P]),
    "ssm_scan_fwd_ex": (_I, [_I64, _I64, _I64, _I64, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P]),
    "ssm_state_update_ex": (_I, [_I64, _I64, _I64, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P]),
    "ssm_scan_fwd_complex": (_I, [_I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P]),
    "ssm_state_update_complex": (_I, [_I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P]),
    "ssm_conv_scan_fwd": (_I, [_I64, _I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P,
                               _P, _P, _P, _P]),
    "ssm_conv_bwd": (_I, [_I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P]),
    "ssm_scan_bwd": (_I, [_I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                          _P, _P, _P, _P, _P]),
    "ssm_scan_bwd_ex": (_I, [_I64, _I64, _I64, _I64, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P,
                             _P, _P, _P, _P, _P, _P, _P]),
    "ssm_scan_bwd_complex": (_I, [_I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P,
                                  _P, _P, _P, _P, _P, _P, _P, _P]),
    "ssm_scan_ckpt_bytes": (_I, [_I64, _I64, _I64, _I64, _I, ctypes.POINTER(_I64)]),
    "ssm_scan_fwd_save": (_I, [_I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P]),
    "ssm_scan_bwd_saved": (_I, [_I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P,
                                _P, _P, _P, _P, _P, _P, _P]),
    "ssm_scan_bwd_saved_noalloc": (_I, [_I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P,
                                        _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "ssm_scan_fwd_plan": (_I, [_I64, _I64, _I64, _I64, _I, ctypes.POINTER(_I), ctypes.POINTER(_I64),
                              ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "ssm_scan_fwd_plan_ex": (_I, [_I64, _I64, _I64, _I64, _I, _I, _I64, ctypes.POINTER(_I), ctypes.POINTER(_I64),
                                 ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "ssm_status_string": (ctypes.c_char_p, [_I]),
    "ssm_last_hip_error": (_I, []),
    "ssm_abi_version": (_I, []),
}


class SsmError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, fn, status, lib):
        self.status = status
        self.name = STATUS_NAMES.get(status, "status %d" % status)
        text = lib.ssm_status_string(status).decode()
        msg = "%s returned %s: %s" % (fn, self.name, text)
        if self.name == "SSM_ERR_HIP":
            msg += " (hipError %d)" % lib.ssm_last_hip_error()
        super().__init__(msg)


_lib = None


def load_library(path=None):
    """Load libssm_scan.so (LIB_PATH unless another path is given) and attach the ctypes signatures."""
    global _lib
    default = path is None or path == LIB_PATH
    path = LIB_PATH if path is None else path
    if _lib is not None and default:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            "libssm_scan.so not found at %s; build it with "
            "`python selective_state_space_65_amd/build.py` (hipcc, gfx950)" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if default:
        _lib = lib
    return lib


def _check(fn, status):
    if status != SSM_OK:
        raise SsmError(fn, status, load_library())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _io_code(dtype):
    import torch
    if dtype == torch.float32:
        return SSM_F32
    if dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError("io tensors must be float32 or bfloat16, got %s" % dtype)


def _need(t, name, shape, dtype, device):
    if t.shape != shape:
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.dtype != dtype:
        raise TypeError("%s: expected %s, got %s" % (name, dtype, t.dtype))
    if t.device != device:
        raise ValueError("%s: expected device %s, got %s" % (name, device, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream(device, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


PATH_NAMES = {0: "split", 1: "segmented", 2: "generic", 3: "chunked"}


def scan_plan(batch, dim, dstate, seqlen, io_dtype, with_path=False, disc="delta_b", conv_width=0):
    """(segments, segment_len, scratch_bytes) the library uses for this shape.

    With with_path=True the kernel path name ("split", "chunked", "segmented" or
    "generic") is prepended to the tuple.  disc and conv_width name the entry
    point: ssm_scan_fwd_ex's discretization, ssm_conv_scan_fwd's conv width.
    """
    lib = load_library()
    path, seg, seglen, scratch = _I(), _I64(), _I64(), _I64()
    st = lib.ssm_scan_fwd_plan_ex(batch, dim, dstate, seqlen, _io_code(io_dtype), DISC_CODES[disc], conv_width,
                                  ctypes.byref(path), ctypes.byref(seg), ctypes.byref(seglen), ctypes.byref(scratch))
    _check("ssm_scan_fwd_plan_ex", st)
    if with_path:
        return PATH_NAMES[path.value], seg.value, seglen.value, scratch.value
    return seg.value, seglen.value, scratch.value


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, h0=None,
             out=None, last_state=None, return_last_state=True, stream=None):
    """Selective scan over the sequence (ssm_scan_fwd); returns (y, last_state).

    u, delta, z: (batch, dim, seqlen); B, C: (batch, dstate, seqlen), all in
    one io dtype (float32 or bfloat16).  A: (dim, dstate), D and delta_bias:
    (dim,), h0: (batch, dim, dstate), all float32.  y has the io dtype;
    last_state is float32 (None when return_last_state is False).  h0 may be
    the same tensor as last_state to carry the state in place.
    """
    return _scan_fwd(None, u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, out, last_state,
                     return_last_state, stream)


def scan_fwd_ex(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, h0=None, disc="zoh",
                out=None, last_state=None, return_last_state=True, stream=None):
    """scan_fwd with a choice of discretization for B (ssm_scan_fwd_ex).

    disc: "zoh" (exact zero-order hold, Bbar = (exp(Delta A) - 1) / A * B) or
    "delta_b" (Bbar = Delta * B, as scan_fwd).  Everything else as scan_fwd.
    """
    if disc not in DISC_CODES:
        raise ValueError("disc must be one of %s" % sorted(DISC_CODES))
    return _scan_fwd(DISC_CODES[disc], u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, out, last_state,
                     return_last_state, stream)


def _scan_fwd(disc, u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, out, last_state, return_last_state,
              stream):
    import torch
    if u.dim() != 3:
        raise ValueError("u must be (batch, dim, seqlen)")
    batch, dim, seqlen = u.shape
    dstate = A.shape[-1]
    dev = u.device
    io = u.dtype
    _need(u, "u", (batch, dim, seqlen), io, dev)
    _need(delta, "delta", (batch, dim, seqlen), io, dev)
    _need(A, "A", (dim, dstate), torch.float32, dev)
    _need(B, "B", (batch, dstate, seqlen), io, dev)
    _need(C, "C", (batch, dstate, seqlen), io, dev)
    if D is not None:
        _need(D, "D", (dim,), torch.float32, dev)
    if z is not None:
        _need(z, "z", (batch, dim, seqlen), io, dev)
    if delta_bias is not None:
        _need(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    if h0 is not None:
        _need(h0, "h0", (batch, dim, dstate), torch.float32, dev)
    if out is None:
        out = torch.empty((batch, dim, seqlen), dtype=io, device=dev)
    else:
        _need(out, "out", (batch, dim, seqlen), io, dev)
    if last_state is None and return_last_state:
        last_state = torch.empty((batch, dim, dstate), dtype=torch.float32, device=dev)
    elif last_state is not None:
        _need(last_state, "last_state", (batch, dim, dstate), torch.float32, dev)
    lib = load_library()
    tail = (_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            1 if delta_softplus else 0, _ptr(h0), _ptr(out), _ptr(last_state), _stream(dev, stream))
    if disc is None:
        _check("ssm_scan_fwd", lib.ssm_scan_fwd(batch, dim, dstate, seqlen, _io_code(io), *tail))
    else:
        _check("ssm_scan_fwd_ex", lib.ssm_scan_fwd_ex(batch, dim, dstate, seqlen, _io_code(io), disc, *tail))
    return out, last_state


def scan_fwd_complex(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, h0=None,
                     out=None, last_state=None, return_last_state=True, stream=None):
    """Selective scan with a complex diagonal A (ssm_scan_fwd_complex); returns (y, last_state).

    Complex arrays are real tensors whose last dimension holds (re, im):
    A (dim, dstate, 2) float32; B, C (batch, dstate, seqlen, 2) in the io dtype;
    h0 and last_state (batch, dim, dstate, 2) float32.  u, delta, z, D,
    delta_bias and y are as in scan_fwd.  dstate counts complex states.
    """
    import torch
    if u.dim() != 3:
        raise ValueError("u must be (batch, dim, seqlen)")
    batch, dim, seqlen = u.shape
    if A.dim() != 3 or A.shape[-1] != 2:
        raise ValueError("A must be (dim, dstate, 2)")
    dstate = A.shape[1]
    dev = u.device
    io = u.dtype
    _need(u, "u", (batch, dim, seqlen), io, dev)
    _need(delta, "delta", (batch, dim, seqlen), io, dev)
    _need(A, "A", (dim, dstate, 2), torch.float32, dev)
    _need(B, "B", (batch, dstate, seqlen, 2), io, dev)
    _need(C, "C", (batch, dstate, seqlen, 2), io, dev)
    if D is not None:
        _need(D, "D", (dim,), torch.float32, dev)
    if z is not None:
        _need(z, "z", (batch, dim, seqlen), io, dev)
    if delta_bias is not None:
        _need(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    if h0 is not None:
        _need(h0, "h0", (batch, dim, dstate, 2), torch.float32, dev)
    if out is None:
        out = torch.empty((batch, dim, seqlen), dtype=io, device=dev)
    else:
        _need(out, "out", (batch, dim, seqlen), io, dev)
    if last_state is None and return_last_state:
        last_state = torch.empty((batch, dim, dstate, 2), dtype=torch.float32, device=dev)
    elif last_state is not None:
        _need(last_state, "last_state", (batch, dim, dstate, 2), torch.float32, dev)
    lib = load_library()
    st = lib.ssm_scan_fwd_complex(batch, dim, dstate, seqlen, _io_code(io), _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                                  _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), 1 if delta_softplus else 0, _ptr(h0),
                                  _ptr(out), _ptr(last_state), _stream(dev, stream))
    _check("ssm_scan_fwd_complex", st)
    return out, last_state


def scan_bwd_complex(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, delta_softplus=False, h0=None,
                     dlast=None, need=("dD", "dz", "ddelta_bias", "dh0"), stream=None):
    """Gradients for scan_fwd_complex (ssm_scan_bwd_complex); complex arrays as real tensors with a trailing
    (re, im) dimension, their gradients as (d/dRe, d/dIm) pairs in the same layout.  Returns a dict as scan_bwd."""
    import torch
    if u.dim() != 3:
        raise ValueError("u must be (batch, dim, seqlen)")
    batch, dim, seqlen = u.shape
    if A.dim() != 3 or A.shape[-1] != 2:
        raise ValueError("A must be (dim, dstate, 2)")
    dstate = A.shape[1]
    dev = u.device
    io = u.dtype
    f32 = torch.float32
    _need(u, "u", (batch, dim, seqlen), io, dev)
    _need(delta, "delta", (batch, dim, seqlen), io, dev)
    _need(A, "A", (dim, dstate, 2), f32, dev)
    _need(B, "B", (batch, dstate, seqlen, 2), io, dev)
    _need(C, "C", (batch, dstate, seqlen, 2), io, dev)
    _need(dy, "dy", (batch, dim, seqlen), io, dev)
    if D is not None:
        _need(D, "D", (dim,), f32, dev)
    if z is not None:
        _need(z, "z", (batch, dim, seqlen), io, dev)
    if delta_bias is not None:
        _need(delta_bias, "delta_bias", (dim,), f32, dev)
    if h0 is not None:
        _need(h0, "h0", (batch, dim, dstate, 2), f32, dev)
    if dlast is not None:
        _need(dlast, "dlast", (batch, dim, dstate, 2), f32, dev)
    g = dict(du=torch.empty_like(u), ddelta=torch.empty_like(u), dA=torch.empty((dim, dstate, 2), dtype=f32, device=dev),
             dB=torch.empty((batch, dstate, seqlen, 2), dtype=f32, device=dev),
             dC=torch.empty((batch, dstate, seqlen, 2), dtype=f32, device=dev),
             dD=torch.empty(dim, dtype=f32, device=dev) if "dD" in need else None,
             dz=torch.empty_like(u) if ("dz" in need and z is not None) else None,
             ddelta_bias=torch.empty(dim, dtype=f32, device=dev) if "ddelta_bias" in need else None,
             dh0=torch.empty((batch, dim, dstate, 2), dtype=f32, device=dev) if "dh0" in need else None)
    lib = load_library()
    st = lib.ssm_scan_bwd_complex(batch, dim, dstate, seqlen, _io_code(io), _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                                  _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), 1 if delta_softplus else 0, _ptr(h0),
                                  _ptr(dy), _ptr(dlast), _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]),
                                  _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["ddelta_bias"]), _ptr(g["dh0"]),
                                  _stream(dev, stream))
    _check("ssm_scan_bwd_complex", st)
    return g


def state_update_complex(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, out=None,
                         stream=None):
    """One decode step with complex A (ssm_state_update_complex), state updated in place; returns y (batch, dim).

    state (batch, dim, dstate, 2) float32; A (dim, dstate, 2) float32; B, C
    (batch, dstate, 2) in the io dtype; u, delta, z (batch, dim).
    """
    import torch
    if state.dim() != 4 or state.shape[-1] != 2:
        raise ValueError("state must be (batch, dim, dstate, 2)")
    batch, dim, dstate, _ = state.shape
    dev = state.device
    io = u.dtype
    _need(state, "state", (batch, dim, dstate, 2), torch.float32, dev)
    _need(u, "u", (batch, dim), io, dev)
    _need(delta, "delta", (batch, dim), io, dev)
    _need(A, "A", (dim, dstate, 2), torch.float32, dev)
    _need(B, "B", (batch, dstate, 2), io, dev)
    _need(C, "C", (batch, dstate, 2), io, dev)
    if D is not None:
        _need(D, "D", (dim,), torch.float32, dev)
    if z is not None:
        _need(z, "z", (batch, dim), io, dev)
    if delta_bias is not None:
        _need(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    if out is None:
        out = torch.empty((batch, dim), dtype=io, device=dev)
    else:
        _need(out, "out", (batch, dim), io, dev)
    lib = load_library()
    st = lib.ssm_state_update_complex(batch, dim, dstate, _io_code(io), _ptr(state), _ptr(u), _ptr(delta), _ptr(A),
                                      _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), 1 if delta_softplus else 0,
                                      _ptr(out), _stream(dev, stream))
    _check("ssm_state_update_complex", st)
    return out


def conv_scan_fwd(x, conv_weight, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
                  conv_bias=None, x_prev=None, conv_silu=True, h0=None, out=None, last_state=None, u_out=None,
                  return_last_state=True, stream=None):
    """Causal depthwise conv (+ silu) fused in front of the scan; returns (y, last_state).

    x: (batch, dim, seqlen) in the io dtype; conv_weight: (dim, K) float32 with
    K in 1..4 (conv_weight[:, K-1] multiplies the current token); conv_bias:
    (dim,) float32; x_prev: (batch, dim, K-1) in the io dtype, the inputs before
    token 0.  u = act(conv(x)) is rounded to the io dtype and scanned as
    scan_fwd would scan it; u_out, when given, receives it.  The other
    arguments are scan_fwd's.
    """
    import torch
    if x.dim() != 3:
        raise ValueError("x must be (batch, dim, seqlen)")
    batch, dim, seqlen = x.shape
    dstate = A.shape[-1]
    dev = x.device
    io = x.dtype
    if conv_weight.dim() != 2:
        raise ValueError("conv_weight must be (dim, K)")
    width = conv_weight.shape[1]
    _need(x, "x", (batch, dim, seqlen), io, dev)
    _need(conv_weight, "conv_weight", (dim, width), torch.float32, dev)
    if conv_bias is not None:
        _need(conv_bias, "conv_bias", (dim,), torch.float32, dev)
    if x_prev is not None and width > 1:
        _need(x_prev, "x_prev", (batch, dim, width - 1), io, dev)
    elif width == 1:
        x_prev = None
    _need(delta, "delta", (batch, dim, seqlen), io, dev)
    _need(A, "A", (dim, dstate), torch.float32, dev)
    _need(B, "B", (batch, dstate, seqlen), io, dev)
    _need(C, "C", (batch, dstate, seqlen), io, dev)
    if D is not None:
        _need(D, "D", (dim,), torch.float32, dev)
    if z is not None:
        _need(z, "z", (batch, dim, seqlen), io, dev)
    if delta_bias is not None:
        _need(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    if h0 is not None:
        _need(h0, "h0", (batch, dim, dstate), torch.float32, dev)
    if out is None:
        out = torch.empty((batch, dim, seqlen), dtype=io, device=dev)
    else:
        _need(out, "out", (batch, dim, seqlen), io, dev)
    if last_state is None and return_last_state:
        last_state = torch.empty((batch, dim, dstate), dtype=torch.float32, device=dev)
    elif last_state is not None:
        _need(last_state, "last_state", (batch, dim, dstate), torch.float32, dev)
    if u_out is not None:
        _need(u_out, "u_out", (batch, dim, seqlen), io, dev)
    lib = load_library()
    st = lib.ssm_conv_scan_fwd(batch, dim, dstate, seqlen, width, _io_code(io), _ptr(x), _ptr(conv_weight),
                               _ptr(conv_bias), _ptr(x_prev), 1 if conv_silu else 0, _ptr(delta), _ptr(A), _ptr(B),
                               _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), 1 if delta_softplus else 0, _ptr(h0),
                               _ptr(out), _ptr(last_state), _ptr(u_out), _stream(dev, stream))
    _check("ssm_conv_scan_fwd", st)
    return out, last_state


def conv_bwd(x, conv_weight, du, conv_bias=None, x_prev=None, conv_silu=True, stream=None):
    """Gradients of the conv of conv_scan_fwd for dL/du = du (ssm_conv_bwd).

    du is the gradient with respect to the u the scan consumed (scan_bwd's du).
    Returns a dict: dx (io dtype, like x), dconv_weight (dim, K) float32,
    dconv_bias (dim,) float32 and dx_prev (batch, dim, K-1) in the io dtype
    (the gradient for the x_prev history; zeros-shaped (batch, dim, 0) when K == 1).
    """
    import torch
    if x.dim() != 3:
        raise ValueError("x must be (batch, dim, seqlen)")
    batch, dim, seqlen = x.shape
    dev = x.device
    io = x.dtype
    if conv_weight.dim() != 2:
        raise ValueError("conv_weight must be (dim, K)")
    width = conv_weight.shape[1]
    _need(x, "x", (batch, dim, seqlen), io, dev)
    _need(du, "du", (batch, dim, seqlen), io, dev)
    _need(conv_weight, "conv_weight", (dim, width), torch.float32, dev)
    if conv_bias is not None:
        _need(conv_bias, "conv_bias", (dim,), torch.float32, dev)
    if x_prev is not None and width > 1:
        _need(x_prev, "x_prev", (batch, dim, width - 1), io, dev)
    elif width == 1:
        x_prev = None
    g = dict(dx=torch.empty_like(x), dconv_weight=torch.empty((dim, width), dtype=torch.float32, device=dev),
             dconv_bias=torch.empty(dim, dtype=torch.float32, device=dev),
             dx_prev=torch.empty((batch, dim, width - 1), dtype=io, device=dev))
    lib = load_library()
    st = lib.ssm_conv_bwd(batch, dim, seqlen, width, _io_code(io), _ptr(x), _ptr(conv_weight), _ptr(conv_bias),
                          _ptr(x_prev), 1 if conv_silu else 0, _ptr(du), _ptr(g["dx"]), _ptr(g["dconv_weight"]),
                          _ptr(g["dconv_bias"]), _ptr(g["dx_prev"]) if width > 1 else None, _stream(dev, stream))
    _check("ssm_conv_bwd", st)
    return g


def scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, delta_softplus=False, h0=None, dlast=None,
             need=("dD", "dz", "ddelta_bias", "dh0"), stream=None):
    """Gradients of sum(dy * y) + sum(dlast * last_state) for the scan of scan_fwd (ssm_scan_bwd).

    Returns a dict: du, ddelta (io dtype, like u); dA (dim, dstate), dB, dC
    (batch, dstate, seqlen) in float32; and, when named in `need`, dD and
    ddelta_bias (dim,) float32, dz (io dtype, only with z) and dh0 (batch, dim,
    dstate) float32.
    """
    return _scan_bwd(None, u, delta, A, B, C, dy, D, z, delta_bias, delta_softplus, h0, dlast, need, stream)


def scan_bwd_ex(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, delta_softplus=False, h0=None, dlast=None,
                disc="zoh", need=("dD", "dz", "ddelta_bias", "dh0"), stream=None):
    """scan_bwd for either discretization of B (ssm_scan_bwd_ex): the gradients of scan_fwd_ex with the same disc."""
    if disc not in DISC_CODES:
        raise ValueError("disc must be one of %s" % sorted(DISC_CODES))
    return _scan_bwd(None, u, delta, A, B, C, dy, D, z, delta_bias, delta_softplus, h0, dlast, need, stream,
                     disc=DISC_CODES[disc])


def scan_bwd_saved(u, delta, A, B, C, dy, ckpt, D=None, z=None, delta_bias=None, delta_softplus=False, dlast=None,
                   need=("dD", "dz", "ddelta_bias", "dh0"), stream=None):
    """scan_bwd reading the checkpoints scan_fwd_save wrote instead of re-running the forward (ssm_scan_bwd_saved)."""
    return _scan_bwd(ckpt, u, delta, A, B, C, dy, D, z, delta_bias, delta_softplus, None, dlast, need, stream)


def scan_bwd_saved_noalloc(u, delta, A, B, C, dy, ckpt, D=None, z=None, delta_bias=None, delta_softplus=False,
                           dlast=None, need=("dD", "dz", "ddelta_bias", "dh0"), stream=None):
    """scan_bwd_saved with its scratch in the library's fixed 64 MiB device array
    (ssm_scan_bwd_saved_noalloc): no device allocation inside the call.  The
    output tensors are still allocated here by torch unless the caller passes
    the C ABI its own."""
    return _scan_bwd(ckpt, u, delta, A, B, C, dy, D, z, delta_bias, delta_softplus, None, dlast, need, stream,
                     noalloc=True)


def ckpt_shape(batch, dim, dstate, seqlen):
    """Shape of the float32 checkpoint tensor of scan_fwd_save / scan_bwd_saved."""
    return ((seqlen + 15) // 16, batch, dstate, dim)


def scan_fwd_save(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, h0=None, out=None,
                  last_state=None, ckpt=None, stream=None):
    """scan_fwd that also writes the backward's checkpoints (ssm_scan_fwd_save); returns (y, last_state, ckpt)."""
    import torch
    if u.dim() != 3:
        raise ValueError("u must be (batch, dim, seqlen)")
    batch, dim, seqlen = u.shape
    dstate = A.shape[-1]
    dev = u.device
    io = u.dtype
    f32 = torch.float32
    _need(u, "u", (batch, dim, seqlen), io, dev)
    _need(delta, "delta", (batch, dim, seqlen), io, dev)
    _need(A, "A", (dim, dstate), f32, dev)
    _need(B, "B", (batch, dstate, seqlen), io, dev)
    _need(C, "C", (batch, dstate, seqlen), io, dev)
    if D is not None:
        _need(D, "D", (dim,), f32, dev)
    if z is not None:
        _need(z, "z", (batch, dim, seqlen), io, dev)
    if delta_bias is not None:
        _need(delta_bias, "delta_bias", (dim,), f32, dev)
    if h0 is not None:
        _need(h0, "h0", (batch, dim, dstate), f32, dev)
    if out is None:
        out = torch.empty((batch, dim, seqlen), dtype=io, device=dev)
    else:
        _need(out, "out", (batch, dim, seqlen), io, dev)
    if last_state is None:
        last_state = torch.empty((batch, dim, dstate), dtype=f32, device=dev)
    else:
        _need(last_state, "last_state", (batch, dim, dstate), f32, dev)
    cs = ckpt_shape(batch, dim, dstate, seqlen)
    if ckpt is None:
        ckpt = torch.empty(cs, dtype=f32, device=dev)
    else:
        _need(ckpt, "ckpt", cs, f32, dev)
    lib = load_library()
    st = lib.ssm_scan_fwd_save(batch, dim, dstate, seqlen, _io_code(io), _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                               _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), 1 if delta_softplus else 0, _ptr(h0),
                               _ptr(out), _ptr(last_state), _ptr(ckpt), _stream(dev, stream))
    _check("ssm_scan_fwd_save", st)
    return out, last_state, ckpt


def _scan_bwd(ckpt, u, delta, A, B, C, dy, D, z, delta_bias, delta_softplus, h0, dlast, need, stream, disc=None,
              noalloc=False):
    import torch
    if u.dim() != 3:
        raise ValueError("u must be (batch, dim, seqlen)")
    batch, dim, seqlen = u.shape
    dstate = A.shape[-1]
    dev = u.device
    io = u.dtype
    f32 = torch.float32
    _need(u, "u", (batch, dim, seqlen), io, dev)
    _need(delta, "delta", (batch, dim, seqlen), io, dev)
    _need(A, "A", (dim, dstate), f32, dev)
    _need(B, "B", (batch, dstate, seqlen), io, dev)
    _need(C, "C", (batch, dstate, seqlen), io, dev)
    _need(dy, "dy", (batch, dim, seqlen), io, dev)
    if D is not None:
        _need(D, "D", (dim,), f32, dev)
    if z is not None:
        _need(z, "z", (batch, dim, seqlen), io, dev)
    if delta_bias is not None:
        _need(delta_bias, "delta_bias", (dim,), f32, dev)
    if h0 is not None:
        _need(h0, "h0", (batch, dim, dstate), f32, dev)
    if dlast is not None:
        _need(dlast, "dlast", (batch, dim, dstate), f32, dev)
    if ckpt is not None:
        _need(ckpt, "ckpt", ckpt_shape(batch, dim, dstate, seqlen), f32, dev)
    g = dict(du=torch.empty_like(u), ddelta=torch.empty_like(u), dA=torch.empty((dim, dstate), dtype=f32, device=dev),
             dB=torch.empty((batch, dstate, seqlen), dtype=f32, device=dev),
             dC=torch.empty((batch, dstate, seqlen), dtype=f32, device=dev),
             dD=torch.empty(dim, dtype=f32, device=dev) if "dD" in need else None,
             dz=torch.empty_like(u) if ("dz" in need and z is not None) else None,
             ddelta_bias=torch.empty(dim, dtype=f32, device=dev) if "ddelta_bias" in need else None,
             dh0=torch.empty((batch, dim, dstate), dtype=f32, device=dev) if "dh0" in need else None)
    lib = load_library()
    head = (batch, dim, dstate, seqlen, _io_code(io), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(delta_bias), 1 if delta_softplus else 0)
    tail = (_ptr(dy), _ptr(dlast), _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
            _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["ddelta_bias"]), _ptr(g["dh0"]), _stream(dev, stream))
    if disc is not None:
        _check("ssm_scan_bwd_ex", lib.ssm_scan_bwd_ex(*head[:5], disc, *head[5:], _ptr(h0), *tail))
    elif ckpt is None:
        _check("ssm_scan_bwd", lib.ssm_scan_bwd(*head, _ptr(h0), *tail))
    elif noalloc:
        _check("ssm_scan_bwd_saved_noalloc", lib.ssm_scan_bwd_saved_noalloc(*head, _ptr(ckpt), *tail))
    else:
        _check("ssm_scan_bwd_saved", lib.ssm_scan_bwd_saved(*head, _ptr(ckpt), *tail))
    return g


def state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, out=None,
                 stream=None):
    """One decode step (ssm_state_update), updating state (batch, dim, dstate) float32 in place; returns y (batch, dim).

    u, delta, z: (batch, dim); B, C: (batch, dstate) in the io dtype.
    """
    return _state_update(None, state, u, delta, A, B, C, D, z, delta_bias, delta_softplus, out, stream)


def state_update_ex(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, disc="zoh",
                    out=None, stream=None):
    """state_update with a choice of discretization for B (ssm_state_update_ex); disc as scan_fwd_ex."""
    if disc not in DISC_CODES:
        raise ValueError("disc must be one of %s" % sorted(DISC_CODES))
    return _state_update(DISC_CODES[disc], state, u, delta, A, B, C, D, z, delta_bias, delta_softplus, out, stream)


def _state_update(disc, state, u, delta, A, B, C, D, z, delta_bias, delta_softplus, out, stream):
    import torch
    if state.dim() != 3:
        raise ValueError("state must be (batch, dim, dstate)")
    batch, dim, dstate = state.shape
    dev = state.device
    io = u.dtype
    _need(state, "state", (batch, dim, dstate), torch.float32, dev)
    _need(u, "u", (batch, dim), io, dev)
    _need(delta, "delta", (batch, dim), io, dev)
    _need(A, "A", (dim, dstate), torch.float32, dev)
    _need(B, "B", (batch, dstate), io, dev)
    _need(C, "C", (batch, dstate), io, dev)
    if D is not None:
        _need(D, "D", (dim,), torch.float32, dev)
    if z is not None:
        _need(z, "z", (batch, dim), io, dev)
    if delta_bias is not None:
        _need(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    if out is None:
        out = torch.empty((batch, dim), dtype=io, device=dev)
    else:
        _need(out, "out", (batch, dim), io, dev)
    lib = load_library()
    tail = (_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            1 if delta_softplus else 0, _ptr(out), _stream(dev, stream))
    if disc is None:
        _check("ssm_state_update", lib.ssm_state_update(batch, dim, dstate, _io_code(io), *tail))
    else:
        _check("ssm_state_update_ex", lib.ssm_state_update_ex(batch, dim, dstate, _io_code(io), disc, *tail))
    return out
