"""fp64 CPU oracle for the selective scan -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package.  The product path (the HIP library and its binding) never
imports it, and it imports nothing from the product: the arithmetic lives in
ssm_oracle.c (plain C, double precision, one sequential loop per channel);
this module only marshals numpy arrays into it.

  Oracle(path)             a loaded oracle library (the default is built from
                           ssm_oracle.c next to this file)
  .scan_f64(...)           full prefill scan, every (batch, channel); zoh=True
                           discretizes B by exact zero-order hold
  .scan_channels_f64(...)  the same scan restricted to chosen (b, d) channels
                           (channels are independent, so a subset is exact)
  .state_update_f64(...)   one-token update of a float64 state, in place
  .state_update_channels_f64(...)  the same for chosen (b, d) channels
  .scan_bwd_f64(...)       gradients of the scan (reverse mode, written out by hand)
  .scan_complex_f64(...)   the scan with complex diagonal A (complex B, C, state)
  .conv1d_f64(...)         the causal depthwise conv (+ silu) in front of the scan
  .conv1d_bwd_f64(...)     its gradients (reverse mode, written out by hand)
  .softplus_f64, .silu_f64 the scalar helpers the C oracle uses
Module-level functions of the same names use the default oracle.
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "ssm_oracle.c")
LIB_PATH = os.path.join(HERE, "libssm_oracle.so")
CFLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra"]


def compile_oracle(source=SOURCE, out=LIB_PATH):
    """gcc -O2 -fopenmp: compile an oracle C source into a shared library."""
    subprocess.run(["gcc"] + CFLAGS + ["-o", out, source, "-lm"], check=True)
    return out


def build():
    """Compile ssm_oracle.c into libssm_oracle.so (always recompiles)."""
    return compile_oracle()


def set_threads(n):
    """Thread count of the oracle's OpenMP channel loop (a call into the OpenMP
    runtime the oracle library links; no arithmetic)."""
    default()
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    def __init__(self, path=LIB_PATH):
        L = ctypes.CDLL(path)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_scan_ex_f64.restype = I
        L.oracle_scan_ex_f64.argtypes = [I64, I64, I64, I64, I] + [P] * 8 + [I, P, P, P]
        L.oracle_state_update_ex_f64.restype = I
        L.oracle_state_update_ex_f64.argtypes = [I64, I64, I64, I] + [P] * 9 + [I, P]
        L.oracle_zoh_b.restype = ctypes.c_double
        L.oracle_zoh_b.argtypes = [ctypes.c_double, ctypes.c_double]
        L.oracle_scan_bwd_ex_f64.restype = I
        L.oracle_scan_bwd_ex_f64.argtypes = [I64, I64, I64, I64, I] + [P] * 8 + [I] + [P] * 12
        L.oracle_zoh_b_da.restype = ctypes.c_double
        L.oracle_zoh_b_da.argtypes = [ctypes.c_double, ctypes.c_double]
        L.oracle_scan_complex_f64.restype = I
        L.oracle_scan_complex_f64.argtypes = [I64, I64, I64, I64] + [P] * 8 + [I, P, P, P]
        L.oracle_scan_complex_bwd_f64.restype = I
        L.oracle_scan_complex_bwd_f64.argtypes = [I64, I64, I64, I64] + [P] * 8 + [I] + [P] * 12
        L.oracle_conv1d_f64.restype = I
        L.oracle_conv1d_f64.argtypes = [I64, I64, I64, I64, P, P, P, P, I, P]
        L.oracle_conv1d_bwd_f64.restype = I
        L.oracle_conv1d_bwd_f64.argtypes = [I64, I64, I64, I64, P, P, P, P, I, P, P, P, P, P]
        L.oracle_softplus.restype = ctypes.c_double
        L.oracle_softplus.argtypes = [ctypes.c_double]
        L.oracle_silu.restype = ctypes.c_double
        L.oracle_silu.argtypes = [ctypes.c_double]
        self.lib = L
        self.path = path

    def softplus_f64(self, x):
        return self.lib.oracle_softplus(float(x))

    def silu_f64(self, x):
        return self.lib.oracle_silu(float(x))

    def zoh_b_f64(self, delta, a):
        return self.lib.oracle_zoh_b(float(delta), float(a))

    def scan_f64(self, u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=False, h0=None, zoh=False):
        """Returns (y, last_state) in float64.  Shapes as in ssm_oracle.c."""
        u, delta, A, B, C, D, z, delta_bias, h0 = map(_f64, (u, delta, A, B, C, D, z, delta_bias, h0))
        batch, dim, seqlen = u.shape
        dstate = A.shape[1]
        y = np.empty((batch, dim, seqlen), np.float64)
        last = np.empty((batch, dim, dstate), np.float64)
        rc = self.lib.oracle_scan_ex_f64(batch, dim, dstate, seqlen, 1 if zoh else 0, _p(u), _p(delta), _p(A), _p(B),
                                         _p(C), _p(D), _p(z), _p(delta_bias), 1 if softplus else 0, _p(h0), _p(y),
                                         _p(last))
        if rc != 0:
            raise ValueError("oracle_scan_f64 rejected the arguments")
        return y, last

    def scan_complex_f64(self, u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=False, h0=None):
        """The scan with complex A (dim, dstate), B and C (batch, dstate, seqlen) and h0 (batch, dim, dstate),
        given as numpy complex arrays; u, delta, z (batch, dim, seqlen), D and delta_bias (dim,) are real.
        Returns (y real (batch, dim, seqlen), last_state complex (batch, dim, dstate))."""
        def ri(a):
            return None if a is None else np.ascontiguousarray(np.stack([np.real(a), np.imag(a)], -1), np.float64)
        u, delta, D, z, delta_bias = map(_f64, (u, delta, D, z, delta_bias))
        A, B, C, h0 = map(ri, (A, B, C, h0))
        batch, dim, seqlen = u.shape
        dstate = A.shape[1]
        y = np.empty((batch, dim, seqlen), np.float64)
        last = np.empty((batch, dim, dstate, 2), np.float64)
        rc = self.lib.oracle_scan_complex_f64(batch, dim, dstate, seqlen, _p(u), _p(delta), _p(A), _p(B), _p(C),
                                              _p(D), _p(z), _p(delta_bias), 1 if softplus else 0, _p(h0), _p(y),
                                              _p(last))
        if rc != 0:
            raise ValueError("oracle_scan_complex_f64 rejected the arguments")
        return y, last[..., 0] + 1j * last[..., 1]

    def scan_complex_bwd_f64(self, u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=False, h0=None,
                             dy=None, dlast=None):
        """Gradients of sum(dy * y) + sum(Re(conj(dlast) last_state)) for scan_complex_f64 (complex arrays as
        numpy complex).  Returns a dict like scan_bwd_f64; dA, dB, dC, dh0 complex (d/dRe + i d/dIm)."""
        def ri(a):
            return None if a is None else np.ascontiguousarray(np.stack([np.real(a), np.imag(a)], -1), np.float64)
        u, delta, D, z, delta_bias, dy = map(_f64, (u, delta, D, z, delta_bias, dy))
        A, B, C, h0, dlast = map(ri, (A, B, C, h0, dlast))
        batch, dim, seqlen = u.shape
        dstate = A.shape[1]
        out = dict(du=np.empty_like(u), ddelta=np.empty_like(u), dA=np.empty((dim, dstate, 2)),
                   dB=np.empty((batch, dstate, seqlen, 2)), dC=np.empty((batch, dstate, seqlen, 2)),
                   dD=None if D is None else np.empty_like(D), dz=None if z is None else np.empty_like(z),
                   ddelta_bias=None if delta_bias is None else np.empty_like(delta_bias),
                   dh0=np.empty((batch, dim, dstate, 2)))
        rc = self.lib.oracle_scan_complex_bwd_f64(batch, dim, dstate, seqlen, _p(u), _p(delta), _p(A), _p(B), _p(C),
                                                  _p(D), _p(z), _p(delta_bias), 1 if softplus else 0, _p(h0), _p(dy),
                                                  _p(dlast), _p(out["du"]), _p(out["ddelta"]), _p(out["dA"]),
                                                  _p(out["dB"]), _p(out["dC"]), _p(out["dD"]), _p(out["dz"]),
                                                  _p(out["ddelta_bias"]), _p(out["dh0"]))
        if rc != 0:
            raise ValueError("oracle_scan_complex_bwd_f64 rejected the arguments")
        for k in ("dA", "dB", "dC", "dh0"):
            out[k] = out[k][..., 0] + 1j * out[k][..., 1]
        return out

    def scan_complex_channels_f64(self, channels, u, delta, A, B, C, D=None, z=None, delta_bias=None,
                                  softplus=False, h0=None):
        """scan_complex_f64 restricted to the listed (b, d) channels (marshalling only)."""
        ys, hs = [], []
        for (b, d) in channels:
            def sl(t):
                return None if t is None else t[b:b + 1, d:d + 1]
            y, h = self.scan_complex_f64(sl(u), sl(delta), A[d:d + 1], B[b:b + 1], C[b:b + 1],
                                         None if D is None else D[d:d + 1], sl(z),
                                         None if delta_bias is None else delta_bias[d:d + 1], softplus, sl(h0))
            ys.append(y[0, 0])
            hs.append(h[0, 0])
        return np.stack(ys), np.stack(hs)

    def zoh_b_da_f64(self, delta, a):
        return self.lib.oracle_zoh_b_da(float(delta), float(a))

    def scan_bwd_f64(self, u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=False, h0=None, dy=None,
                     dlast=None, zoh=False):
        """Gradients of sum(dy * y) + sum(dlast * last_state) with respect to every input (zoh: B by exact
        zero-order hold, as scan_f64).

        Returns a dict with du, ddelta (batch, dim, seqlen), dA (dim, dstate),
        dB, dC (batch, dstate, seqlen), and dD (dim,), dz, ddelta_bias (dim,),
        dh0 (batch, dim, dstate) for the inputs that are given (else None).
        """
        u, delta, A, B, C, D, z, delta_bias, h0, dy, dlast = map(_f64, (u, delta, A, B, C, D, z, delta_bias, h0, dy,
                                                                       dlast))
        batch, dim, seqlen = u.shape
        dstate = A.shape[1]
        out = dict(du=np.empty_like(u), ddelta=np.empty_like(u), dA=np.empty_like(A), dB=np.empty_like(B),
                   dC=np.empty_like(C), dD=None if D is None else np.empty_like(D),
                   dz=None if z is None else np.empty_like(z),
                   ddelta_bias=None if delta_bias is None else np.empty_like(delta_bias),
                   dh0=np.empty((batch, dim, dstate), np.float64))
        rc = self.lib.oracle_scan_bwd_ex_f64(batch, dim, dstate, seqlen, 1 if zoh else 0, _p(u), _p(delta), _p(A),
                                             _p(B), _p(C), _p(D), _p(z), _p(delta_bias), 1 if softplus else 0, _p(h0),
                                             _p(dy), _p(dlast), _p(out["du"]), _p(out["ddelta"]), _p(out["dA"]),
                                             _p(out["dB"]), _p(out["dC"]), _p(out["dD"]), _p(out["dz"]),
                                             _p(out["ddelta_bias"]), _p(out["dh0"]))
        if rc != 0:
            raise ValueError("oracle_scan_bwd_f64 rejected the arguments")
        return out

    def conv1d_f64(self, x, weight, bias=None, x_prev=None, silu=True):
        """u = act(causal depthwise conv of x).  x: (batch, dim, seqlen); weight: (dim, K), K in 1..4;
        bias: (dim,); x_prev: (batch, dim, K-1), the inputs before token 0.  Returns u in float64."""
        x, weight, bias = _f64(x), _f64(weight), _f64(bias)
        batch, dim, seqlen = x.shape
        width = weight.shape[1]
        xp = None if x_prev is None or width == 1 else _f64(x_prev)
        u = np.empty((batch, dim, seqlen), np.float64)
        rc = self.lib.oracle_conv1d_f64(batch, dim, seqlen, width, _p(x), _p(weight), _p(bias), _p(xp),
                                        1 if silu else 0, _p(u))
        if rc != 0:
            raise ValueError("oracle_conv1d_f64 rejected the arguments")
        return u

    def conv1d_bwd_f64(self, x, weight, du, bias=None, x_prev=None, silu=True):
        """Gradients of conv1d_f64 for a loss with dL/du = du: dict of dx (batch, dim, seqlen),
        dweight (dim, K), dbias (dim,) and dx_prev (batch, dim, K-1), all float64."""
        x, weight, bias, du = _f64(x), _f64(weight), _f64(bias), _f64(du)
        batch, dim, seqlen = x.shape
        width = weight.shape[1]
        xp = None if x_prev is None or width == 1 else _f64(x_prev)
        out = dict(dx=np.empty((batch, dim, seqlen), np.float64), dweight=np.empty((dim, width), np.float64),
                   dbias=np.empty(dim, np.float64), dx_prev=np.zeros((batch, dim, width - 1), np.float64))
        rc = self.lib.oracle_conv1d_bwd_f64(batch, dim, seqlen, width, _p(x), _p(weight), _p(bias), _p(xp),
                                            1 if silu else 0, _p(du), _p(out["dx"]), _p(out["dweight"]),
                                            _p(out["dbias"]), _p(out["dx_prev"]) if width > 1 else None)
        if rc != 0:
            raise ValueError("oracle_conv1d_bwd_f64 rejected the arguments")
        return out

    def scan_channels_f64(self, channels, u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=False,
                          h0=None, zoh=False):
        """Scan only the listed (b, d) channels; returns (y[k, seqlen], last_state[k, dstate]).

        Pure marshalling: each channel becomes a batch-1, dim-1 problem with its
        own rows of u/delta/z, its batch row of B/C and its row of A/D/bias.
        """
        ys, hs = [], []
        for (b, d) in channels:
            def sl(t):
                return None if t is None else t[b:b + 1, d:d + 1]
            y, h = self.scan_f64(sl(u), sl(delta), A[d:d + 1], B[b:b + 1], C[b:b + 1],
                                 None if D is None else D[d:d + 1], sl(z),
                                 None if delta_bias is None else delta_bias[d:d + 1], softplus, sl(h0), zoh=zoh)
            ys.append(y[0, 0])
            hs.append(h[0, 0])
        return np.stack(ys), np.stack(hs)

    def state_update_channels_f64(self, channels, state_rows, u, delta, A, B, C, D=None, z=None, delta_bias=None,
                                  softplus=False, zoh=False):
        """One-token update of chosen (b, d) channels only.

        state_rows: float64 (k, dstate), row i belongs to channels[i], updated in
        place; u, delta, z: (batch, dim); B, C: (batch, dstate).  Returns y (k,).
        """
        y = np.empty(len(channels), np.float64)
        for i, (b, d) in enumerate(channels):
            st = state_rows[i:i + 1].reshape(1, 1, -1)  # a view: updated in place
            y[i] = self.state_update_f64(st, u[b:b + 1, d:d + 1], delta[b:b + 1, d:d + 1], A[d:d + 1], B[b:b + 1],
                                         C[b:b + 1], None if D is None else D[d:d + 1],
                                         None if z is None else z[b:b + 1, d:d + 1],
                                         None if delta_bias is None else delta_bias[d:d + 1], softplus, zoh=zoh)[0, 0]
        return y

    def state_update_f64(self, state, u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=False, zoh=False):
        """Advance `state` (float64 (batch, dim, dstate), modified in place) by one token; returns y (batch, dim)."""
        if state.dtype != np.float64 or not state.flags["C_CONTIGUOUS"]:
            raise TypeError("state must be a C-contiguous float64 array (it is updated in place)")
        u, delta, A, B, C, D, z, delta_bias = map(_f64, (u, delta, A, B, C, D, z, delta_bias))
        batch, dim, dstate = state.shape
        y = np.empty((batch, dim), np.float64)
        rc = self.lib.oracle_state_update_ex_f64(batch, dim, dstate, 1 if zoh else 0, _p(state), _p(u), _p(delta),
                                                 _p(A), _p(B), _p(C), _p(D), _p(z), _p(delta_bias),
                                                 1 if softplus else 0, _p(y))
        if rc != 0:
            raise ValueError("oracle_state_update_f64 rejected the arguments")
        return y


_default = None


def default():
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build()
        _default = Oracle(LIB_PATH)
    return _default


def scan_f64(*args, **kw):
    return default().scan_f64(*args, **kw)


def scan_channels_f64(*args, **kw):
    return default().scan_channels_f64(*args, **kw)


def state_update_f64(*args, **kw):
    return default().state_update_f64(*args, **kw)


def state_update_channels_f64(*args, **kw):
    return default().state_update_channels_f64(*args, **kw)


def scan_bwd_f64(*args, **kw):
    return default().scan_bwd_f64(*args, **kw)


def scan_complex_f64(*args, **kw):
    return default().scan_complex_f64(*args, **kw)


def scan_complex_bwd_f64(*args, **kw):
    return default().scan_complex_bwd_f64(*args, **kw)


def scan_complex_channels_f64(*args, **kw):
    return default().scan_complex_channels_f64(*args, **kw)


def conv1d_f64(*args, **kw):
    return default().conv1d_f64(*args, **kw)


def conv1d_bwd_f64(*args, **kw):
    return default().conv1d_bwd_f64(*args, **kw)


def zoh_b_f64(delta, a):
    return default().zoh_b_f64(delta, a)


def softplus_f64(x):
    return default().softplus_f64(x)


def silu_f64(x):
    return default().silu_f64(x)
