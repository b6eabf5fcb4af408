"""fp64 CPU oracle for the Mamba-2 selective state-space layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``libssd.so`` and ``selective_state_space_08_amd``) never imports it and
shares no code with it.

The arithmetic lives in ``ssd_oracle.c`` (plain C, double precision, token by
token, OpenMP over (batch, head)); this module only builds that library and
marshals numpy arrays into it.  Every function is pinned by the CPU tests in
``tests/test_oracle_pins.py`` against forms that do not share its code: the
quadratic (materialised-matrix) SSD form, an independent chunked form,
closed forms (geometric series, prefix sums, conv impulse response, steady
state), special cases (dt = 0, A = 0) and invariants (linearity, group
sharing, split-carry, decode = prefill).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def compile_source(src: str, out: str) -> str:
    """gcc a copy of the oracle source into a shared library (no fast-math, no
    FMA contraction: plain IEEE double arithmetic)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile ssd_oracle.c into liboracle.so."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    return compile_source(_SRC, LIB_PATH)


def _bind(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    I64 = ctypes.c_int64
    lib.oracle_causal_conv1d.argtypes = [P, I64, P, P, P, I, P, P, I, I, I, I]
    lib.oracle_causal_conv1d.restype = I
    lib.oracle_mamba2_fwd.argtypes = [P, I64, P, P, I, P, P, P, P, P, I, P, P, P, P, P,
                                      I, I, I, I, I, I]
    lib.oracle_mamba2_fwd.restype = I
    lib.oracle_mamba2_decode_step.argtypes = [P, P, P, P, P, I, P, P, P, P, I, P, P,
                                              I, I, I, I, I]
    lib.oracle_mamba2_decode_step.restype = I
    lib.oracle_mamba2_bwd.argtypes = [P, I64, P, P, I, P, P, P, P, P, I, P, P, P, P,
                                      P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I]
    lib.oracle_mamba2_bwd.restype = I
    lib.oracle_rmsnorm.argtypes = [P, P, ctypes.c_double, P, I64, I]
    lib.oracle_rmsnorm.restype = I
    lib.oracle_linear.argtypes = [P, P, P, P, I64, I, I]
    lib.oracle_linear.restype = I
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = I
    return lib


def load_library(path: str):
    """Load and bind an oracle library built from ssd_oracle.c at ``path``."""
    return _bind(ctypes.CDLL(path))


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    _lib = load_library(LIB_PATH)
    return _lib


def _in(a):
    """An input as the layer receives it: rounded to fp32, held in fp64
    (exactly) for the C code."""
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32), dtype=np.float64)


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return _load().oracle_num_threads()


def causal_conv1d(xbc, w, bias=None, conv_state_in=None, apply_silu=True):
    """Depthwise causal conv over xbc [B, L, Cdim] with weights w [Cdim, K].

    Returns (out [B, L, Cdim] float64, conv_state_out [B, K-1, Cdim] float64).
    """
    lib = _load()
    x = _in(xbc)
    B, L, C = x.shape
    w = _in(w)
    K = w.shape[1]
    bias = _in(bias)
    hist = _in(conv_state_in)
    out = np.empty((B, L, C), np.float64)
    hist_out = np.empty((B, K - 1, C), np.float64)
    rc = lib.oracle_causal_conv1d(_ptr(x), C, _ptr(w), _ptr(bias), _ptr(hist),
                                  int(bool(apply_silu)), _ptr(out), _ptr(hist_out),
                                  B, L, C, K)
    if rc != 0:
        raise ValueError("oracle_causal_conv1d: bad argument")
    return out, hist_out


def mamba2_fwd(xbc, dt, A, *, nheads, headdim, ngroups, dstate, conv_w=None,
               conv_b=None, conv_state_in=None, D=None, dt_bias=None,
               dt_softplus=True, z=None, h0=None, f64_inputs=False):
    """The layer, token by token in fp64.

    xbc [B, L, Cdim] raw x|B|C (post-conv when conv_w is None); dt [B, L, H];
    A [H]; z [B, L, H, P] or None; h0 [B, H, P, N] or None.
    Inputs are taken as fp32 values (rounded to fp32 first); with f64_inputs
    every input is used unrounded (an fp64 intermediate, as in
    mamba2_block_fwd, or a finite-difference probe).
    Returns (y [B, L, H, P], h_final [B, H, P, N], conv_state_out or None),
    all float64.
    """
    lib = _load()
    act = _f64 if f64_inputs else _in
    x = act(xbc)
    B, L, C = x.shape
    H, P, G, N = nheads, headdim, ngroups, dstate
    if C != H * P + 2 * G * N:
        raise ValueError("xbc channel count %d != H*P + 2*G*N" % C)
    dt = act(dt).reshape(B, L, H)
    A = act(A)
    conv_w = act(conv_w)
    K = 0 if conv_w is None else conv_w.shape[1]
    conv_b = act(conv_b)
    hist = act(conv_state_in)
    D = act(D)
    dt_bias = act(dt_bias)
    z = None if z is None else act(z).reshape(B, L, H, P)
    h0 = None if h0 is None else _f64(h0).reshape(B, H, P, N)
    y = np.empty((B, L, H, P), np.float64)
    hT = np.empty((B, H, P, N), np.float64)
    hist_out = np.empty((B, K - 1, C), np.float64) if conv_w is not None else None
    rc = lib.oracle_mamba2_fwd(_ptr(x), C, _ptr(conv_w), _ptr(conv_b), K, _ptr(hist),
                               _ptr(dt), _ptr(A), _ptr(D), _ptr(dt_bias),
                               int(bool(dt_softplus)), _ptr(z), _ptr(h0), _ptr(y),
                               _ptr(hT), _ptr(hist_out), B, L, H, P, G, N)
    if rc != 0:
        raise ValueError("oracle_mamba2_fwd: bad argument")
    return y, hT, hist_out


def mamba2_bwd(xbc, dt, A, dout, *, nheads, headdim, ngroups, dstate, conv_w=None,
               conv_b=None, conv_state_in=None, D=None, dt_bias=None, dt_softplus=True,
               z=None, h0=None, dh_final=None, f64_inputs=False):
    """The layer's gradients, by reverse-mode differentiation of mamba2_fwd.

    dout [B, L, H, P] and dh_final [B, H, P, N] or None are the gradients of a
    scalar loss with respect to the layer's output and final state; inputs as
    in mamba2_fwd.  Returns a dict of float64 gradients: xbc [B, L, Cdim]
    (raw inputs when conv_w is given), dt [B, L, H], A [H], and, for the
    inputs that are given, z, D, dt_bias, h0, conv_w, conv_b, conv_state_in.
    """
    lib = _load()
    act = _f64 if f64_inputs else _in
    x = act(xbc)
    B, L, C = x.shape
    H, P, G, N = nheads, headdim, ngroups, dstate
    if C != H * P + 2 * G * N:
        raise ValueError("xbc channel count %d != H*P + 2*G*N" % C)
    dt = act(dt).reshape(B, L, H)
    A = act(A)
    conv_w = act(conv_w)
    K = 0 if conv_w is None else conv_w.shape[1]
    conv_b = act(conv_b)
    hist = act(conv_state_in)
    D = act(D)
    dt_bias = act(dt_bias)
    z = None if z is None else act(z).reshape(B, L, H, P)
    h0 = None if h0 is None else _f64(h0).reshape(B, H, P, N)
    dout = _f64(dout).reshape(B, L, H, P)
    dhf = None if dh_final is None else _f64(dh_final).reshape(B, H, P, N)
    g = {"xbc": np.empty((B, L, C)), "dt": np.empty((B, L, H)), "A": np.empty(H)}
    if z is not None:
        g["z"] = np.empty((B, L, H, P))
    if D is not None:
        g["D"] = np.empty(H)
    if dt_bias is not None:
        g["dt_bias"] = np.empty(H)
    g["h0"] = np.empty((B, H, P, N))
    if conv_w is not None:
        g["conv_w"] = np.empty((C, K))
        g["conv_b"] = np.empty(C)
        g["conv_state_in"] = np.empty((B, K - 1, C))
    rc = lib.oracle_mamba2_bwd(
        _ptr(x), C, _ptr(conv_w), _ptr(conv_b), K, _ptr(hist), _ptr(dt), _ptr(A), _ptr(D),
        _ptr(dt_bias), int(bool(dt_softplus)), _ptr(z), _ptr(h0), _ptr(dout), _ptr(dhf),
        _ptr(g["xbc"]), _ptr(g["dt"]), _ptr(g.get("z")), _ptr(g["A"]), _ptr(g.get("D")),
        _ptr(g.get("dt_bias")), _ptr(g["h0"]), _ptr(g.get("conv_w")), _ptr(g.get("conv_b")),
        _ptr(g.get("conv_state_in")), B, L, H, P, G, N)
    if rc != 0:
        raise ValueError("oracle_mamba2_bwd: bad argument")
    return g


def rmsnorm(x, w=None, eps=1e-5):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * w, in fp64.

    x [..., dim]; w [dim] or None.  Returns float64 of x's shape."""
    lib = _load()
    xa = _in(x)
    dim = xa.shape[-1]
    ntok = xa.size // dim
    out = np.empty(xa.shape, np.float64)
    if lib.oracle_rmsnorm(_ptr(xa), _ptr(_in(w)), float(eps), _ptr(out), ntok, dim) != 0:
        raise ValueError("oracle_rmsnorm: bad argument")
    return out


def linear(a, w, residual=None):
    """a @ w^T (+ residual) in fp64, with w stored [out, in].

    a [..., K] (fp64 values are used as given); w [N, K]; residual [..., N]
    or None.  Returns float64 [..., N]."""
    lib = _load()
    aa = _f64(a)
    K = aa.shape[-1]
    M = aa.size // K
    wa = _in(w)
    N = wa.shape[0]
    if wa.shape[1] != K:
        raise ValueError("linear: weight is [%d, %d], input has %d features" % (N, wa.shape[1], K))
    res = None if residual is None else _in(residual).reshape(M, N)
    out = np.empty(aa.shape[:-1] + (N,), np.float64)
    if lib.oracle_linear(_ptr(aa), _ptr(wa), _ptr(res), _ptr(out), M, N, K) != 0:
        raise ValueError("oracle_linear: bad argument")
    return out


def mamba2_block_fwd(h, norm_w, in_proj_w, out_proj_w, A, *, nheads, headdim, ngroups,
                     dstate, conv_w, conv_b=None, conv_state_in=None, D=None,
                     dt_bias=None, dt_softplus=True, h0=None, norm_eps=1e-5):
    """The pre-norm residual block around the layer, in fp64:
    out = h + out_proj(mixer(rmsnorm(h))), with the mixer
    in_proj -> (z | x B C | dt) -> conv + SiLU on x|B|C -> scan, D skip and
    SiLU(z) gate -> out_proj.

    h [B, L, d_model]; norm_w [d_model] or None; in_proj_w
    [2*H*P + 2*G*N + H, d_model] whose output rows are ordered z (H*P),
    x (H*P), B (G*N), C (G*N), dt (H); out_proj_w [d_model, H*P].
    Returns (out [B, L, d_model], h_final, conv_state_out), all float64.
    """
    H, P, G, N = nheads, headdim, ngroups, dstate
    HP, GN = H * P, G * N
    hh = _in(h)
    Bsz, L, dm = hh.shape
    u = rmsnorm(hh, norm_w, norm_eps)
    zxbcdt = linear(u, in_proj_w)
    if zxbcdt.shape[-1] != 2 * HP + 2 * GN + H:
        raise ValueError("in_proj has %d outputs, expected %d" % (zxbcdt.shape[-1], 2 * HP + 2 * GN + H))
    z = zxbcdt[..., :HP].reshape(Bsz, L, H, P)
    xbc = zxbcdt[..., HP:2 * HP + 2 * GN]
    dt = zxbcdt[..., 2 * HP + 2 * GN:]
    y, hT, conv_out = mamba2_fwd(xbc, dt, A, nheads=H, headdim=P, ngroups=G, dstate=N,
                                 conv_w=conv_w, conv_b=conv_b, conv_state_in=conv_state_in,
                                 D=D, dt_bias=dt_bias, dt_softplus=dt_softplus, z=z, h0=h0,
                                 f64_inputs=True)
    out = linear(y.reshape(Bsz, L, HP), out_proj_w, residual=hh)
    return out, hT, conv_out


class DecodeState:
    """fp64 decode carry: the SSM state [B, H, P, N] and the conv ring
    [B, K-1, Cdim] (oldest row first)."""

    def __init__(self, state, ring):
        self.state = _f64(state).copy()
        self.ring = None if ring is None else _f64(ring).copy()


def mamba2_decode_step(carry: DecodeState, xbc, dt, A, *, nheads, headdim, ngroups,
                       dstate, conv_w=None, conv_b=None, D=None, dt_bias=None,
                       dt_softplus=True, z=None):
    """One decode step; updates ``carry`` in place and returns y [B, H*P] float64."""
    lib = _load()
    x = _in(xbc)
    B, C = x.shape
    H, P, G, N = nheads, headdim, ngroups, dstate
    conv_w = _in(conv_w)
    K = 0 if conv_w is None else conv_w.shape[1]
    y = np.empty((B, H * P), np.float64)
    rc = lib.oracle_mamba2_decode_step(
        _ptr(carry.state), _ptr(x), _ptr(carry.ring), _ptr(conv_w), _ptr(_in(conv_b)), K,
        _ptr(_in(dt).reshape(B, H)), _ptr(_in(A)), _ptr(_in(D)), _ptr(_in(dt_bias)),
        int(bool(dt_softplus)), _ptr(None if z is None else _in(z).reshape(B, H * P)),
        _ptr(y), B, H, P, G, N)
    if rc != 0:
        raise ValueError("oracle_mamba2_decode_step: bad argument")
    return y
