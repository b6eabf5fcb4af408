"""Thin Python binding of libssd.so (the C ABI in include/ssd.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Functions carry the C entry points' names and take torch tensors
(device memory) and the current HIP stream.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssd.so")

SSD_F32, SSD_BF16 = 0, 1
SSD_MATH_F32, SSD_MATH_BF16 = 0, 1
STATUS = {0: "SSD_OK", -1: "SSD_ERR_INVALID_ARG", -2: "SSD_ERR_UNSUPPORTED",
          -3: "SSD_ERR_WORKSPACE", -4: "SSD_ERR_HIP"}

# every symbol include/ssd.h declares, with (restype, argtypes)
_V, _I, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "ssd_causal_conv1d_fwd": (_I, [_V, _I64, _I, _V, _V, _V, _V, _V, _I64, _I, _I, _I, _I, _I,
                                   _I, _V]),
    "ssd_chunk_scan_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I, _I]),
    "ssd_chunk_scan_fwd": (_I, [_V, _I64, _V, _I64, _V, _I64, _I, _V, _V, _I, _V, _V, _V, _I64,
                                _V, _I64, _I, _V, _V, _V, _I, _V, _V, _V, _I64, _I, _I, _I, _I,
                                _I, _I, _I, _I, _I, _V, _SZ, _V]),
    "ssd_state_update": (_I, [_V, _V, _I, _V, _V, _V, _I, _V, _V, _I, _V, _V, _V, _I, _V, _I,
                              _I, _I, _I, _I, _I, _V]),
    "ssd_state_update_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "ssd_state_update_ws": (_I, [_V, _V, _I, _V, _V, _V, _I, _V, _V, _I, _V, _V, _V, _I, _V,
                                 _I, _I, _I, _I, _I, _I, _V, _SZ, _V]),
    "ssd_state_update_noalloc": (_I, [_V, _V, _I, _V, _V, _V, _I, _V, _V, _I, _V, _V, _V, _I,
                                      _V, _I, _I, _I, _I, _I, _I, _V]),
    "ssd_decode_cache_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "ssd_chunk_scan_bwd_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "ssd_chunk_scan_bwd": (_I, [_V, _I64, _V, _I64, _V, _I64, _I, _V, _V, _I, _V, _V, _I64, _V,
                                _I64, _I, _V, _V, _V, _I, _V, _V, _I64, _I, _V, _V, _V, _V, _V,
                                _V, _V, _V, _V, _V, _V, _I, _I, _I, _I, _I, _I, _V, _SZ, _V]),
    "ssd_rmsnorm_fwd": (_I, [_V, _I64, _I, _V, ctypes.c_float, _V, _I64, _I, _I64, _I, _V]),
    "ssd_linear_fwd": (_I, [_V, _I64, _V, _I64, _V, _I64, _I, _V, _I64, _I, _I64, _I, _I, _V]),
    "ssd_block_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "ssd_block_fwd": (_I, [_V, _I, _V, ctypes.c_float, _V, _V, _V, _I, _V, _V, _V, _I, _V, _V,
                           _V, _V, _V, _V, _I, _I, _I, _I, _I, _I, _I, _I, _V, _SZ, _V]),
    "ssd_calibrate_stream": (_I, [_V, _V, _SZ, _V]),
    "ssd_calibrate_mfma_bf16": (_I, [_V, _I, _I, _V]),
    "ssd_status_string": (ctypes.c_char_p, [_I]),
    "ssd_last_error": (ctypes.c_char_p, []),
    "ssd_version": (ctypes.c_char_p, []),
}


class SsdError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__("%s: %s" % (STATUS.get(status, status), detail))
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load libssd.so and declare its signatures (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libssd.so is not built (%s); run __graft_entry__.build()" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise SsdError(status, load().ssd_last_error().decode())


def _dt(t: Optional[torch.Tensor]) -> int:
    if t is None:
        return SSD_F32
    if t.dtype == torch.float32:
        return SSD_F32
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    raise TypeError("unsupported dtype %s" % t.dtype)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _tok(t: Optional[torch.Tensor], B: int, L: int, width: int, name: str) -> int:
    """Token stride of a [B, L, ...] tensor whose per-token row is contiguous."""
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    inner = 1
    for d in t.shape[2:]:
        inner *= d
    if tuple(t.shape[:2]) != (B, L) or inner != width:
        raise ValueError("%s has shape %s, want [%d, %d, (%d elements)]"
                         % (name, tuple(t.shape), B, L, width))
    if B == 0 or L == 0:
        return width  # empty: nothing is read or written
    row = t.view(B, L, width)  # raises rather than copies if rows are not contiguous
    if width > 1 and row.stride(2) != 1:
        raise ValueError("%s: per-token rows must be contiguous" % name)
    if B > 1 and L > 0 and row.stride(0) != L * row.stride(1):
        raise ValueError("%s: batch stride must be seqlen * token stride" % name)
    return row.stride(1) if L > 1 or B > 1 else max(row.stride(1), width)


def _dense(t: Optional[torch.Tensor], shape, name: str, dtype=None):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError("%s must be a contiguous device tensor of shape %s" % (name, tuple(shape)))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s" % (name, dtype))


def ssd_calibrate_stream(dst, src):
    """One non-temporal streaming pass dst = src (in place when dst is src);
    moves 2 * nbytes through HBM.  Measurement only."""
    nb = dst.numel() * dst.element_size()
    if src.numel() * src.element_size() != nb:
        raise ValueError("ssd_calibrate_stream: dst and src differ in size")
    _check(load().ssd_calibrate_stream(_p(dst), _p(src), nb, _stream(dst)))


MFMA_CAL_FLOPS_PER_WAVE_ITER = 8 * 16 * 16 * 32 * 2


def ssd_calibrate_mfma_bf16(out, iters):
    """Back-to-back bf16 MFMAs on register operands: out.numel() / 256 blocks
    of 4 waves, iters * 8 products per wave.  Returns the flop count."""
    blocks = out.numel() // 256
    _check(load().ssd_calibrate_mfma_bf16(_p(out), blocks, iters, _stream(out)))
    return blocks * 4 * iters * MFMA_CAL_FLOPS_PER_WAVE_ITER


def ssd_version() -> str:
    return load().ssd_version().decode()


def ssd_decode_cache_bytes(nheads, headdim, ngroups, dstate, width, conv_dtype=torch.bfloat16):
    return load().ssd_decode_cache_bytes(nheads, headdim, ngroups, dstate, width,
                                         SSD_BF16 if conv_dtype == torch.bfloat16 else SSD_F32)


def ssd_chunk_scan_workspace_bytes(batch, seqlen, nheads, headdim=64, ngroups=8, dstate=128,
                                   chunk=128, math="bf16", fused_conv=False):
    return load().ssd_chunk_scan_workspace_bytes(
        batch, seqlen, nheads, headdim, ngroups, dstate, chunk,
        SSD_MATH_BF16 if math == "bf16" else SSD_MATH_F32, int(bool(fused_conv)))


def ssd_causal_conv1d_fwd(x, weight, bias=None, conv_state_in=None, conv_state_out=None,
                          out=None, out_dtype=torch.float32, apply_silu=True):
    """x [B, L, Cdim] -> out [B, L, Cdim] (conv + SiLU); fills conv_state_out."""
    lib = load()
    B, L, C = x.shape
    K = weight.shape[1]
    _dense(weight, (C, K), "weight", torch.float32)
    _dense(bias, (C,), "bias", torch.float32)
    _dense(conv_state_in, (B, K - 1, C), "conv_state_in", x.dtype)
    _dense(conv_state_out, (B, K - 1, C), "conv_state_out", x.dtype)
    if out is None:
        out = torch.empty((B, L, C), dtype=out_dtype, device=x.device)
    xs = _tok(x, B, L, C, "x")
    os_ = _tok(out, B, L, C, "out")
    _check(lib.ssd_causal_conv1d_fwd(_p(x), xs, _dt(x), _p(weight), _p(bias), _p(conv_state_in),
                                     _p(conv_state_out), _p(out), os_, _dt(out), B, L, C, K,
                                     int(bool(apply_silu)), _stream(x)))
    return out


def ssd_chunk_scan_fwd(x, Bm, Cm, dt, A, *, D=None, z=None, dt_bias=None, dt_softplus=True,
                       initial_state=None, final_state=None, conv_w=None, conv_b=None,
                       conv_state_in=None, conv_state_out=None, chunk=128, math="bf16",
                       y=None, y_dtype=torch.float32, workspace=None):
    """Chunked selective scan.  x [B, L, H, P], Bm/Cm [B, L, G, N], dt [B, L, H],
    z [B, L, H, P] or None -> y [B, L, H, P].  With conv_w, x/Bm/Cm are raw
    conv inputs and the conv + SiLU runs inside the scan."""
    lib = load()
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    if Bm.dtype != x.dtype or Cm.dtype != x.dtype:
        raise TypeError("x, Bm, Cm must share a dtype")
    if z is not None and z.dtype != dt.dtype:
        raise TypeError("z and dt must share a dtype")
    xs, bs, cs = _tok(x, B, L, H * P, "x"), _tok(Bm, B, L, G * N, "Bm"), _tok(Cm, B, L, G * N, "Cm")
    dts, zs = _tok(dt, B, L, H, "dt"), _tok(z, B, L, H * P, "z")
    for n, t in (("A", A), ("D", D), ("dt_bias", dt_bias)):
        _dense(t, (H,), n, torch.float32)
    _dense(initial_state, (B, H, P, N), "initial_state", torch.float32)
    _dense(final_state, (B, H, P, N), "final_state", torch.float32)
    K = 0
    if conv_w is not None:
        K = conv_w.shape[1]
        cdim = H * P + 2 * G * N
        _dense(conv_w, (cdim, K), "conv_w", torch.float32)
        _dense(conv_b, (cdim,), "conv_b", torch.float32)
        _dense(conv_state_in, (B, K - 1, cdim), "conv_state_in", x.dtype)
        _dense(conv_state_out, (B, K - 1, cdim), "conv_state_out", x.dtype)
    if y is None:
        y = torch.empty((B, L, H, P), dtype=y_dtype, device=x.device)
    ys = _tok(y, B, L, H * P, "y")
    m = SSD_MATH_BF16 if math == "bf16" else SSD_MATH_F32
    need = lib.ssd_chunk_scan_workspace_bytes(B, L, H, P, G, N, chunk, m, int(conv_w is not None))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ssd_chunk_scan_fwd(
        _p(x), xs, _p(Bm), bs, _p(Cm), cs, _dt(x), _p(conv_w), _p(conv_b), K,
        _p(conv_state_in), _p(conv_state_out), _p(dt), dts, _p(z), zs, _dt(dt), _p(A), _p(D),
        _p(dt_bias), int(bool(dt_softplus)), _p(initial_state), _p(final_state), _p(y), ys,
        _dt(y), B, L, H, P, G, N, chunk, m, _p(workspace), wsz, _stream(x)))
    return y


def _state_update_args(state, xbc, dt, ngroups, conv_state, conv_w, conv_b, z, y, y_dtype):
    """Shape checks shared by both decode entry points; returns (y, B, H, P, G, N, K)."""
    B, H, P, N = state.shape
    G = ngroups
    cdim = H * P + 2 * G * N
    _dense(state, (B, H, P, N), "state", torch.float32)
    _dense(xbc, (B, cdim), "xbc")
    _dense(dt, (B, H), "dt")
    _dense(z, (B, H * P), "z", dt.dtype)
    K = 0
    if conv_w is not None:
        K = conv_w.shape[1]
        _dense(conv_w, (cdim, K), "conv_w", torch.float32)
        _dense(conv_b, (cdim,), "conv_b", torch.float32)
        _dense(conv_state, (B, K - 1, cdim), "conv_state", xbc.dtype)
    if y is None:
        y = torch.empty((B, H * P), dtype=y_dtype, device=state.device)
    _dense(y, (B, H * P), "y")
    return y, B, H, P, G, N, K


def ssd_state_update(state, xbc, dt, A, *, ngroups, conv_state=None, conv_w=None, conv_b=None,
                     z=None, D=None, dt_bias=None, dt_softplus=True, y=None,
                     y_dtype=torch.float32):
    """One decode step, no workspace.  state [B, H, P, N] fp32 (in place),
    xbc [B, Cdim], conv_state [B, K-1, Cdim] (in place), dt [B, H],
    z [B, H*P] -> y [B, H*P]."""
    lib = load()
    y, B, H, P, G, N, K = _state_update_args(state, xbc, dt, ngroups, conv_state, conv_w,
                                             conv_b, z, y, y_dtype)
    _check(lib.ssd_state_update(_p(state), _p(xbc), _dt(xbc), _p(conv_state), _p(conv_w),
                                _p(conv_b), K, _p(dt), _p(z), _dt(dt), _p(A), _p(D),
                                _p(dt_bias), int(bool(dt_softplus)), _p(y), _dt(y), B, H, P, G,
                                N, _stream(state)))
    return y


def ssd_state_update_workspace_bytes(batch, nheads, headdim=64, ngroups=8, dstate=128):
    return load().ssd_state_update_workspace_bytes(batch, nheads, headdim, ngroups, dstate)


def ssd_state_update_ws(state, xbc, dt, A, *, ngroups, conv_state=None, conv_w=None,
                        conv_b=None, z=None, D=None, dt_bias=None, dt_softplus=True, y=None,
                        y_dtype=torch.float32, workspace=None):
    """The same decode step in two kernels through a workspace (allocated
    here when not given; a uint8 device tensor of at least
    ssd_state_update_workspace_bytes bytes)."""
    lib = load()
    y, B, H, P, G, N, K = _state_update_args(state, xbc, dt, ngroups, conv_state, conv_w,
                                             conv_b, z, y, y_dtype)
    need = lib.ssd_state_update_workspace_bytes(B, H, P, G, N)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=state.device)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ssd_state_update_ws(_p(state), _p(xbc), _dt(xbc), _p(conv_state), _p(conv_w),
                                   _p(conv_b), K, _p(dt), _p(z), _dt(dt), _p(A), _p(D),
                                   _p(dt_bias), int(bool(dt_softplus)), _p(y), _dt(y), B, H, P,
                                   G, N, _p(workspace), wsz, _stream(state)))
    return y


def ssd_state_update_noalloc(state, xbc, dt, A, *, ngroups, conv_state=None, conv_w=None,
                             conv_b=None, z=None, D=None, dt_bias=None, dt_softplus=True,
                             y=None, y_dtype=torch.float32):
    """The two-kernel decode step with no workspace and no allocation in the
    library (its scratch is a static device array; batch * Cdim <= 4194304).
    Pass y to allocate nothing here either."""
    lib = load()
    y, B, H, P, G, N, K = _state_update_args(state, xbc, dt, ngroups, conv_state, conv_w,
                                             conv_b, z, y, y_dtype)
    _check(lib.ssd_state_update_noalloc(_p(state), _p(xbc), _dt(xbc), _p(conv_state),
                                        _p(conv_w), _p(conv_b), K, _p(dt), _p(z), _dt(dt), _p(A),
                                        _p(D), _p(dt_bias), int(bool(dt_softplus)), _p(y), _dt(y),
                                        B, H, P, G, N, _stream(state)))
    return y


def _rows(t: torch.Tensor, width: int, name: str):
    """(rows, row stride) of a tensor viewed as [rows, width] with contiguous rows."""
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.shape[-1] != width:
        raise ValueError("%s has %d columns, want %d" % (name, t.shape[-1], width))
    rows = t.numel() // width if width else 0
    if rows == 0:
        return 0, width
    v = t.view(rows, width)  # raises rather than copies for incompatible layouts
    if width > 1 and v.stride(1) != 1:
        raise ValueError("%s: rows must be contiguous" % name)
    return rows, (v.stride(0) if rows > 1 else width)


def ssd_rmsnorm_fwd(x, weight=None, eps=1e-5, out=None, out_dtype=torch.bfloat16):
    """RMSNorm over the last axis of x [..., dim] -> out (same shape)."""
    lib = load()
    dim = x.shape[-1]
    ntok, xs = _rows(x, dim, "x")
    _dense(weight, (dim,), "weight", torch.float32)
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    no, os_ = _rows(out, dim, "out")
    if no != ntok:
        raise ValueError("out has %d rows, x has %d" % (no, ntok))
    _check(lib.ssd_rmsnorm_fwd(_p(x), xs, _dt(x), _p(weight), float(eps), _p(out), os_, _dt(out),
                               ntok, dim, _stream(x)))
    return out


def ssd_linear_fwd(a, w, residual=None, out=None, out_dtype=torch.float32):
    """out = a @ w^T (+ residual) on the matrix cores: a [..., K] bf16,
    w [N, K] bf16, residual [..., N] or None."""
    lib = load()
    N, K = w.shape
    if a.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise TypeError("a and w must be bfloat16")
    M, lda = _rows(a, K, "a")
    _, ldw = _rows(w, K, "w")
    if out is None:
        out = torch.empty(a.shape[:-1] + (N,), dtype=out_dtype, device=a.device)
    mo, ldo = _rows(out, N, "out")
    ldr, rdt = 0, SSD_F32
    if residual is not None:
        mr, ldr = _rows(residual, N, "residual")
        if mr != M:
            raise ValueError("residual has %d rows, a has %d" % (mr, M))
        rdt = _dt(residual)
    if mo != M:
        raise ValueError("out has %d rows, a has %d" % (mo, M))
    _check(lib.ssd_linear_fwd(_p(a), lda, _p(w), ldw, _p(residual), ldr, rdt, _p(out), ldo,
                              _dt(out), M, N, K, _stream(a)))
    return out


def ssd_block_workspace_bytes(batch, seqlen, d_model, nheads, headdim=64, ngroups=8, dstate=128):
    return load().ssd_block_workspace_bytes(batch, seqlen, d_model, nheads, headdim, ngroups,
                                            dstate)


def ssd_block_fwd(h, norm_w, in_proj_w, conv_w, A, out_proj_w, *, nheads, ngroups, conv_b=None,
                  D=None, dt_bias=None, dt_softplus=True, norm_eps=1e-5, conv_state_in=None,
                  conv_state_out=None, initial_state=None, final_state=None, out=None,
                  out_dtype=torch.float32, workspace=None):
    """The pre-norm residual block: out = h + out_proj(mixer(rmsnorm(h))).
    h [B, L, d_model]; in_proj_w [2*H*P + 2*G*N + H, d_model] bf16 (rows
    z | x | B | C | dt); out_proj_w [d_model, H*P] bf16."""
    lib = load()
    B, L, dm = h.shape
    H, G, P, N = nheads, ngroups, 64, 128
    HP, GN = H * P, G * N
    cdim = HP + 2 * GN
    K = conv_w.shape[1]
    if not h.is_contiguous() or not h.is_cuda:
        raise ValueError("h must be a contiguous device tensor")
    _dense(norm_w, (dm,), "norm_w", torch.float32)
    _dense(in_proj_w, (2 * HP + 2 * GN + H, dm), "in_proj_w", torch.bfloat16)
    _dense(out_proj_w, (dm, HP), "out_proj_w", torch.bfloat16)
    _dense(conv_w, (cdim, K), "conv_w", torch.float32)
    _dense(conv_b, (cdim,), "conv_b", torch.float32)
    for n, t in (("A", A), ("D", D), ("dt_bias", dt_bias)):
        _dense(t, (H,), n, torch.float32)
    _dense(conv_state_in, (B, K - 1, cdim), "conv_state_in", torch.bfloat16)
    _dense(conv_state_out, (B, K - 1, cdim), "conv_state_out", torch.bfloat16)
    _dense(initial_state, (B, H, P, N), "initial_state", torch.float32)
    _dense(final_state, (B, H, P, N), "final_state", torch.float32)
    if out is None:
        out = torch.empty((B, L, dm), dtype=out_dtype, device=h.device)
    _dense(out, (B, L, dm), "out")
    need = lib.ssd_block_workspace_bytes(B, L, dm, H, P, G, N)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=h.device)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ssd_block_fwd(
        _p(h), _dt(h), _p(norm_w), float(norm_eps), _p(in_proj_w), _p(conv_w), _p(conv_b), K,
        _p(A), _p(D), _p(dt_bias), int(bool(dt_softplus)), _p(out_proj_w), _p(conv_state_in),
        _p(conv_state_out), _p(initial_state), _p(final_state), _p(out), _dt(out), B, L, dm, H, P,
        G, N, _p(workspace), wsz, _stream(h)))
    return out


def ssd_chunk_scan_bwd_workspace_bytes(batch, seqlen, nheads, headdim=64, ngroups=8, dstate=128,
                                       conv_width=0):
    return load().ssd_chunk_scan_bwd_workspace_bytes(batch, seqlen, nheads, headdim, ngroups,
                                                     dstate, conv_width)


def ssd_chunk_scan_bwd(x, Bm, Cm, dt, A, dout, *, D=None, z=None, dt_bias=None, dt_softplus=True,
                       initial_state=None, d_final_state=None, conv_w=None, conv_b=None,
                       conv_state_in=None, want_initial_state=True, workspace=None):
    """Gradients of ssd_chunk_scan_fwd.  Inputs as there; dout [B, L, H, P] and
    d_final_state [B, H, P, N] or None.  Returns a dict of fp32 device tensors:
    xbc [B, L, Cdim] (raw conv inputs when conv_w is given), dt [B, L, H], A,
    and where applicable z, D, dt_bias, initial_state, conv_w, conv_b,
    conv_state_in."""
    lib = load()
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    dev = x.device
    cdim = H * P + 2 * G * N
    if Bm.dtype != x.dtype or Cm.dtype != x.dtype:
        raise TypeError("x, Bm, Cm must share a dtype")
    if z is not None and z.dtype != dt.dtype:
        raise TypeError("z and dt must share a dtype")
    xs, bs, cs = _tok(x, B, L, H * P, "x"), _tok(Bm, B, L, G * N, "Bm"), _tok(Cm, B, L, G * N, "Cm")
    dts, zs = _tok(dt, B, L, H, "dt"), _tok(z, B, L, H * P, "z")
    ds = _tok(dout, B, L, H * P, "dout")
    for n, t in (("A", A), ("D", D), ("dt_bias", dt_bias)):
        _dense(t, (H,), n, torch.float32)
    _dense(initial_state, (B, H, P, N), "initial_state", torch.float32)
    _dense(d_final_state, (B, H, P, N), "d_final_state", torch.float32)
    K = 0
    if conv_w is not None:
        K = conv_w.shape[1]
        _dense(conv_w, (cdim, K), "conv_w", torch.float32)
        _dense(conv_b, (cdim,), "conv_b", torch.float32)
        _dense(conv_state_in, (B, K - 1, cdim), "conv_state_in", x.dtype)
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"xbc": torch.empty((B, L, cdim), **f32), "dt": torch.empty((B, L, H), **f32),
         "A": torch.empty((H,), **f32), "D": torch.empty((H,), **f32),
         "dt_bias": torch.empty((H,), **f32)}
    if z is not None:
        g["z"] = torch.empty((B, L, H, P), **f32)
    if want_initial_state:
        g["initial_state"] = torch.empty((B, H, P, N), **f32)
    if conv_w is not None:
        g["conv_w"] = torch.empty((cdim, K), **f32)
        g["conv_b"] = torch.empty((cdim,), **f32)
        g["conv_state_in"] = torch.empty((B, K - 1, cdim), **f32)
    need = lib.ssd_chunk_scan_bwd_workspace_bytes(B, L, H, P, G, N, K)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ssd_chunk_scan_bwd(
        _p(x), xs, _p(Bm), bs, _p(Cm), cs, _dt(x), _p(conv_w), _p(conv_b), K, _p(conv_state_in),
        _p(dt), dts, _p(z), zs, _dt(dt), _p(A), _p(D), _p(dt_bias), int(bool(dt_softplus)),
        _p(initial_state), _p(dout), ds, _dt(dout), _p(d_final_state), _p(g["xbc"]), _p(g["dt"]),
        _p(g.get("z")), _p(g["A"]), _p(g["D"]), _p(g["dt_bias"]), _p(g.get("initial_state")),
        _p(g.get("conv_w")), _p(g.get("conv_b")), _p(g.get("conv_state_in")), B, L, H, P, G, N,
        _p(workspace), wsz, _stream(x)))
    return g
