"""Seeded synthetic inputs for the layer.

This is the one module that both the GPU path's tests/benchmark and the CPU
oracle read their inputs from.  It holds none of the layer's arithmetic: it
draws random numbers and rounds them to the workload's dtype, nothing else.

Recipe.  Every block of draws has its own generator,
``Generator(PCG64(SeedSequence([seed, block])))``, so the result does not depend
on how many threads fill it.  Block 0 holds the parameters and states, drawn
in this order (float32 draws; the second argument of N is the std):
  conv_w  [Cdim, K]   ~ N(0, 0.25)
  A       [H]         = -exp(U(ln 1, ln 16))          (A in [-16, -1]),
                        or -U(0.01, 2) for the slow-decay probe
  dt0     [H]         = exp(U(ln 1e-3, ln 1e-1));  dt_bias = dt0 + log(-expm1(-dt0)),
                        the inverse softplus of dt0
  D       [H]         = 1
  h0      [B,H,P,N]   ~ N(0, 0.1)        (workloads with an initial state)
  ring    [B,K-1,Cdim] raw x|B|C draws   (decode only)
Block 1 + i holds token block i: for prefill, tokens [4096 j, 4096 (j+1)) of
sequence b with i = b * ceil(L/4096) + j; for decode, step i.  In each:
  xbc     [.., Cdim]  x part ~ N(0,1); B and C parts ~ N(0,1) / sqrt(d_state)
  z       [.., H, P]  ~ N(0,1)
  dt      [.., H]     ~ 0.5 N(0,1)       (raw: dt_bias and softplus are the layer's)
Activations (xbc, z, dt, ring) are rounded to bf16, ties to even, for bf16
workloads; the rounded values are the ground truth for both sides.
Parameters and states stay fp32.

The block around the layer (make_block) adds, from block 2^31 - 2 of the
seed, in this order:
  norm_w     [d_model]            = 1 + 0.1 N(0,1)             (fp32)
  in_proj_w  [d_in_proj, d_model] ~ N(0,1) times a per-row scale / sqrt(d_model):
                                    1 for the z and x rows, 1/sqrt(d_state) for
                                    the B and C rows, 0.5 for the dt rows, so
                                    that on a unit-RMS input the projection's
                                    outputs have the spread of the layer's
                                    token draws above             (bf16)
  out_proj_w [d_model, d_inner]   ~ N(0, 1/sqrt(d_inner))       (bf16)
and the block input h [B, L, d_model] ~ N(0,1) (bf16) from the token blocks
1 + i as above.  conv_w, A, dt_bias and D are the layer's (block 0).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .workloads import Workload

TOKEN_BLOCK = 4096


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def round_bf16_(a: np.ndarray) -> np.ndarray:
    """Round a float32 array to the nearest bfloat16 value (ties to even), in place."""
    assert a.dtype == np.float32 and a.flags.c_contiguous
    u = a.reshape(-1).view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The bfloat16 bit patterns (uint16) of a float32 array whose values are
    already bf16 values."""
    assert a.dtype == np.float32
    return (np.ascontiguousarray(a).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _rng(seed: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, block])))


def _normal(rng, shape, std=1.0):
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


@dataclass
class Params:
    conv_w: np.ndarray          # [Cdim, K]
    A: np.ndarray               # [H]
    dt_bias: np.ndarray         # [H]
    D: np.ndarray               # [H]
    h0: Optional[np.ndarray]    # [B,H,P,N] or None
    ring: Optional[np.ndarray]  # [B,K-1,Cdim] or None


def _params(wl: Workload, seed: int, slow_decay: bool, decode: bool) -> Params:
    rng = _rng(seed, 0)
    conv_w = _normal(rng, (wl.cdim, wl.width), 0.25)
    if slow_decay:
        A = -rng.uniform(0.01, 2.0, wl.nheads).astype(np.float32)
    else:
        A = -np.exp(rng.uniform(math.log(1.0), math.log(16.0), wl.nheads)).astype(np.float32)
    dt0 = np.exp(rng.uniform(math.log(1e-3), math.log(1e-1), wl.nheads))
    dt_bias = (dt0 + np.log(-np.expm1(-dt0))).astype(np.float32)
    D = np.ones(wl.nheads, np.float32)
    B, H, P, N = wl.batch, wl.nheads, wl.headdim, wl.dstate
    h0 = _normal(rng, (B, H, P, N), 0.1) if (wl.initial_state or decode) else None
    ring = None
    if decode:
        ring = np.empty((B, wl.width - 1, wl.cdim), np.float32)
        _fill_tokens(rng, wl, ring)
        if wl.dtype == "bf16":
            round_bf16_(ring)
    return Params(conv_w, A, dt_bias, D, h0, ring)


def _fill_tokens(rng, wl: Workload, xbc, z=None, dt=None):
    """One block's raw x|B|C, z and dt draws, in that order."""
    xbc[...] = rng.standard_normal(xbc.shape, dtype=np.float32)
    xbc[..., wl.d_inner:] *= np.float32(1.0 / math.sqrt(wl.dstate))
    if z is not None:
        z[...] = rng.standard_normal(z.shape, dtype=np.float32)
    if dt is not None:
        dt[...] = _normal(rng, dt.shape, 0.5)
    if wl.dtype == "bf16":
        for a in (xbc, z, dt):
            if a is not None:
                round_bf16_(a)


def raw_history(wl: Workload, seed: int) -> np.ndarray:
    """A conv history [B, K-1, Cdim] of raw x|B|C values drawn like the tokens
    (its own generator, block -1 of the seed)."""
    h = np.empty((wl.batch, wl.width - 1, wl.cdim), np.float32)
    _fill_tokens(np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2**31 - 1]))),
                 wl, h)
    return h


@dataclass
class PrefillInputs:
    wl: Workload
    conv_w: np.ndarray          # [Cdim, K] f32
    A: np.ndarray               # [H]
    dt_bias: np.ndarray         # [H]
    D: np.ndarray               # [H]
    h0: Optional[np.ndarray]    # [B,H,P,N] or None
    xbc: np.ndarray             # [B,L,Cdim] f32 values (bf16 values for bf16 workloads)
    z: np.ndarray               # [B,L,H,P]
    dt: np.ndarray              # [B,L,H]


def make_prefill(wl: Workload, seed: Optional[int] = None, slow_decay: bool = False,
                 seqlen: Optional[int] = None, batch: Optional[int] = None) -> PrefillInputs:
    if seqlen is not None:
        wl = wl.with_(seqlen=seqlen)
    if batch is not None:
        wl = wl.with_(batch=batch)
    seed = wl.seed if seed is None else seed
    prm = _params(wl, seed, slow_decay, decode=False)
    B, L, H, P = wl.batch, wl.seqlen, wl.nheads, wl.headdim
    xbc = np.empty((B, L, wl.cdim), np.float32)
    z = np.empty((B, L, H, P), np.float32)
    dt = np.empty((B, L, H), np.float32)
    nblk = max(1, -(-L // TOKEN_BLOCK))

    def fill(i):
        b, j = divmod(i, nblk)
        t0, t1 = j * TOKEN_BLOCK, min(L, (j + 1) * TOKEN_BLOCK)
        _fill_tokens(_rng(seed, 1 + i), wl, xbc[b, t0:t1], z[b, t0:t1], dt[b, t0:t1])

    if L > 0:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(B * nblk)))
    return PrefillInputs(wl, prm.conv_w, prm.A, prm.dt_bias, prm.D, prm.h0, xbc, z, dt)


@dataclass
class DecodeInputs:
    wl: Workload
    seed: int
    conv_w: np.ndarray          # [Cdim, K]
    A: np.ndarray
    dt_bias: np.ndarray
    D: np.ndarray
    state: np.ndarray           # [B,H,P,N] f32
    ring: np.ndarray            # [B,K-1,Cdim] raw inputs (bf16 values for bf16)

    def steps(self, s0: int, s1: int):
        """Per-step inputs of steps [s0, s1): xbc [T,B,Cdim], z [T,B,H*P], dt [T,B,H]."""
        wl = self.wl
        T, B = s1 - s0, wl.batch
        xbc = np.empty((T, B, wl.cdim), np.float32)
        z = np.empty((T, B, wl.d_inner), np.float32)
        dt = np.empty((T, B, wl.nheads), np.float32)

        def fill(i):
            _fill_tokens(_rng(self.seed, 1 + s0 + i), wl, xbc[i], z[i], dt[i])

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(T)))
        return xbc, z, dt


def make_decode(wl: Workload, seed: Optional[int] = None,
                batch: Optional[int] = None) -> DecodeInputs:
    if batch is not None:
        wl = wl.with_(batch=batch)
    seed = wl.seed if seed is None else seed
    prm = _params(wl, seed, False, decode=True)
    return DecodeInputs(wl, seed, prm.conv_w, prm.A, prm.dt_bias, prm.D, prm.h0, prm.ring)


@dataclass
class BlockInputs:
    wl: Workload
    h: np.ndarray               # [B,L,d_model] bf16 values (f32 array)
    norm_w: np.ndarray          # [d_model] f32
    in_proj_w: np.ndarray       # [d_in_proj, d_model] bf16 values
    out_proj_w: np.ndarray      # [d_model, d_inner] bf16 values
    conv_w: np.ndarray          # [Cdim, K] f32
    A: np.ndarray               # [H]
    dt_bias: np.ndarray         # [H]
    D: np.ndarray               # [H]


def make_block(wl: Workload, seed: Optional[int] = None, seqlen: Optional[int] = None,
               batch: Optional[int] = None, d_model: Optional[int] = None) -> BlockInputs:
    """Inputs of the pre-norm residual block around the layer (bf16 h and
    projection weights; see the module notes for the recipe)."""
    if seqlen is not None:
        wl = wl.with_(seqlen=seqlen)
    if batch is not None:
        wl = wl.with_(batch=batch)
    seed = wl.seed if seed is None else seed
    dm = wl.d_model if d_model is None else d_model
    prm = _params(wl, seed, slow_decay=False, decode=False)
    HP, GN, H = wl.d_inner, wl.ngroups * wl.dstate, wl.nheads
    rng = _rng(seed, 2**31 - 2)
    norm_w = (1.0 + _normal(rng, (dm,), 0.1)).astype(np.float32)
    scale = np.concatenate([np.ones(2 * HP), np.full(2 * GN, 1.0 / math.sqrt(wl.dstate)),
                            np.full(H, 0.5)]).astype(np.float32) / np.float32(math.sqrt(dm))
    in_proj_w = _normal(rng, (wl.d_in_proj, dm))
    in_proj_w *= scale[:, None]
    round_bf16_(in_proj_w)
    out_proj_w = _normal(rng, (dm, HP), 1.0 / math.sqrt(HP))
    round_bf16_(out_proj_w)
    B, L = wl.batch, wl.seqlen
    h = np.empty((B, L, dm), np.float32)
    nblk = max(1, -(-L // TOKEN_BLOCK))

    def fill(i):
        b, j = divmod(i, nblk)
        t0, t1 = j * TOKEN_BLOCK, min(L, (j + 1) * TOKEN_BLOCK)
        h[b, t0:t1] = _rng(seed, 1 + i).standard_normal((t1 - t0, dm), dtype=np.float32)
        round_bf16_(h[b, t0:t1])

    if L > 0:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(B * nblk)))
    return BlockInputs(wl, h, norm_w, in_proj_w, out_proj_w, prm.conv_w, prm.A, prm.dt_bias,
                       prm.D)
