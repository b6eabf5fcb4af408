"""The Mamba-2 SSD layer's forward paths as sequences of libssd calls.

Argument marshalling only; the arithmetic is in the library's kernels.

* ``prefill``: conv + SiLU over x|B|C, then the chunked scan with D skip and
  SiLU(z) gate.  ``fused=False`` runs ``ssd_causal_conv1d_fwd`` into an fp32
  intermediate and hands views of it to ``ssd_chunk_scan_fwd``; ``fused=True``
  passes the raw x|B|C and the conv weights to ``ssd_chunk_scan_fwd``, which
  convolves inside its prologue.
* ``decode_step``: one ``ssd_state_update_ws`` call (or ``ssd_state_update``).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import ssd

# The prefill path the benchmark times: conv fused into the scan's prologue.
DEFAULT_FUSED = True


@dataclass
class LayerParams:
    nheads: int
    ngroups: int
    conv_w: torch.Tensor              # [Cdim, K] fp32
    A: torch.Tensor                   # [H] fp32
    dt_bias: Optional[torch.Tensor]   # [H] fp32
    D: Optional[torch.Tensor]         # [H] fp32
    conv_b: Optional[torch.Tensor] = None
    headdim: int = 64
    dstate: int = 128
    chunk: int = 128
    dt_softplus: bool = True


def split_xbc(t: torch.Tensor, p: LayerParams):
    """Views x [B,L,H,P], B [B,L,G,N], C [B,L,G,N] of a [B,L,Cdim] buffer."""
    Bsz, L, _ = t.shape
    HP, GN = p.nheads * p.headdim, p.ngroups * p.dstate
    x = t[..., :HP].view(Bsz, L, p.nheads, p.headdim)
    Bm = t[..., HP:HP + GN].view(Bsz, L, p.ngroups, p.dstate)
    Cm = t[..., HP + GN:HP + 2 * GN].view(Bsz, L, p.ngroups, p.dstate)
    return x, Bm, Cm


def prefill(xbc: torch.Tensor, dt: torch.Tensor, z: Optional[torch.Tensor], p: LayerParams, *,
            fused: bool = DEFAULT_FUSED, math: str = "bf16", initial_state=None, final_state=None,
            conv_state_in=None, conv_state_out=None, conv_out=None, y=None,
            y_dtype=torch.float32, workspace=None):
    """xbc [B,L,Cdim] raw, dt [B,L,H], z [B,L,H,P] -> y [B,L,H,P]."""
    if fused:
        x, Bm, Cm = split_xbc(xbc, p)
        return ssd.ssd_chunk_scan_fwd(
            x, Bm, Cm, dt, p.A, D=p.D, z=z, dt_bias=p.dt_bias, dt_softplus=p.dt_softplus,
            initial_state=initial_state, final_state=final_state, conv_w=p.conv_w,
            conv_b=p.conv_b, conv_state_in=conv_state_in, conv_state_out=conv_state_out,
            chunk=p.chunk, math=math, y=y, y_dtype=y_dtype, workspace=workspace)
    conv_out = ssd.ssd_causal_conv1d_fwd(xbc, p.conv_w, p.conv_b, conv_state_in, conv_state_out,
                                         out=conv_out, out_dtype=torch.float32)
    x, Bm, Cm = split_xbc(conv_out, p)
    return ssd.ssd_chunk_scan_fwd(
        x, Bm, Cm, dt, p.A, D=p.D, z=z, dt_bias=p.dt_bias, dt_softplus=p.dt_softplus,
        initial_state=initial_state, final_state=final_state, chunk=p.chunk, math=math, y=y,
        y_dtype=y_dtype, workspace=workspace)


def decode_step(state, xbc, dt, z, conv_state, p: LayerParams, *, y=None,
                y_dtype=torch.float32, workspace=None, fused=False):
    """One token per sequence: state [B,H,P,N] and conv_state [B,K-1,Cdim]
    are updated in place; returns y [B, H*P].  By default the two-kernel step
    through a workspace (allocated per call when not given); fused=True takes
    ssd_state_update, which needs none."""
    if fused:
        return ssd.ssd_state_update(state, xbc, dt, p.A, ngroups=p.ngroups,
                                    conv_state=conv_state, conv_w=p.conv_w, conv_b=p.conv_b,
                                    z=z, D=p.D, dt_bias=p.dt_bias, dt_softplus=p.dt_softplus,
                                    y=y, y_dtype=y_dtype)
    return ssd.ssd_state_update_ws(state, xbc, dt, p.A, ngroups=p.ngroups, conv_state=conv_state,
                                   conv_w=p.conv_w, conv_b=p.conv_b, z=z, D=p.D,
                                   dt_bias=p.dt_bias, dt_softplus=p.dt_softplus, y=y,
                                   y_dtype=y_dtype, workspace=workspace)
