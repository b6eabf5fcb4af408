"""GPU parity of the layer's backward pass (ssd_chunk_scan_bwd) against the
fp64 oracle's (oracle_mamba2_bwd), through the C ABI.

Tolerance: for every gradient tensor, max|gpu - oracle| <= 1e-4 RMS(oracle).
The backward is fp32 throughout; its longest sums (the state's gradient
carried over every chunk, the parameter sums over every token) accumulate
rounding of a few ulps per term with random signs, far inside 1e-4.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from harness import dev, dev32, say
from selective_state_space_08_amd import ssd, synth
from selective_state_space_08_amd.workloads import WORKLOADS, Workload

pytestmark = pytest.mark.gpu

TOL = 1e-4


def views(xbc_t, wl):
    B, L = xbc_t.shape[:2]
    HP, GN = wl.d_inner, wl.ngroups * wl.dstate
    x = xbc_t[:, :, :HP].unflatten(-1, (wl.nheads, wl.headdim))
    Bm = xbc_t[:, :, HP:HP + GN].unflatten(-1, (wl.ngroups, wl.dstate))
    Cm = xbc_t[:, :, HP + GN:].unflatten(-1, (wl.ngroups, wl.dstate))
    return x, Bm, Cm


def run(inp, *, conv=True, gate=True, D=True, bias=True, h0=True, hist=None, dhT=None,
        dout=None, dout_dtype="f32"):
    wl = inp.wl
    dt_ = wl.dtype
    xbc_t = dev(inp.xbc, dt_)
    x, Bm, Cm = views(xbc_t, wl)
    g = ssd.ssd_chunk_scan_bwd(
        x, Bm, Cm, dev(inp.dt, dt_), dev32(inp.A), dev(dout, dout_dtype),
        D=dev32(inp.D) if D else None, z=dev(inp.z, dt_) if gate else None,
        dt_bias=dev32(inp.dt_bias) if bias else None,
        initial_state=dev32(inp.h0) if (h0 and inp.h0 is not None) else None,
        d_final_state=dev32(dhT), conv_w=dev32(inp.conv_w) if conv else None,
        conv_state_in=dev(hist, dt_) if (conv and hist is not None) else None)
    torch.cuda.synchronize()
    return {k: v.double().cpu().numpy() for k, v in g.items()}


def reference(inp, *, conv=True, gate=True, D=True, bias=True, h0=True, hist=None, dhT=None,
              dout=None):
    wl = inp.wl
    return oracle.mamba2_bwd(inp.xbc, inp.dt, inp.A, dout, nheads=wl.nheads, headdim=wl.headdim,
                             ngroups=wl.ngroups, dstate=wl.dstate,
                             conv_w=inp.conv_w if conv else None,
                             conv_state_in=hist if conv else None,
                             D=inp.D if D else None, dt_bias=inp.dt_bias if bias else None,
                             z=inp.z if gate else None,
                             h0=inp.h0 if (h0 and inp.h0 is not None) else None, dh_final=dhT)


def compare(got, ref, keys):
    for k in keys:
        r = ref[k]
        rms = math.sqrt(float(np.mean(r * r))) or 1.0
        err = float(np.max(np.abs(got[k] - r))) / rms
        say("  d%-14s max|err|/RMS %.2e" % (k, err))
        assert err <= TOL, "gradient of %s: %.3e" % (k, err)


def make(B, L, H, G, dtype="bf16", h0=True, seed=3):
    wl = Workload("bwd", batch=B, seqlen=L, nheads=H, ngroups=G, dtype=dtype, initial_state=h0,
                  seed=seed)
    inp = synth.make_prefill(wl)
    rng = np.random.default_rng(seed + 100)
    dout = rng.standard_normal((B, L, H, 64)).astype(np.float32)
    dhT = (0.1 * rng.standard_normal((B, H, 64, 128))).astype(np.float32)
    return inp, dout, dhT


@pytest.mark.parametrize("B,L,H,G,dtype,conv,gate,h0,hist,final", [
    (2, 100, 4, 2, "bf16", True, True, True, True, True),     # everything; ragged last chunk
    (1, 64, 2, 1, "f32", True, False, False, False, False),   # exactly two chunks
    (2, 33, 4, 1, "bf16", False, True, True, False, True),    # post-conv inputs
    (1, 1, 2, 2, "f32", True, True, True, True, True),        # one token: history only
    (3, 32, 8, 2, "bf16", True, True, False, True, False),    # one full chunk
    (1, 300, 16, 4, "bf16", True, True, True, False, True),   # several chunks, 4 heads a group
])
def test_bwd_matches_oracle(B, L, H, G, dtype, conv, gate, h0, hist, final):
    say("bwd B=%d L=%d H=%d G=%d %s conv=%s gate=%s h0=%s hist=%s dhT=%s"
        % (B, L, H, G, dtype, conv, gate, h0, hist, final))
    inp, dout, dhT = make(B, L, H, G, dtype, h0=h0)
    hist_v = synth.raw_history(inp.wl, 77) if hist else None
    kw = dict(conv=conv, gate=gate, h0=h0, hist=hist_v, dhT=dhT if final else None, dout=dout)
    got = run(inp, **kw)
    ref = reference(inp, **kw)
    keys = ["xbc", "dt", "A", "D", "dt_bias", "h0"] + (["z"] if gate else []) + \
           (["conv_w", "conv_b", "conv_state_in"] if conv else [])
    got["h0"] = got.pop("initial_state")
    # (without a history the conv history's gradient is the one at zero)
    compare(got, ref, keys)


def test_bwd_bf16_dout():
    say("bwd with a bf16 output gradient")
    inp, dout, dhT = make(2, 70, 4, 2)
    synth.round_bf16_(dout)
    got = run(inp, dhT=dhT, dout=dout, dout_dtype="bf16")
    ref = reference(inp, dhT=dhT, dout=dout)
    got["h0"] = got.pop("initial_state")
    compare(got, ref, ["xbc", "dt", "z", "A", "D", "dt_bias", "h0", "conv_w", "conv_b"])


def test_bwd_empty_sequence():
    """L = 0: the initial state's gradient is the final state's; the rest are 0."""
    say("bwd empty sequence")
    B, H, G = 2, 4, 2
    wl = Workload("e", batch=B, seqlen=0, nheads=H, ngroups=G)
    cdim = wl.cdim
    e = torch.empty
    x = e((B, 0, H, 64), dtype=torch.bfloat16, device="cuda")
    Bm = e((B, 0, G, 128), dtype=torch.bfloat16, device="cuda")
    dhT = torch.randn(B, H, 64, 128, device="cuda")
    g = ssd.ssd_chunk_scan_bwd(x, Bm, Bm, e((B, 0, H), dtype=torch.bfloat16, device="cuda"),
                               -torch.ones(H, device="cuda"),
                               e((B, 0, H, 64), device="cuda"), d_final_state=dhT,
                               conv_w=torch.ones(cdim, 4, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(g["initial_state"], dhT)
    for k in ("A", "D", "dt_bias", "conv_w", "conv_b", "conv_state_in"):
        assert torch.count_nonzero(g[k]) == 0, k


def test_bwd_bit_stable():
    say("bwd bit-stable")
    inp, dout, dhT = make(2, 100, 4, 2)
    a = run(inp, dhT=dhT, dout=dout)
    b = run(inp, dhT=dhT, dout=dout)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_bwd_full_size_one_group():
    """The Nemotron-3-Nano workload (B=8, L=4096, H=64, G=8) at full size in one
    call; the oracle checks one (sequence, group) -- its 8 heads over the whole
    sequence, with the group's shared B and C -- as a problem of its own."""
    wl = WORKLOADS["nemotron3_nano_b8_l4096"]
    say("bwd full size %s" % wl.name)
    inp = synth.make_prefill(wl)
    B, L, H, G = wl.batch, wl.seqlen, wl.nheads, wl.ngroups
    rng = np.random.default_rng(9)
    dout = rng.standard_normal((B, L, H, 64), dtype=np.float32)
    dhT = (0.1 * rng.standard_normal((B, H, 64, 128))).astype(np.float32)
    got = run(inp, dhT=dhT, dout=dout)
    b, g = 5, 3
    hpg = H // G
    heads = np.arange(g * hpg, (g + 1) * hpg)
    HP, GN, N = wl.d_inner, G * 128, 128
    ch = np.concatenate([(heads[:, None] * 64 + np.arange(64)).ravel(),
                         HP + g * N + np.arange(N), HP + GN + g * N + np.arange(N)])
    ref = oracle.mamba2_bwd(inp.xbc[b:b + 1][:, :, ch], inp.dt[b:b + 1][:, :, heads], inp.A[heads],
                            dout[b:b + 1][:, :, heads], nheads=hpg, headdim=64, ngroups=1,
                            dstate=128, conv_w=inp.conv_w[ch], D=inp.D[heads],
                            dt_bias=inp.dt_bias[heads], z=inp.z[b:b + 1][:, :, heads],
                            h0=inp.h0[b:b + 1][:, heads], dh_final=dhT[b:b + 1][:, heads])
    sub = {"xbc": got["xbc"][b:b + 1][:, :, ch], "dt": got["dt"][b:b + 1][:, :, heads],
           "z": got["z"][b:b + 1][:, :, heads], "h0": got["initial_state"][b:b + 1][:, heads]}
    compare(sub, ref, ["xbc", "dt", "z", "h0"])
