"""GPU parity: libssd's HIP kernels against the fp64 oracle.

Tolerances (max |gpu - oracle| over RMS(oracle output)):
  fp32 path (SSD_MATH_F32, fp32 activations)        <= 1e-4
  bf16 matrix-core path (bf16 in, fp32 accumulate)  <= 2e-2
The SSM term is small next to the D skip under these input distributions,
so every case also runs the "SSM only" probe (D = None, z = None), checked
by relative RMS error: <= 1e-5 on the fp32 path, <= 1e-2 on the bf16 path.
"""
import numpy as np
import pytest
import torch

import oracle
from harness import (dev, dev32, gather_y, gpu_prefill, oracle_pairs, params, pick_pairs,
                     rel_max_err, rel_rms_err, say)
from selective_state_space_08_amd import layer, ssd, synth
from selective_state_space_08_amd.workloads import Workload

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
# SSM-only probes (D = 0, no gate): relative RMS error.  bf16: about 2.6 unit
# roundoffs (u = 2^-9) -- the matrix-core products round C, B, the masked
# C B^T tile, x and the bf16 copy of the state once each, independent errors
# of RMS u / sqrt(3), about 4 per element, RMS ~2.3e-3 -- so that a 1% error
# in the SSM term fails.
PROBE_TOL = {"f32": 1e-5, "bf16": 5e-3}


def small(B, L, H, G, dtype="bf16", h0=True, seed=1):
    wl = Workload("t", batch=B, seqlen=L, nheads=H, ngroups=G, dtype=dtype, initial_state=h0,
                  seed=seed)
    return synth.make_prefill(wl)


# ---------------------------------------------------------------- conv kernel

@pytest.mark.parametrize("B,L,C,K,xd,od,hist,bias", [
    (1, 512, 512, 4, "f32", "f32", False, False),
    (2, 300, 1024, 4, "bf16", "f32", True, True),
    (3, 37, 520, 3, "bf16", "bf16", True, False),
    (2, 45, 260, 4, "bf16", "f32", True, True),     # 4 channels per thread (bf16 -> fp32)
    (2, 45, 262, 4, "bf16", "f32", True, True),     # not a multiple of 4: scalar path
    (1, 70, 260, 3, "bf16", "bf16", True, False),   # not a multiple of 8: scalar path
    (1, 1, 256, 4, "f32", "f32", True, False),
    (2, 2, 264, 4, "f32", "f32", True, True),       # L < K-1: history reaches into the old one
    (1, 33, 128, 1, "f32", "f32", False, False),
    # large enough for 128-token windows (a ragged last window, both vector widths)
    (2, 4200, 8192, 4, "bf16", "f32", True, True),
    (2, 4200, 8192, 3, "f32", "bf16", True, False),
])
def test_conv_kernel(B, L, C, K, xd, od, hist, bias):
    say("conv B=%d L=%d C=%d K=%d %s->%s" % (B, L, C, K, xd, od))
    rng = np.random.default_rng(B * 1000 + L)
    x = rng.standard_normal((B, L, C)).astype(np.float32)
    h = rng.standard_normal((B, K - 1, C)).astype(np.float32) if hist else None
    if xd == "bf16":
        synth.round_bf16_(x)
        if h is not None:
            synth.round_bf16_(h)
    w = (0.5 * rng.standard_normal((C, K))).astype(np.float32)
    bb = rng.standard_normal(C).astype(np.float32) if bias else None
    ref, href = oracle.causal_conv1d(x, w, bb, h)
    tdt = torch.bfloat16 if xd == "bf16" else torch.float32
    hout = torch.empty((B, K - 1, C), dtype=tdt, device="cuda")
    out = ssd.ssd_causal_conv1d_fwd(dev(x, xd), dev32(w), dev32(bb),
                                    dev(h, xd) if h is not None else None, hout,
                                    out_dtype=torch.bfloat16 if od == "bf16" else torch.float32)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    bound = 2e-6 * np.maximum(1.0, np.abs(ref)) if od == "f32" else 2 ** -8 * np.abs(ref) + 1e-6
    assert np.all(np.abs(got - ref) <= bound)
    np.testing.assert_array_equal(hout.double().cpu().numpy(), href)


# ---------------------------------------------------------------- scan kernels

SCAN_SHAPES = [(1, 128, 2, 1), (2, 300, 4, 2), (1, 1, 2, 2), (1, 129, 8, 2), (2, 1000, 2, 1),
               (1, 257, 4, 4)]


@pytest.mark.parametrize("math_mode", ["f32", "bf16"])
@pytest.mark.parametrize("B,L,H,G", SCAN_SHAPES)
def test_scan_post_conv(math_mode, B, L, H, G):
    """x, B, C given as post-conv values (no conv in the call)."""
    dtype = "f32" if math_mode == "f32" else "bf16"
    inp = small(B, L, H, G, dtype)
    say("scan %s B=%d L=%d H=%d G=%d" % (math_mode, B, L, H, G))
    wl = inp.wl
    pairs = [(b, h) for b in range(B) for h in range(H)]
    for probe in (False, True):
        xbc = dev(inp.xbc, dtype)
        p = params(inp, D=not probe)
        x, Bm, Cm = layer.split_xbc(xbc, p)
        fs = torch.empty((B, H, 64, 128), device="cuda")
        y = ssd.ssd_chunk_scan_fwd(x, Bm, Cm, dev(inp.dt, dtype), p.A, D=p.D,
                                   z=None if probe else dev(inp.z, dtype), dt_bias=p.dt_bias,
                                   initial_state=dev32(inp.h0), final_state=fs,
                                   chunk=128, math=math_mode)
        torch.cuda.synchronize()
        yr, hr = oracle_pairs(inp, pairs, conv=False, D=not probe, z=not probe)
        yg = gather_y(y, pairs)
        hg = np.stack([fs[b, h].double().cpu().numpy() for b, h in pairs])
        if probe:
            assert rel_rms_err(yg, yr) <= PROBE_TOL[math_mode]
        else:
            assert rel_max_err(yg, yr) <= TOL[math_mode]
        assert rel_max_err(hg, hr) <= TOL[math_mode]


@pytest.mark.parametrize("math_mode", ["f32", "bf16"])
@pytest.mark.parametrize("xd,ad,yd", [("bf16", "f32", "f32"), ("f32", "bf16", "bf16"),
                                      ("bf16", "bf16", "bf16")])
def test_prefill_dtype_mix(math_mode, xd, ad, yd):
    """The fused prefill with x|B|C in one dtype, dt and z in another and y in
    a third: every typed instance of both scan paths against the oracle on
    the same (rounded) values.  A bf16 y adds its own rounding, at most 2^-8
    of each element, which is bounded per element."""
    inp = small(2, 300, 4, 2, "f32", seed=43)
    inp.xbc = np.array(inp.xbc)
    inp.dt = np.array(inp.dt)
    inp.z = np.array(inp.z)
    if xd == "bf16":
        synth.round_bf16_(inp.xbc)
    if ad == "bf16":
        synth.round_bf16_(inp.dt)
        synth.round_bf16_(inp.z)
    say("prefill dtypes %s: %s x|B|C, %s dt/z, %s y" % (math_mode, xd, ad, yd))
    p = params(inp)
    fs = torch.empty((2, 4, 64, 128), device="cuda")
    y = layer.prefill(dev(inp.xbc, xd), dev(inp.dt, ad), dev(inp.z, ad).view(2, 300, 4, 64), p,
                      fused=True, math=math_mode, initial_state=dev32(inp.h0), final_state=fs,
                      y_dtype=torch.bfloat16 if yd == "bf16" else torch.float32)
    torch.cuda.synchronize()
    pairs = [(b, h) for b in range(2) for h in range(4)]
    yr, hr = oracle_pairs(inp, pairs)
    yg = gather_y(y, pairs)
    rms = float(np.sqrt(np.mean(yr * yr)))
    slack = 2.0 ** -8 * np.abs(yr) if yd == "bf16" else 0.0
    assert float(np.max(np.abs(yg - yr) - slack)) <= TOL[math_mode] * rms
    hg = np.stack([fs[b, h].double().cpu().numpy() for b, h in pairs])
    assert rel_max_err(hg, hr) <= TOL[math_mode]


@pytest.mark.parametrize("math_mode", ["f32", "bf16"])
@pytest.mark.parametrize("shift", [6.0, 40.0])
def test_scan_strong_decay(math_mode, shift):
    """Raw dt shifted far up (delta ~ shift, delta*A down to about -16*shift
    per token, |Lam| up to ~10^4 within a chunk): the decay factors underflow
    within a few tokens and only the most recent tokens contribute.  Every
    output stays finite and matches the oracle, the SSM part included (D = 0,
    no gate probe).  This also pins the decay of a partial last chunk to its
    last real token (an ulp of Lam there is a visible factor on the state).

    With delta ~ 40 the SSM term dominates y, whose max error then measures
    the bf16 rounding of the decayed C B^T tile (2^-9 relative, R26): that
    case is held to the relative-RMS bound instead."""
    dtype = "f32" if math_mode == "f32" else "bf16"
    inp = small(1, 300, 4, 2, dtype, seed=31)
    inp.dt = inp.dt + np.float32(shift)
    if dtype == "bf16":
        synth.round_bf16_(inp.dt)
    say("strong decay %s shift %g" % (math_mode, shift))
    pairs = [(0, h) for h in range(4)]
    for probe in (False, True):
        p = params(inp, D=not probe)
        x, Bm, Cm = layer.split_xbc(dev(inp.xbc, dtype), p)
        fs = torch.empty((1, 4, 64, 128), device="cuda")
        y = ssd.ssd_chunk_scan_fwd(x, Bm, Cm, dev(inp.dt, dtype), p.A, D=p.D,
                                   z=None if probe else dev(inp.z, dtype), dt_bias=p.dt_bias,
                                   initial_state=dev32(inp.h0), final_state=fs,
                                   chunk=128, math=math_mode)
        torch.cuda.synchronize()
        assert torch.isfinite(y).all() and torch.isfinite(fs).all()
        yr, hr = oracle_pairs(inp, pairs, conv=False, D=not probe, z=not probe)
        yg = gather_y(y, pairs)
        hg = np.stack([fs[b, h].double().cpu().numpy() for b, h in pairs])
        if probe or (math_mode == "bf16" and shift > 10):
            assert rel_rms_err(yg, yr) <= PROBE_TOL[math_mode]
        else:
            assert rel_max_err(yg, yr) <= TOL[math_mode]
        assert rel_max_err(hg, hr) <= TOL[math_mode]


@pytest.mark.parametrize("chunk", [32, 64, 256])
def test_scan_f32_other_chunks(chunk):
    inp = small(1, 300, 2, 1, "f32")
    say("scan f32 chunk %d" % chunk)
    p = params(inp)
    x, Bm, Cm = layer.split_xbc(dev(inp.xbc, "f32"), p)
    fs = torch.empty((1, 2, 64, 128), device="cuda")
    y = ssd.ssd_chunk_scan_fwd(x, Bm, Cm, dev(inp.dt, "f32"), p.A, D=p.D, z=dev(inp.z, "f32"),
                               dt_bias=p.dt_bias, initial_state=dev32(inp.h0), final_state=fs,
                               chunk=chunk, math="f32")
    torch.cuda.synchronize()
    pairs = [(0, 0), (0, 1)]
    yr, hr = oracle_pairs(inp, pairs, conv=False)
    assert rel_max_err(gather_y(y, pairs), yr) <= TOL["f32"]


@pytest.mark.parametrize("math_mode", ["f32", "bf16"])
@pytest.mark.parametrize("fused", [False, True])
def test_layer_with_conv_history(math_mode, fused):
    """Raw x|B|C with a nonzero conv history and conv bias; conv state out."""
    dtype = "f32" if math_mode == "f32" else "bf16"
    inp = small(2, 300, 4, 2, dtype, seed=5)
    wl = inp.wl
    rng = np.random.default_rng(9)
    hist = synth.raw_history(wl, 9)
    conv_b = (0.01 * rng.standard_normal(wl.cdim)).astype(np.float32)
    say("layer %s fused=%s" % (math_mode, fused))
    y, fs, cso = gpu_prefill(inp, fused=fused, math_mode=math_mode, conv_state_in=hist,
                             conv_state_out=True, conv_b=conv_b)
    pairs = [(b, h) for b in range(2) for h in range(4)]
    yr, hr = oracle_pairs(inp, pairs, conv_state_in=hist, conv_b=conv_b)
    assert rel_max_err(gather_y(y, pairs), yr) <= TOL[math_mode]
    hg = np.stack([fs[b, h].double().cpu().numpy() for b, h in pairs])
    assert rel_max_err(hg, hr) <= TOL[math_mode]
    series = np.concatenate([hist, inp.xbc], axis=1)
    np.testing.assert_array_equal(cso.float().cpu().numpy(), series[:, -3:])


@pytest.mark.parametrize("math_mode", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 2, 3])
def test_layer_narrow_conv(math_mode, K):
    """The fused prefill with conv widths below the layer's 4 (the boundary
    takes 1 to 4): a ragged sequence over several chunks, a nonzero conv
    history and bias, y and the final state against the oracle, and the conv
    state out equal to the last K-1 raw rows."""
    dtype = "f32" if math_mode == "f32" else "bf16"
    wl = Workload("t", batch=2, seqlen=300, nheads=4, ngroups=2, dtype=dtype, initial_state=True,
                  seed=40 + K, width=K)
    inp = synth.make_prefill(wl)
    hist = synth.raw_history(wl, 41 + K) if K > 1 else None
    conv_b = (0.01 * np.random.default_rng(K).standard_normal(wl.cdim)).astype(np.float32)
    say("narrow conv K=%d %s" % (K, math_mode))
    y, fs, cso = gpu_prefill(inp, fused=True, math_mode=math_mode, conv_state_in=hist,
                             conv_state_out=K > 1, conv_b=conv_b)
    pairs = [(b, h) for b in range(2) for h in range(4)]
    yr, hr = oracle_pairs(inp, pairs, conv_state_in=hist, conv_b=conv_b)
    assert rel_max_err(gather_y(y, pairs), yr) <= TOL[math_mode]
    hg = np.stack([fs[b, h].double().cpu().numpy() for b, h in pairs])
    assert rel_max_err(hg, hr) <= TOL[math_mode]
    if K > 1:
        series = np.concatenate([hist, inp.xbc], axis=1)
        np.testing.assert_array_equal(cso.float().cpu().numpy(), series[:, -(K - 1):])


@pytest.mark.parametrize("math_mode", ["f32", "bf16"])
@pytest.mark.parametrize("L1", [1, 128, 200])
def test_split_carry(math_mode, L1):
    """[0, L1) then [L1, L) with the SSM state and conv history carried equals
    the oracle over [0, L)."""
    dtype = "f32" if math_mode == "f32" else "bf16"
    inp = small(1, 300, 4, 2, dtype, seed=7)
    wl = inp.wl
    say("split-carry %s L1=%d" % (math_mode, L1))
    p = params(inp)
    xbc = dev(inp.xbc, dtype)
    dt = dev(inp.dt, dtype)
    z = dev(inp.z, dtype)
    cdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    hA = torch.empty((1, 4, 64, 128), device="cuda")
    cA = torch.empty((1, 3, wl.cdim), device="cuda", dtype=cdt)
    ya = layer.prefill(xbc[:, :L1].contiguous(), dt[:, :L1].contiguous(), z[:, :L1].contiguous(),
                       p, fused=True, math=math_mode, initial_state=dev32(inp.h0),
                       final_state=hA, conv_state_out=cA)
    hB = torch.empty_like(hA)
    yb = layer.prefill(xbc[:, L1:].contiguous(), dt[:, L1:].contiguous(), z[:, L1:].contiguous(),
                       p, fused=True, math=math_mode, initial_state=hA, final_state=hB,
                       conv_state_in=cA)
    torch.cuda.synchronize()
    pairs = [(0, h) for h in range(4)]
    yr, hr = oracle_pairs(inp, pairs)
    y = torch.cat([ya, yb], dim=1)
    assert rel_max_err(gather_y(y, pairs), yr) <= TOL[math_mode]
    assert rel_max_err(np.stack([hB[0, h].double().cpu().numpy() for h in range(4)]), hr) <= \
        TOL[math_mode]


@pytest.mark.parametrize("fused", [False, True])
def test_sequence_split_segments(fused):
    """Few heads and a long sequence: the matrix-core scan splits the sequence
    into segments (state-only pass, segment combine, full pass)."""
    inp = small(1, 128 * 40 + 17, 4, 2, "bf16", seed=11)
    wl = inp.wl
    need = ssd.ssd_chunk_scan_workspace_bytes(1, wl.seqlen, 4, ngroups=2, fused_conv=fused)
    assert need > 0, "this shape should be split"
    say("segments fused=%s ws=%d" % (fused, need))
    for probe in (False, True):
        y, fs, _ = gpu_prefill(inp, fused=fused, math_mode="bf16", D=not probe, z=not probe)
        pairs = [(0, h) for h in range(4)]
        yr, hr = oracle_pairs(inp, pairs, D=not probe, z=not probe)
        yg = gather_y(y, pairs)
        if probe:
            assert rel_rms_err(yg, yr) <= PROBE_TOL["bf16"]
        else:
            assert rel_max_err(yg, yr) <= TOL["bf16"]
        assert rel_max_err(np.stack([fs[0, h].double().cpu().numpy() for h in range(4)]), hr) <= \
            TOL["bf16"]


@pytest.mark.parametrize("math_mode,L", [("f32", 300), ("bf16", 300), ("bf16", 128 * 40 + 17)])
def test_no_decay(math_mode, L):
    """A = 0: every decay factor is exp(0) = 1, so the state is the running
    sum h0 + sum_{s <= t} delta_s x_s B_s^T (the recurrence of "Hybrid
    Architectures for Language Models", section 2 Background, with the
    transition at 1; the oracle's own A = 0 pin checks that form).  Outputs
    and the final state match the oracle, the SSM part included (D = 0, no
    gate probe).  The long bf16 case is split into segments, whose combine
    then scales each carried state by exp(0)."""
    dtype = "f32" if math_mode == "f32" else "bf16"
    inp = small(1, L, 4, 2, dtype, seed=41)
    inp.A = np.zeros_like(inp.A)
    if L > 1000:
        assert ssd.ssd_chunk_scan_workspace_bytes(1, L, 4, ngroups=2, fused_conv=True) > 0
    say("no decay %s L=%d" % (math_mode, L))
    pairs = [(0, h) for h in range(4)]
    for probe in (False, True):
        y, fs, _ = gpu_prefill(inp, fused=True, math_mode=math_mode, D=not probe, z=not probe)
        yr, hr = oracle_pairs(inp, pairs, D=not probe, z=not probe)
        yg = gather_y(y, pairs)
        hg = np.stack([fs[0, h].double().cpu().numpy() for h in range(4)])
        e, eh = rel_max_err(yg, yr), rel_max_err(hg, hr)
        say("  probe=%s max|e|/RMS(y) %.3e rel RMS %.3e final state %.3e"
            % (probe, e, rel_rms_err(yg, yr), eh))
        if probe:
            assert rel_rms_err(yg, yr) <= PROBE_TOL[math_mode]
        else:
            assert e <= TOL[math_mode]
        assert eh <= TOL[math_mode]


@pytest.mark.parametrize("math_mode", ["f32", "bf16"])
def test_scan_at_largest_batch(math_mode):
    """The largest batch the scan takes (65535: the grid dimension the B|C
    pack and the conv spread sequences over), on short sequences (3 tokens,
    one ragged chunk, conv fused); sampled sequences, the last included,
    against the oracle, with the final state."""
    dtype = "f32" if math_mode == "f32" else "bf16"
    B = 65535
    inp = small(B, 3, 2, 1, dtype, h0=False, seed=51)
    say("largest batch %s B=%d" % (math_mode, B))
    pairs = [(0, 0), (B - 1, 1), (B - 1, 0), (12345, 1), (40000, 0)]
    y, fs, _ = gpu_prefill(inp, fused=True, math_mode=math_mode)
    yr, hr = oracle_pairs(inp, pairs)
    assert rel_max_err(gather_y(y, pairs), yr) <= TOL[math_mode]
    assert rel_max_err(np.stack([fs[b, h].double().cpu().numpy() for b, h in pairs]), hr) <= \
        TOL[math_mode]


def test_in_place_state_with_segments():
    """initial_state and final_state may be one buffer, also when split."""
    inp = small(1, 128 * 24, 2, 1, "bf16", seed=13)
    say("in-place state")
    p = params(inp)
    st = dev32(inp.h0)
    y = layer.prefill(dev(inp.xbc, "bf16"), dev(inp.dt, "bf16"), dev(inp.z, "bf16"), p,
                      fused=True, initial_state=st, final_state=st)
    torch.cuda.synchronize()
    pairs = [(0, 0), (0, 1)]
    yr, hr = oracle_pairs(inp, pairs)
    assert rel_max_err(gather_y(y, pairs), yr) <= TOL["bf16"]
    assert rel_max_err(np.stack([st[0, h].double().cpu().numpy() for h in range(2)]), hr) <= \
        TOL["bf16"]


@pytest.mark.parametrize("math_mode", ["f32", "bf16"])
def test_bit_stable(math_mode):
    dtype = "f32" if math_mode == "f32" else "bf16"
    inp = small(2, 700, 8, 2, dtype, seed=17)
    say("bit-stable %s" % math_mode)
    outs = [gpu_prefill(inp, fused=True, math_mode=math_mode) for _ in range(2)]
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


def test_empty_sequence_hands_states_through():
    inp = small(2, 0, 4, 2, "bf16")
    wl = inp.wl
    hist = synth.raw_history(wl, 3)
    say("empty sequence")
    y, fs, cso = gpu_prefill(inp, fused=True, math_mode="bf16", conv_state_in=hist,
                             conv_state_out=True)
    assert y.shape == (2, 0, 4, 64)
    np.testing.assert_array_equal(fs.cpu().numpy(), inp.h0)
    np.testing.assert_array_equal(cso.float().cpu().numpy(), hist)


def test_zero_dt_keeps_state():
    """dt = 0, no bias, no softplus: h_t = h0, y = (C_t h0 + D x_t) silu(z_t)."""
    inp = small(1, 200, 4, 2, "f32", seed=19)
    say("dt = 0")
    p = params(inp)
    p.dt_bias = None
    p.dt_softplus = False
    xbc = dev(inp.xbc, "f32")
    x, Bm, Cm = layer.split_xbc(xbc, p)
    fs = torch.empty((1, 4, 64, 128), device="cuda")
    zero = torch.zeros((1, 200, 4), device="cuda")
    y = ssd.ssd_chunk_scan_fwd(x, Bm, Cm, zero, p.A, D=p.D, z=dev(inp.z, "f32"), dt_bias=None,
                               dt_softplus=False, initial_state=dev32(inp.h0), final_state=fs,
                               math="f32")
    torch.cuda.synchronize()
    np.testing.assert_allclose(fs.cpu().numpy(), inp.h0, rtol=0, atol=0)
    want = np.empty((200, 4, 64))
    from pinforms import silu
    for h in range(4):
        g = h // 2
        Cv = inp.xbc[0, :, 256 + 256 + g * 128:256 + 256 + (g + 1) * 128].astype(np.float64)
        want[:, h] = (Cv @ inp.h0[0, h].astype(np.float64).T +
                      inp.xbc[0, :, h * 64:(h + 1) * 64]) * silu(inp.z[0, :, h].astype(np.float64))
    assert rel_max_err(y[0].double().cpu().numpy(), want) <= 1e-5


# ---------------------------------------------------------------- decode

DECODE_CASES = [  # (dtype, B, H, G, steps, gated, conv width; 0: no conv)
    ("f32", 3, 16, 4, 40, True, 4), ("bf16", 3, 16, 4, 40, True, 4),
    # 128 heads in one group: the fused kernel's per-group LDS (x, gate,
    # per-head scalars) exceeds 64 KiB
    ("bf16", 2, 128, 1, 6, True, 4),
    # one head per group, no gate
    ("f32", 2, 8, 8, 12, False, 4),
    # shorter conv windows: a ring of one row, and no ring at all
    ("bf16", 2, 8, 2, 8, True, 2), ("f32", 2, 8, 2, 6, True, 1),
    # post-conv inputs (no conv in the step)
    ("f32", 2, 8, 2, 6, True, 0),
    # one sequence at the serving head count
    ("bf16", 1, 128, 8, 4, True, 4),
]
DECODE_ENTRIES = {"fused": ssd.ssd_state_update, "ws": ssd.ssd_state_update_ws}


@pytest.mark.parametrize("entry", sorted(DECODE_ENTRIES))
@pytest.mark.parametrize("dtype,B,H,G,T,gated,K", DECODE_CASES,
                         ids=["%s-B%d-H%d-G%d-%s-K%d" % (c[0], c[1], c[2], c[3],
                                                         "gate" if c[5] else "nogate", c[6])
                              for c in DECODE_CASES])
def test_state_update_chain(dtype, B, H, G, T, gated, K, entry):
    wl = Workload("d", batch=B, seqlen=1, nheads=H, ngroups=G, dtype=dtype, decode_steps=T,
                  initial_state=True, seed=23 + H + G + K, width=max(K, 1))
    inp = synth.make_decode(wl)
    xbc, z, dt = inp.steps(0, T)
    say("decode chain %s %s B=%d H=%d G=%d gated=%s K=%d" % (entry, dtype, B, H, G, gated, K))
    p = params(inp)
    st = dev32(inp.state)
    ring = dev(inp.ring, dtype) if K > 1 else None
    conv_w = p.conv_w if K > 0 else None
    call = DECODE_ENTRIES[entry]
    ys = []
    for t in range(T):
        ys.append(call(
            st, dev(xbc[t], dtype), dev(dt[t], dtype), p.A, ngroups=G, conv_state=ring,
            conv_w=conv_w, z=dev(z[t], dtype) if gated else None, D=p.D,
            dt_bias=p.dt_bias).double().cpu().numpy())
    torch.cuda.synchronize()
    carry = oracle.DecodeState(inp.state, inp.ring if K > 0 else None)
    yr = []
    for t in range(T):
        yr.append(oracle.mamba2_decode_step(carry, xbc[t], dt[t], inp.A, nheads=H, headdim=64,
                                            ngroups=G, dstate=128,
                                            conv_w=inp.conv_w if K > 0 else None, D=inp.D,
                                            dt_bias=inp.dt_bias, z=z[t] if gated else None))
    tol = TOL[dtype]
    assert rel_max_err(np.stack(ys), np.stack(yr)) <= tol
    assert rel_max_err(st.cpu().numpy(), carry.state) <= tol
    if K > 1:
        np.testing.assert_array_equal(ring.float().cpu().numpy(), carry.ring)


def test_state_update_ws_matches_fused_at_full_size():
    """The two-kernel step and the fused step agree at the serving shape
    (256 sequences, 128 heads, 8 groups, bf16 activations): the ring bit for
    bit, the state and y within 1e-5 of their RMS (the kernels round alike
    but fuse multiplies and adds into FMAs differently, and sum h C in
    different orders; 1e-5 is about 100 fp32 ulps at RMS), over three chained
    steps with one workspace reused (two calls in a row, then a smaller batch
    through the same workspace)."""
    wl = Workload("d", batch=256, seqlen=1, nheads=128, ngroups=8, dtype="bf16",
                  decode_steps=3, initial_state=True, seed=31)
    inp = synth.make_decode(wl)
    xbc, z, dt = inp.steps(0, 3)
    say("decode ws vs fused B=256 H=128 G=8")
    p = params(inp)
    need = ssd.ssd_state_update_workspace_bytes(256, 128, 64, 8, 128)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for Bn in (256, 256, 97):
        st_a, st_b = dev32(inp.state[:Bn]), dev32(inp.state[:Bn])
        ring_a, ring_b = dev(inp.ring[:Bn], "bf16"), dev(inp.ring[:Bn], "bf16")
        for t in range(3):
            args = (dev(xbc[t][:Bn], "bf16"), dev(dt[t][:Bn], "bf16"), p.A)
            kw = dict(ngroups=8, conv_w=p.conv_w, z=dev(z[t][:Bn], "bf16"), D=p.D,
                      dt_bias=p.dt_bias)
            ya = ssd.ssd_state_update(st_a, *args, conv_state=ring_a, **kw)
            yb = ssd.ssd_state_update_ws(st_b, *args, conv_state=ring_b, workspace=ws, **kw)
            torch.cuda.synchronize()
            assert torch.equal(ring_a, ring_b)
            assert rel_max_err(yb.double().cpu().numpy(), ya.double().cpu().numpy()) <= 1e-5
            assert rel_max_err(st_b.cpu().numpy(), st_a.cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("entry", sorted(DECODE_ENTRIES))
@pytest.mark.parametrize("xd,ad,yd", [("bf16", "f32", "f32"), ("f32", "bf16", "bf16"),
                                      ("bf16", "bf16", "bf16")])
def test_state_update_dtype_mix(xd, ad, yd, entry):
    """x|B|C and its ring in one dtype, dt and z in another, y in a third:
    every typed instance of both entry points against the oracle on the same
    (rounded) values."""
    wl = Workload("d", batch=3, seqlen=1, nheads=16, ngroups=4, dtype="f32", decode_steps=5,
                  initial_state=True, seed=41)
    inp = synth.make_decode(wl)
    xbc, z, dt = (np.array(v) for v in inp.steps(0, 5))
    ring0 = np.array(inp.ring)
    if xd == "bf16":
        synth.round_bf16_(xbc)
        synth.round_bf16_(ring0)
    if ad == "bf16":
        synth.round_bf16_(z)
        synth.round_bf16_(dt)
    say("decode dtypes %s x|B|C, %s dt/z, %s y (%s)" % (xd, ad, yd, entry))
    p = params(inp)
    st = dev32(inp.state)
    ring = dev(ring0, xd)
    ydt = torch.bfloat16 if yd == "bf16" else torch.float32
    ys = []
    for t in range(5):
        ys.append(DECODE_ENTRIES[entry](
            st, dev(xbc[t], xd), dev(dt[t], ad), p.A, ngroups=4, conv_state=ring,
            conv_w=p.conv_w, z=dev(z[t], ad), D=p.D, dt_bias=p.dt_bias,
            y_dtype=ydt).double().cpu().numpy())
    torch.cuda.synchronize()
    carry = oracle.DecodeState(inp.state, ring0)
    yr = [oracle.mamba2_decode_step(carry, xbc[t], dt[t], inp.A, nheads=16, headdim=64,
                                    ngroups=4, dstate=128, conv_w=inp.conv_w, D=inp.D,
                                    dt_bias=inp.dt_bias, z=z[t]) for t in range(5)]
    # Both sides compute in fp32 or better from the same rounded inputs, so
    # the fp32 bound holds before y is stored.  A bf16 y then adds its own
    # rounding, at most 2^-8 of each element (8 significant bits, round to
    # nearest even), which for the largest elements exceeds any fraction of
    # RMS(y) worth stating: that part is bounded per element instead.
    got, want = np.stack(ys), np.stack(yr)
    rms = float(np.sqrt(np.mean(want * want)))
    slack = 2.0 ** -8 * np.abs(want) if yd == "bf16" else 0.0
    assert float(np.max(np.abs(got - want) - slack)) <= 2 * TOL["f32"] * rms
    assert rel_max_err(st.cpu().numpy(), carry.state) <= TOL["f32"]
    np.testing.assert_array_equal(ring.float().cpu().numpy(), carry.ring)


@pytest.mark.parametrize("entry", sorted(DECODE_ENTRIES))
def test_decode_zero_dt_keeps_state(entry):
    """dt = 0, no bias, no softplus, post-conv inputs: the decay is exp(0) = 1
    and the input term 0, so the state comes back bit for bit, and
    y = (C h + D x) silu(z) from that state (closed form, not the oracle)."""
    B, H, G = 2, 8, 2
    wl = Workload("d", batch=B, seqlen=1, nheads=H, ngroups=G, dtype="f32", decode_steps=1,
                  initial_state=True, seed=47)
    inp = synth.make_decode(wl)
    xbc, z, _ = inp.steps(0, 1)
    say("decode dt = 0 (%s)" % entry)
    st = dev32(inp.state)
    y = DECODE_ENTRIES[entry](st, dev(xbc[0], "f32"), torch.zeros((B, H), device="cuda"),
                              dev32(inp.A), ngroups=G, z=dev(z[0], "f32"), D=dev32(inp.D),
                              dt_bias=None, dt_softplus=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(st.cpu().numpy(), inp.state)
    from pinforms import silu
    HP = H * 64
    want = np.empty((B, H, 64))
    for h in range(H):
        g = h // (H // G)
        Cv = xbc[0][:, HP + G * 128 + g * 128:HP + G * 128 + (g + 1) * 128].astype(np.float64)
        hs = inp.state[:, h].astype(np.float64)                      # [B, P, N]
        xv = xbc[0][:, h * 64:(h + 1) * 64].astype(np.float64)
        want[:, h] = (np.einsum("bpn,bn->bp", hs, Cv) + inp.D[h] * xv) * \
            silu(z[0][:, h * 64:(h + 1) * 64].astype(np.float64))
    assert rel_max_err(y.double().cpu().numpy().reshape(B, H, 64), want) <= 1e-5


@pytest.mark.parametrize("entry", sorted(DECODE_ENTRIES))
def test_decode_bit_stable(entry):
    """The same step from the same state, ring and inputs gives the same bytes
    (y, state and ring) on a second run: no atomics, fixed reduction order."""
    wl = Workload("d", batch=16, seqlen=1, nheads=128, ngroups=8, dtype="bf16", decode_steps=2,
                  initial_state=True, seed=37)
    inp = synth.make_decode(wl)
    xbc, z, dt = inp.steps(0, 2)
    say("decode bit-stable %s" % entry)
    p = params(inp)
    outs = []
    for _ in range(2):
        st = dev32(inp.state)
        ring = dev(inp.ring, "bf16")
        ys = [DECODE_ENTRIES[entry](st, dev(xbc[t], "bf16"), dev(dt[t], "bf16"), p.A, ngroups=8,
                                    conv_state=ring, conv_w=p.conv_w, z=dev(z[t], "bf16"),
                                    D=p.D, dt_bias=p.dt_bias) for t in range(2)]
        torch.cuda.synchronize()
        outs.append((torch.stack(ys).cpu(), st.cpu(), ring.cpu()))
    for a_, b_ in zip(outs[0], outs[1]):
        assert torch.equal(a_, b_)


def test_decode_equals_prefill_on_gpu():
    """64 one-token steps of ssd_state_update equal one prefill call over the
    same tokens from the same state and conv history (fp32 path)."""
    wl = Workload("d", batch=2, seqlen=1, nheads=4, ngroups=2, dtype="f32", decode_steps=64,
                  initial_state=True, seed=29)
    inp = synth.make_decode(wl)
    T = 64
    xbc, z, dt = inp.steps(0, T)
    say("decode = prefill")
    p = params(inp)
    st = dev32(inp.state)
    ring = dev(inp.ring, "f32")
    yd = torch.stack([layer.decode_step(st, dev(xbc[t], "f32"), dev(dt[t], "f32"),
                                        dev(z[t], "f32"), ring, p) for t in range(T)], dim=1)
    fs = torch.empty_like(st)
    yp = layer.prefill(dev(np.ascontiguousarray(xbc.transpose(1, 0, 2)), "f32"),
                       dev(np.ascontiguousarray(dt.transpose(1, 0, 2)), "f32"),
                       dev(np.ascontiguousarray(z.transpose(1, 0, 2)), "f32").view(2, T, 4, 64),
                       p, fused=True, math="f32", initial_state=dev32(inp.state), final_state=fs,
                       conv_state_in=dev(inp.ring, "f32"))
    torch.cuda.synchronize()
    assert rel_max_err(yd.double().cpu().numpy(), yp.view(2, T, -1).double().cpu().numpy()) <= 1e-5
    assert rel_max_err(st.cpu().numpy(), fs.cpu().numpy()) <= 1e-5
