"""Pins for the fp64 oracle (CPU only).

The pages print no worked numerical example, so each pin is a form the
mathematics fixes and that does not share the oracle's code: the quadratic
SSD matrix form, an independent chunked form, numpy's correlate for the conv,
closed forms (geometric series, prefix sums, steady state, conv impulse
response), special cases (dt = 0, A = 0), library routines (softplus via
logaddexp) and invariants (linearity, group sharing, split-carry,
decode = prefill).  Each is chosen so that a plausible mistake in the oracle
-- a dropped term, a wrong sign or index, a transposed operand, the wrong
head-to-group map, reading the state before instead of after the update --
fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle
from pinforms import (conv_correlate, pack_xbc, silu, softplus, ssd_chunked,
                      ssd_quadratic)

TOL = 1e-12


def rel_max_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    rms = math.sqrt(float(np.mean(b * b))) or 1.0
    return float(np.max(np.abs(a - b))) / rms


def rand_problem(rng, B, L, H, P, G, N, *, h0=True, z=True, grid=False):
    """Random post-conv SSM inputs.  grid=True puts x on a coarse binary grid so
    that small integer combinations stay exact in float32."""
    if grid:
        x = rng.integers(-64, 65, (B, L, H, P)).astype(np.float32) / 16
    else:
        x = rng.standard_normal((B, L, H, P)).astype(np.float32)
    Bm = (rng.standard_normal((B, L, G, N)) / math.sqrt(N)).astype(np.float32)
    Cm = (rng.standard_normal((B, L, G, N)) / math.sqrt(N)).astype(np.float32)
    dt = (0.5 * rng.standard_normal((B, L, H))).astype(np.float32)
    A = -np.exp(rng.uniform(0, math.log(16), H)).astype(np.float32)
    dt_bias = rng.uniform(-4, -1, H).astype(np.float32)
    D = rng.uniform(0.5, 1.5, H).astype(np.float32)
    zz = rng.standard_normal((B, L, H, P)).astype(np.float32) if z else None
    hh = (0.1 * rng.standard_normal((B, H, P, N))).astype(np.float32) if h0 else None
    return dict(x=x, Bm=Bm, Cm=Cm, dt=dt, A=A, dt_bias=dt_bias, D=D, z=zz, h0=hh)


def run_oracle(pr, **over):
    p = dict(pr)
    p.update(over)
    x, Bm, Cm = p["x"], p["Bm"], p["Cm"]
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    y, hT, _ = oracle.mamba2_fwd(pack_xbc(x, Bm, Cm), p["dt"], p["A"], nheads=H, headdim=P,
                                 ngroups=G, dstate=N, D=p["D"], dt_bias=p["dt_bias"],
                                 dt_softplus=p.get("dt_softplus", True), z=p["z"],
                                 h0=p["h0"])
    return y, hT


# --------------------------------------------------------------------------- conv

def test_conv_matches_numpy_correlate():
    rng = np.random.default_rng(1)
    B, L, C, K = 2, 37, 19, 4
    x = rng.standard_normal((B, L, C)).astype(np.float32)
    w = rng.standard_normal((C, K)).astype(np.float32)
    bias = rng.standard_normal(C).astype(np.float32)
    hist = rng.standard_normal((B, K - 1, C)).astype(np.float32)
    for hh, bb, act in [(None, None, True), (hist, bias, True), (hist, None, False)]:
        out, _ = oracle.causal_conv1d(x, w, bb, hh, apply_silu=act)
        ref = conv_correlate(x, w, bb, hh, apply_silu=act)
        assert rel_max_err(out, ref) < TOL


def test_conv_impulse_response():
    """A unit impulse at t0 gives silu(w[c, K-1-j]) at t0 + j and silu(0) = 0
    elsewhere: the current token meets the last tap."""
    rng = np.random.default_rng(2)
    C, K, L, t0 = 5, 4, 12, 3
    w = rng.standard_normal((C, K)).astype(np.float32)
    x = np.zeros((1, L, C), np.float32)
    x[0, t0, :] = 1.0
    out, _ = oracle.causal_conv1d(x, w)
    for c in range(C):
        for t in range(L):
            j = t - t0
            want = float(silu(np.float64(w[c, K - 1 - j]))) if 0 <= j < K else 0.0
            assert abs(out[0, t, c] - want) < 1e-15


@pytest.mark.parametrize("L", [0, 1, 2, 3, 9])
def test_conv_history_out(L):
    """The carried history is the last K-1 raw inputs, oldest first, reaching
    into the old history when L < K-1."""
    rng = np.random.default_rng(3)
    C, K = 6, 4
    x = rng.standard_normal((2, L, C)).astype(np.float32)
    hist = rng.standard_normal((2, K - 1, C)).astype(np.float32)
    _, hout = oracle.causal_conv1d(x, rng.standard_normal((C, K)).astype(np.float32), None, hist)
    series = np.concatenate([hist, x], axis=1)
    np.testing.assert_array_equal(hout, series[:, -(K - 1):, :].astype(np.float64))


# --------------------------------------------------------------------------- scan

@pytest.mark.parametrize("B,L,H,P,G,N", [(1, 9, 1, 3, 1, 5), (2, 24, 4, 4, 2, 6),
                                          (1, 40, 4, 2, 4, 3), (1, 20, 2, 64, 1, 128)])
def test_quadratic_form(B, L, H, P, G, N):
    rng = np.random.default_rng(10 + L)
    pr = rand_problem(rng, B, L, H, P, G, N)
    y, _ = run_oracle(pr)
    yq = ssd_quadratic(pr["x"], pr["Bm"], pr["Cm"], pr["dt"], pr["A"], D=pr["D"], z=pr["z"],
                       dt_bias=pr["dt_bias"], h0=pr["h0"])
    assert rel_max_err(y, yq) < TOL
    # the SSM part alone (no skip, no gate, zero state) -- the skip must not
    # mask an error in the scan
    y2, _ = run_oracle(pr, D=None, z=None, h0=None)
    yq2 = ssd_quadratic(pr["x"], pr["Bm"], pr["Cm"], pr["dt"], pr["A"], dt_bias=pr["dt_bias"])
    assert rel_max_err(y2, yq2) < TOL


@pytest.mark.parametrize("chunk", [1, 7, 64, 128, 256, 1000])
def test_chunked_form_any_chunk(chunk):
    """Chunk-size independence: the chunked form at any chunk length, ragged
    tails included, equals the recurrence; so does its final state."""
    rng = np.random.default_rng(20)
    pr = rand_problem(rng, 1, 300, 2, 8, 1, 16)
    y, hT = run_oracle(pr)
    yc, hc = ssd_chunked(pr["x"], pr["Bm"], pr["Cm"], pr["dt"], pr["A"], chunk, D=pr["D"],
                         z=pr["z"], dt_bias=pr["dt_bias"], h0=pr["h0"])
    assert rel_max_err(y, yc) < TOL
    assert rel_max_err(hT, hc) < TOL


def test_dt_zero_keeps_state():
    """dt = 0 with no softplus and no bias: Abar = 1, Bbar = 0, so h_t = h0 and
    y_t = (h0 C_t + D x_t) * silu(z_t); with h0 = 0, y = D x silu(z)."""
    rng = np.random.default_rng(30)
    pr = rand_problem(rng, 2, 17, 4, 5, 2, 7)
    zero = np.zeros_like(pr["dt"])
    y, hT = run_oracle(pr, dt=zero, dt_bias=None, dt_softplus=False)
    B, L, H, P = pr["x"].shape
    G = pr["Bm"].shape[2]
    want = np.zeros_like(y)
    for h in range(H):
        g = h * G // H
        hc = np.einsum("bpn,bln->blp", pr["h0"][:, h].astype(np.float64),
                       pr["Cm"][:, :, g].astype(np.float64))
        want[:, :, h] = (hc + np.float64(pr["D"][h]) * pr["x"][:, :, h].astype(np.float64)) * \
            silu(pr["z"][:, :, h].astype(np.float64))
    assert rel_max_err(y, want) < TOL
    assert rel_max_err(hT, pr["h0"]) < TOL
    y0, _ = run_oracle(pr, dt=zero, dt_bias=None, dt_softplus=False, h0=None)
    want0 = (pr["D"].astype(np.float64)[None, None, :, None] * pr["x"].astype(np.float64) *
             silu(pr["z"].astype(np.float64)))
    assert rel_max_err(y0, want0) < TOL


def test_A_zero_is_prefix_sum():
    """A = 0 removes the decay: h_t = h0 + sum_{s<=t} delta_s x_s B_s^T, i.e.
    unnormalised causal linear attention, computed here with cumsum."""
    rng = np.random.default_rng(40)
    pr = rand_problem(rng, 1, 33, 2, 4, 1, 6, z=False)
    A0 = np.zeros_like(pr["A"])
    y, hT = run_oracle(pr, A=A0)
    delta = softplus(pr["dt"].astype(np.float64) + pr["dt_bias"])
    x = pr["x"].astype(np.float64)
    Bm = pr["Bm"].astype(np.float64)[:, :, 0]
    Cm = pr["Cm"].astype(np.float64)[:, :, 0]
    for h in range(2):
        outer = np.einsum("l,lp,ln->lpn", delta[0, :, h], x[0, :, h], Bm[0])
        hs = pr["h0"][0, h].astype(np.float64)[None] + np.cumsum(outer, axis=0)
        want = np.einsum("lpn,ln->lp", hs, Cm[0]) + np.float64(pr["D"][h]) * x[0, :, h]
        assert rel_max_err(y[0, :, h], want) < TOL
        assert rel_max_err(hT[0, h], hs[-1]) < TOL


def test_scalar_geometric_series():
    """H = P = N = G = 1, constant delta and A, B = C = x = 1, D = 0, no gate:
    h_t = a^(t+1) h0 + delta (1 - a^(t+1)) / (1 - a), a = exp(delta A), and the
    read-out y_t equals h_t (the state after the token's update)."""
    L, delta, A, h0 = 50, 0.07, -3.0, 0.8
    ones = np.ones((1, L, 1, 1), np.float32)
    xbc = pack_xbc(ones, ones, ones)
    dt = np.full((1, L, 1), delta, np.float32)
    y, hT, _ = oracle.mamba2_fwd(xbc, dt, np.array([A], np.float32), nheads=1, headdim=1,
                                 ngroups=1, dstate=1, dt_softplus=False,
                                 h0=np.full((1, 1, 1, 1), h0))
    d = float(np.float32(delta))
    a = math.exp(d * A)
    for t in range(L):
        k = t + 1
        want = a ** k * h0 + d * (1 - a ** k) / (1 - a)
        assert abs(y[0, t, 0, 0] - want) < 1e-13 * abs(want)
    assert abs(hT[0, 0, 0, 0] - y[0, L - 1, 0, 0]) == 0.0


def test_softplus_values():
    """With h0 = 0 and B = C = x = 1 the first output is delta itself, so it
    must equal softplus(dt + dt_bias) from numpy's logaddexp, in both tails."""
    v = np.array([-40.0, -5.0, -0.3, 0.0, 2.5, 40.0], np.float32)
    H = v.size
    ones = np.ones((1, 1, H, 1), np.float32)
    one_g = np.ones((1, 1, 1, 1), np.float32)
    xbc = pack_xbc(ones, one_g, one_g)
    y, _, _ = oracle.mamba2_fwd(xbc, np.zeros((1, 1, H), np.float32),
                                np.full(H, -2.0, np.float32), nheads=H, headdim=1, ngroups=1,
                                dstate=1, dt_bias=v, dt_softplus=True)
    want = softplus(v.astype(np.float64))
    np.testing.assert_allclose(y[0, 0, :, 0], want, rtol=1e-14, atol=0)


def test_linear_in_x():
    """With delta, B, C fixed (post-conv inputs), no gate and zero state, the
    scan is linear in x."""
    rng = np.random.default_rng(50)
    pr = rand_problem(rng, 1, 21, 2, 3, 1, 4, z=False, h0=False, grid=True)
    x2 = (rng.integers(-64, 65, pr["x"].shape).astype(np.float32) / 16)
    y1, _ = run_oracle(pr)
    y2, _ = run_oracle(pr, x=x2)
    y3, _ = run_oracle(pr, x=(2 * pr["x"] - 3 * x2).astype(np.float32))
    assert rel_max_err(y3, 2 * y1 - 3 * y2) < TOL


def test_group_sharing_and_permutation():
    """Heads in one group with the same x, dt, A, D see the same B and C and so
    give the same output; swapping the two groups' B and C swaps the outputs
    of the heads that read them (heads 0,1 -> group 0, heads 2,3 -> group 1)."""
    rng = np.random.default_rng(60)
    pr = rand_problem(rng, 1, 15, 4, 3, 2, 5, h0=False)
    for k in ("x", "z"):
        pr[k][:, :, 1] = pr[k][:, :, 0]
        pr[k][:, :, 3] = pr[k][:, :, 2]
    pr["dt"][:, :, 1] = pr["dt"][:, :, 0]
    pr["dt"][:, :, 3] = pr["dt"][:, :, 2]
    for k in ("A", "dt_bias", "D"):
        pr[k][1] = pr[k][0]
        pr[k][3] = pr[k][2]
    y, _ = run_oracle(pr)
    np.testing.assert_array_equal(y[:, :, 0], y[:, :, 1])
    np.testing.assert_array_equal(y[:, :, 2], y[:, :, 3])
    assert np.max(np.abs(y[:, :, 0] - y[:, :, 2])) > 0
    # swap the groups' B and C and the per-head inputs of heads {0,1} <-> {2,3}
    perm = [2, 3, 0, 1]
    sw = dict(pr)
    sw["Bm"] = pr["Bm"][:, :, ::-1].copy()
    sw["Cm"] = pr["Cm"][:, :, ::-1].copy()
    for k in ("x", "z", "dt"):
        sw[k] = pr[k][:, :, perm].copy()
    for k in ("A", "dt_bias", "D"):
        sw[k] = pr[k][perm].copy()
    ys, _ = run_oracle(sw)
    np.testing.assert_array_equal(ys, y[:, :, perm])


def test_constant_input_steady_state():
    """Constant delta, x, B: the state tends to h* = delta x B^T / (1 - a)."""
    L, H, P, N = 400, 1, 3, 4
    rng = np.random.default_rng(70)
    x = np.broadcast_to(rng.standard_normal(P).astype(np.float32), (1, L, H, P)).copy()
    Bv = rng.standard_normal(N).astype(np.float32)
    Cv = rng.standard_normal(N).astype(np.float32)
    Bm = np.broadcast_to(Bv, (1, L, 1, N)).copy()
    Cm = np.broadcast_to(Cv, (1, L, 1, N)).copy()
    dt = np.full((1, L, H), 0.25, np.float32)
    A = np.array([-0.5], np.float32)
    y, hT, _ = oracle.mamba2_fwd(pack_xbc(x, Bm, Cm), dt, A, nheads=H, headdim=P, ngroups=1,
                                 dstate=N, dt_softplus=False)
    a = math.exp(0.25 * -0.5)
    hstar = 0.25 * np.outer(x[0, 0, 0].astype(np.float64), Bv.astype(np.float64)) / (1 - a)
    assert np.max(np.abs(hT[0, 0] - hstar)) < 1e-10 * np.max(np.abs(hstar))
    assert np.max(np.abs(y[0, -1, 0] - hstar @ Cv.astype(np.float64))) < 1e-10 * np.max(np.abs(hstar))


# ------------------------------------------------------------- layer and decode

def layer_problem(rng, B, L, H, P, G, N, K=4):
    C = H * P + 2 * G * N
    xbc = rng.standard_normal((B, L, C)).astype(np.float32)
    xbc[..., H * P:] /= math.sqrt(N)
    return dict(
        xbc=xbc, dt=(0.5 * rng.standard_normal((B, L, H))).astype(np.float32),
        A=-np.exp(rng.uniform(0, math.log(16), H)).astype(np.float32),
        dt_bias=rng.uniform(-5, -2, H).astype(np.float32), D=np.ones(H, np.float32),
        z=rng.standard_normal((B, L, H, P)).astype(np.float32),
        conv_w=(0.5 * rng.standard_normal((C, K))).astype(np.float32),
        conv_b=(0.1 * rng.standard_normal(C)).astype(np.float32),
        h0=(0.1 * rng.standard_normal((B, H, P, N))),
        hist=rng.standard_normal((B, K - 1, C)).astype(np.float32))


def layer(lp, sl, h0, hist, dims):
    H, P, G, N = dims
    return oracle.mamba2_fwd(lp["xbc"][:, sl], lp["dt"][:, sl], lp["A"], nheads=H, headdim=P,
                             ngroups=G, dstate=N, conv_w=lp["conv_w"], conv_b=lp["conv_b"],
                             conv_state_in=hist, D=lp["D"], dt_bias=lp["dt_bias"],
                             z=lp["z"][:, sl], h0=h0)


def test_layer_equals_conv_then_scan():
    """The layer with the conv inside equals the conv (pinned above against
    numpy) followed by the scan on post-conv channels (pinned against the
    quadratic form)."""
    rng = np.random.default_rng(80)
    dims = (4, 3, 2, 5)
    H, P, G, N = dims
    lp = layer_problem(rng, 2, 19, *dims)
    y, hT, hout = layer(lp, slice(None), lp["h0"], lp["hist"], dims)
    conv = conv_correlate(lp["xbc"], lp["conv_w"], lp["conv_b"], lp["hist"])
    HP = H * P
    x = conv[..., :HP].reshape(2, 19, H, P)
    Bm = conv[..., HP:HP + G * N].reshape(2, 19, G, N)
    Cm = conv[..., HP + G * N:].reshape(2, 19, G, N)
    yq = ssd_quadratic(x, Bm, Cm, lp["dt"], lp["A"], D=lp["D"], z=lp["z"],
                       dt_bias=lp["dt_bias"], h0=lp["h0"])
    assert rel_max_err(y, yq) < TOL
    np.testing.assert_array_equal(hout, lp["xbc"][:, -3:].astype(np.float64))


@pytest.mark.parametrize("L1", [1, 3, 127, 128, 300])
def test_split_carry(L1):
    """Running [0, L) at once equals [0, L1) then [L1, L) with the SSM state and
    the conv history carried across the split."""
    rng = np.random.default_rng(90)
    dims = (2, 4, 1, 6)
    lp = layer_problem(rng, 1, 301, *dims)
    y, hT, hout = layer(lp, slice(None), lp["h0"], lp["hist"], dims)
    ya, ha, hista = layer(lp, slice(0, L1), lp["h0"], lp["hist"], dims)
    yb, hb, histb = layer(lp, slice(L1, None), ha, hista.astype(np.float32), dims)
    assert rel_max_err(np.concatenate([ya, yb], axis=1), y) < TOL
    assert rel_max_err(hb, hT) < TOL
    np.testing.assert_array_equal(histb, hout)


def test_decode_equals_prefill():
    """T one-token decode steps (conv ring + state) reproduce a prefill over the
    same T tokens started from the same state and conv history."""
    rng = np.random.default_rng(100)
    dims = (4, 3, 2, 5)
    H, P, G, N = dims
    T, B = 1000, 3
    lp = layer_problem(rng, B, T, *dims)
    y, hT, hout = layer(lp, slice(None), lp["h0"], lp["hist"], dims)
    carry = oracle.DecodeState(lp["h0"], lp["hist"])
    for t in range(T):
        yt = oracle.mamba2_decode_step(carry, lp["xbc"][:, t], lp["dt"][:, t], lp["A"],
                                       nheads=H, headdim=P, ngroups=G, dstate=N,
                                       conv_w=lp["conv_w"], conv_b=lp["conv_b"], D=lp["D"],
                                       dt_bias=lp["dt_bias"], z=lp["z"][:, t])
        assert rel_max_err(yt, y[:, t].reshape(B, -1)) < TOL
    assert rel_max_err(carry.state, hT) < TOL
    np.testing.assert_array_equal(carry.ring, hout)


def test_decode_without_conv_matches_closed_step():
    """conv_w = None: the step reads post-conv inputs directly and leaves the
    ring alone; one step from h is a h + delta x B^T, read out through C."""
    rng = np.random.default_rng(110)
    H, P, G, N, B = 2, 3, 1, 4, 2
    C = H * P + 2 * G * N
    xbc = rng.standard_normal((B, C)).astype(np.float32)
    dt = rng.standard_normal((B, H)).astype(np.float32)
    A = np.array([-1.5, -0.25], np.float32)
    h = rng.standard_normal((B, H, P, N))
    carry = oracle.DecodeState(h, None)
    y = oracle.mamba2_decode_step(carry, xbc, dt, A, nheads=H, headdim=P, ngroups=G,
                                  dstate=N, dt_softplus=True)
    for b in range(B):
        for hh in range(H):
            d = softplus(np.float64(dt[b, hh]))
            a = math.exp(d * A[hh])
            x = xbc[b, hh * P:(hh + 1) * P].astype(np.float64)
            Bv = xbc[b, H * P:H * P + N].astype(np.float64)
            Cv = xbc[b, H * P + N:].astype(np.float64)
            hn = a * h[b, hh] + d * np.outer(x, Bv)
            assert np.max(np.abs(carry.state[b, hh] - hn)) < 1e-14
            assert np.max(np.abs(y[b, hh * P:(hh + 1) * P] - hn @ Cv)) < 1e-13
