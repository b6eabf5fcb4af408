"""Pins of the oracle's backward (oracle_mamba2_bwd): its gradients against
central finite differences of the forward oracle in fp64, for every input
element of tiny layers, through the loss
    sum(dout * y) + sum(dh_final * h_final).
A finite difference differentiates the forward recurrence itself, so it
shares nothing with the reverse-mode code but the forward oracle, which is
pinned on its own (test_oracle_pins.py).
"""
import numpy as np
import pytest

import oracle


def case(seed, B=2, L=6, H=2, P=3, G=1, N=2, K=3, conv=True, z=True, D=True, bias=True,
         h0=True, hist=True, softplus=True):
    rng = np.random.default_rng(seed)
    C = H * P + 2 * G * N
    inp = dict(xbc=rng.standard_normal((B, L, C)), dt=0.5 * rng.standard_normal((B, L, H)),
               A=-rng.uniform(0.5, 2.0, H))
    kw = dict(nheads=H, headdim=P, ngroups=G, dstate=N, dt_softplus=softplus)
    opt = {}
    if conv:
        opt["conv_w"] = 0.5 * rng.standard_normal((C, K))
        opt["conv_b"] = 0.1 * rng.standard_normal(C)
        if hist:
            opt["conv_state_in"] = rng.standard_normal((B, K - 1, C))
    if z:
        opt["z"] = rng.standard_normal((B, L, H, P))
    if D:
        opt["D"] = rng.uniform(0.5, 1.5, H)
    if bias:
        opt["dt_bias"] = rng.uniform(-1.0, 0.5, H)
    if h0:
        opt["h0"] = 0.3 * rng.standard_normal((B, H, P, N))
    dout = rng.standard_normal((B, L, H, P))
    dhf = rng.standard_normal((B, H, P, N))
    return inp, opt, kw, dout, dhf


def loss(inp, opt, kw, dout, dhf):
    y, hT, _ = oracle.mamba2_fwd(inp["xbc"], inp["dt"], inp["A"], **kw, **opt, f64_inputs=True)
    return float(np.sum(dout * y) + np.sum(dhf * hT))


def check_fd(inp, opt, kw, dout, dhf):
    g = oracle.mamba2_bwd(inp["xbc"], inp["dt"], inp["A"], dout, **kw, **opt, dh_final=dhf,
                          f64_inputs=True)
    names = list(inp) + list(opt)
    for name in names:
        src = inp if name in inp else opt
        arr = src[name]
        got = g[name]
        assert got.shape == arr.shape, name
        fd = np.empty_like(arr)
        flat, fflat = arr.reshape(-1), fd.reshape(-1)
        for i in range(flat.size):
            v = flat[i]
            eps = 1e-6 * max(1.0, abs(v))
            flat[i] = v + eps
            lp = loss(inp, opt, kw, dout, dhf)
            flat[i] = v - eps
            lm = loss(inp, opt, kw, dout, dhf)
            flat[i] = v
            fflat[i] = (lp - lm) / (2 * eps)
        err = np.abs(got - fd)
        assert np.all(err <= 1e-7 + 1e-6 * np.abs(fd)), \
            "%s: max err %.3e (max |grad| %.3e)" % (name, float(err.max()), float(np.abs(fd).max()))


def test_bwd_full_layer():
    """conv with bias and history, gate, skip, bias, initial state"""
    check_fd(*case(1))


def test_bwd_groups_share_B_and_C():
    """two heads per group: the B and C gradients of a group add up"""
    check_fd(*case(2, H=4, G=2, P=2, N=3, L=5))


def test_bwd_post_conv_inputs_no_gate_no_softplus():
    check_fd(*case(3, conv=False, z=False, softplus=False, L=7))


def test_bwd_no_skip_no_bias_no_state():
    check_fd(*case(4, D=False, bias=False, h0=False, hist=False, K=4, L=5))


def test_bwd_linear_in_dout():
    """The gradients are linear in (dout, dh_final): g(a u + v) = a g(u) + g(v)."""
    inp, opt, kw, d1, h1 = case(5)
    _, _, _, d2, h2 = case(6)
    run = lambda d, h: oracle.mamba2_bwd(inp["xbc"], inp["dt"], inp["A"], d, **kw, **opt,
                                         dh_final=h, f64_inputs=True)
    g1, g2, g12 = run(d1, h1), run(d2, h2), run(3.0 * d1 + d2, 3.0 * h1 + h2)
    for k in g1:
        assert np.allclose(g12[k], 3.0 * g1[k] + g2[k], rtol=1e-12, atol=1e-12), k
