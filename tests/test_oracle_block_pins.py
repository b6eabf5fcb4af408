"""Pins of the oracle's block around the layer (RMSNorm, the linear map, the
pre-norm residual block x + mamba(norm(x)) of "Nemotron-H style Hybrid
Mamba-Transformer 3B feasibility study", section 3.2), against values and
forms that do not share its code: a hand-computed example, closed forms,
invariants, numpy's matrix product, and an independent composition of the
block from numpy and the quadratic SSD form.
"""
import math

import numpy as np
import pytest

import oracle
from pinforms import conv_correlate, ssd_quadratic


# ------------------------------------------------------------------ RMSNorm

def test_rmsnorm_worked_example():
    """x = (3, 4): mean square 12.5, so the row becomes (3, 4) / sqrt(12.5)."""
    out = oracle.rmsnorm(np.array([[3.0, 4.0]]), None, eps=0.0)
    r = math.sqrt(12.5)
    assert np.allclose(out, [[3.0 / r, 4.0 / r]], rtol=0, atol=1e-15)


@pytest.mark.parametrize("c,eps", [(-2.5, 0.25), (1e-3, 1e-5), (7.0, 0.0)])
def test_rmsnorm_constant_row(c, eps):
    """A constant row c maps to c / sqrt(c^2 + eps) in every channel, times w."""
    dim = 24
    c = float(np.float32(c))  # the oracle takes its inputs as fp32 values
    w = np.linspace(0.5, 2.0, dim).astype(np.float32)
    out = oracle.rmsnorm(np.full((3, dim), c), w, eps=eps)
    want = c / math.sqrt(c * c + eps) * w.astype(np.float64)
    assert np.allclose(out, np.broadcast_to(want, out.shape), rtol=1e-14, atol=0)


def test_rmsnorm_unit_rms_and_scale_invariance():
    """With eps = 0 and no weight each output row has RMS exactly 1, and the
    norm ignores a positive scale of its input."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 64)).astype(np.float32)
    out = oracle.rmsnorm(x, None, eps=0.0)
    assert np.allclose(np.sqrt(np.mean(out ** 2, axis=1)), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(oracle.rmsnorm(x * np.float32(8.0), None, eps=0.0), out, rtol=1e-14, atol=0)
    # eps > 0 shrinks every row below unit RMS
    assert np.all(np.sqrt(np.mean(oracle.rmsnorm(x, None, eps=0.5) ** 2, axis=1)) < 1.0)


def test_rmsnorm_weight_scales_each_channel():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4, 16)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, 16).astype(np.float32)
    base = oracle.rmsnorm(x, None, eps=1e-5)
    assert np.allclose(oracle.rmsnorm(x, w, eps=1e-5), base * w.astype(np.float64), rtol=1e-14, atol=0)


# ------------------------------------------------------------------ linear

def test_linear_matches_numpy_matmul():
    """Non-square shapes, so a transposed weight or swapped index fails."""
    rng = np.random.default_rng(5)
    a = rng.standard_normal((7, 24))
    w = rng.standard_normal((10, 24)).astype(np.float32)
    r = rng.standard_normal((7, 10)).astype(np.float32)
    want = a @ w.astype(np.float64).T
    assert np.allclose(oracle.linear(a, w), want, rtol=1e-13, atol=1e-13)
    assert np.allclose(oracle.linear(a, w, residual=r), want + r.astype(np.float64),
                       rtol=1e-13, atol=1e-13)
    # leading axes are kept
    assert oracle.linear(a.reshape(7, 1, 24), w).shape == (7, 1, 10)


def test_linear_identity_and_one_hot():
    rng = np.random.default_rng(6)
    a = rng.standard_normal((5, 8))
    assert np.array_equal(oracle.linear(a, np.eye(8, dtype=np.float32)), a)
    w = np.zeros((3, 8), np.float32)
    w[0, 5] = 1.0
    w[2, 1] = -2.0
    out = oracle.linear(a, w)
    assert np.array_equal(out[:, 0], a[:, 5])
    assert np.array_equal(out[:, 1], np.zeros(5))
    assert np.array_equal(out[:, 2], -2.0 * a[:, 1])


# ------------------------------------------------------------------ the block

def small_block(seed=7, B=2, L=12, dm=16, H=2, P=8, G=1, N=4, K=4):
    rng = np.random.default_rng(seed)
    HP, GN = H * P, G * N
    cdim = HP + 2 * GN
    d_in = 2 * HP + 2 * GN + H
    f32 = lambda a: np.asarray(a, np.float32)
    return dict(
        h=f32(rng.standard_normal((B, L, dm))),
        norm_w=f32(rng.uniform(0.5, 1.5, dm)),
        in_proj_w=f32(rng.standard_normal((d_in, dm)) / math.sqrt(dm)),
        out_proj_w=f32(rng.standard_normal((dm, HP)) / math.sqrt(HP)),
        A=f32(-rng.uniform(0.5, 4.0, H)),
        conv_w=f32(0.4 * rng.standard_normal((cdim, K))),
        conv_b=f32(0.1 * rng.standard_normal(cdim)),
        D=f32(rng.uniform(0.5, 1.5, H)),
        dt_bias=f32(rng.uniform(-2.0, 0.0, H)),
        dims=dict(nheads=H, headdim=P, ngroups=G, dstate=N),
    )


def block_oracle(p, **over):
    kw = dict(conv_w=p["conv_w"], conv_b=p["conv_b"], D=p["D"], dt_bias=p["dt_bias"], norm_eps=1e-5)
    kw.update(over)
    return oracle.mamba2_block_fwd(p["h"], p["norm_w"], p["in_proj_w"], p["out_proj_w"], p["A"],
                                   **p["dims"], **kw)


def test_block_matches_independent_composition():
    """numpy RMSNorm and matrix products, np.correlate conv and the quadratic
    SSD form, with in_proj's outputs sliced as z | x | B | C | dt."""
    p = small_block()
    H, P, G, N = (p["dims"][k] for k in ("nheads", "headdim", "ngroups", "dstate"))
    HP, GN = H * P, G * N
    h = p["h"].astype(np.float64)
    Bt, L, dm = h.shape
    u = h / np.sqrt(np.mean(h ** 2, axis=-1, keepdims=True) + 1e-5) * p["norm_w"].astype(np.float64)
    zx = u @ p["in_proj_w"].astype(np.float64).T
    z = zx[..., :HP]
    xbc = zx[..., HP:2 * HP + 2 * GN]
    dt = zx[..., 2 * HP + 2 * GN:]
    post = conv_correlate(xbc, p["conv_w"], p["conv_b"])
    x = post[..., :HP].reshape(Bt, L, H, P)
    Bm = post[..., HP:HP + GN].reshape(Bt, L, G, N)
    Cm = post[..., HP + GN:].reshape(Bt, L, G, N)
    y = ssd_quadratic(x, Bm, Cm, dt, p["A"], D=p["D"], z=z.reshape(Bt, L, H, P),
                      dt_bias=p["dt_bias"])
    want = h + y.reshape(Bt, L, HP) @ p["out_proj_w"].astype(np.float64).T
    got, _, _ = block_oracle(p)
    mix = want - h
    assert np.abs(got - want).max() <= 1e-12 * np.sqrt(np.mean(mix ** 2))


def test_block_zero_out_proj_is_identity():
    p = small_block(seed=8)
    p["out_proj_w"] = np.zeros_like(p["out_proj_w"])
    got, _, _ = block_oracle(p)
    assert np.array_equal(got, p["h"].astype(np.float64))


def test_block_linear_in_out_proj():
    """The block minus its residual is linear in out_proj's weight."""
    p = small_block(seed=9)
    # weights on a 2^-10 grid, so that w1 + w2 is exact in fp32 as well
    grid = lambda a: (np.round(a * 1024.0) / 1024.0).astype(np.float32)
    w1 = grid(p["out_proj_w"])
    w2 = grid(0.5 * np.random.default_rng(1).standard_normal(w1.shape))
    h = p["h"].astype(np.float64)
    m1 = block_oracle(dict(p, out_proj_w=w1))[0] - h
    m2 = block_oracle(dict(p, out_proj_w=w2))[0] - h
    m12 = block_oracle(dict(p, out_proj_w=w1 + w2))[0] - h
    assert np.abs(m12 - (m1 + m2)).max() <= 1e-12 * np.abs(m12).max()


def test_block_split_carry():
    """Two calls carrying the SSM state and the conv state over the split equal
    one call over the whole sequence."""
    p = small_block(seed=10, L=20)
    full, hT, cso = block_oracle(p)
    a = dict(p, h=p["h"][:, :7])
    b = dict(p, h=p["h"][:, 7:])
    ya, ha, ca = block_oracle(a)
    yb, hb, cb = block_oracle(b, h0=ha, conv_state_in=ca)
    assert np.abs(np.concatenate([ya, yb], axis=1) - full).max() <= 1e-12 * np.abs(full).max()
    assert np.abs(hb - hT).max() <= 1e-12 * np.abs(hT).max()
    assert np.array_equal(cb, cso)
