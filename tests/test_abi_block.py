"""The C ABI of the block around the layer (RMSNorm, the matrix-core
projection and the whole pre-norm residual block), on the CPU: workspace
sizes in closed form, and host-side rejection of bad arguments before any
device call (fake, aligned addresses; nothing is dereferenced).
"""
import ctypes

import pytest

from selective_state_space_08_amd import ssd
from test_abi import Fake, OK, INVALID, UNSUPPORTED, WORKSPACE


def r256(n):
    return (n + 255) // 256 * 256


@pytest.mark.parametrize("B,L,dm,H,G", [(4, 8192, 4096, 128, 8), (2, 300, 512, 8, 2),
                                        (1, 5, 64, 4, 1), (3, 17, 1024, 12, 4)])
def test_block_workspace_closed_form(B, L, dm, H, G):
    """normed input, in_proj output (rows padded to 8 elements) and layer
    output in bf16, each 256-byte aligned, then the layer's own workspace."""
    lib = ssd.load()
    T, HP, GN = B * L, H * 64, G * 128
    ld_in = (2 * HP + 2 * GN + H + 7) // 8 * 8
    scan = lib.ssd_chunk_scan_workspace_bytes(B, L, H, 64, G, 128, 128, 1, 1)
    want = r256(T * dm * 2) + r256(T * ld_in * 2) + r256(T * HP * 2) + r256(scan)
    assert lib.ssd_block_workspace_bytes(B, L, dm, H, 64, G, 128) == want


def test_block_workspace_rejects_bad_shapes():
    lib = ssd.load()
    assert lib.ssd_block_workspace_bytes(0, 10, 64, 4, 64, 1, 128) == 0
    assert lib.ssd_block_workspace_bytes(1, 10, 64, 4, 32, 1, 128) == 0
    assert lib.ssd_block_workspace_bytes(1, 10, 64, 6, 64, 4, 128) == 0


def rms_call(**over):
    f = Fake()
    a = dict(x=f(), xs=512, xd=1, w=f(), eps=1e-5, out=f(), os=512, od=1, n=100, dim=512,
             stream=None)
    a.update(over)
    return ssd.load().ssd_rmsnorm_fwd(*[a[k] for k in ["x", "xs", "xd", "w", "eps", "out", "os",
                                                        "od", "n", "dim", "stream"]])


@pytest.mark.parametrize("over,status", [
    (dict(dim=500), UNSUPPORTED), (dict(dim=0), INVALID), (dict(n=-1), INVALID),
    (dict(eps=-1.0), INVALID), (dict(eps=float("nan")), INVALID), (dict(xs=504), INVALID),
    (dict(os=508), INVALID), (dict(xd=3), INVALID), (dict(x=None), INVALID),
    (dict(x=ctypes.c_void_p((1 << 40) + 8)), INVALID), (dict(w=ctypes.c_void_p((1 << 41) + 4)), INVALID),
])
def test_rmsnorm_validation(over, status):
    assert rms_call(**over) == status
    assert ssd.load().ssd_last_error().decode() != ""


def test_rmsnorm_overlap_rules():
    f = Fake()
    x = f()
    # exact in-place (same dtype and stride) passes validation; a shifted out does not
    assert rms_call(x=x, out=ctypes.c_void_p(x.value + 512), od=1) == INVALID
    assert rms_call(x=x, out=x, od=0) == INVALID  # same address, other dtype
    assert rms_call(n=0, x=None, out=None) == OK


def lin_call(**over):
    f = Fake()
    a = dict(a=f(), lda=4096, w=f(), ldw=4096, r=None, ldr=0, rd=0, out=f(), ldo=1024, od=0,
             M=300, N=1024, K=4096, stream=None)
    a.update(over)
    return ssd.load().ssd_linear_fwd(*[a[k] for k in ["a", "lda", "w", "ldw", "r", "ldr", "rd",
                                                       "out", "ldo", "od", "M", "N", "K",
                                                       "stream"]])


@pytest.mark.parametrize("over,status", [
    (dict(K=4092, lda=4092, ldw=4092), UNSUPPORTED), (dict(K=0), INVALID), (dict(N=0), INVALID),
    (dict(M=-1), INVALID), (dict(lda=4088), INVALID), (dict(ldw=100), INVALID),
    (dict(ldo=1000), INVALID), (dict(od=2), INVALID), (dict(w=None), INVALID),
    (dict(a=None), INVALID), (dict(lda=4100), INVALID),  # 8200-byte rows: not 16-byte multiples
    (dict(a=ctypes.c_void_p((1 << 40) + 2)), INVALID),
    (dict(r=ctypes.c_void_p(1 << 44), ldr=1000), INVALID),
    (dict(r=ctypes.c_void_p(1 << 44), ldr=1024, rd=5), INVALID),
])
def test_linear_validation(over, status):
    assert lin_call(**over) == status
    assert ssd.load().ssd_last_error().decode() != ""


def test_linear_overlap_rules():
    f = Fake()
    a, out = f(), f()
    assert lin_call(a=a, out=ctypes.c_void_p(a.value + 4096)) == INVALID
    # out on the residual: only the exact in-place form (same dtype, same stride)
    assert lin_call(out=out, r=ctypes.c_void_p(out.value + 16), ldr=1024) == INVALID
    assert lin_call(out=out, r=out, ldr=2048, ldo=1024) == INVALID
    assert lin_call(M=0, a=None, out=None) == OK


def block_args(**over):
    f = Fake()
    B, L, dm, H, G = 2, 300, 512, 8, 2
    cdim = H * 64 + 2 * G * 128
    a = dict(h=f(), hd=1, nw=f(), eps=1e-5, win=f(), cw=f(), cb=None, K=4, A=f(), D=f(),
             dtb=f(), sp=1, wout=f(), csi=None, cso=None, h0=None, hT=None, out=f(), od=0,
             B=B, L=L, dm=dm, H=H, P=64, G=G, N=128, ws=f(), wsb=1 << 29, stream=None)
    a.update(over)
    return a


def call_block(a):
    order = ["h", "hd", "nw", "eps", "win", "cw", "cb", "K", "A", "D", "dtb", "sp", "wout",
             "csi", "cso", "h0", "hT", "out", "od", "B", "L", "dm", "H", "P", "G", "N", "ws",
             "wsb", "stream"]
    return ssd.load().ssd_block_fwd(*[a[k] for k in order])


BLOCK_CASES = [
    ("headdim 32", dict(P=32), UNSUPPORTED), ("dstate 64", dict(N=64), UNSUPPORTED),
    ("d_model 500", dict(dm=500), UNSUPPORTED), ("H % G", dict(G=3), INVALID),
    ("conv width 5", dict(K=5), UNSUPPORTED), ("conv width 0", dict(K=0), INVALID),
    ("null in_proj", dict(win=None), INVALID), ("null out_proj", dict(wout=None), INVALID),
    ("null conv_w", dict(cw=None), INVALID), ("null A", dict(A=None), INVALID),
    ("null h", dict(h=None), INVALID), ("dt_softplus 2", dict(sp=2), INVALID),
    ("bad eps", dict(eps=-1.0), INVALID), ("bad dtype", dict(od=4), INVALID),
    ("misaligned conv state", dict(csi=ctypes.c_void_p((1 << 46) + 8)), INVALID),
    ("misaligned final state", dict(hT=ctypes.c_void_p((1 << 46) + 4)), INVALID),
    ("no workspace", dict(ws=None, wsb=0), WORKSPACE),
    ("small workspace", dict(wsb=1 << 10), WORKSPACE),
    ("misaligned workspace", dict(ws=ctypes.c_void_p((1 << 47) + 16)), INVALID),
]


@pytest.mark.parametrize("name,over,status", BLOCK_CASES, ids=[c[0] for c in BLOCK_CASES])
def test_block_validation(name, over, status):
    assert call_block(block_args(**over)) == status
    assert ssd.load().ssd_last_error().decode() != ""


def test_block_overlap_rules():
    a = block_args()
    a["out"] = ctypes.c_void_p(a["h"].value + 1024)
    assert call_block(a) == INVALID              # out partly over h
    a = block_args(hd=1, od=0)
    a["out"] = a["h"]
    assert call_block(a) == INVALID              # same address, other dtype
    a = block_args()
    a["out"] = a["win"]
    assert call_block(a) == INVALID              # out over a weight
    a = block_args()
    a["ws"] = ctypes.c_void_p(a["h"].value)
    assert call_block(a) == INVALID              # workspace over h
    a = block_args(csi=ctypes.c_void_p(1 << 46))
    a["cso"] = ctypes.c_void_p((1 << 46) + 256)
    assert call_block(a) == INVALID              # conv_state_out over conv_state_in
    a = block_args(L=0, ws=None, wsb=0)
    assert call_block(a) == OK                   # nothing to do: no launch
