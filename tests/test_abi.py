"""The C ABI on the CPU: libssd.so loads, exports every symbol include/ssd.h
declares, and rejects bad arguments on the host before touching a device.

The pointers passed here are fake, aligned addresses: every call below fails
validation, which runs before any HIP call, so nothing is dereferenced and no
device is needed.
"""
import ctypes
import os
import re

import pytest

from selective_state_space_08_amd import ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "ssd.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = ssd.load()
    names = declared_symbols()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), "libssd.so does not export %s" % n
        assert n in ssd.SIGNATURES, "binding does not declare %s" % n
    assert set(ssd.SIGNATURES) == set(names)


def test_status_strings_and_version():
    lib = ssd.load()
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, -4):
        assert lib.ssd_status_string(code).decode() not in ("", "unknown status")
    assert lib.ssd_status_string(42).decode() == "unknown status"
    assert "gfx950" in ssd.ssd_version()


@pytest.mark.parametrize("H,G,K,dtype,es", [(128, 8, 4, 1, 2), (64, 8, 4, 0, 4), (4, 1, 2, 1, 2)])
def test_decode_cache_bytes_closed_form(H, G, K, dtype, es):
    """fp32 state 4*H*P*N plus K-1 conv rows of Cdim = H*P + 2*G*N elements: the
    fixed-size Mamba cache of the hybrid-architecture analysis (Appendix C),
    with an fp32 state."""
    P, N = 64, 128
    want = 4 * H * P * N + (K - 1) * (H * P + 2 * G * N) * es
    assert ssd.load().ssd_decode_cache_bytes(H, P, G, N, K, dtype) == want
    # independent of sequence position: nothing in the signature depends on it


def test_decode_cache_bytes_rejects_bad_input():
    lib = ssd.load()
    assert lib.ssd_decode_cache_bytes(0, 64, 8, 128, 4, 1) == 0
    assert lib.ssd_decode_cache_bytes(12, 64, 8, 128, 4, 1) == 0   # H % G != 0
    assert lib.ssd_decode_cache_bytes(8, 64, 8, 128, 0, 1) == 0
    assert lib.ssd_decode_cache_bytes(8, 64, 8, 128, 4, 9) == 0


def test_workspace_query():
    lib = ssd.load()
    # fp32 path and short sequences never need a workspace
    for fused in (0, 1):
        assert lib.ssd_chunk_scan_workspace_bytes(1, 131072, 80, 64, 8, 128, 128, 0, fused) == 0
    # matrix cores, per (sequence, group, chunk): C [t][n] and B^T hi/lo
    # [n][s] in bf16, and the 36 causal 16x16 tiles of B C^T in fp32
    pack = 3 * 128 * 128 * 2 + 36 * 256 * 4
    for fused in (0, 1):
        assert lib.ssd_chunk_scan_workspace_bytes(4, 128, 128, 64, 8, 128, 128, 1, fused) == \
            4 * 8 * 1 * pack
        assert lib.ssd_chunk_scan_workspace_bytes(4, 8192, 128, 64, 8, 128, 128, 1, fused) == \
            4 * 8 * 64 * pack
    # a ragged last chunk is stored whole
    assert lib.ssd_chunk_scan_workspace_bytes(2, 129, 128, 64, 2, 128, 128, 1, 1) == \
        2 * 2 * 2 * pack
    # one long sequence with few heads is split into segments: per-segment states
    ws = lib.ssd_chunk_scan_workspace_bytes(1, 131072, 80, 64, 8, 128, 128, 1, 0)
    assert ws >= 80 * 2 * 64 * 128 * 4
    assert lib.ssd_chunk_scan_workspace_bytes(0, 128, 8, 64, 8, 128, 128, 1, 0) == 0


@pytest.mark.parametrize("Q", [64, 256])
def test_workspace_query_other_chunks(Q):
    """The pack per (sequence, group, chunk) for chunk lengths 64 and 256: C
    and B^T hi/lo for Q tokens in bf16, and the Q/16 (Q/16 + 1) / 2 causal
    tiles of B C^T in fp32."""
    lib = ssd.load()
    ntri = (Q // 16) * (Q // 16 + 1) // 2
    pack = 3 * Q * 128 * 2 + ntri * 256 * 4
    assert lib.ssd_chunk_scan_workspace_bytes(4, 8192, 128, 64, 8, 128, Q, 1, 1) == \
        4 * 8 * (8192 // Q) * pack
    assert lib.ssd_chunk_scan_workspace_bytes(2, Q + 1, 128, 64, 2, 128, Q, 1, 0) == \
        2 * 2 * 2 * pack
    # an unsupported chunk length on the matrix cores needs (and gets) nothing
    assert lib.ssd_chunk_scan_workspace_bytes(2, 4096, 8, 64, 2, 128, 32, 1, 0) == 0


# ------------------------------------------------------------------ validation

class Fake:
    """Distinct, 256-byte aligned, non-overlapping fake device addresses."""

    def __init__(self):
        self.next = 1 << 32

    def __call__(self, nbytes=1 << 30):
        p = self.next
        self.next += (nbytes + (1 << 20)) // 256 * 256 + 256
        return ctypes.c_void_p(p)


def scan_args(**over):
    f = Fake()
    B, L, H, G = 2, 300, 8, 2
    a = dict(x=f(), xs=H * 64, Bm=f(), bs=G * 128, Cm=f(), cs=G * 128, xd=1, conv_w=None,
             conv_b=None, K=0, csi=None, cso=None, dt=f(), dts=H, z=f(), zs=H * 64, ad=1,
             A=f(), D=f(), dt_bias=f(), sp=1, h0=f(), hT=f(), y=f(), ys=H * 64, yd=0, B=B, L=L,
             H=H, P=64, G=G, N=128, Q=128, math=1, ws=None, wsb=0, stream=None)
    a.update(over)
    return a


def call_scan(a):
    lib = ssd.load()
    order = ["x", "xs", "Bm", "bs", "Cm", "cs", "xd", "conv_w", "conv_b", "K", "csi", "cso",
             "dt", "dts", "z", "zs", "ad", "A", "D", "dt_bias", "sp", "h0", "hT", "y", "ys",
             "yd", "B", "L", "H", "P", "G", "N", "Q", "math", "ws", "wsb", "stream"]
    return lib.ssd_chunk_scan_fwd(*[a[k] for k in order])


SCAN_CASES = [
    ("headdim 32", dict(P=32), UNSUPPORTED),
    ("dstate 64", dict(N=64), UNSUPPORTED),
    ("H % G", dict(G=3), INVALID),
    ("chunk 100 on matrix cores", dict(Q=100), UNSUPPORTED),
    ("chunk 32 on matrix cores", dict(Q=32), UNSUPPORTED),
    ("x stride past 32-bit chunk offsets", dict(xs=1 << 23), UNSUPPORTED),
    ("chunk 96 on fp32", dict(Q=96, math=0), UNSUPPORTED),
    ("chunk 0", dict(Q=0), INVALID),
    ("negative seqlen", dict(L=-1), INVALID),
    ("null x", dict(x=None), INVALID),
    ("null A", dict(A=None), INVALID),
    ("null y", dict(y=None), INVALID),
    ("x stride below width", dict(xs=8 * 64 - 1), INVALID),
    ("dt stride below width", dict(dts=7), INVALID),
    ("misaligned x", dict(x=ctypes.c_void_p((1 << 40) + 8)), INVALID),
    ("odd token stride bytes", dict(xs=8 * 64 + 4), INVALID),
    ("bad xbc dtype", dict(xd=7), INVALID),
    ("bad math", dict(math=5), INVALID),
    ("dt_softplus 2", dict(sp=2), INVALID),
    ("conv_b without conv_w", dict(conv_b=ctypes.c_void_p(1 << 45)), INVALID),
    ("conv state without conv_w", dict(csi=ctypes.c_void_p(1 << 45)), INVALID),
    ("conv width 5", dict(conv_w=ctypes.c_void_p(1 << 45), K=5), UNSUPPORTED),
    ("conv width 0", dict(conv_w=ctypes.c_void_p(1 << 45), K=0), INVALID),
]


@pytest.mark.parametrize("name,over,status", SCAN_CASES, ids=[c[0] for c in SCAN_CASES])
def test_scan_validation(name, over, status):
    assert call_scan(scan_args(**over)) == status
    assert ssd.load().ssd_last_error().decode() != ""


def test_scan_rejects_y_overlapping_x():
    a = scan_args()
    a["y"] = ctypes.c_void_p(a["x"].value + 64)
    assert call_scan(a) == INVALID


def test_scan_rejects_y_overlapping_state():
    a = scan_args()
    a["y"] = a["h0"]
    assert call_scan(a) == INVALID


def test_scan_rejects_workspace_overlapping_y():
    lib = ssd.load()
    need = lib.ssd_chunk_scan_workspace_bytes(1, 65536, 8, 64, 2, 128, 128, 1, 0)
    a = scan_args(B=1, L=65536)
    a["ws"] = ctypes.c_void_p(a["y"].value)
    a["wsb"] = need
    assert call_scan(a) == INVALID


def test_scan_rejects_conv_state_out_on_conv_state_in():
    a = scan_args(conv_w=ctypes.c_void_p(1 << 45), K=4)
    a["csi"] = ctypes.c_void_p(1 << 46)
    a["cso"] = ctypes.c_void_p((1 << 46) + 256)
    assert call_scan(a) == INVALID


def test_scan_rejects_final_state_partly_on_initial_state():
    """final_state may be initial_state itself, but any other overlap races:
    the workgroup of head h + 1 would read initial[h + 1] while the one of h
    writes final[h] over it."""
    a = scan_args()
    a["hT"] = ctypes.c_void_p(a["h0"].value + 64 * 128 * 4)
    assert call_scan(a) == INVALID
    assert "initial_state" in ssd.load().ssd_last_error().decode()


def test_scan_rejects_batch_beyond_grid():
    assert call_scan(scan_args(B=65536, L=1)) == UNSUPPORTED
    assert conv_call(B=65536, L=1) == UNSUPPORTED


def test_scan_workspace_required():
    """One long sequence with few heads needs a workspace for the sequence
    split; without it (or with too little) the call fails with SSD_ERR_WORKSPACE."""
    lib = ssd.load()
    need = lib.ssd_chunk_scan_workspace_bytes(1, 65536, 8, 64, 2, 128, 128, 1, 0)
    assert need > 0
    assert call_scan(scan_args(B=1, L=65536)) == WORKSPACE
    assert call_scan(scan_args(B=1, L=65536, ws=ctypes.c_void_p(1 << 47), wsb=need - 1)) == WORKSPACE
    assert call_scan(scan_args(B=1, L=65536, ws=ctypes.c_void_p((1 << 47) + 16), wsb=need)) == INVALID


def conv_call(**over):
    f = Fake()
    a = dict(x=f(), xs=512, xd=1, w=f(), bias=None, hin=f(), hout=f(), out=f(), os=512, od=0,
             B=2, L=100, C=512, K=4, silu=1, stream=None)
    a.update(over)
    lib = ssd.load()
    return lib.ssd_causal_conv1d_fwd(*[a[k] for k in ["x", "xs", "xd", "w", "bias", "hin", "hout",
                                                       "out", "os", "od", "B", "L", "C", "K",
                                                       "silu", "stream"]])


@pytest.mark.parametrize("over,status", [
    (dict(K=0), INVALID), (dict(K=5), UNSUPPORTED), (dict(xs=511), INVALID),
    (dict(w=None), INVALID), (dict(x=None), INVALID), (dict(xd=3), INVALID),
    (dict(silu=2), INVALID), (dict(C=0), INVALID), (dict(B=-1), INVALID)])
def test_conv_validation(over, status):
    assert conv_call(**over) == status


def test_conv_rejects_aliasing():
    base = 1 << 40
    assert conv_call(x=ctypes.c_void_p(base), out=ctypes.c_void_p(base + 1024)) == INVALID
    assert conv_call(hin=ctypes.c_void_p(base), hout=ctypes.c_void_p(base)) == INVALID


def update_call(**over):
    f = Fake()
    a = dict(state=f(), xbc=f(), xd=1, ring=f(), w=f(), cb=None, K=4, dt=f(), z=f(), ad=1, A=f(),
             D=f(), dtb=f(), sp=1, y=f(), yd=0, B=4, H=16, P=64, G=2, N=128, stream=None)
    a.update(over)
    return ssd.load().ssd_state_update(*[a[k] for k in ["state", "xbc", "xd", "ring", "w", "cb",
                                                        "K", "dt", "z", "ad", "A", "D", "dtb",
                                                        "sp", "y", "yd", "B", "H", "P", "G", "N",
                                                        "stream"]])


@pytest.mark.parametrize("over,status", [
    (dict(P=32), UNSUPPORTED), (dict(G=3), INVALID), (dict(ring=None), INVALID),
    (dict(w=None), INVALID), (dict(K=5), UNSUPPORTED), (dict(state=None), INVALID),
    (dict(state=ctypes.c_void_p((1 << 40) + 4)), INVALID), (dict(yd=2), INVALID),
    (dict(sp=-1), INVALID)])
def test_state_update_validation(over, status):
    assert update_call(**over) == status


def test_state_update_rejects_y_on_state():
    f = Fake()
    s = f()
    assert update_call(state=s, y=s) == INVALID


def update_ws_call(ws=0, wsz=None, **over):
    f = Fake()
    a = dict(state=f(), xbc=f(), xd=1, ring=f(), w=f(), cb=None, K=4, dt=f(), z=f(), ad=1, A=f(),
             D=f(), dtb=f(), sp=1, y=f(), yd=0, B=4, H=16, P=64, G=2, N=128, stream=None)
    a.update(over)
    need = ssd.load().ssd_state_update_workspace_bytes(a["B"], a["H"], a["P"], a["G"], a["N"])
    ptr = f() if ws == 0 else ws
    return ssd.load().ssd_state_update_ws(
        *[a[k] for k in ["state", "xbc", "xd", "ring", "w", "cb", "K", "dt", "z", "ad", "A",
                         "D", "dtb", "sp", "y", "yd", "B", "H", "P", "G", "N"]],
        ptr, need if wsz is None else wsz, a["stream"])


@pytest.mark.parametrize("B,H,G", [(1, 16, 2), (256, 128, 8), (3, 8, 8), (0, 8, 1)])
def test_state_update_workspace_bytes_closed_form(B, H, G):
    # one fp32 per post-conv channel of each sequence: H*P x, G*N B, G*N C
    assert ssd.load().ssd_state_update_workspace_bytes(B, H, 64, G, 128) == \
        4 * B * (H * 64 + 2 * G * 128)


def test_state_update_workspace_bytes_rejects_bad_input():
    lib = ssd.load()
    assert lib.ssd_state_update_workspace_bytes(4, 12, 64, 8, 128) == 0   # H % G != 0
    assert lib.ssd_state_update_workspace_bytes(4, 16, 32, 2, 128) == 0   # P unsupported
    assert lib.ssd_state_update_workspace_bytes(-1, 16, 64, 2, 128) == 0


@pytest.mark.parametrize("over,status", [
    (dict(P=32), UNSUPPORTED), (dict(G=3), INVALID), (dict(ring=None), INVALID),
    (dict(w=None), INVALID), (dict(K=5), UNSUPPORTED), (dict(state=None), INVALID),
    (dict(yd=2), INVALID), (dict(sp=-1), INVALID), (dict(B=70000), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(wsz=1024), WORKSPACE),
    (dict(ws=ctypes.c_void_p((1 << 41) + 16)), INVALID)])
def test_state_update_ws_validation(over, status):
    assert update_ws_call(**over) == status
    assert ssd.load().ssd_last_error().decode().startswith("state_update_ws")


def test_state_update_ws_rejects_workspace_on_a_tensor():
    f = Fake()
    s = f()
    assert update_ws_call(state=s, ws=s) == INVALID
    assert update_ws_call(y=s, ws=s) == INVALID


def test_state_update_empty_batch_is_a_no_op():
    # batch 0: nothing to read or write, so NULL tensors and no workspace pass
    # validation and nothing is launched (no device needed)
    none = dict(state=None, xbc=None, dt=None, z=None, y=None, A=None, D=None, dtb=None, B=0)
    assert update_call(**none) == OK
    assert update_ws_call(ws=None, wsz=0, **none) == OK


def test_state_update_rejects_huge_batch():
    assert update_call(B=70000) == UNSUPPORTED


def test_binding_refuses_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(ssd, "_lib", None)
    with pytest.raises(ImportError):
        ssd.load(str(tmp_path / "missing.so"))
