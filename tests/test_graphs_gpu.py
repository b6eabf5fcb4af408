"""The decode step and the prefill call captured in HIP graphs.

A serving loop replays a captured step instead of launching its kernels one
by one.  The library's calls record into a capture as they are: they take
caller-owned buffers (a workspace where they need one), make no host
synchronisation and no allocation, and hand states through with copy
kernels rather than memset or memcpy nodes.  So a replayed graph must give
exactly what the same calls give eagerly.  Each test replays its graph
several times, with the caller's own eager work and synchronisations between
the replays (new inputs copied into the captured buffers, states reset), and
checks every replay bit for bit against eager calls on the same inputs.
"""
import pytest
import torch

from harness import dev, dev32, params, say
from selective_state_space_08_amd import layer, ssd, synth
from selective_state_space_08_amd.workloads import Workload

pytestmark = pytest.mark.gpu

REPLAYS = 4


def capture(fn):
    """fn run once on a side stream (the usual warm-up before a capture),
    then captured into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def same(a, b, what):
    assert torch.equal(a, b), "%s differs from the eager result" % what


@pytest.mark.parametrize("entry", ["state_update", "state_update_ws", "state_update_noalloc"])
def test_decode_chain_replays(entry):
    """Four decode steps in one graph, replayed from the same starting state:
    every replay's outputs, state and conv ring are the eager chain's."""
    wl = Workload("graph_decode", batch=8, seqlen=1, nheads=8, ngroups=2, dtype="bf16",
                  decode_steps=4, seed=17)
    T = wl.decode_steps
    inp = synth.make_decode(wl)
    xbc, z, dt = inp.steps(0, T)
    xbc, z, dt = dev(xbc, "bf16"), dev(z, "bf16"), dev(dt, "bf16")
    p = layer.LayerParams(nheads=wl.nheads, ngroups=wl.ngroups, conv_w=dev32(inp.conv_w),
                          A=dev32(inp.A), dt_bias=dev32(inp.dt_bias), D=dev32(inp.D))
    st0, ring0 = dev32(inp.state), dev(inp.ring, "bf16")
    st, ring = st0.clone(), ring0.clone()
    y = torch.zeros((T, wl.batch, wl.d_inner), device="cuda")
    ws = torch.empty(ssd.ssd_state_update_workspace_bytes(wl.batch, wl.nheads, 64, wl.ngroups,
                                                          128), dtype=torch.uint8, device="cuda")
    fn = getattr(ssd, "ssd_" + entry)
    extra = {"workspace": ws} if entry == "state_update_ws" else {}

    def chain():
        for t in range(T):
            fn(st, xbc[t], dt[t], p.A, ngroups=wl.ngroups, conv_state=ring, conv_w=p.conv_w,
               z=z[t], D=p.D, dt_bias=p.dt_bias, y=y[t], **extra)

    chain()
    torch.cuda.synchronize()
    ref = (y.clone(), st.clone(), ring.clone())
    g = capture(chain)
    for r in range(REPLAYS):
        st.copy_(st0)
        ring.copy_(ring0)
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("%s: replay %d" % (entry, r))
        same(y, ref[0], "y")
        same(st, ref[1], "the state")
        same(ring, ref[2], "the conv ring")


@pytest.mark.parametrize("B,L,H,G", [(2, 300, 4, 2), (1, 40 * 128 + 17, 2, 1)])
def test_prefill_replays(B, L, H, G):
    """One fused prefill call in a graph (the second shape splits the sequence
    into segments: state-only pass, combine, full pass), replayed on two input
    sets in turn: every replay gives the eager call's y, final state and conv
    history for the inputs then in the captured buffers."""
    sets = [synth.make_prefill(Workload("graph_prefill", batch=B, seqlen=L, nheads=H, ngroups=G,
                                        dtype="bf16", initial_state=True, seed=23 + k))
            for k in range(2)]
    wl = sets[0].wl
    p = params(sets[0])  # the parameters of the first set serve both
    K, cdim = wl.width, wl.cdim
    xbc = dev(sets[0].xbc, "bf16")
    dt = dev(sets[0].dt, "bf16")
    z = dev(sets[0].z, "bf16")
    h0 = dev32(sets[0].h0)
    y = torch.zeros((B, L, H, 64), device="cuda")
    hT = torch.zeros((B, H, 64, 128), device="cuda")
    cso = torch.zeros((B, K - 1, cdim), dtype=torch.bfloat16, device="cuda")
    need = ssd.ssd_chunk_scan_workspace_bytes(B, L, H, ngroups=G, chunk=wl.chunk,
                                              fused_conv=True, math="bf16")
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    def load(k):
        xbc.copy_(dev(sets[k].xbc, "bf16"))
        dt.copy_(dev(sets[k].dt, "bf16"))
        z.copy_(dev(sets[k].z, "bf16"))
        h0.copy_(dev32(sets[k].h0))

    def call():
        layer.prefill(xbc, dt, z, p, fused=True, math="bf16", initial_state=h0, final_state=hT,
                      conv_state_out=cso, y=y, workspace=ws)

    refs = []
    for k in range(2):
        load(k)
        call()
        torch.cuda.synchronize()
        refs.append((y.clone(), hT.clone(), cso.clone()))
    assert not torch.equal(refs[0][0], refs[1][0])  # (the two input sets differ)
    g = capture(call)
    for r in range(REPLAYS):
        k = r % 2
        load(k)
        y.zero_()
        hT.zero_()
        cso.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("prefill B=%d L=%d H=%d: replay %d (input set %d)" % (B, L, H, r, k))
        same(y, refs[k][0], "y")
        same(hT, refs[k][1], "the final state")
        same(cso, refs[k][2], "the conv history")
