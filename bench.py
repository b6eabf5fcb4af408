#!/usr/bin/env python3
"""Benchmark of the Mamba-2 SSD layer on one MI355X.

One step = one prefill of the Nemotron-H-8B-shaped Mamba-2 layer (batch 4 x
8192 tokens, 128 heads x 64, d_state 128, 8 groups, chunk 128, conv 4 + SiLU,
SiLU(z) gate; bf16 activations, fp32 state and output) through libssd: the
causal conv, the chunked scan and the gated epilogue.  `value` is prefill
tokens/s with every input already resident in HBM.  The same run times the
other prefill workloads (tiny fp32 prefill; the Nemotron-3-Nano layer with
an initial state; the 131072-token long-context sequence) under "configs",
each with its own roofline; the decode workload (256 sequences x 1000
chained one-token steps, fp32 state) through ssd_state_update_ws and
ssd_state_update under "decode"; the pre-norm residual block around the
layer (RMSNorm, in_proj, the layer, out_proj + residual; d_model 4096) under
"block", with the MFMA roofline of its projections; and the backward pass.
Measured peaks (HBM streaming, back-to-back bf16 MFMAs) come from the
library's calibration kernels, beside the published ones.

Kernel durations come from HIP events recorded on the stream the kernels are
launched on (torch's current stream, which the binding passes to libssd).
The CPU baseline is the fp64 oracle timed on a bounded sample of the same
workload on this host's cores.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 MFMA, TFLOP/s


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def src_hash(*names):
    """Hash of the named csrc files and the compiler options each is built
    with: counters taken on other code, or the same code built otherwise, do
    not match it."""
    from selective_state_space_08_amd import build as libbuild
    common = [f for f in libbuild.FLAGS if not f.startswith("-I")]  # (paths differ per machine)
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "selective_state_space_08_amd", "csrc", n), "rb") as f:
            h.update(f.read())
        h.update(" ".join(common + libbuild.FILE_FLAGS.get(n, [])).encode())
    return h.hexdigest()[:16]


def prefill_alg_bytes_per_token(wl, fused: bool) -> float:
    """Minimum HBM traffic of the layer per token: raw x|B|C, z and dt read once
    (in the workload's activation dtype), y written once (fp32), and, where
    the workload has them, the fp32 initial state read and final state
    written once per sequence (spread over its tokens).  The unfused path
    adds the fp32 conv intermediate's write and re-read."""
    e, o = (4 if wl.dtype == "f32" else 2), 4
    b = e * wl.cdim + e * wl.d_inner + e * wl.nheads + o * wl.d_inner
    if wl.initial_state:
        b += 2 * 4 * wl.nheads * wl.headdim * wl.dstate / wl.seqlen
    if not fused:
        b += 2 * 4 * wl.cdim
    return float(b)


def prefill_alg_flops_per_token(wl) -> float:
    """Matrix-product work of the chunked form per token, counting the causal
    lower triangles: 4 H N P (chunk state + inter-chunk read-out) +
    (Q+1) (G N + H P) (C B^T per group and M X per head)."""
    H, N, P, G, Q = wl.nheads, wl.dstate, wl.headdim, wl.ngroups, wl.chunk
    return 4.0 * H * N * P + (Q + 1) * (G * N + H * P)


def decode_alg_bytes_per_step(wl) -> float:
    B, H, P, N, K = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.width
    state = 2 * 4 * B * H * P * N                 # fp32 state read + write
    ring = 2 * 2 * B * (K - 1) * wl.cdim          # bf16 ring rows read + written
    io = 2 * B * wl.cdim + 2 * B * wl.d_inner + 2 * B * H + 4 * B * wl.d_inner
    return float(state + ring + io)


def traffic_record(kernel_key: str, current_hash: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path)).get(kernel_key)
    except Exception:
        return None
    if not rec or rec.get("source_hash") != current_hash:
        return None
    return rec.get("bytes_per_launch")


def time_prefill(args, wl, torch, layer, synth, dev, dev32, steps=None, warmup=None,
                 fused=None):
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    math_mode = "f32" if wl.dtype == "f32" else "bf16"
    log("prefill %s: generating inputs" % wl.name)
    t0 = time.time()
    inp = synth.make_prefill(wl)
    log("  generated in %.1fs; uploading" % (time.time() - t0))
    from selective_state_space_08_amd import ssd
    xbc = dev(inp.xbc, wl.dtype)
    dt = dev(inp.dt, wl.dtype)
    z = dev(inp.z, wl.dtype)
    p = layer.LayerParams(nheads=wl.nheads, ngroups=wl.ngroups, conv_w=dev32(inp.conv_w),
                          A=dev32(inp.A), dt_bias=dev32(inp.dt_bias), D=dev32(inp.D),
                          chunk=wl.chunk)
    h0 = dev32(inp.h0)
    hT = torch.empty((wl.batch, wl.nheads, wl.headdim, wl.dstate), device="cuda")
    y = torch.empty((wl.batch, wl.seqlen, wl.nheads, wl.headdim), device="cuda")
    fused = (not args.unfused) if fused is None else fused
    conv_out = None if fused else torch.empty((wl.batch, wl.seqlen, wl.cdim), device="cuda")
    need = ssd.ssd_chunk_scan_workspace_bytes(wl.batch, wl.seqlen, wl.nheads,
                                              ngroups=wl.ngroups, fused_conv=fused,
                                              math=math_mode)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    del inp

    def step():
        layer.prefill(xbc, dt, z, p, fused=fused, math=math_mode, initial_state=h0,
                      final_state=hT, conv_out=conv_out, y=y, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(stop)
    per = sorted(a.elapsed_time(b) for a, b in ev)
    step_ms = total_ms / steps
    log("prefill %s: %.3f ms/step (events), median step %.3f ms, wall %.3f s" %
        (wl.name, step_ms, per[len(per) // 2], t_wall))
    del xbc, dt, z, y, ws, conv_out
    return dict(step_ms=step_ms, median_ms=per[len(per) // 2], fused=fused, math=math_mode,
                nseg_workspace=need)


def time_decode(args, wl, torch, layer, synth, dev, dev32):
    from selective_state_space_08_amd import ssd
    T = args.decode_steps
    log("decode %s: generating %d steps of inputs" % (wl.name, T))
    inp = synth.make_decode(wl)
    xbc = torch.empty((T, wl.batch, wl.cdim), dtype=torch.bfloat16, device="cuda")
    z = torch.empty((T, wl.batch, wl.d_inner), dtype=torch.bfloat16, device="cuda")
    dt = torch.empty((T, wl.batch, wl.nheads), dtype=torch.bfloat16, device="cuda")
    BLK = 100
    for s0 in range(0, T, BLK):
        s1 = min(T, s0 + BLK)
        a, b, c = inp.steps(s0, s1)
        xbc[s0:s1] = dev(a, "bf16")
        z[s0:s1] = dev(b, "bf16")
        dt[s0:s1] = dev(c, "bf16")
    p = layer.LayerParams(nheads=wl.nheads, ngroups=wl.ngroups, conv_w=dev32(inp.conv_w),
                          A=dev32(inp.A), dt_bias=dev32(inp.dt_bias), D=dev32(inp.D))
    st0 = dev32(inp.state)
    ring0 = dev(inp.ring, "bf16")
    st, ring = st0.clone(), ring0.clone()
    y = torch.empty((T, wl.batch, wl.d_inner), device="cuda")
    ws = torch.empty(ssd.ssd_state_update_workspace_bytes(wl.batch, wl.nheads, wl.headdim,
                                                          wl.ngroups, wl.dstate),
                     dtype=torch.uint8, device="cuda")
    log("decode: inputs resident (%.1f GB)" % ((xbc.numel() + z.numel()) * 2 / 1e9))

    def run(fused):
        """The chain of T steps from the seeded state and ring, through
        ssd_state_update_ws (fused=False) or ssd_state_update (fused=True)."""
        for t in range(min(T, 20)):
            layer.decode_step(st, xbc[t], dt[t], z[t], ring, p, y=y[t], workspace=ws,
                              fused=fused)
        torch.cuda.synchronize()
        st.copy_(st0)
        ring.copy_(ring0)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(T + 1)]
        marks[0].record(stream)
        for t in range(T):
            layer.decode_step(st, xbc[t], dt[t], z[t], ring, p, y=y[t], workspace=ws,
                              fused=fused)
            marks[t + 1].record(stream)
        torch.cuda.synchronize()
        total_ms = marks[0].elapsed_time(marks[T])
        steps = [marks[t].elapsed_time(marks[t + 1]) for t in range(T)]
        first = sum(steps[:10]) / 10
        last = sum(steps[-10:]) / 10
        log("decode (%s): %.3f ms per step; first 10 %.3f ms, last 10 %.3f ms" %
            ("ssd_state_update" if fused else "ssd_state_update_ws", total_ms / T, first, last))
        return dict(chain_ms=total_ms, step_ms=total_ms / T, first10_ms=first, last10_ms=last)

    res = run(False)
    res["fused"] = run(True)
    return res


def bwd_alg_bytes_per_call(wl) -> float:
    """Bytes a backward call must move at least: raw x|B|C, dt, z and dout in
    (bf16), dxbc, ddt and dz out (fp32), and the initial-state gradient."""
    T, H, P, N = wl.tokens, wl.nheads, wl.headdim, wl.dstate
    reads = 2.0 * T * (wl.cdim + H + 2 * wl.d_inner)
    writes = 4.0 * T * (wl.cdim + H + wl.d_inner) + 4.0 * wl.batch * H * P * N
    return reads + writes


def bwd_flops_per_token(wl, Q: int = 32) -> float:
    """Flops per token of the backward pass in its chunked form (chunks of Q
    tokens), counting each contraction once (causal ones at half): per head,
    the intra-chunk C B^T and its gradient products, the inter-chunk read-out
    and its gradients, the state products, and the forward state pass."""
    P, N = wl.headdim, wl.dstate
    per_head = 2.0 * (Q / 2 * N + P * N + Q / 2 * P + Q / 2 * P + P * N + Q * N + Q * N
                      + P * N + P * N + Q / 2 * P + P * N) + 2.0 * P * N
    return per_head * wl.nheads


def time_backward(args, wl, torch, ssd, synth, dev, dev32):
    """ssd_chunk_scan_bwd at the prefill workload's shape (conv fused, gate,
    skip, bias; bf16 inputs and output gradient)."""
    log("backward %s: generating inputs" % wl.name)
    inp = synth.make_prefill(wl)
    B, L, H, G = wl.batch, wl.seqlen, wl.nheads, wl.ngroups
    HP, GN = wl.d_inner, G * wl.dstate
    xbc = dev(inp.xbc, "bf16")
    x = xbc[:, :, :HP].unflatten(-1, (H, wl.headdim))
    Bm = xbc[:, :, HP:HP + GN].unflatten(-1, (G, wl.dstate))
    Cm = xbc[:, :, HP + GN:].unflatten(-1, (G, wl.dstate))
    dt, z = dev(inp.dt, "bf16"), dev(inp.z, "bf16")
    A, D, dtb, cw = dev32(inp.A), dev32(inp.D), dev32(inp.dt_bias), dev32(inp.conv_w)
    del inp
    dout = torch.randn(B, L, H, wl.headdim, device="cuda").to(torch.bfloat16)
    ws = torch.empty(ssd.ssd_chunk_scan_bwd_workspace_bytes(B, L, H, wl.headdim, G, wl.dstate,
                                                            wl.width), dtype=torch.uint8,
                     device="cuda")
    ms = events_ms(torch, lambda: ssd.ssd_chunk_scan_bwd(x, Bm, Cm, dt, A, dout, D=D, z=z,
                                                         dt_bias=dtb, conv_w=cw, workspace=ws),
                   max(2, args.steps // 10), 1)
    log("backward: %.3f ms per call" % ms)
    return ms


def time_conv(args, wl, torch, ssd, synth, dev, dev32):
    """The standalone conv (ssd_causal_conv1d_fwd) over the workload's raw
    x|B|C: bf16 in, the fp32 post-conv values out (the first step of the
    unfused prefill)."""
    inp = synth.make_prefill(wl)
    xbc = dev(inp.xbc, "bf16")
    cw = dev32(inp.conv_w)
    del inp
    out = torch.empty(xbc.shape, device="cuda")
    ms = events_ms(torch, lambda: ssd.ssd_causal_conv1d_fwd(xbc, cw, out=out), args.steps,
                   args.warmup)
    log("conv: %.3f ms per call" % ms)
    del xbc, out
    return ms


def events_ms(torch, fn, steps: int, warmup: int):
    """Mean duration of fn() over `steps` calls, from HIP events on the stream
    the library launches on (torch's current stream)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def time_block(args, wl, torch, ssd, synth, dev, dev32):
    """The block h + out_proj(mixer(rmsnorm(h))) at the layer's shape, and its
    two projections alone (the dominant kernels)."""
    dm = wl.d_model
    log("block %s d_model %d: generating inputs" % (wl.name, dm))
    bi = synth.make_block(wl)
    h = dev(bi.h, "bf16")
    norm_w, win, wout = dev32(bi.norm_w), dev(bi.in_proj_w, "bf16"), dev(bi.out_proj_w, "bf16")
    conv_w, A, D, dtb = dev32(bi.conv_w), dev32(bi.A), dev32(bi.D), dev32(bi.dt_bias)
    del bi
    out = torch.empty((wl.batch, wl.seqlen, dm), device="cuda")
    ws = torch.empty(ssd.ssd_block_workspace_bytes(wl.batch, wl.seqlen, dm, wl.nheads, 64,
                                                   wl.ngroups, 128), dtype=torch.uint8,
                     device="cuda")
    steps, warm = max(3, args.steps // 4), 2
    call_ms = events_ms(torch, lambda: ssd.ssd_block_fwd(
        h, norm_w, win, conv_w, A, wout, nheads=wl.nheads, ngroups=wl.ngroups, D=D,
        dt_bias=dtb, out=out, workspace=ws), steps, warm)
    T = wl.tokens
    u = h.view(T, dm)
    zx = torch.empty((T, wl.d_in_proj), dtype=torch.bfloat16, device="cuda")
    in_ms = events_ms(torch, lambda: ssd.ssd_linear_fwd(u, win, out=zx), steps, warm)
    del zx
    # a seeded random layer output (an all-zero operand would let the matrix
    # cores run at a lower power and a higher clock than real data does)
    gen = torch.Generator(device="cuda").manual_seed(wl.seed + 7)
    y = torch.randn((T, wl.d_inner), generator=gen, device="cuda").to(torch.bfloat16)
    o2 = out.view(T, dm)
    out_ms = events_ms(torch, lambda: ssd.ssd_linear_fwd(y, wout, residual=u, out=o2), steps, warm)
    log("block: %.3f ms per call; in_proj %.3f ms, out_proj %.3f ms" % (call_ms, in_ms, out_ms))
    return dict(call_ms=call_ms, in_ms=in_ms, out_ms=out_ms)


def measure_peaks(torch, ssd, nbytes: int = 1 << 30, reps: int = 20):
    """The rates this GPU reaches, measured with the library's calibration
    kernels after warm-up: HBM streaming over a buffer of nbytes (four times
    the last-level cache), in place (read and written back at the same
    addresses, the decode state's pattern) and as a copy, each as reps passes
    back to back between two events (as the decode chain is timed); and
    back-to-back bf16 MFMAs on register operands (8 independent chains per
    wave, 8 waves per SIMD).  Measurement only.
    Returns (GB/s of the faster streaming form, its name, TFLOP/s)."""
    n = nbytes // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    stream = torch.cuda.current_stream()
    best = {}
    for name, dst, src in (("in place", a, a), ("copy", b, a)):
        for _ in range(3):
            ssd.ssd_calibrate_stream(dst, src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            ssd.ssd_calibrate_stream(dst, src)
        e1.record(stream)
        torch.cuda.synchronize()
        best[name] = 2 * nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
        log("stream %s: %.0f GB/s (%d passes back to back, 2 x %d MiB each)" %
            (name, best[name], reps, nbytes >> 20))
    del a, b
    out = torch.empty(2048 * 256, device="cuda")
    iters = 4096
    ssd.ssd_calibrate_mfma_bf16(out, iters)
    times = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        flops = ssd.ssd_calibrate_mfma_bf16(out, iters)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    tflops = flops / (min(times) / 1e3) / 1e12
    log("bf16 MFMA loop: %.0f TFLOP/s (best of 5)" % tflops)
    del out
    form = max(best, key=best.get)
    return best[form], form, tflops


def rebase_measured_hbm(out):
    """The streaming rate this GPU was seen to reach is at least the fastest
    HBM-bound rate any timed launch in the run reached: when a kernel's
    algorithmic rate beats the calibration stream, that rate becomes the
    measured HBM peak and every HBM roofline's frac_of_measured is taken
    against it (so none exceeds 1)."""
    recs = []
    def walk(o):
        if isinstance(o, dict):
            r = o.get("roofline")
            if isinstance(r, dict) and r.get("unit") == "GB/s":
                recs.append(r)
            for v in o.values():
                walk(v)
    walk(out)
    peaks = out["measured_peaks"]
    best = max(recs, key=lambda r: r["achieved"], default=None)
    if best is None or best["achieved"] <= peaks["hbm_gbs"]:
        return
    peaks["hbm_gbs_stream"] = peaks["hbm_gbs"]
    peaks["hbm_gbs"] = best["achieved"]
    peaks["hbm_form"] = "algorithmic rate of %s (above the stream kernel's)" % best["kernel"]
    for r in recs:
        r["measured_peak"] = best["achieved"]
        r["frac_of_measured"] = r["achieved"] / best["achieved"]


def calibrate_copy(torch, ssd, nbytes: int = 1 << 30):
    """A plain copy kernel of known size (the library's calibration stream,
    dst != src) for scaling the HBM byte counters of a rocprofv3 --pmc run.
    Returns the bytes read (= bytes written) per call."""
    a = torch.ones(nbytes // 4, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        ssd.ssd_calibrate_stream(b, a)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    return nbytes


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s: float):
    """The fp64 oracle on a bounded sample of the prefill workload: whole
    sequences of sampled (sequence, head) pairs, conv included."""
    import numpy as np
    import oracle
    from selective_state_space_08_amd import synth
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from harness import oracle_pairs
    inp = synth.make_prefill(wl)
    everything = [(b, h) for b in range(wl.batch) for h in range(wl.nheads)]
    order = np.random.default_rng(100).permutation(len(everything))
    n, done, elapsed = 16, 0, 0.0
    while done < len(everything):
        pairs = [everything[i] for i in order[done:done + n]]
        t0 = time.perf_counter()
        oracle_pairs(inp, pairs)
        elapsed += time.perf_counter() - t0
        done += len(pairs)
        if elapsed >= budget_s:
            break
        n = max(16, int(done * (budget_s - elapsed) / max(elapsed, 1e-3)))
    frac = done / len(everything)
    tok_s = wl.tokens * frac / elapsed
    return dict(value=tok_s, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                cpu=cpu_model(), host_cpus=os.cpu_count(),
                sample="%d of %d (sequence, head) pairs of %s, each over all %d tokens with its "
                       "conv channels; %.1f s of oracle time, scaled by the sampled fraction" %
                       (done, len(everything), wl.name, wl.seqlen, elapsed))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other prefill workloads (tiny fp32, Nemotron-3-Nano, long context)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the layer's backward pass")
    ap.add_argument("--no-conv", action="store_true",
                    help="skip the standalone conv timing")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the block around the layer (RMSNorm + projections)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--unfused", action="store_true",
                    help="conv kernel + scan kernel instead of the fused scan")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain copy kernel of known size (for scaling the HBM "
                         "byte counters of a rocprofv3 --pmc run) and print its size")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(asked for --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_state_space_08_amd import layer, ssd, synth
    from selective_state_space_08_amd.workloads import DECODE_MAIN, PREFILL_MAIN, WORKLOADS
    from selective_state_space_08_amd.devio import dev, dev32

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ssd.load()
    if args.calibrate_copy:
        nbytes = calibrate_copy(torch, ssd)
        print(json.dumps({"calibration": "stream_kernel (copy)", "bytes_read": nbytes,
                          "bytes_written": nbytes, "calls": 3}), flush=True)
        return
    # the headline first, then the reference rates (their long MFMA loop and
    # streaming passes are not allowed to set the clock it runs at)
    wl = WORKLOADS[PREFILL_MAIN]
    pre = time_prefill(args, wl, torch, layer, synth, dev, dev32)
    copy_gbs, stream_form, gemm_tflops = measure_peaks(torch, ssd)
    tok_s = wl.tokens / (pre["step_ms"] / 1e3)
    bpt = prefill_alg_bytes_per_token(wl, pre["fused"])
    fpt = prefill_alg_flops_per_token(wl)
    kernel_ms = pre["median_ms"]
    achieved = bpt * wl.tokens / (kernel_ms / 1e3) / 1e9
    peaks = {"hbm_gbs": copy_gbs, "hbm_form": "stream kernel, " + stream_form,
             "bf16_mfma_tflops": gemm_tflops, "mfma_form": "MFMA loop on register operands"}
    # The measured unit is one ssd_chunk_scan_fwd call: the B|C pack kernel
    # (conv of B and C once per group, their matrix-core layouts and the
    # chunk's C B^T tiles into the workspace) and then the scan walker;
    # unfused, the step is the conv kernel over x|B|C followed by that call.
    kfile = ("scan_bf16.hip", "conv1d.hip", "api.hip")
    key = "prefill_fused_call" if pre["fused"] else "prefill_unfused_step"
    traffic = traffic_record(key, src_hash(*kfile))
    out = {
        "metric": "Mamba-2 SSD prefill tokens/s + decode steps/s; % of MFMA / HBM peak",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the Nemotron-H-8B Mamba-2 layer)",
        "config": {"workload": wl.name, "batch": wl.batch, "seqlen": wl.seqlen,
                   "nheads": wl.nheads, "headdim": wl.headdim, "dstate": wl.dstate,
                   "ngroups": wl.ngroups, "chunk": wl.chunk, "conv_width": wl.width,
                   "activations": "bf16", "state_and_output": "fp32",
                   "path": "fused conv+scan" if pre["fused"] else "conv kernel + scan kernel",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": key,
                     "launches": (["bc_pack_kernel", "scan_bf16_kernel"] if pre["fused"] else
                                  ["causal_conv1d_kernel (x|B|C)", "bc_pack_kernel",
                                   "scan_bf16_kernel"]),
                     "alg_bytes_per_token": bpt, "tokens_per_launch": wl.tokens,
                     "launch_ms": kernel_ms, "measured_peak": copy_gbs,
                     "frac_of_measured": achieved / copy_gbs},
        "mfma": {"alg_flops_per_token": fpt,
                 "achieved_tflops": fpt * wl.tokens / (kernel_ms / 1e3) / 1e12,
                 "peak_tflops": BF16_PEAK_TFLOPS,
                 "frac": fpt * wl.tokens / (kernel_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
                 "measured_peak_tflops": gemm_tflops,
                 "frac_of_measured": fpt * wl.tokens / (kernel_ms / 1e3) / 1e12 / gemm_tflops},
    }
    out["measured_peaks"] = peaks
    if not args.no_configs:
        out["configs"] = {}
        for name in [n for n in WORKLOADS if n not in (PREFILL_MAIN, DECODE_MAIN)]:
            cwl = WORKLOADS[name]
            r = time_prefill(args, cwl, torch, layer, synth, dev, dev32, fused=True)
            cb = prefill_alg_bytes_per_token(cwl, True)
            cf = prefill_alg_flops_per_token(cwl)
            ms = r["median_ms"]
            gbs = cb * cwl.tokens / (ms / 1e3) / 1e9
            tf = cf * cwl.tokens / (ms / 1e3) / 1e12
            mpeak = BF16_PEAK_TFLOPS if r["math"] == "bf16" else FP32_MFMA_PEAK_TFLOPS
            out["configs"][name] = {
                "batch": cwl.batch, "seqlen": cwl.seqlen, "nheads": cwl.nheads,
                "ngroups": cwl.ngroups, "activations": cwl.dtype, "math": r["math"],
                "initial_state": cwl.initial_state, "ms_per_call": r["step_ms"],
                "median_ms": ms, "tokens_per_s": cwl.tokens / (r["step_ms"] / 1e3),
                "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                             "kernel": "prefill_fused_call", "alg_bytes_per_token": cb,
                             "tokens_per_launch": cwl.tokens, "launch_ms": ms,
                             "measured_peak": copy_gbs, "frac_of_measured": gbs / copy_gbs},
                "mfma": {"alg_flops_per_token": cf, "achieved_tflops": tf, "peak_tflops": mpeak,
                         "frac": tf / mpeak},
            }
    if not args.no_conv:
        cms = time_conv(args, wl, torch, ssd, synth, dev, dev32)
        cbytes = (2.0 + 4.0) * wl.cdim * wl.tokens  # bf16 in, fp32 out, each element once
        cgbs = cbytes / (cms / 1e3) / 1e9
        out["conv"] = {
            "workload": wl.name + " x|B|C (bf16 in, fp32 out)", "ms_per_call": cms,
            "tokens_per_s": wl.tokens / (cms / 1e3),
            "roofline": {"bound": "hbm", "achieved": cgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": cgbs / HBM_PEAK_GBS,
                         "traffic": traffic_record("conv_fwd", src_hash("conv1d.hip", "api.hip")),
                         "kernel": "causal_conv1d_kernel", "alg_bytes_per_call": cbytes,
                         "measured_peak": copy_gbs, "frac_of_measured": cgbs / copy_gbs}}
    if not args.no_decode:
        dwl = WORKLOADS[DECODE_MAIN].with_(decode_steps=args.decode_steps)
        dec = time_decode(args, dwl, torch, layer, synth, dev, dev32)
        dbytes = decode_alg_bytes_per_step(dwl)
        fz, wsr = dec["fused"], dec

        def droof(r, key, kernel):
            ach = dbytes / (r["step_ms"] / 1e3) / 1e9
            return {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": ach / HBM_PEAK_GBS,
                    "traffic": traffic_record(key, src_hash("state_update.hip", "api.hip")),
                    "kernel": kernel, "measured_peak": copy_gbs,
                    "frac_of_measured": ach / copy_gbs, "alg_bytes_per_step": dbytes}
        # ssd_state_update (no workspace) is the decode entry point; the
        # workspace form is timed beside it
        out["decode"] = {"workload": dwl.name, "entry": "ssd_state_update",
                         "steps_per_s": 1e3 / fz["step_ms"],
                         "tokens_per_s": dwl.batch * 1e3 / fz["step_ms"],
                         "ms_per_step": fz["step_ms"], "first10_ms": fz["first10_ms"],
                         "last10_ms": fz["last10_ms"],
                         "roofline": droof(fz, "decode_fused_state_update",
                                           "state_conv_stream_kernel + ring_shift_bc_kernel")}
        out["decode"]["ssd_state_update_ws"] = {
            "steps_per_s": 1e3 / wsr["step_ms"], "ms_per_step": wsr["step_ms"],
            "first10_ms": wsr["first10_ms"], "last10_ms": wsr["last10_ms"],
            "roofline": droof(wsr, "decode_state_update",
                              "conv_step_kernel + state_stream_kernel")}
    if not args.no_block:
        blk = time_block(args, wl, torch, ssd, synth, dev, dev32)
        T, dm, HP, din = wl.tokens, wl.d_model, wl.d_inner, wl.d_in_proj
        f_in, f_out = 2.0 * T * dm * din, 2.0 * T * HP * dm
        tf_in = f_in / (blk["in_ms"] / 1e3) / 1e12
        out["block"] = {
            "workload": "nemotron_h_8b_block_b4_l8192_d4096",
            "ms_per_call": blk["call_ms"], "tokens_per_s": T / (blk["call_ms"] / 1e3),
            "launches": ["rmsnorm_kernel", "gemm_bf16_kernel (in_proj)", "bc_pack_kernel",
                         "scan_bf16_kernel", "gemm_bf16_kernel (out_proj + residual)"],
            "projection_flops_per_call": f_in + f_out,
            "roofline": {"bound": "mfma", "achieved": tf_in, "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf_in / BF16_PEAK_TFLOPS,
                         "traffic": traffic_record("block_in_proj", src_hash("gemm.hip", "api.hip")),
                         "kernel": "gemm_bf16_kernel (in_proj, M=%d N=%d K=%d)" % (T, din, dm),
                         "alg_flops_per_launch": f_in, "launch_ms": blk["in_ms"],
                         "measured_peak": gemm_tflops, "frac_of_measured": tf_in / gemm_tflops},
            "out_proj": {"ms": blk["out_ms"],
                         "tflops": f_out / (blk["out_ms"] / 1e3) / 1e12,
                         "frac": f_out / (blk["out_ms"] / 1e3) / 1e12 / BF16_PEAK_TFLOPS},
        }
    if not args.no_backward:
        bms = time_backward(args, wl, torch, ssd, synth, dev, dev32)
        fpt_b = bwd_flops_per_token(wl)
        tf_b = fpt_b * wl.tokens / (bms / 1e3) / 1e12
        out["backward"] = {
            "workload": wl.name, "ms_per_call": bms, "tokens_per_s": wl.tokens / (bms / 1e3),
            "dtype": "f32",
            "roofline": {"bound": "mfma", "achieved": tf_b, "peak": FP32_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf_b / FP32_MFMA_PEAK_TFLOPS,
                         "traffic": traffic_record(
                             "backward_call", src_hash("scan_bwd.hip", "conv1d.hip", "api.hip")),
                         "kernel": "ssd_chunk_scan_bwd call (6 kernels)",
                         "alg_flops_per_token": fpt_b,
                         "alg_bytes_per_call": bwd_alg_bytes_per_call(wl)},
        }
    rebase_measured_hbm(out)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
        log("cpu baseline: %.1f tokens/s on %d threads" % (out["cpu_baseline"]["value"],
                                                           out["cpu_baseline"]["cores"]))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
