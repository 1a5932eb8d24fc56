"""Benchmark of the gated delta-rule memory on one MI355X.

Default workload (the headline): Gated DeltaNet chunked forward, bf16
inputs, fp32 state, B=8, H=8, L=2048, d_k=d_v=128, C=64.  One step is one
gdr_fwd_chunked call over one batch (all of its kernels).  Further legs of
the default run, each reported in its own sub-object: the channel-gate
(Kimi-style) forward at B=4, H=16, L=4096 ("kda"); the fixed-token
sequence-length sweep, 65,536 tokens x 16 heads at (B, L) = (32, 2048),
(8, 8192), (2, 32768), (1, 65536) ("sweep": time per call vs L); and the
single-token decode step on 256 sequences x 16 heads (d=128, fp32 state of
512 MiB) over 1024 consecutive steps, with its HBM rate ("decode").

Inputs are drawn on the GPU and resident in HBM before timing starts.  The
chunked legs rotate over several input copies so a working set is not
served from the 256 MB Infinity Cache.  Every rate of a chunked leg comes
from one timing: HIP events around K back-to-back calls on the stream the
library launches on, divided by K.  The CPU baseline runs the fp64 oracle
on a bounded sample of the headline workload on the host cores, and on
one thread.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import itertools
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

import gdr_inputs as gi  # noqa: E402

METRIC = "tokens/s chunked GDN fwd (L=2048,H=8,d=128) + % MFMA peak; decode HBM GB/s"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3     # MI355X fp32 matrix

# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE passes, scaled by
# the same counters read for a 1 GiB device copy (FETCH_SIZE x 2, WRITE_SIZE x 1
# on this chip), with a digest of the kernel sources they were taken on: a
# figure whose sources have changed since is reported as null.
# (the segment-combining kernels of gdr_segment.hip run only for shapes that
# split their scan, which none of the measured workloads below does)
FWD_SOURCES = ('gdr_wy.hip', 'gdr_scan.hip', 'gdr_pipe.h', 'gdr_chunk.h', 'gdr_tri.h',
               'gdr_fwd.hip', 'gdr_device.h', 'gdr_internal.h')
BWD_SOURCES = FWD_SOURCES + ('gdr_bwd.hip', 'gdr_bwd_chain.hip', 'gdr_bwd.h')
MEASURED_TRAFFIC = {
    ("gdn_bf16_B8_H8_L2048_d128", "chunk_wy_kernel + chunk_scan_kernel"):
        dict(sources=FWD_SOURCES, digest="ea5aecb629206c78", read=154.78e6, written=56.67e6),
    ("kda_bf16_B4_H16_L4096_d128", "chunk_wy_channel_kernel + chunk_scan_kernel"):
        dict(sources=FWD_SOURCES, digest="ea5aecb629206c78", read=576.35e6, written=310.38e6),
    ("gdn_decode_bf16_N256_H16_d128", "decode_step_kernel"):
        dict(sources=('gdr_decode.hip', 'gdr_device.h', 'gdr_internal.h'), digest="ceeaddb62259d5a3", read=274.34e6, written=269.49e6),
    ("gdn_bf16_B8_H8_L2048_d128 backward", "chunk_wy_kernel + chunk_scan_kernel + chunk_bwd_chain_pipe_kernel + chunk_bwd_grad_kernel"):
        dict(sources=BWD_SOURCES, digest="9945b68ce4c3165b", read=507.47e6, written=284.17e6),
    ("kda_bf16_B4_H16_L4096_d128 backward", "chunk_wy_channel_kernel + chunk_scan_kernel + chunk_bwd_chain_pipe_kernel + chunk_bwd_grad_channel_kernel"):
        dict(sources=BWD_SOURCES, digest="9945b68ce4c3165b", read=1608.63e6, written=890.25e6),
}


def source_digest(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "gated_delta_rule_88_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch measured with counters, or None if not measured on
    the current kernel sources."""
    m = MEASURED_TRAFFIC.get((workload, kernel))
    if m is None or source_digest(m["sources"]) != m["digest"]:
        return None
    return m["read"] + m["written"]


WORKLOADS = {w.name: w for w in (gi.DELTANET_FP32, gi.GDN_BF16, gi.KDA_BF16, *gi.GDN_SWEEP)}


def chunked_algorithmic(w: gi.ChunkedWorkload, step: int) -> tuple[float, float]:
    """(bytes, flops) the method itself must move and compute for one call.

    Bytes per head-token: q, k, v read and o written in the input dtype,
    beta and log alpha read (4 B each, or 4 d_k B for channel gates).  Bytes
    per (b, h): the final state written (4 d_k d_v).  Flops per head-token
    on the triangular count with C = the token step the kernels execute:
    5 C d + 3 d + 6 d^2 + C^2 / 3 (d = d_k = d_v; 1 FMA = 2 flops)."""
    es = 2 if w.dtype == torch.bfloat16 else 4
    ht = w.B * w.H * w.L
    gate = 0 if w.mode == gi.ALPHA_NONE else (4 if w.mode == gi.ALPHA_SCALAR else 4 * w.dk)
    per_tok = es * (2 * w.dk + 2 * w.dv) + 4 + gate
    state = 4 * w.dk * w.dv * (w.B * w.H) * (2 if w.s0_std > 0 else 1)
    d, C = w.dk, step
    flops = ht * (5 * C * d + 3 * d + 6 * d * d + C * C / 3)
    return float(ht * per_tok + state), float(flops)


def decode_algorithmic(w: gi.DecodeWorkload) -> float:
    """Bytes per decode step: state read + written (fp32), q, k, v read and
    o written (dtype), beta and log alpha read."""
    es = 2 if w.dtype == torch.bfloat16 else 4
    nh = w.N * w.H
    gate = 0 if w.mode == gi.ALPHA_NONE else (4 if w.mode == gi.ALPHA_SCALAR else 4 * w.dk)
    return float(nh * (2 * 4 * w.dk * w.dv + es * (2 * w.dk + 2 * w.dv) + 4 + gate))


def chunked_kernel_name(w) -> str:
    """The kernels one gdr_fwd_chunked call launches for this workload (the
    roofline unit is the whole call: both launches)."""
    if w.mode == gi.ALPHA_CHANNEL:
        return "chunk_wy_channel_kernel + chunk_scan_kernel"
    return "chunk_wy_kernel + chunk_scan_kernel"


def copy_probe(mib: int, reps: int = 5):
    """Plain device copies of a known size, for scaling the HBM byte counters
    (FETCH_SIZE, WRITE_SIZE) a profiler reads for the kernels above.  Each
    copy is also timed (an event pair on the current stream, after one
    untimed copy of each kind): the read + write rate a plain streaming
    kernel reaches on this device, the practical ceiling of a kernel that
    reads and writes its bytes once, as the decode step does."""
    dev = torch.device("cuda:0")
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.neg(src, out=dst)
    rate = {}
    for name, fn in (("copy_", lambda: dst.copy_(src)), ("neg", lambda: torch.neg(src, out=dst))):
        ev = _events(2 * reps)
        for i in range(reps):
            ev[2 * i].record()
            fn()
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        ms = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps))
        rate[name] = {"median_ms": ms[reps // 2], "GB_per_s": 2 * n / (ms[reps // 2] * 1e-3) / 1e9}
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "reps": reps,
                      "kernels": ["copy_", "neg"], "rate": rate}))


def _events(n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def bench_chunked(w, steps, warmup, copies, prologue=0):
    """prologue != 0: raw inputs, and the library applies those input-side
    steps itself (gdr_fwd_chunked_ex)."""
    import gated_delta_rule_88_amd as gdr

    dev = torch.device("cuda:0")
    sets = []
    for c in range(copies):
        if prologue:
            x = gi.raw_inputs((w.B, w.H), w.L, w.dk, w.dv, w.dtype, w.mode, w.seed + 1000 * c,
                              w.s0_std, raw_qk=bool(prologue & 1), raw_gates=bool(prologue & 2))
        else:
            # drawn on the GPU: the same recipe, without minutes of host-side
            # drawing for the larger workloads
            x = gi.chunked_inputs(w.B, w.H, w.L, w.dk, w.dv, w.dtype, w.mode,
                                  w.seed + 1000 * c, w.s0_std, device=dev)
        sets.append({k: (None if t is None else t.to(dev)) for k, t in x.items()})
    mode = w.mode
    code = gdr.GDR_BF16 if w.dtype == torch.bfloat16 else gdr.GDR_F32
    need = gdr.gdr_fwd_chunked_workspace_size(w.B, w.H, w.L, w.dk, w.dv, w.C, code, mode)
    outs = [torch.empty((w.B, w.H, w.L, w.dv), dtype=w.dtype, device=dev) for _ in range(copies)]
    finals = [torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device=dev)
              for _ in range(copies)]
    wss = [torch.empty(max(need, 1), dtype=torch.uint8, device=dev) for _ in range(copies)]

    # one checked call per input copy, replayed (the C call per step; the
    # Python-side argument checks would otherwise cost as much host time as
    # the GPU spends on the call)
    calls = [gdr.FwdChunkedCall(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"], w.C,
                                o=outs[c], S_final=finals[c], workspace=wss[c],
                                prologue=prologue)
             for c, d in enumerate(sets)]

    def call(i):
        calls[i % copies]()

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    # whole-job timing: K calls back to back, HIP events on the stream the
    # library launches on (the current stream), bracketed by synchronisations
    t0 = time.perf_counter()
    e0, e1 = _events(2)
    e0.record()
    for i in range(steps):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = e0.elapsed_time(e1)
    # for reference: durations of calls timed one at a time (an event pair
    # around each call), which include the gap an event inserts
    n_each = min(steps, 50)
    ev = _events(2 * n_each)
    for i in range(n_each):
        ev[2 * i].record()
        call(i)
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    per_call = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n_each))
    del sets, outs, finals, wss, calls
    return dict(total_ms=total_ms, wall_s=wall, call_ms=total_ms / steps,
                isolated_ms_mean=sum(per_call) / n_each, isolated_ms_median=per_call[n_each // 2])


def bench_varlen(w, steps, warmup, copies):
    """The packed variable-length forward over one fixed length mix."""
    import gated_delta_rule_88_amd as gdr

    dev = torch.device("cuda:0")
    lens = gi.varlen_lengths(w.N, w.T, w.seed)
    cu = torch.tensor([0] + list(itertools.accumulate(lens)), dtype=torch.int32, device=dev)
    sets = []
    for c in range(copies):
        x = gi.chunked_inputs(1, w.H, w.T, w.dk, w.dv, w.dtype, w.mode, w.seed + 1000 * c)
        sets.append({k: (None if t is None else t[0].to(dev)) for k, t in x.items()})
    code = gdr.GDR_BF16 if w.dtype == torch.bfloat16 else gdr.GDR_F32
    need = gdr.gdr_fwd_varlen_workspace_size(w.N, w.H, w.T, w.dk, w.dv, w.C, code, w.mode)
    outs = [torch.empty((w.H, w.T, w.dv), dtype=w.dtype, device=dev) for _ in range(copies)]
    finals = [torch.empty((w.N, w.H, w.dv, w.dk), dtype=torch.float32, device=dev)
              for _ in range(copies)]
    wss = [torch.empty(max(need, 1), dtype=torch.uint8, device=dev) for _ in range(copies)]

    def call(i):
        d = sets[i % copies]
        gdr.gdr_fwd_varlen(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], None, cu, w.C,
                           o=outs[i % copies], S_final=finals[i % copies],
                           workspace=wss[i % copies])

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    e0, e1 = _events(2)
    e0.record()
    for i in range(steps):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    return dict(total_ms=e0.elapsed_time(e1), lengths=lens)


def bench_backward(w, steps, warmup, copies, train=True):
    """gdr_bwd_chunked on the workload's inputs with a random output gradient
    (the forward is recomputed inside every call)."""
    import gated_delta_rule_88_amd as gdr

    dev = torch.device("cuda:0")
    sets = []
    for c in range(copies):
        x = gi.chunked_inputs(w.B, w.H, w.L, w.dk, w.dv, w.dtype, w.mode, w.seed + 1000 * c,
                              w.s0_std)
        g = torch.Generator().manual_seed(w.seed + 1000 * c + 7)
        x["dO"] = torch.randn(w.B, w.H, w.L, w.dv, generator=g).to(w.dtype)
        sets.append({k: (None if t is None else t.to(dev)) for k, t in x.items()})
    code = gdr.GDR_BF16 if w.dtype == torch.bfloat16 else gdr.GDR_F32
    need = gdr.gdr_bwd_chunked_workspace_size(w.B, w.H, w.L, w.dk, w.dv, w.C, code, w.mode)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def call(i):
        d = sets[i % copies]
        gdr.gdr_bwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"], d["dO"],
                            None, w.C, workspace=ws)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    e0, e1 = _events(2)
    e0.record()
    for i in range(steps):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    total = e0.elapsed_time(e1)
    if not train:
        return dict(total_ms=total, ws_bytes=need, train=None)

    # a training step both ways: the forward, then the backward recomputing
    # it; or the keeping forward, then the backward from what it kept
    o = torch.empty((w.B, w.H, w.L, w.dv), dtype=w.dtype, device=dev)
    fws = torch.empty(max(gdr.gdr_fwd_chunked_workspace_size(w.B, w.H, w.L, w.dk, w.dv, w.C, code, w.mode), 1),
                      dtype=torch.uint8, device=dev)

    def step_recompute(i):
        d = sets[i % copies]
        gdr.gdr_fwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"], w.C, o=o,
                            write_final=False, workspace=fws)
        call(i)

    def step_kept(i):
        d = sets[i % copies]
        gdr.gdr_fwd_chunked_keep(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"], w.C, o=o,
                                 write_final=False, workspace=ws)
        gdr.gdr_bwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["S0"], d["dO"], None,
                            w.C, workspace=ws, kept=True)

    def timed(fn, n):
        for i in range(max(2, warmup // 2)):
            fn(i)
        torch.cuda.synchronize()
        a, b = _events(2)
        a.record()
        for i in range(n):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3

    n = max(steps // 2, 5)
    train = {"forward_then_backward_us": timed(step_recompute, n),
             "keep_forward_then_kept_backward_us": timed(step_kept, n)}
    return dict(total_ms=total, ws_bytes=need, train=train)


def backward_bytes(w):
    """(algorithmic bytes per backward call, the kernels it launches)."""
    es = 2 if w.dtype == torch.bfloat16 else 4
    ht = w.B * w.H * w.L
    gate = {gi.ALPHA_NONE: 0, gi.ALPHA_SCALAR: 4, gi.ALPHA_CHANNEL: 4 * w.dk}[w.mode]
    # read q, k, v, dO, beta, log alpha; write dq, dk, dv, dbeta, dlog alpha
    nbytes = ht * (es * (4 * w.dk + 3 * w.dv) + 8 + 2 * gate)
    pipe = w.dtype == torch.bfloat16 and w.C >= 32   # 32-token steps: the pipelined chain
    kernel = " + ".join((
        "chunk_wy_channel_kernel" if w.mode == gi.ALPHA_CHANNEL else "chunk_wy_kernel",
        "chunk_scan_kernel",
        "chunk_bwd_chain_pipe_kernel" if pipe else "chunk_bwd_chain_kernel",
        "chunk_bwd_grad_channel_kernel" if w.mode == gi.ALPHA_CHANNEL else "chunk_bwd_grad_kernel"))
    return nbytes, kernel


def bench_decode(w, steps, prologue=0):
    import gated_delta_rule_88_amd as gdr

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(w.seed)
    N, H, dk, dv = w.N, w.H, w.dk, w.dv

    def unit(x):   # the caller-side normalisation, unless the library does it
        if prologue & 1:
            return x
        return x / torch.clamp(x.norm(dim=-1, keepdim=True), min=1e-6)

    q = unit(torch.randn(steps, N, H, dk, generator=g, device=dev)).to(w.dtype)
    k = unit(torch.randn(steps, N, H, dk, generator=g, device=dev)).to(w.dtype)
    v = torch.randn(steps, N, H, dv, generator=g, device=dev).to(w.dtype)
    b = torch.randn(steps, N, H, generator=g, device=dev)
    a = -(torch.randn(steps, N, H, generator=g, device=dev) + 2.0)
    if prologue & 2:   # raw pre-activations: the library applies the gates
        beta, la = b, a
    else:
        beta, la = torch.sigmoid(b), -torch.nn.functional.softplus(-a)
    S = torch.randn(N, H, dv, dk, generator=g, device=dev) * w.s0_std
    o = torch.empty(steps, N, H, dv, dtype=w.dtype, device=dev)
    Sw = S.clone()
    for i in range(64):  # warm-up on a scratch copy of the state
        t = i % steps
        gdr.gdr_decode_step(q[t], k[t], v[t], beta[t], la[t], Sw, o[t], prologue=prologue)
    del Sw
    torch.cuda.synchronize()
    e0, e1 = _events(2)
    e0.record()
    for t in range(steps):
        gdr.gdr_decode_step(q[t], k[t], v[t], beta[t], la[t], S, o[t], prologue=prologue)
    e1.record()
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    ok = bool(torch.isfinite(S).all().item())
    return dict(total_ms=total_ms, step_ms=total_ms / steps, finite=ok)


def _host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, chains: int, min_seconds: float, single_seconds: float):
    """fp64 oracle on the first `chains` (b, h) chains of the workload, on all
    the host threads OpenMP is given, repeated until `min_seconds` have
    passed; then on one thread over two chains for `single_seconds`.  Both
    are tokens/s of the chains run (a chain's tokens count once per head, as
    the workload's tokens/s does)."""
    import oracle

    x = gi.workload_inputs(w)
    bh = w.B * w.H
    chains = min(chains, bh)
    flat = lambda t, n: None if t is None else t.reshape((bh,) + tuple(t.shape[2:]))[:n]

    def timed(n, threads, seconds):
        args = [flat(x[k], n) for k in ("q", "k", "v", "beta", "log_alpha", "S0")]
        reps = 0
        t0 = time.perf_counter()
        while True:
            oracle.run(*args, mode=w.mode, nthreads=threads)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= seconds:
                break
        return w.tokens * n / bh * reps / dt, reps, dt

    threads = oracle.max_threads()
    value, reps, dt = timed(chains, threads, min_seconds)
    one, reps1, dt1 = timed(min(2, bh), 1, single_seconds)
    return dict(value=value, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{chains} of {bh} (batch, head) chains at full L={w.L}, run {reps} times: "
                       f"{dt:.1f} s wall on {threads} threads; tokens/s of those chains scaled "
                       f"to the workload's {w.tokens} tokens per call",
                single_thread=dict(value=one, unit="tokens/s", cores=1,
                                   sample=f"{min(2, bh)} chains, run {reps1} times: {dt1:.1f} s on "
                                          "one thread"),
                nproc=os.cpu_count(), host_cpu=_host_cpu_model())


def sweep_leg(steps: int, warmup: int):
    """The fixed-token sequence-length sweep (65,536 tokens x 16 heads per
    call): time per call vs L, one line per (B, L) point."""
    import gated_delta_rule_88_amd as gdr

    pts = []
    for w in gi.GDN_SWEEP:
        r = bench_chunked(w, steps, warmup, 2)
        step = gdr.gdr_fwd_chunked_token_step(w.C, gdr.GDR_BF16, w.mode)
        nbytes, flops = chunked_algorithmic(w, step)
        call_s = r["call_ms"] / 1e3
        pts.append({"workload": w.name, "B": w.B, "L": w.L, "us_per_call": r["call_ms"] * 1e3,
                    "tokens_per_s": w.tokens / call_s, "hbm_frac": nbytes / call_s / 1e9 / HBM_PEAK_GBS,
                    "mfma_frac": flops / call_s / 1e12 / BF16_PEAK_TFLOPS, "token_step": step})
        torch.cuda.empty_cache()
    return pts


def chunked_summary(w, r, step, prologue=0):
    """Throughput and roofline of one chunked workload from one timing (the
    back-to-back per-call time of bench_chunked)."""
    nbytes, flops = chunked_algorithmic(w, step)
    call_s = r["call_ms"] / 1e3
    gbs = nbytes / call_s / 1e9
    tflops = flops / call_s / 1e12
    mfma_peak = BF16_PEAK_TFLOPS if w.dtype == torch.bfloat16 else FP32_PEAK_TFLOPS
    return {
        "tokens_per_s": w.tokens / call_s,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": (None if prologue else
                                 measured_traffic(w.name, chunked_kernel_name(w))),
                     "kernel": chunked_kernel_name(w),
                     "algorithmic_bytes_per_call": nbytes,
                     "call_ms": r["call_ms"],
                     "isolated_call_ms_mean": r["isolated_ms_mean"]},
        "mfma": {"achieved": tflops, "peak": mfma_peak, "unit": "TFLOP/s",
                 "frac": tflops / mfma_peak, "algorithmic_flops_per_call": flops,
                 "count": f"triangular, at the executed {step}-token step",
                 # the most this call's MFMA fraction could be: its flops done in
                 # the time its algorithmic bytes take at peak HBM bandwidth
                 "ceiling_at_hbm_floor": flops / (nbytes / (HBM_PEAK_GBS * 1e9)) / 1e12 / mfma_peak},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed calls first (200 x 66 us brings the GPU to its steady clock; "
                         "with 20 the first timed calls run up to 8 %% slower)")
    ap.add_argument("--workload", default=gi.GDN_BF16.name, choices=sorted(WORKLOADS))
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--cpu-chains", type=int, default=32)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-single-seconds", type=float, default=4.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the channel-gate and sequence-length-sweep legs of the default run "
                         "(with --backward: the training-step timings)")
    ap.add_argument("--backward", action="store_true",
                    help="time the chunked backward (gradients) on --workload instead (one JSON "
                         "line of its own)")
    ap.add_argument("--varlen", action="store_true",
                    help="time the packed variable-length forward on its length-mix workload "
                         "instead (one JSON line of its own)")
    ap.add_argument("--prologue", type=int, default=0, choices=(0, 1, 2, 3),
                    help="time the fused input-side prologue on raw inputs: 1 = L2-normalise "
                         "q, k; 2 = sigmoid gates; 3 = both")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run plain copies of this many MiB (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the per-(batch, head) chains are independent, so "
              "several GPUs would each run this same kernel on their own share; run with "
              "--gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.backward:
        w = WORKLOADS[args.workload]
        r = bench_backward(w, args.steps, args.warmup, min(args.copies, 2), train=not args.no_legs)
        ms = r["total_ms"] / args.steps
        nbytes, bwd_kernel = backward_bytes(w)
        print(json.dumps({
            "metric": "tokens/s chunked gated delta-rule backward (gradients; forward recomputed "
                      "inside)",
            "value": w.tokens / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
            "data": "synthetic",
            "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "d_k": w.dk, "d_v": w.dv,
                       "C": w.C, "alpha": gi.MODE_NAMES[w.mode], "workspace_bytes": r["ws_bytes"]},
            "roofline": {"bound": "hbm", "achieved": nbytes / (ms / 1e3) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": measured_traffic(w.name + " backward", bwd_kernel),
                         "kernel": bwd_kernel,
                         "algorithmic_bytes_per_call": nbytes},
            # µs per training step (forward + backward, same inputs): with the
            # backward recomputing the forward (the line above), and with the
            # forward keeping its records and states for the backward
            "training_step": r["train"],
        }))
        return
    if args.varlen:
        vw = gi.VARLEN_GDN_BF16
        r = bench_varlen(vw, args.steps, args.warmup, args.copies)
        ms = r["total_ms"] / args.steps
        vb = vw.H * vw.T * (2 * (2 * vw.dk + 2 * vw.dv) + 8) + vw.N * vw.H * 4 * vw.dk * vw.dv
        print(json.dumps({
            "metric": "tokens/s packed variable-length GDN fwd", "value": vw.tokens / (ms / 1e3),
            "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": vw.name, "N": vw.N, "H": vw.H, "T": vw.T, "d_k": vw.dk,
                       "d_v": vw.dv, "C": vw.C, "lengths": r["lengths"],
                       "input_copies": args.copies},
            "roofline": {"bound": "hbm", "achieved": vb / (ms / 1e3) / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": vb / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": None, "kernel": "chunk_wy_kernel + chunk_scan_kernel",
                         "algorithmic_bytes_per_call": vb},
        }))
        return
    import gated_delta_rule_88_amd as gdr

    w = WORKLOADS[args.workload]
    code = gdr.GDR_BF16 if w.dtype == torch.bfloat16 else gdr.GDR_F32
    step = gdr.gdr_fwd_chunked_token_step(w.C, code, w.mode)
    r = bench_chunked(w, args.steps, args.warmup, args.copies, args.prologue)
    summ = chunked_summary(w, r, step, args.prologue)
    ms_step = r["call_ms"]
    out = {
        "metric": METRIC,
        "value": summ["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "d_k": w.dk, "d_v": w.dv,
                   "C": w.C, "token_step": step, "alpha": gi.MODE_NAMES[w.mode],
                   "input_copies": args.copies, "prologue": args.prologue},
        "roofline": summ["roofline"],
        "mfma": summ["mfma"],
    }
    torch.cuda.empty_cache()
    if not args.no_legs and args.workload == gi.GDN_BF16.name and not args.prologue:
        kw = gi.KDA_BF16
        kstep = gdr.gdr_fwd_chunked_token_step(kw.C, gdr.GDR_BF16, kw.mode)
        kr = bench_chunked(kw, max(args.steps // 4, 20), max(args.warmup // 4, 20), 2)
        ks = chunked_summary(kw, kr, kstep)
        out["kda"] = {"workload": kw.name, "token_step": kstep, "ms_per_call": kr["call_ms"],
                      **ks}
        torch.cuda.empty_cache()
        out["sweep"] = sweep_leg(max(args.steps // 10, 10), max(args.warmup // 10, 10))
        torch.cuda.empty_cache()
        # the backward on the headline workload (forward recomputed inside),
        # and a training step both ways
        bw = gi.GDN_BF16
        nb = max(args.steps // 10, 20)
        br = bench_backward(bw, nb, max(args.warmup // 20, 5), 2)
        bms = br["total_ms"] / nb
        bbytes, bkern = backward_bytes(bw)
        out["backward"] = {
            "workload": bw.name, "us_per_call": bms * 1e3, "tokens_per_s": bw.tokens / (bms / 1e3),
            "roofline": {"bound": "hbm", "achieved": bbytes / (bms / 1e3) / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": bbytes / (bms / 1e3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": measured_traffic(bw.name + " backward", bkern), "kernel": bkern,
                         "algorithmic_bytes_per_call": bbytes},
            "training_step": br["train"],
        }
    if not args.no_decode:
        dw = gi.DECODE_BF16
        dr = bench_decode(dw, args.decode_steps, args.prologue)
        db = decode_algorithmic(dw)
        dgbs = db / (dr["step_ms"] / 1e3) / 1e9
        out["decode"] = {
            "workload": dw.name, "steps": args.decode_steps, "ms_per_step": dr["step_ms"],
            "tokens_per_s": dw.N / (dr["step_ms"] / 1e3),
            "roofline": {"bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": dgbs / HBM_PEAK_GBS,
                         "traffic": (None if args.prologue else
                                     measured_traffic(dw.name, "decode_step_kernel")),
                         "kernel": "decode_step_kernel", "algorithmic_bytes_per_step": db},
            "state_finite": dr["finite"],
        }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_chains, args.cpu_seconds,
                                           args.cpu_single_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
