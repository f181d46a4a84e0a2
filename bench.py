"""Selective-scan benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one mamba_scan_fwd over the large-model prefill workload (batch 8,
L 4096, d_inner 5120, d_state 16, bf16 u/delta/z/B/C, fp32 A/D/bias, silu gate,
final state returned): every row of the fused path -- input streaming, softplus
step size, discretisation, recurrence, readout, D term, gate, output store and
final state -- runs inside the timed region on inputs already resident in HBM.

Prints ONE JSON line: throughput as GB/s of minimum algorithmic traffic (each
input read once, each output written once), with channel-steps/s and the
fraction of the 8 TB/s HBM peak; the roofline of the dominant kernel; the fp64
oracle timed on the host cores on a bounded sample; and the other workloads
(small prefill, long sequence, decode step, and the causal conv1d + SiLU that
produces the scan's input, prefill and decode token) measured briefly.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "selective-scan GB/s + Gchan-steps/s (B·L·D) and % of MI355X HBM peak"
# Plain-ALU roofline of the scan (no MFMA, no packed FP32).  One state update (b, t, d, n)
# needs one v_exp_f32 and four fp32 VALU operations: Delta*A' (an FMA with the exp bias
# shift), (Delta u)*B, the recurrence FMA and the readout FMA -- 6 flops counting a
# multiply as 1 and an FMA as 2 (the exp is not counted).  The peak is what the chip's
# 256 CUs x 4 SIMDs issue of that mix at the rates the probes measure in the same run
# (mamba_probe_issue): v_exp_f32 at R_exp and the VALU forms at R_fma (all operands in
# vector registers, the cheaper form), both in wave instructions per second over the chip:
#   peak = 6 flops x 64 lanes / (1 / R_exp + 4 / R_fma).
ALU_FLOPS_PER_UPDATE = 6
ALU_VALU_PER_UPDATE = 4


# Sources that determine the dominant kernel's code; HBM traffic measured with counters is
# reported only while their digest matches the one recorded with the counters.
KERNEL_SOURCES = ("selective_state_space_72_amd/csrc/scan_scalar.hip",
                  "selective_state_space_72_amd/csrc/device_math.h",
                  "selective_state_space_72_amd/csrc/scan_common.h")
TRAFFIC_PROFILE = "profiles/scan_scalar_kernel_c3_hbm_traffic.txt"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_digest():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch of the scan kernel from the committed counter summary, or None
    when the summary is missing or was taken on different kernel sources."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_digest") != kernel_source_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU's clock ramps up over the first ~40 ms of sustained work: the default warmup
    # covers that, so the timed steps measure the steady state.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--only-main", action="store_true", help="alias of --no-extra --no-cpu-baseline")
    ap.add_argument("--bwd-only", action="store_true",
                    help="time only the backward pass on the large prefill (for profiling) and "
                         "print its JSON summary")
    ap.add_argument("--bwd-variant", choices=("zoh", "trapezoid", "rotation"),
                    help="with --bwd-only: time the backward of this discretisation option "
                         "instead (for profiling)")
    ap.add_argument("--bwd-config", choices=("c2", "c3", "c4"), default="c3",
                    help="with --bwd-only --bwd-variant: the workload (default: the large "
                         "prefill)")
    ap.add_argument("--ssd-only", action="store_true",
                    help="time only the Mamba-2 SSD scan on its large shape (for profiling) and "
                         "print its JSON summary")
    ap.add_argument("--workload", choices=("c2", "c3", "c4"),
                    help="time only this prefill workload (small prefill, large prefill, long "
                         "sequence) and print its JSON summary (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 512 MiB device copy three times (the reference kernel for "
                         "scaling FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def to_dev(a, dev):
    import numpy as np
    import torch
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(dev)


class ScanCase:
    """A scan workload resident on the GPU with preallocated outputs and workspace."""

    def __init__(self, cfg, dev, with_h_last=True, trapezoid=False, rotation=False, **opts):
        import torch
        import selective_state_space_72_amd as ms
        from selective_state_space_72_amd import synth
        self.cfg = cfg
        self.opts = opts
        inp = synth.make_scan_inputs(cfg)
        p = inp.params
        self.t = {k: to_dev(v, dev) for k, v in dict(u=inp.u, delta=inp.delta, z=inp.z, B=inp.B,
                                                      C=inp.C, A=p.A, D=p.D, bias=p.bias,
                                                      h0=inp.h0).items()}
        self.ext = {}
        extra_bytes = 0
        if trapezoid or rotation:
            m3 = synth.make_mamba3_inputs(cfg)
            es = 4 if cfg.dtype == synth.F32 else 2
            if trapezoid:
                self.ext.update(lam=to_dev(m3.lam, dev), u_prev=to_dev(m3.u_prev, dev),
                                B_prev=to_dev(m3.B_prev, dev))
                extra_bytes += m3.lam.size * es + m3.u_prev.size * es + m3.B_prev.size * es
            if rotation:
                self.ext["theta"] = to_dev(m3.theta, dev)
                extra_bytes += m3.theta.size * es
        act = self.t["u"].dtype
        self.y = torch.empty((cfg.batch, cfg.seqlen, cfg.d_inner), dtype=act, device=dev)
        self.h_last = (torch.empty((cfg.batch, cfg.d_inner, cfg.d_state), dtype=torch.float32,
                                   device=dev) if with_h_last else None)
        nws = ms.mamba_scan_fwd_workspace_size(cfg.batch, cfg.seqlen, cfg.d_inner,
                                               cfg.d_state, trapezoid=trapezoid,
                                               rotation=rotation, **opts)
        self.ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        self.n_spans_auto = nws > 0
        self.min_bytes = cfg.min_bytes(with_h_last=with_h_last) + extra_bytes
        self.inp = inp

    def step(self):
        import selective_state_space_72_amd as ms
        t = self.t
        ms.mamba_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                          delta_bias=t["bias"], h0=t["h0"], out=self.y,
                          h_last_out=self.h_last, workspace=self.ws, **self.ext, **self.opts)


class BwdCase:
    """A backward-pass workload resident on the GPU: the scan's inputs, the upstream
    gradients dy and dh_last, preallocated gradient outputs and workspace."""

    def __init__(self, cfg, dev, discretization="euler", trapezoid=False, rotation=False):
        import torch
        import selective_state_space_72_amd as ms
        from selective_state_space_72_amd import synth
        self.cfg = cfg
        inp = synth.make_scan_inputs(cfg)
        g = synth.make_upstream_grads(cfg)
        p = inp.params
        self.t = {k: to_dev(v, dev) for k, v in dict(u=inp.u, delta=inp.delta, z=inp.z, B=inp.B,
                                                      C=inp.C, A=p.A, D=p.D, bias=p.bias,
                                                      h0=inp.h0, dy=g.dy,
                                                      dh_last=g.dh_last).items()}
        es = 4 if cfg.dtype == synth.F32 else 2
        # Mamba-3 options: their inputs, and their gradients among the outputs
        self.ext = {"discretization": discretization}
        extra_bytes = 0
        if trapezoid or rotation:
            m3 = synth.make_mamba3_inputs(cfg)
            if trapezoid:
                self.ext.update(lam=to_dev(m3.lam, dev), u_prev=to_dev(m3.u_prev, dev),
                                B_prev=to_dev(m3.B_prev, dev))
                extra_bytes += 2 * es * (m3.lam.size + m3.u_prev.size + m3.B_prev.size)
            if rotation:
                self.ext["theta"] = to_dev(m3.theta, dev)
                extra_bytes += 2 * es * m3.theta.size
            self.ws = None  # (sized by the binding; torch's caching allocator keeps it)
        else:
            nws = ms.mamba_scan_bwd_workspace_size(cfg.batch, cfg.seqlen, cfg.d_inner,
                                                   cfg.d_state, discretization=discretization)
            self.ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        self.out = None
        self.step()
        bld = cfg.batch * cfg.seqlen * cfg.d_inner
        bln = cfg.batch * cfg.seqlen * cfg.d_state
        bdn = cfg.batch * cfg.d_inner * cfg.d_state
        dn = cfg.d_inner * cfg.d_state
        act = 3 if cfg.gate else 2
        # each input read once, each gradient written once: u, delta, z, dy in and du,
        # ddelta, dz out; B, C in and dB, dC out; A, D, bias in and their gradients out;
        # h0 in, dh_last in, dh0 out
        self.min_bytes = (bld * es * (act + 1) + bld * es * act + bln * es * 4 +
                          (dn + 2 * cfg.d_inner) * 4 * 2 + bdn * 4 * (3 if cfg.h0 else 2) +
                          extra_bytes)

    def step(self):
        import selective_state_space_72_amd as ms
        t = self.t
        self.out = ms.mamba_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["dy"],
                                     D=t["D"], z=t["z"], delta_bias=t["bias"], h0=t["h0"],
                                     dh_last=t["dh_last"], out=self.out, workspace=self.ws,
                                     **self.ext)


class CkptTrainCase(BwdCase):
    """The training path with checkpoints: the forward scan also stores the state entering
    every 8-step segment (mamba_scan_fwd(..., ckpt=)), and the backward reads them instead of
    running a forward pass of its own (mamba_scan_bwd(..., ckpt=))."""

    def __init__(self, cfg, dev):
        import ctypes
        import torch
        import selective_state_space_72_amd as ms
        self.ck = ms.mamba_scan_ckpt_buffer(cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state, dev)
        lib = ms.load_library()
        ext = ms.ScanExt(None, None, None, None, 1)  # (only the option's presence matters)
        nf = lib.mamba_scan_fwd_workspace_size_ext(cfg.batch, cfg.seqlen, cfg.d_inner,
                                                   cfg.d_state, ctypes.byref(ext), None)
        self.fws = torch.empty(max(int(nf), 1), dtype=torch.uint8, device=dev)
        self._dev = dev
        self.y = self.hl = None
        super().__init__(cfg, dev)
        nws = ms.mamba_scan_bwd_workspace_size(cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state,
                                               with_ckpt=True)
        self.ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        self.forward()
        self.step()

    def forward(self):
        import selective_state_space_72_amd as ms
        t = self.t
        self.y, self.hl = ms.mamba_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"],
                                            D=t["D"], z=t["z"], delta_bias=t["bias"],
                                            h0=t["h0"], return_last_state=True, out=self.y,
                                            h_last_out=self.hl, workspace=self.fws,
                                            ckpt=self.ck)

    def step(self):
        import selective_state_space_72_amd as ms
        if self.y is None:  # (the base class's first step: checkpoints not written yet)
            self.forward()
        t = self.t
        self.out = ms.mamba_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["dy"],
                                     D=t["D"], z=t["z"], delta_bias=t["bias"], h0=t["h0"],
                                     dh_last=t["dh_last"], out=self.out, workspace=self.ws,
                                     ckpt=self.ck)


def time_steps(fn, steps, warmup, flush=None, warm_ms=0.0):
    """Event-timed steps on the current stream.  Returns (ms/step over the back-to-back
    loop, median ms of single steps each preceded by a MALL flush, wall ms/step).
    Warmup runs `warmup` steps and then keeps going until `warm_ms` have passed."""
    import torch
    w0 = time.perf_counter()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while (time.perf_counter() - w0) * 1e3 < warm_ms:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - w0) * 1e3 / steps
    loop_ms = e0.elapsed_time(e1) / steps
    singles = []
    if flush is not None:
        for _ in range(min(steps, 10)):
            flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            singles.append(a.elapsed_time(b))
    med = sorted(singles)[len(singles) // 2] if singles else None
    return loop_ms, med, wall


def make_flush(dev):
    """Writing 1 GiB evicts the 256 MB Infinity Cache (MALL) between timed runs."""
    import torch
    buf = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def flush():
        buf.fill_(1.0)
    return flush


def cpu_baseline(cfg, rows=4):
    """The fp64 oracle on the host cores, on the first `rows` batch rows of the workload."""
    import numpy as np
    import oracle
    from selective_state_space_72_amd import synth
    inp = synth.make_scan_inputs(cfg, batch=rows)
    f = lambda a: synth.to_f64(a, cfg.dtype)  # noqa: E731
    p = inp.params
    args = (f(inp.u), f(inp.delta), p.A.astype(np.float64), f(inp.B), f(inp.C))
    kw = dict(D=p.D.astype(np.float64), z=f(inp.z), bias=p.bias.astype(np.float64))
    orc = oracle.load()
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    orc.scan(*args, **kw, nthreads=threads)
    sec = time.perf_counter() - t0
    chan_steps = rows * cfg.seqlen * cfg.d_inner
    bytes_per_cs = cfg.min_bytes() / cfg.chan_steps
    return {"value": round(chan_steps / sec * bytes_per_cs / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"batch rows 0-{rows - 1} of the workload ({chan_steps} channel-steps, "
                      f"{chan_steps * cfg.d_state} state updates), {sec:.2f} s wall on "
                      f"{threads} threads",
            "gchan_steps_per_s": round(chan_steps / sec / 1e9, 5)}


def extra_workloads(dev, flush, steps):
    import numpy as np
    import torch
    import selective_state_space_72_amd as ms
    from selective_state_space_72_amd import synth
    out = {}
    variants = (("c2", {}), ("c4", {}), ("c3_zoh", dict(discretization="zoh")),
                ("c3_trapezoid", dict(trapezoid=True)), ("c3_rotation", dict(rotation=True)),
                ("c4_rotation", dict(rotation=True)))
    labels = {"discretization": ", zero-order-hold discretisation",
              "trapezoid": ", exponential-trapezoidal rule (lam, u_prev, B_prev)",
              "rotation": ", data-dependent rotation of state pairs (theta)"}
    for name, opts in variants:
        cfg = synth.CONFIGS[name.split("_")[0]]
        case = ScanCase(cfg, dev, **opts)
        loop_ms, med, _ = time_steps(case.step, steps, 10, flush, warm_ms=100.0)
        ms_used = med if med is not None else loop_ms
        out[name] = {"workload": f"{cfg.desc}: batch {cfg.batch}, L {cfg.seqlen}, d_inner "
                                 f"{cfg.d_inner}, d_state {cfg.d_state}, {cfg.dtype}"
                                 + "".join(labels[k] for k in opts),
                     "ms": round(ms_used, 4), "ms_back_to_back": round(loop_ms, 4),
                     "GB_s": round(case.min_bytes / (ms_used * 1e-3) / 1e9, 1),
                     "gchan_steps_per_s": round(cfg.chan_steps / (ms_used * 1e-3) / 1e9, 2),
                     "hbm_frac": round(case.min_bytes / (ms_used * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del case
        torch.cuda.empty_cache()
    # backward pass (gradients of every input) on the three prefill shapes
    for name in ("c3", "c2", "c4"):
        cfg = synth.CONFIGS[name]
        case = BwdCase(cfg, dev)
        loop_ms, med, _ = time_steps(case.step, max(10, steps // 4), 3, flush, warm_ms=100.0)
        ms_used = med if med is not None else loop_ms
        out[name + "_bwd"] = {
            "workload": f"backward of the {cfg.desc}: batch {cfg.batch}, L {cfg.seqlen}, "
                        f"d_inner {cfg.d_inner}, d_state {cfg.d_state}, {cfg.dtype}; du, "
                        "ddelta, dz, dB, dC, dA, dD, dbias, dh0 from dy and dh_last",
            "ms": round(ms_used, 4), "ms_back_to_back": round(loop_ms, 4),
            "GB_s": round(case.min_bytes / (ms_used * 1e-3) / 1e9, 1),
            "gchan_steps_per_s": round(cfg.chan_steps / (ms_used * 1e-3) / 1e9, 2),
            "hbm_frac": round(case.min_bytes / (ms_used * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del case
        torch.cuda.empty_cache()
    # backward of the large prefill with the discretisation variants, and of the long
    # sequence with the trapezoid (a sequence split)
    for name, opts in (("c3_bwd_zoh", dict(discretization="zoh")),
                       ("c3_bwd_trapezoid", dict(trapezoid=True)),
                       ("c3_bwd_rotation", dict(rotation=True)),
                       ("c4_bwd_trapezoid", dict(trapezoid=True))):
        cfg = synth.CONFIGS[name.split("_")[0]]
        case = BwdCase(cfg, dev, **opts)
        loop_ms, med, _ = time_steps(case.step, max(10, steps // 4), 3, flush, warm_ms=100.0)
        ms_used = med if med is not None else loop_ms
        out[name] = {
            "workload": f"backward of the {cfg.desc}: batch {cfg.batch}, L {cfg.seqlen}, "
                        f"d_inner {cfg.d_inner}, d_state {cfg.d_state}, {cfg.dtype}"
                        + "".join(labels[k] for k in opts) + "; all gradients",
            "ms": round(ms_used, 4), "ms_back_to_back": round(loop_ms, 4),
            "GB_s": round(case.min_bytes / (ms_used * 1e-3) / 1e9, 1),
            "gchan_steps_per_s": round(cfg.chan_steps / (ms_used * 1e-3) / 1e9, 2),
            "hbm_frac": round(case.min_bytes / (ms_used * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del case
        torch.cuda.empty_cache()
    # training path with checkpoints on the large prefill: forward storing them, backward
    # reading them
    cfg = synth.CONFIGS["c3"]
    case = CkptTrainCase(cfg, dev)
    f_loop, f_med, _ = time_steps(case.forward, max(10, steps // 4), 3, flush, warm_ms=100.0)
    b_loop, b_med, _ = time_steps(case.step, max(10, steps // 4), 3, flush, warm_ms=100.0)
    fm = f_med if f_med is not None else f_loop
    bm = b_med if b_med is not None else b_loop
    out["c3_train_ckpt"] = {
        "workload": f"training path of the {cfg.desc} (batch {cfg.batch}, L {cfg.seqlen}, "
                    f"d_inner {cfg.d_inner}, d_state {cfg.d_state}, {cfg.dtype}): the forward "
                    "storing a state every 8 steps, then the backward reading them",
        "fwd_ckpt_ms": round(fm, 4), "fwd_ckpt_ms_back_to_back": round(f_loop, 4),
        "bwd_from_ckpt_ms": round(bm, 4), "bwd_from_ckpt_ms_back_to_back": round(b_loop, 4),
        "train_step_ms": round(fm + bm, 4),
        "ckpt_bytes": int(case.ck.numel() * 4)}
    del case
    torch.cuda.empty_cache()
    # causal depthwise conv1d + SiLU producing the scan's u, on the large-prefill shape
    ci = synth.make_conv_inputs(8, 4096, 5120, 4, synth.BF16)
    cx, cw, cb = to_dev(ci.x, dev), to_dev(ci.w, dev), to_dev(ci.bias, dev)
    cs_in, cs_out = to_dev(ci.state, dev), to_dev(ci.state, dev).clone()
    cu = torch.empty_like(cx)

    def cstep():
        ms.mamba_conv1d_silu_fwd(cx, cw, cb, cs_in, out=cu, state_out=cs_out)
    loop_ms, med, _ = time_steps(cstep, steps, 10, flush, warm_ms=100.0)
    cbytes = (cx.numel() * 2 * 2 + cw.numel() * 4 + cb.numel() * 4 + cs_in.numel() * 2 * 2)
    out["conv1d_silu"] = {
        "workload": "causal depthwise conv1d (d_conv 4) + SiLU: x (8, 4096, 5120) bf16 -> u, "
                    "with carried state in and out",
        "ms": round(med, 4), "ms_back_to_back": round(loop_ms, 4),
        "GB_s": round(cbytes / (med * 1e-3) / 1e9, 1),
        "GB_s_back_to_back": round(cbytes / (loop_ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(cbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del cx, cu, ci
    torch.cuda.empty_cache()
    # its decode token on the decode shape (256, 5120)
    dx = to_dev(synth.make_conv_step(0, 256, 5120), dev)
    dstate = to_dev(synth.make_conv_inputs(256, 0, 5120, 4).state, dev)
    du_out = torch.empty_like(dx)

    def cdstep():
        ms.mamba_conv1d_silu_update(dstate, dx, cw, cb, out=du_out)
    loop_ms, med, _ = time_steps(cdstep, max(steps, 50), 10, flush, warm_ms=100.0)
    dcb = dx.numel() * 2 * 2 + dstate.numel() * 2 * 2 + cw.numel() * 4 + cb.numel() * 4
    out["conv1d_silu_decode"] = {
        "workload": "conv1d + SiLU decode token: x (256, 5120) bf16, state (256, 5120, 3) bf16",
        "ms": round(med, 5), "ms_chained_cache_warm": round(loop_ms, 5),
        "GB_s": round(dcb / (med * 1e-3) / 1e9, 1),
        "hbm_frac": round(dcb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    # decode: one-token state update on the (256, 5120, 16) fp32 state
    dc = synth.DECODE
    p, h = synth.make_decode_state()
    st = synth.make_decode_step(0)
    t = {k: to_dev(v, dev) for k, v in dict(u=st.u, delta=st.delta, z=st.z, B=st.B, C=st.C,
                                              A=p.A, D=p.D, bias=p.bias, h=h).items()}
    y = torch.empty((dc["batch"], dc["d_inner"]), dtype=torch.bfloat16, device=dev)

    def dstep():
        ms.mamba_state_update(t["h"], t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"],
                              z=t["z"], delta_bias=t["bias"], out=y)
    loop_ms, med, _ = time_steps(dstep, max(steps, 50), 10, flush, warm_ms=100.0)
    bd = dc["batch"] * dc["d_inner"]
    dbytes = bd * dc["d_state"] * 8 + bd * 2 * 4 + dc["batch"] * dc["d_state"] * 2 * 2 + \
        dc["d_inner"] * (dc["d_state"] + 2) * 4
    out["c5"] = {"workload": "decode step: state (256, 5120, 16) fp32, bf16 token inputs",
                 "ms": round(med, 5), "ms_chained_cache_warm": round(loop_ms, 5),
                 "GB_s": round(dbytes / (med * 1e-3) / 1e9, 1),
                 "GB_s_chained_cache_warm": round(dbytes / (loop_ms * 1e-3) / 1e9, 1),
                 "gchan_steps_per_s": round(bd / (med * 1e-3) / 1e9, 2),
                 "hbm_frac": round(dbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del t, y
    torch.cuda.empty_cache()
    # Mamba-2 SSD scan (chunked, on the matrix cores) on its large shape, and its decode token
    out["ssd_large"] = ssd_workload(dev, flush, steps)
    out["ssd_one_row"] = ssd_workload(dev, flush, steps, batch=1, seqlen=16384)
    out["ssd_decode"] = ssd_decode_workload(dev, flush, steps)
    return out


def ssd_workload(dev, flush, steps, batch=None, seqlen=None):
    """The SSD scan on the large shape: batch 8, L 4096, 80 heads of 64 channels, d_state
    128, bf16 activations, gated, final state returned (or another batch and length of the
    same heads).  Bytes: x, z and y once each, dt, B and C once, the final state; flops: the
    chunked form's products over their causal part (C B^T and M X over s <= t, C H_in and
    B^T X in full), 64-step chunks."""
    import torch
    import selective_state_space_72_amd as ms
    from selective_state_space_72_amd import synth
    sc = dict(synth.SSD_LARGE)
    if batch is not None:
        sc["batch"], sc["seqlen"] = batch, seqlen
    si = synth.make_ssd_inputs(sc["batch"], sc["seqlen"], sc["n_heads"], sc["head_dim"],
                               sc["d_state"], sc["dtype"], sc["gate"], sc["h0"], sc["seed"])
    sa = [to_dev(v, dev) for v in (si.x, si.dt, si.A, si.B, si.C)]
    kw = dict(D=to_dev(si.D, dev), z=to_dev(si.z, dev), dt_bias=to_dev(si.dt_bias, dev))
    need = ms.mamba_ssd_workspace_size(sc["batch"], sc["seqlen"], sc["n_heads"],
                                       sc["head_dim"], sc["d_state"], sc["dtype"])
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    kw["workspace"] = ws
    y, h = ms.mamba_ssd_fwd(*sa, **kw, return_last_state=True)

    def sstep():
        ms.mamba_ssd_fwd(*sa, **kw, out=y, h_last_out=h)
    loop_ms, med, _ = time_steps(sstep, steps, 10, flush, warm_ms=100.0)
    ms_used = med if med is not None else loop_ms
    tok, H, P, N, Q = sc["batch"] * sc["seqlen"], sc["n_heads"], sc["head_dim"], sc["d_state"], 64
    es = 2
    nbytes = tok * (3 * H * P * es + H * es + 2 * N * es) + sc["batch"] * H * P * N * 4
    flop = tok * H * ((Q + 1) * (N + P) + 4 * N * P)
    tf = flop / (ms_used * 1e-3) / 1e12
    gbs = nbytes / (ms_used * 1e-3) / 1e9
    return {"workload": f"Mamba-2 SSD scan: batch {sc['batch']}, L {sc['seqlen']}, 80 heads x "
                        "head_dim 64, d_state 128, bf16 x/dt/B/C/z and y, fp32 A/D/dt_bias and "
                        "state, gated, final state returned",
            "ms": round(ms_used, 4), "ms_back_to_back": round(loop_ms, 4),
            "GB_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "TFLOP_s": round(tf, 1), "mfma_bf16_frac": round(tf / 2500.0, 4),
            "bytes_per_step": nbytes, "flop_per_step": flop,
            "workspace_bytes": need}


def ssd_decode_workload(dev, flush, steps):
    """One Mamba-2 decode token on a persistent fp32 state of 64 rows x 80 heads x 64 x
    d_state 128 (the SSD large shape's heads), bf16 token inputs, gated.  Bytes: the
    state read and written, the token's x, z, y, dt, B, C and the per-head parameters."""
    import torch
    import selective_state_space_72_amd as ms
    from selective_state_space_72_amd import synth
    batch, H, P, N = 64, 80, 64, 128
    si = synth.make_ssd_inputs(batch, 1, H, P, N, synth.BF16, True, True, 7220)
    t = {k: to_dev(v, dev) for k, v in dict(x=si.x[:, 0], dt=si.dt[:, 0], B=si.B[:, 0],
                                              C=si.C[:, 0], z=si.z[:, 0], A=si.A, D=si.D,
                                              bias=si.dt_bias, h=si.h0).items()}
    y = torch.empty((batch, H * P), dtype=torch.bfloat16, device=dev)

    def dstep():
        ms.mamba_ssd_state_update(t["h"], t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"],
                                  z=t["z"], dt_bias=t["bias"], out=y, head_dim=P)
    loop_ms, med, _ = time_steps(dstep, max(steps, 50), 10, flush, warm_ms=100.0)
    nbytes = batch * H * P * N * 8 + batch * H * P * 2 * 3 + batch * H * 2 + \
        batch * N * 2 * 2 + H * 4 * 3
    del t, y
    torch.cuda.empty_cache()
    return {"workload": "Mamba-2 SSD decode token: state (64, 80 x 64, 128) fp32, bf16 token "
                        "inputs, gated",
            "ms": round(med, 5), "ms_chained_cache_warm": round(loop_ms, 5),
            "GB_s": round(nbytes / (med * 1e-3) / 1e9, 1),
            "GB_s_chained_cache_warm": round(nbytes / (loop_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def probe_rates(dev):
    """The measured ceilings: issue rates of the update's instruction forms (chip-wide wave
    instructions per second, 8 waves per SIMD) and the bandwidth of a 512 MiB device copy
    (best over a few grid sizes)."""
    import ctypes
    import torch
    import selective_state_space_72_amd as ms
    lib = ms.load_library()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream(dev).cuda_stream
    sink = torch.empty(cus * 8 * 256, dtype=torch.float32, device=dev)
    out = {"compute_units": cus, "waves_per_simd": 8}

    def timed(launch, reps=5):
        for _ in range(2):
            launch()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            launch()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return sorted(ts)[len(ts) // 2]
    forms = (("fma_vgpr", 0, 4096), ("fma_sgpr", 1, 4096), ("fma_dpp", 4, 4096),
             ("exp", 2, 2048), ("update", 3, 256), ("update_dpp", 5, 256))
    for name, kind, iters in forms:
        n = ctypes.c_uint64(0)

        def launch(kind=kind, iters=iters, n=n):
            st = lib.mamba_probe_issue(kind, 8, iters, cus, ctypes.c_void_p(sink.data_ptr()),
                                       ctypes.byref(n), ctypes.c_void_p(stream))
            if st != 0:
                raise ms.MambaError(st, "mamba_probe_issue")
        sec = timed(launch)
        rate = n.value / sec
        out[name] = {"wave_instr_per_s": float(f"{rate:.4e}"),
                     "simd_cycles_at_2_4_ghz": round(cus * 4 * 2.4e9 / rate, 3)}
    out["update"]["unit"] = out["update_dpp"]["unit"] = "wave-level state updates"
    nbytes = 512 << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    best = 0.0
    for blocks in (1024, 2048, 4096, 16384):
        def launch(blocks=blocks):
            st = lib.mamba_probe_copy(ctypes.c_void_p(src.data_ptr()),
                                      ctypes.c_void_p(dst.data_ptr()), nbytes, blocks,
                                      ctypes.c_void_p(stream))
            if st != 0:
                raise ms.MambaError(st, "mamba_probe_copy")
        sec = timed(launch, reps=7)
        best = max(best, 2 * nbytes / sec / 1e9)
    out["copy_512MiB_GB_s"] = round(best, 1)
    del src, dst, sink
    torch.cuda.empty_cache()
    r_exp, r_fma = out["exp"]["wave_instr_per_s"], out["fma_vgpr"]["wave_instr_per_s"]
    out["alu_peak_tflops"] = round(ALU_FLOPS_PER_UPDATE * 64 /
                                   (1.0 / r_exp + ALU_VALU_PER_UPDATE / r_fma) / 1e12, 2)
    out["update_pattern_tflops"] = round(
        ALU_FLOPS_PER_UPDATE * 64 * out["update"]["wave_instr_per_s"] / 1e12, 2)
    return out


def copy_calibration(dev):
    """Three 512 MiB device copies: the reference kernel that FETCH_SIZE / WRITE_SIZE
    counters of the measured kernels are scaled by."""
    import torch
    src = torch.ones(1 << 27, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def main():
    args = parse()
    if args.only_main:
        args.no_extra = args.no_cpu_baseline = True
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the scan shards over channels with no communication: see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from selective_state_space_72_amd import build as hip_build
    hip_build.ensure_built()
    import selective_state_space_72_amd as ms
    from selective_state_space_72_amd import synth
    ms.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    cfg = synth.CONFIGS["c3"]
    if args.workload:
        wcfg = synth.CONFIGS[args.workload]
        log(f"bench: {wcfg.desc} only")
        case = ScanCase(wcfg, dev)
        loop_ms, _, _ = time_steps(case.step, args.steps, args.warmup, warm_ms=100.0)
        if args.copy_calibration:
            copy_calibration(dev)
        print(json.dumps({"workload": f"{wcfg.desc}: batch {wcfg.batch}, L {wcfg.seqlen}, "
                                      f"d_inner {wcfg.d_inner}, d_state {wcfg.d_state}",
                          "steps": args.steps, "ms_per_step": round(loop_ms, 4),
                          "min_bytes_per_step": case.min_bytes,
                          "GB_s": round(case.min_bytes / (loop_ms * 1e-3) / 1e9, 1)}), flush=True)
        return
    if args.ssd_only:
        log("bench: SSD scan on its large shape")
        res = ssd_workload(dev, make_flush(dev), args.steps)
        if args.copy_calibration:
            copy_calibration(dev)
        print(json.dumps(res), flush=True)
        return
    if args.bwd_only and args.bwd_variant:
        opts = {"zoh": dict(discretization="zoh"), "trapezoid": dict(trapezoid=True),
                "rotation": dict(rotation=True)}[args.bwd_variant]
        bcfg = synth.CONFIGS[args.bwd_config]
        log(f"bench: backward pass on the {bcfg.desc}, {args.bwd_variant}")
        bcase = BwdCase(bcfg, dev, **opts)
        loop_ms, _, _ = time_steps(bcase.step, args.steps, args.warmup)
        if args.copy_calibration:
            copy_calibration(dev)
        print(json.dumps({"workload": f"backward of the {bcfg.desc}, {args.bwd_variant}",
                          "steps": args.steps, "ms_per_step": round(loop_ms, 4),
                          "min_bytes_per_step": bcase.min_bytes,
                          "GB_s": round(bcase.min_bytes / (loop_ms * 1e-3) / 1e9, 1)}),
              flush=True)
        return
    if args.bwd_only:
        log("bench: backward pass on the large prefill (own states, then from checkpoints)")
        bcase = BwdCase(cfg, dev)
        loop_ms, _, _ = time_steps(bcase.step, args.steps, args.warmup)
        min_bytes = bcase.min_bytes
        del bcase
        torch.cuda.empty_cache()
        ccase = CkptTrainCase(cfg, dev)
        f_ms, _, _ = time_steps(ccase.forward, args.steps, args.warmup)
        b_ms, _, _ = time_steps(ccase.step, args.steps, args.warmup)
        if args.copy_calibration:
            copy_calibration(dev)
        print(json.dumps({"workload": "backward of the large-model prefill scan",
                          "steps": args.steps, "ms_per_step": round(loop_ms, 4),
                          "min_bytes_per_step": min_bytes,
                          "GB_s": round(min_bytes / (loop_ms * 1e-3) / 1e9, 1),
                          "fwd_ckpt_ms": round(f_ms, 4), "bwd_from_ckpt_ms": round(b_ms, 4)}),
              flush=True)
        return
    log(f"bench: generating {cfg.name} inputs")
    case = ScanCase(cfg, dev)
    flush = make_flush(dev)
    log("bench: timing")
    # the warmup runs for at least 100 ms: the clock ramps over the first ~40 ms of load
    loop_ms, med_ms, wall_ms = time_steps(case.step, args.steps, args.warmup, flush,
                                          warm_ms=100.0)
    ms_per_step = loop_ms
    gbs = case.min_bytes / (ms_per_step * 1e-3) / 1e9
    gcs = cfg.chan_steps / (ms_per_step * 1e-3) / 1e9
    elems = cfg.chan_steps * cfg.d_state

    # A step is the B/C staging pass (~0.3% of the time) plus one scan launch (no sequence
    # split on this workload); the event-timed step time is charged to the scan kernel,
    # which slightly understates its rate.
    kernel_ms = ms_per_step
    kbytes = case.min_bytes
    del case
    torch.cuda.empty_cache()
    log("bench: probes (issue rates, device copy)")
    probes = probe_rates(dev)
    alu_peak = probes["alu_peak_tflops"]
    tflops = elems * ALU_FLOPS_PER_UPDATE / (kernel_ms * 1e-3) / 1e12
    roof = {"bound": "alu", "achieved": round(tflops, 3), "peak": alu_peak,
            "unit": "TFLOP/s", "frac": round(tflops / alu_peak, 4),
            "traffic": recorded_traffic(),
            "kernel": "scan_scalar_kernel<bf16, d_state 16, 8 waves, chunk 8> (+ stage_bc_kernel)",
            "peak_source": "1 v_exp_f32 + 4 fp32 VALU (6 flops) per state update at the probe "
                           "rates of this run: 6 x 64 / (1/R_exp + 4/R_fma_vgpr)",
            "update_pattern_peak": probes["update_pattern_tflops"],
            "hbm": {"achieved": round(kbytes / (kernel_ms * 1e-3) / 1e9, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(kbytes / (kernel_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "copy_probe_GB_s": probes["copy_512MiB_GB_s"]},
            "alu_time_floor_ms": round(elems * ALU_FLOPS_PER_UPDATE / (alu_peak * 1e12) * 1e3, 4),
            "hbm_time_floor_ms": round(kbytes / HBM_PEAK_GBS / 1e9 * 1e3, 4)}
    line = {"metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": "large-model prefill scan: batch 8, L 4096, d_inner 5120, "
                                   "d_state 16, bf16 u/delta/z/B/C and y, fp32 A/D/bias and "
                                   "state, silu gate, final state returned",
                       "batch": cfg.batch, "seq_len": cfg.seqlen, "d_inner": cfg.d_inner,
                       "d_state": cfg.d_state, "io_dtype": "bf16", "parallelism": "none"},
            "gchan_steps_per_s": round(gcs, 2),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "min_bytes_per_step": kbytes,
            "ms_single_step_mall_flushed": round(med_ms, 4) if med_ms else None,
            "wall_ms_per_step": round(wall_ms, 4),
            "roofline": roof,
            "probes": probes}
    if args.copy_calibration:
        copy_calibration(dev)
    if not args.no_extra:
        log("bench: other workloads")
        line["other_workloads"] = extra_workloads(dev, flush, args.steps)
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(cfg, rows=cfg.batch)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
