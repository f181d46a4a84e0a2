"""Shared helpers for the GPU parity tests: move synthetic inputs to the device,
run the HIP path through the C-ABI binding, run the oracle on the same bits, and
compare with the tolerance metric.

Metric: M(x, r) = max_i |x_i - r_i| / max(|r_i|, rms(r)).  It is the stated
relative error where |r_i| is at least the output RMS and an RMS-relative error
where r_i is small (cancellation in sum_n C h can make r_i ~ 0).  Bounds:
1e-5 for fp32 inputs, 2e-2 for bf16 inputs with the fp32 state.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import selective_state_space_72_amd as ms
from selective_state_space_72_amd import synth

TOL = {synth.F32: 1e-5, synth.BF16: 2e-2}
DEV = torch.device("cuda:0")


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def metric(x, r) -> float:
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    if rms == 0.0:
        return float(np.max(np.abs(x - r)))
    return float(np.max(np.abs(x - r) / np.maximum(np.abs(r), rms)))


def rms_metric(x, r) -> float:
    """Literal max|x - r| / rms(r), reported alongside."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    return float(np.max(np.abs(x - r)) / rms) if rms > 0 else float(np.max(np.abs(x - r)))


def to_dev(a):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(DEV)


def from_dev(t) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


class DevInputs:
    def __init__(self, inp: synth.ScanInputs):
        self.inp = inp
        p = inp.params
        self.u, self.delta, self.z = to_dev(inp.u), to_dev(inp.delta), to_dev(inp.z)
        self.B, self.C = to_dev(inp.B), to_dev(inp.C)
        self.A, self.D, self.bias = to_dev(p.A), to_dev(p.D), to_dev(p.bias)
        self.h0 = to_dev(inp.h0)

    def run(self, *, gate=True, use_D=True, use_bias=True, use_h0=True, **opts):
        y, h = ms.mamba_scan_fwd(self.u, self.delta, self.A, self.B, self.C,
                                 D=self.D if use_D else None,
                                 z=self.z if gate else None,
                                 delta_bias=self.bias if use_bias else None,
                                 h0=self.h0 if use_h0 else None,
                                 return_last_state=True, **opts)
        torch.cuda.synchronize()
        return y, h


def oracle_scan(inp: synth.ScanInputs, bs=None, ds=None, *, gate=True, use_D=True,
                use_bias=True, use_h0=True, zoh=False):
    """Oracle on the sub-grid of batch rows bs x channels ds (all if None)."""
    dt = inp.dtype
    p = inp.params
    bs = np.arange(inp.cfg.batch) if bs is None else np.asarray(bs)
    ds = np.arange(inp.cfg.d_inner) if ds is None else np.asarray(ds)
    f = lambda a: synth.to_f64(a, dt)  # noqa: E731
    sub = lambda a: np.ascontiguousarray(a[bs][:, :, ds])  # noqa: E731 -- slice before widening
    u = f(sub(inp.u))
    delta = f(sub(inp.delta))
    z = f(sub(inp.z)) if (gate and inp.z is not None) else None
    B = f(inp.B[bs])
    C = f(inp.C[bs])
    h0 = (inp.h0[bs][:, ds].astype(np.float64) if (use_h0 and inp.h0 is not None) else None)
    return oracle.load().scan(u, delta, p.A[ds].astype(np.float64), B, C,
                              D=p.D[ds].astype(np.float64) if use_D else None, z=z,
                              bias=p.bias[ds].astype(np.float64) if use_bias else None, h0=h0,
                              zoh=zoh)
