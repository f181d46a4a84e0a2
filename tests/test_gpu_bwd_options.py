"""GPU parity of the backward pass with the zero-order hold (mamba_scan_bwd(...,
discretization="zoh")) against the fp64 oracle's gradients of that rule
(oracle.scan_bwd_ext(zoh=True), pinned by finite differences).  Metric and bounds of
gpu_helpers: 1e-5 for fp32 inputs, 2e-2 for bf16.  Shapes span several 8-step segments,
64-channel tiles with a ragged tail, sequence splits, and a d_state that runs padded.
"""
from __future__ import annotations

import ctypes
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_72_amd as ms
from selective_state_space_72_amd import synth
from gpu_helpers import DEV, TOL, from_dev, log, metric, to_dev

pytestmark = pytest.mark.gpu

GRADS = ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dbias", "dh0")


def case(n, dtype, *, batch=2, seqlen=150, d_inner=72, gate=True, seed=None):
    cfg = dataclasses.replace(synth.CONFIGS["c3"], d_state=n, dtype=dtype, h0=True, gate=gate,
                              batch=batch, seqlen=seqlen, d_inner=d_inner,
                              seed=500 + n if seed is None else seed)
    inp = synth.make_scan_inputs(cfg)
    return inp, synth.make_upstream_grads(inp.cfg)


def check(label, inp, g, **opts):
    p = inp.params
    log(f"case {label}: batch {inp.cfg.batch} L {inp.cfg.seqlen} D {inp.cfg.d_inner} "
        f"N {inp.cfg.d_state} {inp.dtype} {opts}")
    out = ms.mamba_scan_bwd(to_dev(inp.u), to_dev(inp.delta), to_dev(p.A), to_dev(inp.B),
                            to_dev(inp.C), to_dev(g.dy), D=to_dev(p.D), z=to_dev(inp.z),
                            delta_bias=to_dev(p.bias), h0=to_dev(inp.h0),
                            dh_last=to_dev(g.dh_last), discretization="zoh", **opts)
    torch.cuda.synchronize()
    f = lambda a: synth.to_f64(a, inp.dtype)  # noqa: E731
    ref = oracle.load().scan_bwd_ext(
        f(inp.u), f(inp.delta), p.A.astype(np.float64), f(inp.B), f(inp.C), f(g.dy),
        D=p.D.astype(np.float64), z=f(inp.z) if inp.z is not None else None,
        bias=p.bias.astype(np.float64), h0=inp.h0.astype(np.float64),
        dh_last=g.dh_last.astype(np.float64), zoh=True)
    worst = {k: metric(from_dev(out[k]), ref[k]) for k in GRADS if out.get(k) is not None}
    log(f"  {label}: " + ", ".join(f"{k} {v:.1e}" for k, v in worst.items()))
    assert max(worst.values()) <= TOL[inp.dtype], worst


@pytest.mark.parametrize("n", [4, 8, 16, 32, 12])
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_zoh_backward(n, dtype):
    inp, g = case(n, dtype)
    check(f"zoh N={n}", inp, g)


@pytest.mark.parametrize("n_spans", [2, 5])
def test_zoh_backward_split(n_spans):
    inp, g = case(16, synth.F32, batch=1, seqlen=300, d_inner=130, gate=False)
    check(f"zoh split {n_spans}", inp, g, n_spans=n_spans)


def test_zoh_backward_auto_split_past_one_round():
    """More (batch row, tile) units than one round of two blocks per compute unit (576 on
    256 CUs): the planner splits the zero-order hold's backward into spans by itself; every
    gradient agrees with the unsplit run within the bf16 bound."""
    inp, g = case(16, synth.BF16, batch=9, seqlen=256, d_inner=4096, seed=91)
    p = inp.params
    args = [to_dev(a) for a in (inp.u, inp.delta, p.A, inp.B, inp.C, g.dy)]
    kw = dict(D=to_dev(p.D), z=to_dev(inp.z), delta_bias=to_dev(p.bias), h0=to_dev(inp.h0),
              dh_last=to_dev(g.dh_last), discretization="zoh")
    log("zoh backward 9 x 256 x 4096: automatic plan against one span")
    auto = ms.mamba_scan_bwd(*args, **kw)
    one = ms.mamba_scan_bwd(*args, **kw, n_spans=1)
    torch.cuda.synchronize()
    worst = {k: metric(from_dev(auto[k]), from_dev(one[k])) for k in GRADS
             if auto.get(k) is not None}
    log("  " + ", ".join(f"{k} {v:.1e}" for k, v in worst.items()))
    assert max(worst.values()) <= TOL[synth.BF16], worst


def test_zoh_backward_small_decays():
    """|Delta A| below and above the 1/16 switch of the series: A spread over decades."""
    inp, g = case(16, synth.F32, seed=77)
    rng = np.random.default_rng(3)
    inp.params.A = -np.exp(rng.uniform(np.log(1e-3), np.log(30.0), inp.params.A.shape)).astype(
        np.float32)
    check("zoh A over decades", inp, g)


def test_zoh_backward_refuses_stored_checkpoints():
    inp, g = case(16, synth.F32, batch=1, seqlen=64, d_inner=64)
    p = inp.params
    ck = ms.mamba_scan_ckpt_buffer(1, 64, 64, 16, DEV)
    with pytest.raises(RuntimeError):
        ms.mamba_scan_bwd(to_dev(inp.u), to_dev(inp.delta), to_dev(p.A), to_dev(inp.B),
                          to_dev(inp.C), to_dev(g.dy), ckpt=ck, discretization="zoh")


# ---- the Mamba-3 options: trapezoid (lam, u_prev, B_prev) and rotation (theta) ------------

M3_GRADS = GRADS + ("dlam", "du_prev", "dB_prev", "dtheta")


def check_m3(label, inp, g, m3, *, trap, rot, zoh=False, prev=True, n_spans=0, ends=True):
    p = inp.params
    log(f"case {label}: batch {inp.cfg.batch} L {inp.cfg.seqlen} D {inp.cfg.d_inner} "
        f"N {inp.cfg.d_state} {inp.dtype} trap {trap} rot {rot} zoh {zoh} spans {n_spans}")
    out = ms.mamba_scan_bwd(to_dev(inp.u), to_dev(inp.delta), to_dev(p.A), to_dev(inp.B),
                            to_dev(inp.C), to_dev(g.dy), D=to_dev(p.D), z=to_dev(inp.z),
                            delta_bias=to_dev(p.bias), h0=to_dev(inp.h0) if ends else None,
                            dh_last=to_dev(g.dh_last) if ends else None,
                            discretization="zoh" if zoh else "euler",
                            lam=to_dev(m3.lam) if trap else None,
                            u_prev=to_dev(m3.u_prev) if (trap and prev) else None,
                            B_prev=to_dev(m3.B_prev) if (trap and prev) else None,
                            theta=to_dev(m3.theta) if rot else None, n_spans=n_spans)
    torch.cuda.synchronize()
    f = lambda a: synth.to_f64(a, inp.dtype)  # noqa: E731
    ref = oracle.load().scan_bwd_ext(
        f(inp.u), f(inp.delta), p.A.astype(np.float64), f(inp.B), f(inp.C), f(g.dy),
        D=p.D.astype(np.float64), z=f(inp.z) if inp.z is not None else None,
        bias=p.bias.astype(np.float64), h0=inp.h0.astype(np.float64) if ends else None,
        dh_last=g.dh_last.astype(np.float64) if ends else None, zoh=zoh,
        lam=f(m3.lam) if trap else None,
        u_prev=f(m3.u_prev) if (trap and prev) else None,
        B_prev=f(m3.B_prev) if (trap and prev) else None,
        theta=f(m3.theta) if rot else None)
    worst = {}
    for k in M3_GRADS:
        if out.get(k) is None:
            continue
        if k in ("du_prev", "dB_prev") and not prev:
            continue
        assert tuple(out[k].shape) == ref[k].shape, (k, out[k].shape, ref[k].shape)
        worst[k] = metric(from_dev(out[k]), ref[k])
    log(f"  {label}: " + ", ".join(f"{k} {v:.1e}" for k, v in worst.items()))
    assert max(worst.values()) <= TOL[inp.dtype], worst


M3_CASES = [(16, True, False, False), (16, False, True, False), (16, True, True, False),
            (16, False, True, True), (4, True, True, False), (8, False, True, False),
            (32, True, False, False), (32, False, True, False)]


@pytest.mark.parametrize("n,trap,rot,zoh", M3_CASES)
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_m3_backward(n, trap, rot, zoh, dtype):
    inp, g = case(n, dtype, batch=2, seqlen=77, d_inner=96)
    m3 = synth.make_mamba3_inputs(inp.cfg)
    check_m3(f"m3 N={n}", inp, g, m3, trap=trap, rot=rot, zoh=zoh)


def test_m3_backward_without_prev_and_gate():
    inp, g = case(16, synth.F32, batch=1, seqlen=130, d_inner=70, gate=False)
    m3 = synth.make_mamba3_inputs(inp.cfg)
    check_m3("m3 no prev, no gate", inp, g, m3, trap=True, rot=True, prev=False)


# Sequence splits: 203 steps in 2 spans (104 + 99) or 3 (72 + 72 + 59), so the step before
# each span is inside a segment and the last span ends in a partial segment.  With the
# rotation a split needs d_state 16 or 32.
M3_SPLIT_CASES = [(16, True, False, False), (16, False, True, False), (16, True, True, False),
                  (16, False, True, True), (32, True, True, False), (8, True, False, False)]


@pytest.mark.parametrize("n_spans", [2, 3])
@pytest.mark.parametrize("n,trap,rot,zoh", M3_SPLIT_CASES)
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_m3_backward_split(n, trap, rot, zoh, dtype, n_spans):
    inp, g = case(n, dtype, batch=2, seqlen=203, d_inner=96)
    m3 = synth.make_mamba3_inputs(inp.cfg)
    check_m3(f"m3 split N={n}", inp, g, m3, trap=trap, rot=rot, zoh=zoh, n_spans=n_spans)


def test_m3_backward_split_without_prev_and_gate():
    inp, g = case(16, synth.F32, batch=1, seqlen=300, d_inner=70, gate=False)
    m3 = synth.make_mamba3_inputs(inp.cfg)
    check_m3("m3 split, no prev, no gate", inp, g, m3, trap=True, rot=True, prev=False,
             n_spans=5)


def test_m3_backward_split_without_h0_and_dh_last():
    # the spans' entering state from a zero h0, the adjoint from a zero dh_last
    inp, g = case(16, synth.BF16, batch=2, seqlen=203, d_inner=96)
    m3 = synth.make_mamba3_inputs(inp.cfg)
    check_m3("m3 split, no h0, no dh_last", inp, g, m3, trap=True, rot=True, n_spans=3,
             ends=False)


def test_m3_backward_auto_split_long_sequence():
    # one batch row of two channel tiles: the planner splits the sequence by itself
    inp, g = case(16, synth.BF16, batch=1, seqlen=1024, d_inner=128)
    m3 = synth.make_mamba3_inputs(inp.cfg)
    lib = ms.load_library()
    e = ms.ScanExt(1, None, None, 1)  # (only the options' presence matters for the size)
    auto = lib.mamba_scan_bwd_ext_workspace_size(1, 1024, 128, 16, ctypes.byref(e), None)
    one = lib.mamba_scan_bwd_ext_workspace_size(1, 1024, 128, 16, ctypes.byref(e),
                                                ctypes.byref(ms.ScanOpts(0, 0, 1, 0, 0, 0)))
    assert auto > one  # the span regions: the call is split
    check_m3("m3 auto split", inp, g, m3, trap=True, rot=True)


def m3_oracle_rows(inp, g, m3, ds, rows):
    """Oracle gradients of the options' backward on batch rows `rows` and channel subset ds
    (channels are independent; B, C, theta, B_prev are shared, so dB, dC, dtheta, dB_prev
    are the sums over ds only)."""
    p = inp.params
    f = lambda a: synth.to_f64(a, inp.dtype)  # noqa: E731
    ch = lambda a: np.ascontiguousarray(a[rows][:, :, ds])  # noqa: E731
    return oracle.load().scan_bwd_ext(
        f(ch(inp.u)), f(ch(inp.delta)), p.A[ds].astype(np.float64), f(inp.B[rows]),
        f(inp.C[rows]), f(ch(g.dy)), D=p.D[ds].astype(np.float64), z=f(ch(inp.z)),
        bias=p.bias[ds].astype(np.float64),
        h0=None if inp.h0 is None else inp.h0[rows][:, ds].astype(np.float64),
        dh_last=None if g.dh_last is None else g.dh_last[rows][:, ds].astype(np.float64),
        lam=f(ch(m3.lam)), u_prev=f(np.ascontiguousarray(m3.u_prev[rows][:, ds])),
        B_prev=f(m3.B_prev[rows]), theta=f(m3.theta[rows]))


def test_m3_backward_c3_full_size_sampled():
    """The large prefill (8 x 4096 x 5120, bf16) with the trapezoid and the rotation, in the
    launch configuration the benchmark times: the per-channel gradients on sampled channels
    of every lane and tile position, and dB, dC, dtheta, dB_prev of batch row 0 from the
    oracle over all channels (in groups run in parallel, partial sums added in fp64)."""
    import concurrent.futures
    cfg = synth.CONFIGS["c3"]
    inp = synth.make_scan_inputs(cfg)
    g = synth.make_upstream_grads(cfg)
    m3 = synth.make_mamba3_inputs(cfg)
    p = inp.params
    log("m3 backward, c3 full size: running the GPU backward")
    out = ms.mamba_scan_bwd(to_dev(inp.u), to_dev(inp.delta), to_dev(p.A), to_dev(inp.B),
                            to_dev(inp.C), to_dev(g.dy), D=to_dev(p.D), z=to_dev(inp.z),
                            delta_bias=to_dev(p.bias), h0=to_dev(inp.h0),
                            dh_last=to_dev(g.dh_last), lam=to_dev(m3.lam),
                            u_prev=to_dev(m3.u_prev), B_prev=to_dev(m3.B_prev),
                            theta=to_dev(m3.theta))
    torch.cuda.synchronize()
    ds = np.array([0, 1, 15, 16, 63, 64, 2047, 2600, 4095, 5119])
    di = torch.from_numpy(ds).to(DEV)
    sub = {"du": out["du"][:, :, di], "ddelta": out["ddelta"][:, :, di],
           "dz": out["dz"][:, :, di], "dlam": out["dlam"][:, :, di],
           "du_prev": out["du_prev"][:, di], "dA": out["dA"][di], "dD": out["dD"][di],
           "dbias": out["dbias"][di], "dh0": out["dh0"][:, di]}
    sub = {k: from_dev(v.contiguous()) for k, v in sub.items()}
    row0 = {k: from_dev(out[k][:1].contiguous()) for k in ("dB", "dC", "dtheta", "dB_prev")}
    del out
    ref = m3_oracle_rows(inp, g, m3, ds, slice(None))
    worst = {k: metric(sub[k], ref[k]) for k in sub}
    log("  sampled channels: " + ", ".join(f"{k} {v:.1e}" for k, v in worst.items()))
    assert max(worst.values()) <= TOL[synth.BF16], worst
    groups = np.array_split(np.arange(cfg.d_inner), 16)
    with concurrent.futures.ThreadPoolExecutor(16) as ex:
        parts = list(ex.map(lambda dsg: m3_oracle_rows(inp, g, m3, dsg, slice(0, 1)), groups))
    worst = {k: metric(row0[k], sum(pp[k] for pp in parts)) for k in row0}
    log("  row 0 over all channels: " + ", ".join(f"{k} {v:.1e}" for k, v in worst.items()))
    assert max(worst.values()) <= TOL[synth.BF16], worst

