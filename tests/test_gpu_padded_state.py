"""d_state values without kernels of their own (1..64 other than 4, 8, 16, 32, 64).

They run at the next compiled size with the state-indexed arrays padded (A with -1, B, C,
h0, theta, B_prev with 0) and the state-indexed results cut back.  The padded states start
at zero and get zero input, so they stay exactly zero and add exactly zero to the readout:
the checks are the oracle (which takes any d_state) at the usual bounds -- 1e-5 for fp32
inputs, 2e-2 for bf16 -- for the scan, the decode step, the Mamba-3 options and the
backward pass, and bitwise equality with a call at the compiled size on inputs padded by
hand.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_72_amd as ms
from selective_state_space_72_amd import synth
from gpu_helpers import DEV, TOL, DevInputs, from_dev, log, metric, oracle_scan, to_dev

pytestmark = pytest.mark.gpu


def case(n, dtype, *, batch=2, seqlen=333, d_inner=72, seed=None, base="c3"):
    cfg = dataclasses.replace(synth.CONFIGS[base], d_state=n, dtype=dtype, h0=True, gate=True,
                              batch=batch, seqlen=seqlen, d_inner=d_inner,
                              seed=1000 + n if seed is None else seed)
    return synth.make_scan_inputs(cfg)


def check_fwd(label, inp, **opts):
    log(f"case {label}: batch {inp.cfg.batch} L {inp.cfg.seqlen} D {inp.cfg.d_inner} "
        f"N {inp.cfg.d_state} {inp.dtype} {opts}")
    y, h = DevInputs(inp).run(**opts)
    yr, hr = oracle_scan(inp)
    ey, eh = metric(from_dev(y), yr), metric(from_dev(h), hr)
    log(f"  {label}: y {ey:.2e}, h_last {eh:.2e}")
    assert ey <= TOL[inp.dtype] and eh <= TOL[inp.dtype], (label, ey, eh)
    assert h.shape == (inp.cfg.batch, inp.cfg.d_inner, inp.cfg.d_state)


@pytest.mark.parametrize("n", [1, 3, 5, 12, 24, 40, 63])
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_forward_matches_oracle(n, dtype):
    inp = case(n, dtype)
    check_fwd(f"N={n} auto", inp)
    check_fwd(f"N={n} split", inp, n_spans=3)


@pytest.mark.parametrize("n,kernel", [(12, "scalar"), (12, "rows"), (12, "block"),
                                      (5, "scalar"), (40, "rows"), (63, "block")])
def test_padding_is_exact(n, kernel):
    """The call at d_state n equals, bit for bit, the call at the compiled size on inputs
    padded by hand; the padded states' final values are exactly zero there."""
    inp = case(n, synth.F32, batch=2, seqlen=200, d_inner=130)
    np_ = 4
    while np_ < n:
        np_ *= 2
    di = DevInputs(inp)
    y, h = di.run(kernel=kernel)
    pad_n = lambda t, fill=0.0: torch.nn.functional.pad(t, (0, np_ - n), value=fill)  # noqa: E731
    yp, hp = ms.mamba_scan_fwd(di.u, di.delta, pad_n(di.A, -1.0).contiguous(),
                               pad_n(di.B).contiguous(), pad_n(di.C).contiguous(), D=di.D,
                               z=di.z, delta_bias=di.bias, h0=pad_n(di.h0).contiguous(),
                               return_last_state=True, kernel=kernel)
    torch.cuda.synchronize()
    log(f"N={n} ({kernel}) against N={np_} padded by hand")
    assert torch.equal(y, yp)
    assert torch.equal(h, hp[..., :n])
    assert torch.count_nonzero(hp[..., n:]) == 0


def test_relay_with_padding():
    """The relay's hand-off and its fault word sit behind the padded arrays."""
    B, L, Dn, n = 3, 1000, 200, 12
    inp = case(n, synth.BF16, batch=B, seqlen=L, d_inner=Dn, seed=77)
    di = DevInputs(inp)
    opts = dict(kernel="scalar", n_spans=1)
    need = ms.mamba_scan_fwd_workspace_size(B, L, Dn, n, relay=2, **opts)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    y1, h1 = di.run(relay=1, **opts)
    y2, h2 = di.run(relay=2, workspace=ws, **opts)
    assert ms.mamba_scan_fwd_relay_faults(ws, B, L, Dn, n, relay=2, **opts) == 0
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    yw, hw = di.run(relay=-2, workspace=ws, **opts)
    faults = ms.mamba_scan_fwd_relay_faults(ws, B, L, Dn, n, relay=-2, **opts)
    log(f"relay N={n}: {faults} faults when withheld")
    assert faults == 12 and torch.isnan(hw).all()


# ---- Mamba-3 options --------------------------------------------------------------------

def m3_case(n, *, seqlen=77):
    cfg = dataclasses.replace(synth.CONFIGS["c1"], d_state=n, batch=2, seqlen=seqlen,
                              d_inner=96, gate=True, h0=True, seed=300 + n)
    inp = synth.make_scan_inputs(cfg)
    return inp, synth.make_mamba3_inputs(inp.cfg)


def m3_oracle(inp, m3, *, trap, rot, zoh=False):
    f = lambda a: synth.to_f64(a, inp.dtype)  # noqa: E731
    p = inp.params
    return oracle.load().scan(
        f(inp.u), f(inp.delta), p.A.astype(np.float64), f(inp.B), f(inp.C),
        D=p.D.astype(np.float64), z=f(inp.z), bias=p.bias.astype(np.float64),
        h0=inp.h0.astype(np.float64), zoh=zoh, lam=f(m3.lam) if trap else None,
        u_prev=f(m3.u_prev) if trap else None, B_prev=f(m3.B_prev) if trap else None,
        theta=f(m3.theta) if rot else None)


@pytest.mark.parametrize("n,trap,rot,zoh", [(12, True, True, False), (10, False, True, True),
                                            (5, True, False, False), (7, False, False, True)])
def test_mamba3_options(n, trap, rot, zoh):
    inp, m3 = m3_case(n)
    p = inp.params
    y, h = ms.mamba_scan_fwd(to_dev(inp.u), to_dev(inp.delta), to_dev(p.A), to_dev(inp.B),
                             to_dev(inp.C), D=to_dev(p.D), z=to_dev(inp.z),
                             delta_bias=to_dev(p.bias), h0=to_dev(inp.h0),
                             return_last_state=True,
                             discretization="zoh" if zoh else "euler",
                             lam=to_dev(m3.lam) if trap else None,
                             u_prev=to_dev(m3.u_prev) if trap else None,
                             B_prev=to_dev(m3.B_prev) if trap else None,
                             theta=to_dev(m3.theta) if rot else None)
    torch.cuda.synchronize()
    yr, hr = m3_oracle(inp, m3, trap=trap, rot=rot, zoh=zoh)
    ey, eh = metric(from_dev(y), yr), metric(from_dev(h), hr)
    log(f"N={n} trap {trap} rot {rot} zoh {zoh}: y {ey:.2e}, h_last {eh:.2e}")
    assert ey <= TOL[synth.F32] and eh <= TOL[synth.F32]


def test_rotation_needs_even_d_state():
    inp, m3 = m3_case(5)
    p = inp.params
    with pytest.raises(RuntimeError):
        ms.mamba_scan_fwd(to_dev(inp.u), to_dev(inp.delta), to_dev(p.A), to_dev(inp.B),
                          to_dev(inp.C), theta=to_dev(np.zeros((2, 77, 2), np.float32)))


# ---- decode step ------------------------------------------------------------------------

@pytest.mark.parametrize("n,trap,rot", [(3, False, False), (12, True, True), (40, False, False),
                                        (63, True, False)])
def test_decode_chain(n, trap, rot):
    """Chained decode steps at d_state n against the oracle's scan of the same tokens."""
    inp, m3 = m3_case(n, seqlen=20)
    p = inp.params
    dev = lambda a: to_dev(np.ascontiguousarray(a))  # noqa: E731
    h = to_dev(inp.h0).clone()
    ys = []
    for t in range(20):
        up = m3.u_prev if t == 0 else inp.u[:, t - 1]
        bp = m3.B_prev if t == 0 else inp.B[:, t - 1]
        y = ms.mamba_state_update(h, dev(inp.u[:, t]), dev(inp.delta[:, t]), to_dev(p.A),
                                  dev(inp.B[:, t]), dev(inp.C[:, t]), D=to_dev(p.D),
                                  z=dev(inp.z[:, t]), delta_bias=to_dev(p.bias),
                                  lam=dev(m3.lam[:, t]) if trap else None,
                                  u_prev=dev(up) if trap else None,
                                  B_prev=dev(bp) if trap else None,
                                  theta=dev(m3.theta[:, t]) if rot else None)
        ys.append(from_dev(y))
    torch.cuda.synchronize()
    yr, hr = m3_oracle(inp, m3, trap=trap, rot=rot)
    ey, eh = metric(np.stack(ys, axis=1), yr), metric(from_dev(h), hr)
    log(f"decode chain N={n} trap {trap} rot {rot}: y {ey:.2e}, h {eh:.2e}")
    assert ey <= TOL[synth.F32] and eh <= TOL[synth.F32]


# ---- backward pass ----------------------------------------------------------------------

GRADS = ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dbias", "dh0")


def bwd_oracle(inp, g):
    f = lambda a: synth.to_f64(a, inp.dtype)  # noqa: E731
    p = inp.params
    return oracle.load().scan_bwd(
        f(inp.u), f(inp.delta), p.A.astype(np.float64), f(inp.B), f(inp.C), f(g.dy),
        D=p.D.astype(np.float64), z=f(inp.z), bias=p.bias.astype(np.float64),
        h0=inp.h0.astype(np.float64), dh_last=g.dh_last.astype(np.float64))


@pytest.mark.parametrize("n,dtype,ckpt", [(3, synth.F32, False), (12, synth.F32, False),
                                          (20, synth.BF16, False), (12, synth.BF16, True)])
def test_backward(n, dtype, ckpt):
    inp = case(n, dtype, batch=2, seqlen=150, d_inner=72)
    g = synth.make_upstream_grads(inp.cfg)
    p = inp.params
    args = [to_dev(a) for a in (inp.u, inp.delta, p.A, inp.B, inp.C, g.dy)]
    kw = dict(D=to_dev(p.D), z=to_dev(inp.z), delta_bias=to_dev(p.bias), h0=to_dev(inp.h0),
              dh_last=to_dev(g.dh_last))
    extra = {}
    if ckpt:
        B_, L, D_ = inp.u.shape
        ck = ms.mamba_scan_ckpt_buffer(B_, L, D_, n, DEV)
        ms.mamba_scan_fwd(*args[:5], D=kw["D"], z=kw["z"], delta_bias=kw["delta_bias"],
                          h0=kw["h0"], ckpt=ck)
        extra["ckpt"] = ck
    out = ms.mamba_scan_bwd(*args, **kw, **extra)
    torch.cuda.synchronize()
    ref = bwd_oracle(inp, g)
    worst = {}
    for k in GRADS:
        if out.get(k) is None:
            continue
        assert tuple(out[k].shape) == ref[k].shape, (k, out[k].shape, ref[k].shape)
        worst[k] = metric(from_dev(out[k]), ref[k])
    log(f"backward N={n} {dtype} ckpt {ckpt}: " +
        ", ".join(f"{k} {v:.1e}" for k, v in worst.items()))
    assert max(worst.values()) <= TOL[dtype], worst
