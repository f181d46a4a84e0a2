"""GPU parity of the checkpointed training path.

``mamba_scan_fwd(..., ckpt=)`` stores the state entering every 8-step segment of each
(batch row, 64-channel tile); ``mamba_scan_bwd(..., ckpt=)`` (mamba_scan_bwd_ckpt) reads
those states instead of running a forward pass of its own.  Checked here: the stored states
equal the oracle's states at the segment boundaries (oracle runs over the prefixes), and the
gradients computed from them equal the oracle's gradients (metric and bounds of the other
backward tests: 1e-5 fp32, 2e-2 bf16), for unsplit and split sequences on either side, the
relay of the forward, every d_state of the backward, and the large prefill sampled.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_72_amd as ms
from selective_state_space_72_amd import synth
from gpu_helpers import DEV, TOL, from_dev, log, metric, to_dev
from test_gpu_bwd import ALL, compare, make_case, oracle_bwd

pytestmark = pytest.mark.gpu


def fwd_ckpt(inp, **opts):
    p = inp.params
    cfg = inp.cfg
    ck = ms.mamba_scan_ckpt_buffer(cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state, DEV)
    y, h = ms.mamba_scan_fwd(to_dev(inp.u), to_dev(inp.delta), to_dev(p.A), to_dev(inp.B),
                             to_dev(inp.C), D=to_dev(p.D), z=to_dev(inp.z),
                             delta_bias=to_dev(p.bias), h0=to_dev(inp.h0),
                             return_last_state=True, ckpt=ck, **opts)
    return y, h, ck


def bwd_from(inp, grads, ck, n_spans=0, raw=False):
    p = inp.params
    r = ms.mamba_scan_bwd(to_dev(inp.u), to_dev(inp.delta), to_dev(p.A), to_dev(inp.B),
                          to_dev(inp.C), to_dev(grads.dy), D=to_dev(p.D), z=to_dev(inp.z),
                          delta_bias=to_dev(p.bias), h0=to_dev(inp.h0),
                          dh_last=to_dev(grads.dh_last), want=ALL, n_spans=n_spans, ckpt=ck)
    torch.cuda.synchronize()
    if raw:
        return r
    return {k: (from_dev(v) if v is not None else None) for k, v in r.items()}


def check(inp, grads, label, fwd_opts=None, n_spans=0):
    log(f"case {label}: batch {inp.cfg.batch} L {inp.cfg.seqlen} D {inp.cfg.d_inner} "
        f"N {inp.cfg.d_state} {inp.dtype} fwd {fwd_opts or {}} bwd spans {n_spans}")
    y, h, ck = fwd_ckpt(inp, **(fwd_opts or {}))
    out = bwd_from(inp, grads, ck, n_spans=n_spans)
    ref = oracle_bwd(inp, grads)
    names = [n for n in ALL if not (n == "dz" and inp.z is None)]
    compare(out, ref, TOL[inp.dtype], names, label)
    return y, h, ck


def test_ckpt_holds_the_states():
    """Stored states against the oracle's state after 8s steps (prefix runs), every
    segment boundary, two tiles (the second ragged)."""
    inp, g = make_case("c1", batch=2, seqlen=77, d_inner=96, gate=True, h0=True)
    cfg = inp.cfg
    _, _, ck = fwd_ckpt(inp)
    torch.cuda.synchronize()
    N, tiles, nseg = cfg.d_state, (cfg.d_inner + 63) // 64, (cfg.seqlen + 7) // 8
    ckv = from_dev(ck)[:cfg.batch * tiles * nseg * N * 64]
    ckv = ckv.reshape(tiles, cfg.batch, nseg, N, 64)                 # [tile][b][seg][n][lane]
    f = lambda a: synth.to_f64(a, inp.dtype)  # noqa: E731
    p = inp.params
    worst = 0.0
    for s in range(1, nseg):
        t = 8 * s
        _, hr = oracle.load().scan(
            f(inp.u[:, :t]), f(inp.delta[:, :t]), p.A.astype(np.float64), f(inp.B[:, :t]),
            f(inp.C[:, :t]), D=p.D.astype(np.float64), z=f(inp.z[:, :t]),
            bias=p.bias.astype(np.float64), h0=inp.h0.astype(np.float64))
        got = np.transpose(ckv[:, :, s], (1, 0, 3, 2)).reshape(cfg.batch, tiles * 64, N)
        assert np.all(np.isfinite(got))                               # tail lanes too
        worst = max(worst, metric(got[:, :cfg.d_inner], hr))
    log(f"checkpoints vs oracle states: {worst:.2e}")
    assert worst <= TOL[synth.F32]


@pytest.mark.parametrize("d_state", [4, 8, 16, 32])
def test_bwd_from_ckpt_fp32(d_state):
    inp, g = make_case("c1", batch=2, seqlen=70, d_inner=100, d_state=d_state, gate=True,
                       h0=True)
    check(inp, g, f"fp32 N={d_state} from checkpoints")


@pytest.mark.parametrize("fwd_spans,bwd_spans", [(1, 3), (3, 1), (4, 5)])
def test_bwd_from_ckpt_split(fwd_spans, bwd_spans):
    """The forward split into spans (checkpoints written by its full-output pass from the
    carried state) and the backward split independently (a span's state is its first
    checkpoint)."""
    inp, g = make_case("c1", batch=2, seqlen=203, d_inner=96, gate=True, h0=True)
    check(inp, g, f"fp32, forward {fwd_spans} spans, backward {bwd_spans} spans",
          fwd_opts=dict(n_spans=fwd_spans), n_spans=bwd_spans)


def test_bwd_from_ckpt_relay():
    inp, g = make_case("c1", batch=2, seqlen=130, d_inner=130, gate=True, h0=True)
    check(inp, g, "fp32, forward relayed in 3 parts", fwd_opts=dict(relay=3))


def test_bwd_from_ckpt_bf16_auto():
    inp, g = make_case("c3", batch=2, seqlen=300, d_inner=160, h0=True)
    check(inp, g, "bf16 automatic plans")


def test_ckpt_leaves_forward_outputs_unchanged():
    inp, _ = make_case("c1", batch=2, seqlen=100, d_inner=96, gate=True, h0=True)
    y, h, _ = fwd_ckpt(inp)
    p = inp.params
    y0, h0_ = ms.mamba_scan_fwd(to_dev(inp.u), to_dev(inp.delta), to_dev(p.A), to_dev(inp.B),
                                to_dev(inp.C), D=to_dev(p.D), z=to_dev(inp.z),
                                delta_bias=to_dev(p.bias), h0=to_dev(inp.h0),
                                return_last_state=True, kernel="scalar")
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(h, h0_)


def test_bwd_from_ckpt_large_prefill_sampled():
    """The large prefill (8 x 4096 x 5120, bf16) as the benchmark's training step runs it:
    the forward with checkpoints, then the backward from them; per-channel gradients on
    sampled channels against the oracle, and bitwise-close agreement of every gradient
    with the backward that recomputes its own states."""
    cfg = synth.CONFIGS["c3"]
    inp = synth.make_scan_inputs(cfg)
    g = synth.make_upstream_grads(cfg)
    _, _, ck = fwd_ckpt(inp)
    r = bwd_from(inp, g, ck, raw=True)
    ds = np.array([0, 1, 63, 64, 2600, 5056, 5119])
    di = torch.from_numpy(ds).to(DEV)
    sub = {"du": r["du"][:, :, di], "ddelta": r["ddelta"][:, :, di], "dz": r["dz"][:, :, di],
           "dA": r["dA"][di], "dD": r["dD"][di], "dbias": r["dbias"][di],
           "dh0": r["dh0"][:, di]}
    sub = {k: from_dev(v.contiguous()) for k, v in sub.items()}
    ref = oracle_bwd(inp, g, ds=ds)
    compare(sub, ref, TOL[synth.BF16], list(sub), "c3 from checkpoints, sampled channels")
    del ck
    p = inp.params
    own = ms.mamba_scan_bwd(to_dev(inp.u), to_dev(inp.delta), to_dev(p.A), to_dev(inp.B),
                            to_dev(inp.C), to_dev(g.dy), D=to_dev(p.D), z=to_dev(inp.z),
                            delta_bias=to_dev(p.bias), h0=to_dev(inp.h0),
                            dh_last=to_dev(g.dh_last), want=ALL)
    torch.cuda.synchronize()
    for k in ALL:
        m = metric(from_dev(r[k]), from_dev(own[k]))
        log(f"c3 {k}: from checkpoints vs own recomputation {m:.2e}")
        assert m <= TOL[synth.BF16]
