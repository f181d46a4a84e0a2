"""A relay hand-off that never arrives is reported, not silently wrong.

The relay splits a (batch row, channel tile) unit -- or, for the SSD, a (batch row, head)
unit -- in time across two blocks, the second continuing from the first's final state (the
carry of the segment scan, "Mamba slides" section 3.2).  The wait for that state is bounded.
The failure test (relay = -2) makes every first part withhold its hand-off from the host
side, so every second part's wait gives up after a short bound; every kernel still exits
normally.  The tests check that the give-ups are counted in the workspace, that the parts
that lost their state produce NaN (and so does the final state), that the first parts are
untouched, and that the next normal call on the same workspace reports no fault again.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import selective_state_space_72_amd as ms
from selective_state_space_72_amd import synth
from gpu_helpers import DEV, DevInputs, log, to_dev

pytestmark = pytest.mark.gpu


def test_scan_relay_give_up_is_counted_and_poisons_outputs():
    B, L, Dn, N = 3, 1000, 200, 16  # 3 x 4 channel tiles = 12 units, all relayed in 2 parts
    log(f"relay fault: scan {B}x{L}x{Dn}")
    inp = synth.make_scan_inputs(synth.CONFIGS["c3"], batch=B, seqlen=L, d_inner=Dn, seed=61)
    inp.h0 = np.random.default_rng(62).standard_normal((B, Dn, N), dtype=np.float32)
    di = DevInputs(inp)
    opts = dict(kernel="scalar", n_spans=1)
    need = ms.mamba_scan_fwd_workspace_size(B, L, Dn, N, relay=2, **opts)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)

    y_ref, h_ref = di.run(**opts, relay=1)
    y2, h2 = di.run(**opts, relay=2, workspace=ws)
    assert ms.mamba_scan_fwd_relay_faults(ws, B, L, Dn, N, relay=2, **opts) == 0
    assert torch.equal(y2, y_ref) and torch.equal(h2, h_ref)

    yw, hw = di.run(**opts, relay=-2, workspace=ws)
    faults = ms.mamba_scan_fwd_relay_faults(ws, B, L, Dn, N, relay=-2, **opts)
    log(f"  withheld hand-offs: {faults} faults")
    assert faults == 12
    # the parts are whole 8-step chunks: 1000 / 2 -> 504 steps in the first part
    mid = 504
    assert torch.equal(yw[:, :mid], y_ref[:, :mid]), "first parts must be unaffected"
    assert torch.isnan(yw[:, mid:].float()).all(), "second parts must be NaN"
    assert torch.isnan(hw).all(), "final states must be NaN"

    # the next normal call clears the fault word and is exact again
    y3, h3 = di.run(**opts, relay=2, workspace=ws)
    assert ms.mamba_scan_fwd_relay_faults(ws, B, L, Dn, N, relay=2, **opts) == 0
    assert torch.equal(y3, y_ref) and torch.equal(h3, h_ref)


def test_scan_without_relay_reports_no_fault():
    # no relay planned: nothing can time out and no workspace word is read
    assert ms.mamba_scan_fwd_relay_faults(None, 3, 1000, 200, 16, kernel="scalar", n_spans=1,
                                          relay=1, device=DEV) == 0


def test_ssd_relay_give_up_is_counted_and_poisons_outputs():
    b, L, H, P, N = 2, 256, 4, 64, 128  # 8 units, all relayed; second parts from step 128
    log(f"relay fault: ssd {b}x{L}, {H} heads x {P}, N {N}")
    s = synth.make_ssd_inputs(b, L, H, P, N, synth.BF16, gate=True, h0=True, seed=63)
    args = [to_dev(a) for a in (s.x, s.dt, s.A, s.B, s.C)]
    kw = dict(D=to_dev(s.D), z=to_dev(s.z), dt_bias=to_dev(s.dt_bias), h0=to_dev(s.h0),
              return_last_state=True, head_dim=P)
    need = ms.mamba_ssd_workspace_size(b, L, H, P, N, torch.bfloat16, relay="force", n_spans=1)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)

    y_ref, h_ref = ms.mamba_ssd_fwd(*args, **kw, relay="off", n_spans=1)
    y2, h2 = ms.mamba_ssd_fwd(*args, **kw, relay="force", n_spans=1, workspace=ws)
    assert ms.mamba_ssd_relay_faults(ws, b, L, H, P, N, torch.bfloat16, relay="force",
                                     n_spans=1) == 0
    assert torch.equal(y2, y_ref) and torch.equal(h2, h_ref)

    yw, hw = ms.mamba_ssd_fwd(*args, **kw, relay="force_withheld", n_spans=1, workspace=ws)
    faults = ms.mamba_ssd_relay_faults(ws, b, L, H, P, N, torch.bfloat16,
                                       relay="force_withheld", n_spans=1)
    log(f"  withheld hand-offs: {faults} faults")
    assert faults == 8
    mid = 128
    assert torch.equal(yw[:, :mid], y_ref[:, :mid]), "first parts must be unaffected"
    assert torch.isnan(yw[:, mid:].float()).all(), "second parts must be NaN"
    assert torch.isnan(hw).all(), "final states must be NaN"

    y3, h3 = ms.mamba_ssd_fwd(*args, **kw, relay="force", n_spans=1, workspace=ws)
    assert ms.mamba_ssd_relay_faults(ws, b, L, H, P, N, torch.bfloat16, relay="force",
                                     n_spans=1) == 0
    assert torch.equal(y3, y_ref) and torch.equal(h3, h_ref)
