"""GPU parity of the Mamba-2 SSD scan (chunked, matrix cores) against the fp64 oracle.

The SSD recurrence is the selective scan with the step size and A shared by the channels
of a head, so the reference is the scan oracle on inputs expanded per channel
(tests/ssd_reference.py, pinned against the dual form in tests/test_ssd_reference.py).  Shapes cover
several 64-step chunks with a ragged last chunk, several heads, both compiled d_state
values, h0 and the gate; the large shape in the benchmark's configuration is checked on
sampled heads.  Metric and bounds as for the scan (1e-5 fp32, 2e-2 bf16 inputs).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import selective_state_space_72_amd as ms
from selective_state_space_72_amd import synth
from gpu_helpers import TOL, from_dev, log, metric, to_dev
from ssd_reference import ssd_oracle

pytestmark = pytest.mark.gpu


def run_gpu(s, *, use_D=True, use_bias=True, use_h0=True, relay="auto", n_spans=0):
    y, h = ms.mamba_ssd_fwd(to_dev(s.x), to_dev(s.dt), to_dev(s.A), to_dev(s.B), to_dev(s.C),
                            D=to_dev(s.D) if use_D else None, z=to_dev(s.z),
                            dt_bias=to_dev(s.dt_bias) if use_bias else None,
                            h0=to_dev(s.h0) if use_h0 else None, return_last_state=True,
                            head_dim=s.head_dim, relay=relay, n_spans=n_spans)
    torch.cuda.synchronize()
    return y, h


def run_oracle(s, heads=None, **flags):
    return ssd_oracle(s, heads, **flags)


def check(s, label, **flags):
    log(f"case {label}")
    y, h = run_gpu(s, **flags)
    (yr, hr), _ = run_oracle(s, **flags)
    ey, eh = metric(from_dev(y), yr), metric(from_dev(h), hr)
    log(f"{label}: y {ey:.2e}, h_last {eh:.2e}")
    tol = TOL[s.dtype]
    assert ey <= tol and eh <= tol, (label, ey, eh)


@pytest.mark.parametrize("d_state", [64, 128])
def test_ssd_fp32(d_state):
    s = synth.make_ssd_inputs(2, 200, 3, d_state=d_state, dtype=synth.F32, h0=True)
    check(s, f"ssd fp32 N={d_state}")


@pytest.mark.parametrize("seqlen", [1, 63, 64, 65, 300])
def test_ssd_bf16_lengths(seqlen):
    s = synth.make_ssd_inputs(2, seqlen, 4, d_state=128, dtype=synth.BF16, h0=True)
    check(s, f"ssd bf16 L={seqlen}")


def test_ssd_no_optional_inputs():
    s = synth.make_ssd_inputs(1, 150, 2, d_state=64, dtype=synth.F32, gate=False, h0=False)
    check(s, "ssd fp32, no gate/D/bias/h0", use_D=False, use_bias=False, use_h0=False)


def test_ssd_split_continues_state():
    """Two calls, the second starting from the first's h_last, equal one call."""
    s = synth.make_ssd_inputs(1, 256, 2, d_state=64, dtype=synth.F32, h0=True)
    y, h = run_gpu(s)
    dev = lambda a: to_dev(np.ascontiguousarray(a))  # noqa: E731
    y1, h1 = ms.mamba_ssd_fwd(dev(s.x[:, :100]), dev(s.dt[:, :100]), to_dev(s.A),
                              dev(s.B[:, :100]), dev(s.C[:, :100]), D=to_dev(s.D),
                              z=dev(s.z[:, :100]), dt_bias=to_dev(s.dt_bias), h0=to_dev(s.h0),
                              return_last_state=True)
    y2, h2 = ms.mamba_ssd_fwd(dev(s.x[:, 100:]), dev(s.dt[:, 100:]), to_dev(s.A),
                              dev(s.B[:, 100:]), dev(s.C[:, 100:]), D=to_dev(s.D),
                              z=dev(s.z[:, 100:]), dt_bias=to_dev(s.dt_bias), h0=h1,
                              return_last_state=True)
    torch.cuda.synchronize()
    yy = torch.cat([y1, y2], dim=1)
    assert metric(from_dev(yy), from_dev(y)) <= 1e-5
    assert metric(from_dev(h2), from_dev(h)) <= 1e-5


def test_ssd_unsupported():
    s = synth.make_ssd_inputs(1, 16, 2, head_dim=32, d_state=64, dtype=synth.F32)
    with pytest.raises(ms.MambaError, match="UNSUPPORTED"):
        ms.mamba_ssd_fwd(to_dev(s.x), to_dev(s.dt), to_dev(s.A), to_dev(s.B), to_dev(s.C),
                         head_dim=32)


def test_ssd_large_sampled():
    """8 x 4096 x (80 heads of 64), d_state 128, bf16, in the benchmark's configuration:
    sampled heads (first, middle, last) against the oracle."""
    c = synth.SSD_LARGE
    s = synth.make_ssd_inputs(c["batch"], c["seqlen"], c["n_heads"], c["head_dim"],
                              c["d_state"], c["dtype"], c["gate"], c["h0"], c["seed"])
    y, h = run_gpu(s)
    heads = [0, 37, 79]
    (yr, hr), ch = run_oracle(s, heads)
    chd = torch.from_numpy(ch).to(y.device)
    ey = metric(from_dev(y[:, :, chd].contiguous()), yr)
    eh = metric(from_dev(h[:, chd].contiguous()), hr)
    log(f"ssd large, heads {heads}: y {ey:.2e}, h_last {eh:.2e}")
    assert ey <= TOL[synth.BF16] and eh <= TOL[synth.BF16]


def test_ssd_bf16_d_state_64():
    """bf16 with d_state 64, h0, no gate; 3 x 8 = 24 blocks (a multiple of 8: the blocks
    are renumbered so each XCD takes a contiguous range) and a ragged last chunk."""
    s = synth.make_ssd_inputs(3, 130, 8, d_state=64, dtype=synth.BF16, gate=False, h0=True)
    check(s, "ssd bf16 N=64, 24 blocks")


def test_ssd_fp32_remapped_grid():
    s = synth.make_ssd_inputs(2, 70, 4, d_state=128, dtype=synth.F32, h0=True)
    check(s, "ssd fp32 N=128, 8 blocks")


@pytest.mark.parametrize("dtype,d_state,seqlen,gate,h0", [
    (synth.F32, 64, 200, True, True),      # 4 chunks, ragged last
    (synth.BF16, 128, 130, False, False),  # 3 chunks: parts of 2 and 1
    (synth.BF16, 64, 128, True, True),     # 2 whole chunks: one each
])
def test_ssd_relay_forced(dtype, d_state, seqlen, gate, h0):
    """Every unit in two parts (the second from the middle chunk, continuing from the
    first's final state handed over through the workspace): against the oracle, and
    bitwise equal to the call without relay."""
    s = synth.make_ssd_inputs(2, seqlen, 3, d_state=d_state, dtype=dtype, gate=gate, h0=h0)
    need = ms.mamba_ssd_workspace_size(2, seqlen, 3, 64, d_state, dtype, relay="force")
    assert need == 256 + 6 * 64 * d_state * 4
    label = f"ssd relay forced, {dtype} N={d_state} L={seqlen}"
    log(f"case {label}")
    y, h = run_gpu(s, relay="force", n_spans=1)
    (yr, hr), _ = run_oracle(s)
    ey, eh = metric(from_dev(y), yr), metric(from_dev(h), hr)
    log(f"{label}: y {ey:.2e}, h_last {eh:.2e}")
    assert ey <= TOL[dtype] and eh <= TOL[dtype]
    y0, h0_ = run_gpu(s, relay="off", n_spans=1)
    assert torch.equal(y, y0) and torch.equal(h, h0_)


def test_ssd_relay_mixed_grid():
    """576 units (8 batch rows x 72 heads), 8 chunks: on a device with 512 block slots
    (MI355X, two blocks per compute unit) the 64 units past the full round run in two
    parts beside 512 whole units.  Bitwise equal to the call without relay; sampled heads
    (whole and relayed units) against the oracle."""
    s = synth.make_ssd_inputs(8, 512, 72, d_state=128, dtype=synth.BF16, gate=True, h0=True)
    need = ms.mamba_ssd_workspace_size(8, 512, 72, 64, 128, synth.BF16)
    log(f"ssd 576 units: relay workspace {need} bytes")
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        # 64 flags and the fault word (260 bytes, in 256-byte blocks), 64 states
        assert need == 512 + 64 * 64 * 128 * 4
    y, h = run_gpu(s)
    y0, h0_ = run_gpu(s, relay="off", n_spans=1)
    assert torch.equal(y, y0) and torch.equal(h, h0_)
    heads = [0, 35, 71]  # head 35 and 71 of batch row 7 are relayed units
    (yr, hr), ch = run_oracle(s, heads)
    chd = torch.from_numpy(ch).to(y.device)
    ey = metric(from_dev(y[:, :, chd].contiguous()), yr)
    eh = metric(from_dev(h[:, chd].contiguous()), hr)
    log(f"ssd 576 units, heads {heads}: y {ey:.2e}, h_last {eh:.2e}")
    assert ey <= TOL[synth.BF16] and eh <= TOL[synth.BF16]


def test_ssd_large_relay_equals_unrelayed():
    """The large shape (640 units; relayed on MI355X) equals the unrelayed call bitwise."""
    c = synth.SSD_LARGE
    s = synth.make_ssd_inputs(c["batch"], c["seqlen"], c["n_heads"], c["head_dim"],
                              c["d_state"], c["dtype"], c["gate"], c["h0"], c["seed"])
    need = ms.mamba_ssd_workspace_size(c["batch"], c["seqlen"], c["n_heads"], c["head_dim"],
                                       c["d_state"], c["dtype"])
    log(f"ssd large: relay workspace {need} bytes")
    y, h = run_gpu(s)
    y0, h0_ = run_gpu(s, relay="off", n_spans=1)
    assert torch.equal(y, y0) and torch.equal(h, h0_)


@pytest.mark.parametrize("dtype,d_state,seqlen,n_spans,gate,h0", [
    (synth.F32, 64, 200, 3, True, True),      # 4 chunks: spans of 2, 2
    (synth.F32, 128, 1000, 5, False, True),   # 16 chunks, 4 per span, ragged last chunk
    (synth.BF16, 128, 1000, 4, True, False),
    (synth.BF16, 64, 130, 8, True, True),     # 3 chunks: 3 spans of one
])
def test_ssd_split_forced(dtype, d_state, seqlen, n_spans, gate, h0):
    """The sequence split into spans (span passes from zero, the carry, the output pass
    from each span's true state): against the oracle, and against the unsplit call within
    the same bounds."""
    s = synth.make_ssd_inputs(2, seqlen, 3, d_state=d_state, dtype=dtype, gate=gate, h0=h0)
    label = f"ssd split {n_spans} spans, {dtype} N={d_state} L={seqlen}"
    log(f"case {label}")
    y, h = run_gpu(s, relay="off", n_spans=n_spans)
    (yr, hr), _ = run_oracle(s)
    ey, eh = metric(from_dev(y), yr), metric(from_dev(h), hr)
    y0, h0_ = run_gpu(s, relay="off", n_spans=1)
    e0 = max(metric(from_dev(y), from_dev(y0)), metric(from_dev(h), from_dev(h0_)))
    log(f"{label}: y {ey:.2e}, h_last {eh:.2e}; against unsplit {e0:.2e}")
    assert ey <= TOL[dtype] and eh <= TOL[dtype] and e0 <= TOL[dtype]


def test_ssd_split_one_step_last_span():
    """257 steps in 5 spans of one chunk: the last span holds a single step; no h0, no gate;
    and the same call without the final state (h_last not written)."""
    s = synth.make_ssd_inputs(2, 257, 3, d_state=64, dtype=synth.F32, gate=False, h0=False)
    y, h = run_gpu(s, relay="off", n_spans=5)
    (yr, hr), _ = run_oracle(s)
    ey, eh = metric(from_dev(y), yr), metric(from_dev(h), hr)
    log(f"ssd split, one-step last span: y {ey:.2e}, h_last {eh:.2e}")
    assert ey <= TOL[synth.F32] and eh <= TOL[synth.F32]
    y2, h2 = ms.mamba_ssd_fwd(to_dev(s.x), to_dev(s.dt), to_dev(s.A), to_dev(s.B), to_dev(s.C),
                              D=to_dev(s.D), dt_bias=to_dev(s.dt_bias), relay="off", n_spans=5)
    torch.cuda.synchronize()
    assert h2 is None and torch.equal(y2, y)


def test_ssd_split_auto_few_units():
    """One batch row of 4 heads over 2048 steps: 4 units on a device of 512 block slots
    (MI355X) are split automatically (4 spans of 8 chunks); against the oracle."""
    s = synth.make_ssd_inputs(1, 2048, 4, d_state=128, dtype=synth.BF16, gate=True, h0=True)
    need = ms.mamba_ssd_workspace_size(1, 2048, 4, 64, 128, synth.BF16)
    log(f"ssd 4 units x 2048 steps: workspace {need} bytes")
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert need == 3 * 4 * (64 * 128 + 1) * 4
    y, h = run_gpu(s)
    (yr, hr), _ = run_oracle(s)
    ey, eh = metric(from_dev(y), yr), metric(from_dev(h), hr)
    log(f"ssd 4 units auto split: y {ey:.2e}, h_last {eh:.2e}")
    assert ey <= TOL[synth.BF16] and eh <= TOL[synth.BF16]


def test_ssd_empty_sequence_returns_h0():
    s = synth.make_ssd_inputs(2, 0, 3, d_state=64, dtype=synth.BF16, h0=True)
    y, h = run_gpu(s)
    assert y.shape == (2, 0, 3 * 64)
    assert torch.equal(h.cpu(), torch.from_numpy(s.h0))


# ---- the decode token (mamba_ssd_state_update) ----------------------------------------

def step_gpu(s, t, h, *, use_D=True, use_bias=True, use_z=True):
    """Token t of the inputs s through mamba_ssd_state_update on the device state h."""
    sl = lambda a: to_dev(a[:, t]) if a is not None else None  # noqa: E731
    return ms.mamba_ssd_state_update(h, sl(s.x), sl(s.dt), to_dev(s.A), sl(s.B), sl(s.C),
                                     D=to_dev(s.D) if use_D else None,
                                     z=sl(s.z) if use_z else None,
                                     dt_bias=to_dev(s.dt_bias) if use_bias else None,
                                     head_dim=s.head_dim)


@pytest.mark.parametrize("dtype,d_state,gate,opt", [
    (synth.F32, 64, True, True),
    (synth.F32, 128, False, False),
    (synth.BF16, 128, True, True),
    (synth.BF16, 64, True, False),
])
def test_ssd_step_one_token(dtype, d_state, gate, opt):
    """One token on a nonzero state against the oracle's one-step scan from that state."""
    s = synth.make_ssd_inputs(3, 1, 5, d_state=d_state, dtype=dtype, gate=gate, h0=True)
    h = to_dev(s.h0)
    y = step_gpu(s, 0, h, use_D=opt, use_bias=opt)
    torch.cuda.synchronize()
    (yr, hr), _ = run_oracle(s, use_D=opt, use_bias=opt)
    ey, eh = metric(from_dev(y), yr[:, 0]), metric(from_dev(h), hr)
    log(f"ssd step {dtype} N={d_state} gate={gate} D/bias={opt}: y {ey:.2e}, h {eh:.2e}")
    assert ey <= TOL[dtype] and eh <= TOL[dtype]


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_ssd_step_chain_equals_scan(dtype):
    """200 chained tokens against the oracle's scan of the same 200 steps (every output
    and the final state), and against the chunked scan on the device (same bounds)."""
    L = 200
    s = synth.make_ssd_inputs(2, L, 3, d_state=128, dtype=dtype, gate=True, h0=True)
    h = to_dev(s.h0)
    ys = [step_gpu(s, t, h) for t in range(L)]
    torch.cuda.synchronize()
    y = torch.stack(ys, dim=1)
    (yr, hr), _ = run_oracle(s)
    ey, eh = metric(from_dev(y), yr), metric(from_dev(h), hr)
    yc, hc = run_gpu(s)
    ec = metric(from_dev(y), from_dev(yc))
    log(f"ssd {dtype} 200 chained tokens: y {ey:.2e}, h {eh:.2e}; against the chunked scan "
        f"{ec:.2e}")
    assert ey <= TOL[dtype] and eh <= TOL[dtype] and ec <= TOL[dtype]


def test_ssd_step_large_sampled():
    """The decode shape of the benchmark (64 rows x 80 heads x 64, d_state 128, bf16):
    sampled heads against the oracle."""
    s = synth.make_ssd_inputs(64, 1, 80, d_state=128, dtype=synth.BF16, gate=True, h0=True)
    h = to_dev(s.h0)
    y = step_gpu(s, 0, h)
    torch.cuda.synchronize()
    heads = [0, 41, 79]
    (yr, hr), ch = run_oracle(s, heads)
    chd = torch.from_numpy(ch).to(y.device)
    ey = metric(from_dev(y[:, chd].contiguous()), yr[:, 0])
    eh = metric(from_dev(h[:, chd].contiguous()), hr)
    log(f"ssd step 64 x 80 heads, heads {heads}: y {ey:.2e}, h {eh:.2e}")
    assert ey <= TOL[synth.BF16] and eh <= TOL[synth.BF16]
