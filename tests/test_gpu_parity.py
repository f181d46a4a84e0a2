"""HIP selective scan and decode step vs the fp64 oracle (needs an MI355X).

Every call goes through the C-ABI library (libmambascan.so) via the binding.
Tolerances (metric in gpu_helpers.metric): 1e-5 for fp32 inputs, 2e-2 for bf16
inputs with the fp32 state; y and the final state are checked the same way.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import (DEV, TOL, DevInputs, from_dev, log, metric, oracle_scan, rms_metric,
                         to_dev)
import oracle
import selective_state_space_72_amd as ms
from selective_state_space_72_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selective_state_space_72_amd import build as hip_build
    hip_build.ensure_built()
    ms.load_library()


def check(name, y, h, yr, hr, dtype):
    ey, eh = metric(y, yr), metric(h, hr)
    log(f"  {name}: y M={ey:.3e} (max/rms {rms_metric(y, yr):.3e}), h_last M={eh:.3e}, "
        f"|y|max/rms={np.max(np.abs(yr)) / max(np.sqrt(np.mean(yr ** 2)), 1e-300):.1f}")
    assert ey <= TOL[dtype], f"{name}: y error {ey:.3e} > {TOL[dtype]}"
    assert eh <= TOL[dtype], f"{name}: h_last error {eh:.3e} > {TOL[dtype]}"


def full_check(name, inp, **kw):
    opts = {k: kw.pop(k) for k in ("chunk_len", "waves", "n_spans", "kernel", "relay",
                                   "discretization") if k in kw}
    if opts.get("discretization") == "zoh":
        kw["zoh"] = True
    log(f"case {name}: batch={inp.cfg.batch} L={inp.cfg.seqlen} D={inp.cfg.d_inner} "
        f"N={inp.cfg.d_state} {inp.dtype} opts={opts} {kw}")
    di = DevInputs(inp)
    y, h = di.run(**{k: v for k, v in kw.items() if k != "zoh"}, **opts)
    yr, hr = oracle_scan(inp, **kw)
    check(name, from_dev(y), from_dev(h), yr, hr, inp.dtype)
    return y, h


# ----------------------------------------------------------------------------
# the configurations
# ----------------------------------------------------------------------------

def test_c1_tiny_fp32():
    inp = synth.make_scan_inputs(synth.CONFIGS["c1"])
    full_check("c1", inp, gate=False)


def test_c2_small_prefill_full():
    inp = synth.make_scan_inputs(synth.CONFIGS["c2"])
    full_check("c2", inp)


def sampled_check(name, cfg, bs, ds, gate):
    log(f"case {name}: full size, sampled channels batch rows {list(bs)} x {len(ds)} channels")
    inp = synth.make_scan_inputs(cfg)
    di = DevInputs(inp)
    y, h = di.run(gate=gate)
    tb, td = torch.as_tensor(bs, device=DEV), torch.as_tensor(ds, device=DEV)
    y = y.index_select(0, tb).index_select(2, td)
    h = h.index_select(0, tb).index_select(1, td)
    del di
    yr, hr = oracle_scan(inp, bs, ds, gate=gate)
    check(name, from_dev(y), from_dev(h), yr, hr, inp.dtype)


def test_c3_large_prefill_full():
    """Every output and final-state element of the large prefill (8 x 4096 x 5120, bf16,
    gated) in the launch configuration the benchmark times, against the threaded oracle."""
    full_check("c3", synth.make_scan_inputs(synth.CONFIGS["c3"]), gate=True)


def test_c4_long_sequence_full():
    """Every element of the long sequence (1 x 131072 x 2048, h0, no gate): split into spans
    joined by the carry pass, as the benchmark runs it."""
    full_check("c4", synth.make_scan_inputs(synth.CONFIGS["c4"]), gate=False)


def test_c3_sampled_rows_and_edges():
    """Channel tile edges and the relayed units' boundary channels of the large prefill."""
    cfg = synth.CONFIGS["c3"]
    rng = np.random.default_rng(1)
    ds = np.unique(np.concatenate([[0, 63, 64, 5119], rng.choice(cfg.d_inner, 44, replace=False)]))
    sampled_check("c3 sampled", cfg, np.array([0, 3, 7]), ds, gate=True)


def test_c5_decode_1024_chained_steps():
    cfg = synth.DECODE
    p, h = synth.make_decode_state()
    rng = np.random.default_rng(3)
    bs = np.array([0, 101, 255])
    ds = np.unique(np.concatenate([[0, 5119], rng.choice(cfg["d_inner"], 30, replace=False)]))
    log(f"case c5: {cfg['steps']} chained steps, state {h.shape}, checking {len(bs)}x{len(ds)}")
    A, D, bias = to_dev(p.A), to_dev(p.D), to_dev(p.bias)
    h_dev = to_dev(h)
    tb, td = torch.as_tensor(bs, device=DEV), torch.as_tensor(ds, device=DEV)
    h_ref = h[bs][:, ds].astype(np.float64)
    orc = oracle.load()
    g = lambda a: synth.to_f64(a, synth.BF16)  # noqa: E731
    y_err = 0.0
    for step in range(cfg["steps"]):
        st = synth.make_decode_step(step)
        y = ms.mamba_state_update(h_dev, to_dev(st.u), to_dev(st.delta), A, to_dev(st.B),
                                  to_dev(st.C), D=D, z=to_dev(st.z), delta_bias=bias)
        sub = lambda a: np.ascontiguousarray(a[bs][:, ds])  # noqa: E731
        yr, h_ref = orc.step(h_ref, g(sub(st.u)), g(sub(st.delta)),
                             p.A[ds].astype(np.float64), g(st.B[bs]), g(st.C[bs]),
                             D=p.D[ds].astype(np.float64), z=g(sub(st.z)),
                             bias=p.bias[ds].astype(np.float64))
        if step % 128 == 0 or step == cfg["steps"] - 1:
            e = metric(from_dev(y.index_select(0, tb).index_select(1, td)), yr)
            y_err = max(y_err, e)
            log(f"  step {step}: y M={e:.3e}")
    torch.cuda.synchronize()
    eh = metric(from_dev(h_dev.index_select(0, tb).index_select(1, td)), h_ref)
    log(f"  c5 final state M={eh:.3e}; worst sampled y M={y_err:.3e}")
    assert y_err <= TOL[synth.BF16]
    assert eh <= TOL[synth.BF16]


# ----------------------------------------------------------------------------
# internal split, chunk and wave settings; edge cases
# ----------------------------------------------------------------------------

VARIANTS = [dict(waves=8, chunk_len=16), dict(waves=8, chunk_len=8), dict(waves=4, chunk_len=16),
            dict(waves=4, chunk_len=32), dict(n_spans=2), dict(n_spans=7), dict(n_spans=64),
            dict(waves=4, chunk_len=16, n_spans=5), dict(kernel="block"), dict(kernel="rows"),
            dict(kernel="rows", n_spans=3), dict(kernel="rows", n_spans=64),
            dict(kernel="scalar"), dict(kernel="scalar", chunk_len=4),
            dict(kernel="scalar", n_spans=5), dict(kernel="scalar", n_spans=64)]


@pytest.mark.parametrize("n_spans", [12, 24, 40])
def test_carry_span_counts(n_spans):
    """Span counts whose carry pass runs 16- and 32-lane segments (the other tests cover 1,
    2, 4, 8 and 64), over 1120 state columns: the last 64-column block of the carry is
    partial, as is the last channel tile."""
    inp = synth.make_scan_inputs(synth.CONFIGS["c3"], batch=1, seqlen=2000, d_inner=70, seed=13)
    inp.h0 = np.random.default_rng(6).standard_normal((1, 70, 16), dtype=np.float32)
    full_check(f"carry n_spans={n_spans}", inp, kernel="scalar", n_spans=n_spans)


@pytest.mark.parametrize("opts", VARIANTS, ids=[str(v) for v in VARIANTS])
def test_variants_agree_with_oracle(opts):
    inp = synth.make_scan_inputs(synth.CONFIGS["c3"], batch=3, seqlen=1000, d_inner=200, seed=11)
    inp.h0 = np.random.default_rng(5).standard_normal((3, 200, 16), dtype=np.float32)
    full_check(f"variant {opts}", inp, **opts)


@pytest.mark.parametrize("kernel", ["block", "rows", "scalar"])
@pytest.mark.parametrize("n", [4, 8, 16, 32, 64])
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_other_state_sizes(n, dtype, kernel):
    if kernel == "scalar" and n == 64:
        pytest.skip("the scalar kernel family has no d_state 64 variant")
    import dataclasses
    cfg = dataclasses.replace(synth.CONFIGS["c3"], d_state=n, dtype=dtype, h0=True)
    inp = synth.make_scan_inputs(cfg, batch=2, seqlen=333, d_inner=72, seed=20 + n)
    full_check(f"N={n} {dtype} {kernel}", inp, kernel=kernel)
    full_check(f"N={n} {dtype} {kernel} split", inp, n_spans=3, kernel=kernel)


@pytest.mark.parametrize("kernel", ["block", "rows", "scalar"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 1, 64), (2, 7, 65), (3, 17, 130),
                                   (1, 4097, 64), (5, 129, 40), (2, 6, 17)])
def test_ragged_shapes_fp32(shape, kernel):
    import dataclasses
    b, L, d = shape
    cfg = dataclasses.replace(synth.CONFIGS["c1"], h0=True, gate=True)
    inp = synth.make_scan_inputs(cfg, batch=b, seqlen=L, d_inner=d, seed=b * 1000 + L + d)
    full_check(f"fp32 {shape} {kernel}", inp, kernel=kernel)
    full_check(f"fp32 {shape} {kernel} no D/bias/h0/z", inp, gate=False, use_D=False,
               use_bias=False, use_h0=False, kernel=kernel)


def test_empty_sequence_returns_h0():
    h0 = torch.randn(2, 64, 16, device=DEV)
    A = -torch.rand(64, 16, device=DEV) - 0.5
    e = torch.empty(2, 0, 64, dtype=torch.bfloat16, device=DEV)
    eb = torch.empty(2, 0, 16, dtype=torch.bfloat16, device=DEV)
    y, h = ms.mamba_scan_fwd(e, e, A, eb, eb, h0=h0, return_last_state=True)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 64) and torch.equal(h, h0)
    y, h = ms.mamba_scan_fwd(e, e, A, eb, eb, return_last_state=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(h) == 0


@pytest.mark.parametrize("kernel", ["block", "rows", "scalar"])
@pytest.mark.parametrize("n_spans", [1, 4])
def test_in_place_state_continuation(n_spans, kernel):
    """h_last may be h0 itself: scanning two halves in place equals one scan."""
    inp = synth.make_scan_inputs(synth.CONFIGS["c4"], batch=1, seqlen=1024, d_inner=128, seed=9)
    di = DevInputs(inp)
    y_full, h_full = di.run(gate=False, n_spans=n_spans, kernel=kernel)
    h = di.h0.clone()
    ys = []
    for lo, hi in ((0, 400), (400, 1024)):
        sl = lambda t: t[:, lo:hi].contiguous()  # noqa: E731
        y, _ = ms.mamba_scan_fwd(sl(di.u), sl(di.delta), di.A, sl(di.B), sl(di.C), D=di.D,
                                 delta_bias=di.bias, h0=h, h_last_out=h, n_spans=n_spans,
                                 kernel=kernel)
        ys.append(y)
    torch.cuda.synchronize()
    y2 = torch.cat(ys, dim=1)
    assert metric(from_dev(y2), from_dev(y_full)) <= 1e-2
    assert metric(from_dev(h), from_dev(h_full)) <= 1e-5


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("parts", [2, 3, 8])
def test_relay_parts_agree_with_oracle(parts, dtype):
    """Units split in time across blocks, each part handing its state to the next."""
    import dataclasses
    # each dtype with its own config's recipe: the fp32 one (A = -(n+1), D = 1) for fp32,
    # the large-prefill one for bf16; gate and h0 on in both
    base = synth.CONFIGS["c1"] if dtype == synth.F32 else synth.CONFIGS["c3"]
    cfg = dataclasses.replace(base, dtype=dtype, h0=True, gate=True)
    inp = synth.make_scan_inputs(cfg, batch=3, seqlen=1001, d_inner=200, seed=30 + parts)
    full_check(f"relay {parts} {dtype}", inp, kernel="scalar", n_spans=1, relay=parts)
    # 17 steps in chunks of 8: parts of 8, 8 and 1 step
    inp = synth.make_scan_inputs(cfg, batch=2, seqlen=17, d_inner=70, seed=40 + parts)
    full_check(f"relay {parts} {dtype} short", inp, kernel="scalar", n_spans=1, relay=parts)


def test_relay_is_bitwise_identical_to_one_block_per_unit():
    inp = synth.make_scan_inputs(synth.CONFIGS["c3"], batch=2, seqlen=640, d_inner=192, seed=5)
    inp.h0 = np.random.default_rng(6).standard_normal((2, 192, 16), dtype=np.float32)
    di = DevInputs(inp)
    y1, h1 = di.run(kernel="scalar", n_spans=1, relay=1)
    for parts in (2, 5):
        y2, h2 = di.run(kernel="scalar", n_spans=1, relay=parts)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(h1, h2), f"relay {parts} differs"


def test_relay_in_place_continuation():
    """h_last == h0 with relay: part 0 reads h0 before the last part overwrites it."""
    inp = synth.make_scan_inputs(synth.CONFIGS["c3"], batch=2, seqlen=512, d_inner=128, seed=8)
    inp.h0 = np.random.default_rng(9).standard_normal((2, 128, 16), dtype=np.float32)
    di = DevInputs(inp)
    y_ref, h_ref = di.run(kernel="scalar", n_spans=1, relay=1)
    h = di.h0.clone()
    y, _ = ms.mamba_scan_fwd(di.u, di.delta, di.A, di.B, di.C, D=di.D, z=di.z,
                             delta_bias=di.bias, h0=h, h_last_out=h, kernel="scalar",
                             n_spans=1, relay=4)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(h, h_ref)


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("opts", [dict(), dict(n_spans=1), dict(n_spans=4), dict(n_spans=1, relay=3),
                                  dict(chunk_len=4)], ids=str)
def test_zoh_agrees_with_oracle(opts, dtype):
    """Zero-order-hold discretisation (Bbar = (exp(Delta A) - 1) / A B)."""
    import dataclasses
    base = synth.CONFIGS["c1"] if dtype == synth.F32 else synth.CONFIGS["c3"]
    cfg = dataclasses.replace(base, dtype=dtype, h0=True, gate=True)
    inp = synth.make_scan_inputs(cfg, batch=2, seqlen=333, d_inner=200, seed=50)
    full_check(f"zoh {opts} {dtype}", inp, discretization="zoh", **opts)


def test_zoh_both_branches_and_zero_A():
    """A spread so that Delta A falls on both sides of the series / decay-factor switch
    (|Delta A| = 1/16), plus exactly zero entries (the Euler limit)."""
    import dataclasses
    cfg = dataclasses.replace(synth.CONFIGS["c1"], h0=True, gate=True)
    inp = synth.make_scan_inputs(cfg, batch=2, seqlen=200, d_inner=72, seed=51)
    rng = np.random.default_rng(52)
    A = -np.exp(rng.uniform(np.log(1e-3), np.log(30.0), size=inp.params.A.shape))
    A[::7, ::5] = 0.0
    inp.params.A = A.astype(np.float32)
    full_check("zoh spread A", inp, discretization="zoh")
    full_check("euler spread A", inp)


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_zoh_decode_steps(dtype):
    """Chained zero-order-hold decode steps against the oracle's, and against the ZOH scan."""
    import dataclasses
    base = synth.CONFIGS["c1"] if dtype == synth.F32 else synth.CONFIGS["c3"]
    cfg = dataclasses.replace(base, dtype=dtype, h0=True, gate=True)
    inp = synth.make_scan_inputs(cfg, batch=3, seqlen=40, d_inner=96, seed=53)
    di = DevInputs(inp)
    y_scan, h_scan = di.run(discretization="zoh")
    yr, hr = oracle_scan(inp, zoh=True)
    h = di.h0.clone()
    ys = []
    for t in range(40):
        y = ms.mamba_state_update(h, di.u[:, t].contiguous(), di.delta[:, t].contiguous(), di.A,
                                  di.B[:, t].contiguous(), di.C[:, t].contiguous(), D=di.D,
                                  z=di.z[:, t].contiguous(), delta_bias=di.bias,
                                  discretization="zoh")
        ys.append(y)
    torch.cuda.synchronize()
    y_dec = torch.stack(ys, dim=1)
    check("zoh decode", from_dev(y_dec), from_dev(h), yr, hr, dtype)
    assert metric(from_dev(y_dec), from_dev(y_scan)) <= TOL[dtype]
    assert metric(from_dev(h), from_dev(h_scan)) <= TOL[dtype]


def test_deterministic():
    inp = synth.make_scan_inputs(synth.CONFIGS["c2"], batch=2, seqlen=700, d_inner=256, seed=4)
    di = DevInputs(inp)
    for opts in (dict(), dict(n_spans=3), dict(kernel="rows"), dict(kernel="rows", n_spans=3),
                 dict(kernel="scalar"), dict(kernel="scalar", n_spans=3)):
        y1, h1 = di.run(**opts)
        y2, h2 = di.run(**opts)
        assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_decode_steps_equal_scan():
    """L chained single-token updates give the scan's outputs and final state."""
    inp = synth.make_scan_inputs(synth.CONFIGS["c3"], batch=2, seqlen=50, d_inner=128, seed=8)
    inp.h0 = np.random.default_rng(6).standard_normal((2, 128, 16), dtype=np.float32)
    di = DevInputs(inp)
    y_scan, h_scan = di.run()
    h = di.h0.clone()
    ys = []
    for t in range(50):
        ys.append(ms.mamba_state_update(h, di.u[:, t].contiguous(), di.delta[:, t].contiguous(),
                                        di.A, di.B[:, t].contiguous(), di.C[:, t].contiguous(),
                                        D=di.D, z=di.z[:, t].contiguous(), delta_bias=di.bias))
    torch.cuda.synchronize()
    y_dec = torch.stack(ys, dim=1)
    # both are fp32 internally; bf16 outputs may differ by a rounding step
    assert metric(from_dev(y_dec), from_dev(y_scan)) <= 1e-2
    assert metric(from_dev(h), from_dev(h_scan)) <= 1e-5
    yr, hr = oracle_scan(inp)
    assert metric(from_dev(y_dec), yr) <= TOL[synth.BF16]
    assert metric(from_dev(h), hr) <= TOL[synth.BF16]


def test_decode_other_sizes_fp32():
    for n in (4, 8, 32, 64):
        p, h = synth.make_decode_state(batch=3, d_inner=80, d_state=n, seed=30 + n)
        st = synth.make_decode_step(0, batch=3, d_inner=80, d_state=n, dtype=synth.F32,
                                    seed=30 + n)
        log(f"case decode N={n} fp32")
        h_dev = to_dev(h)
        y = ms.mamba_state_update(h_dev, to_dev(st.u), to_dev(st.delta), to_dev(p.A),
                                  to_dev(st.B), to_dev(st.C), D=to_dev(p.D), z=to_dev(st.z),
                                  delta_bias=to_dev(p.bias))
        torch.cuda.synchronize()
        f = lambda a: a.astype(np.float64)  # noqa: E731
        yr, hr = oracle.load().step(f(h), f(st.u), f(st.delta), f(p.A), f(st.B), f(st.C),
                                    D=f(p.D), z=f(st.z), bias=f(p.bias))
        assert metric(from_dev(y), yr) <= TOL[synth.F32]
        assert metric(from_dev(h_dev), hr) <= TOL[synth.F32]


def test_step_size_softplus_accuracy():
    """L = 1, h0 = 0, u = B = 1, C = 1/N, no D or gate: y = Delta = softplus(delta + bias),
    so the kernel's softplus is compared directly with the fp64 value over a wide range."""
    n, d = 16, 4096
    delta = np.linspace(-40.0, 40.0, d).astype(np.float32)
    u = torch.ones(1, 1, d, device=DEV)
    dl = torch.from_numpy(delta).view(1, 1, d).to(DEV)
    A = -torch.ones(d, n, device=DEV)
    B = torch.ones(1, 1, n, device=DEV)
    C = torch.full((1, 1, n), 1.0 / n, device=DEV)
    y, _ = ms.mamba_scan_fwd(u, dl, A, B, C)
    torch.cuda.synchronize()
    ref = np.logaddexp(0.0, delta.astype(np.float64))
    rel = np.abs(from_dev(y).ravel() - ref) / ref
    log(f"  softplus: max rel err {rel.max():.3e} at delta={delta[rel.argmax()]:.3f}")
    assert rel.max() < 2e-6


def test_step_size_softplus_accuracy_bf16():
    """bf16 activations take the softplus without the log1p compensation term.  L = 1,
    h0 = 0, u = B = 1: the fp32 final state is h_last[d, n] = Delta exactly, compared with
    the fp64 softplus of the same bf16 delta: absolute error near 1e-7 (the rounding of
    1 + e^-|v| and of v_log_f32), far below the bf16 rounding of delta itself."""
    n, d = 16, 4096
    delta = torch.linspace(-40.0, 40.0, d).to(torch.bfloat16)
    dl = delta.view(1, 1, d).to(DEV)
    u = torch.ones(1, 1, d, device=DEV, dtype=torch.bfloat16)
    A = -torch.ones(d, n, device=DEV)
    B = torch.ones(1, 1, n, device=DEV, dtype=torch.bfloat16)
    C = torch.full((1, 1, n), 1.0 / n, device=DEV, dtype=torch.bfloat16)
    _, h = ms.mamba_scan_fwd(u, dl, A, B, C, return_last_state=True)
    torch.cuda.synchronize()
    ref = np.logaddexp(0.0, delta.float().numpy().astype(np.float64))
    hd = from_dev(h).reshape(d, n).astype(np.float64)
    err = np.abs(hd - ref[:, None])
    assert np.all(hd == hd[:, :1])
    log(f"  bf16 softplus: max abs err {err.max():.3e}, "
        f"max rel err above Delta 1e-3 {(err / ref[:, None])[ref >= 1e-3].max():.3e}")
    assert np.all(err <= 2e-7 + 2e-7 * ref[:, None])


def test_long_fp32_decay_error_growth():
    """u = 0, h0 = 1 over 4096 steps (fp32): y_t = sum_n C exp(A_n S_t); the error of the
    running product of v_exp_f32 values grows with t and is reported per quarter."""
    import dataclasses
    cfg = dataclasses.replace(synth.CONFIGS["c1"], h0=True, seqlen=4096, d_inner=64)
    inp = synth.make_scan_inputs(cfg, seed=77)
    inp.u = np.zeros_like(inp.u)
    inp.h0 = np.ones_like(inp.h0)
    inp.C = np.abs(inp.C)
    di = DevInputs(inp)
    y, h = di.run(gate=False)
    yr, hr = oracle_scan(inp, gate=False)
    yd = from_dev(y)
    for q in range(4):
        sl = slice(q * 1024, (q + 1) * 1024)
        rel = np.max(np.abs(yd[:, sl] - yr[:, sl]) / np.abs(yr[:, sl]).clip(1e-30))
        log(f"  decay t in [{q * 1024}, {(q + 1) * 1024}): max rel err {rel:.3e}")
    e = metric(yd, yr)
    log(f"  decay: y M={e:.3e}")
    assert e <= TOL[synth.F32]
