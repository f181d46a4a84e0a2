"""Seeded synthetic workloads for the selective scan.

This module only draws numbers and stores them in the two storage formats the
library accepts (fp32 and bf16).  It holds none of the scan's arithmetic, and it
is the only code shared between the HIP path and the fp64 oracle: both sides are
fed the very same bits.

Recipe (every config):
  * Parameters come from ``numpy.random.default_rng(seed)``, drawn in the order
    A jitter, dt, D.
  * Activations u, delta, z, B, C, h0 (tensor ids 0..5) are standard normal
    draws made directly in float32.  Tensor k is filled in blocks of 2**18
    values; block j is drawn by ``Generator(PCG64(SeedSequence(seed,
    spawn_key=(k, j))))``, so the values do not depend on how many threads fill
    the blocks.  For bf16 configs they are rounded to bf16 with
    round-to-nearest-even and carried as raw ``uint16`` bits.
  * Decode steps use spawn keys (1000 + step, k) for u, delta, z, B, C.
  * Parameters are computed in float64 and rounded once to float32:
      - A[d, n] = -exp(A_log[d, n]) with A_log = log(n + 1) (S4D-real, the
        "A = -exp(A_log)" parameterisation of "Understanding Mamba"
        (aiattnstudio.link), section 5.2), plus N(0, 0.1) jitter where the
        config asks for it;
      - dt bias = inverse softplus of dt, dt log-uniform in [1e-3, 1e-1] (the
        0.001-0.1 initial step range of the hnwysp.cn Mamba slides, section
        4.1): bias = log(expm1(dt));
      - D = 1, or U(0.5, 1.5) where the config asks for it.

Shapes follow the pages' workloads: d_state 16, expand 2 (d_model 768 -> d_inner
1536; d_model 2560 -> d_inner 5120), packed length 4096, 128K-token sequences.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Optional

import numpy as np

BLOCK = 1 << 18
_THREADS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
                      else (os.cpu_count() or 1)))

F32 = "f32"
BF16 = "bf16"


# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    nan = np.isnan(x)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = bits + np.uint32(0x7FFF) + lsb
    out = (rounded >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits (uint16) to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(arr: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    """Exact float64 expansion of a stored array (fp32 values or bf16 bits)."""
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def _store(x_f32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return f32_to_bf16_bits(x_f32)
    return np.ascontiguousarray(x_f32, dtype=np.float32)


# ----------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class ScanConfig:
    name: str
    desc: str
    batch: int
    seqlen: int
    d_inner: int
    d_state: int
    dtype: str
    a_jitter: bool      # A_log = log(n+1) + N(0, 0.1)
    d_uniform: bool     # D ~ U(0.5, 1.5) instead of 1
    gate: bool          # z given
    h0: bool            # nonzero initial state h0 ~ N(0, 1)
    seed: int

    @property
    def chan_steps(self) -> int:
        return self.batch * self.seqlen * self.d_inner

    def min_bytes(self, with_h_last: bool = True) -> int:
        """Each input read once and each output written once, in stored dtype."""
        es = 4 if self.dtype == F32 else 2
        bld = self.batch * self.seqlen * self.d_inner
        bln = self.batch * self.seqlen * self.d_state
        dn = self.d_inner * self.d_state
        bdn = self.batch * dn
        n = bld * es * (2 + (1 if self.gate else 0))      # u, delta, z
        n += 2 * bln * es                                 # B, C
        n += dn * 4 + 2 * self.d_inner * 4                # A, D, bias
        n += bdn * 4 if self.h0 else 0                    # h0
        n += bld * es                                     # y
        n += bdn * 4 if with_h_last else 0                # h_last
        return n


CONFIGS = {
    "c1": ScanConfig("c1", "tiny scan, fp32", 1, 64, 32, 16, F32,
                     a_jitter=False, d_uniform=False, gate=False, h0=False, seed=7201),
    "c2": ScanConfig("c2", "small-model prefill scan", 4, 2048, 1536, 16, BF16,
                     a_jitter=False, d_uniform=False, gate=True, h0=False, seed=7202),
    "c3": ScanConfig("c3", "large-model prefill scan", 8, 4096, 5120, 16, BF16,
                     a_jitter=True, d_uniform=True, gate=True, h0=False, seed=7203),
    "c4": ScanConfig("c4", "long-sequence scan", 1, 131072, 2048, 16, BF16,
                     a_jitter=False, d_uniform=False, gate=False, h0=True, seed=7204),
}

# recurrent decode: persistent state (256, 5120, 16), 1024 chained one-token steps
DECODE = dict(name="c5", batch=256, d_inner=5120, d_state=16, dtype=BF16, steps=1024, seed=7205)


@dataclasses.dataclass
class Params:
    A: np.ndarray       # (D, N) float32
    D: np.ndarray       # (D,) float32
    bias: np.ndarray    # (D,) float32


@dataclasses.dataclass
class ScanInputs:
    cfg: ScanConfig
    params: Params
    u: np.ndarray
    delta: np.ndarray
    z: Optional[np.ndarray]
    B: np.ndarray
    C: np.ndarray
    h0: Optional[np.ndarray]

    @property
    def dtype(self) -> str:
        return self.cfg.dtype


def draw_params(rng: np.random.Generator, d_inner: int, d_state: int,
                a_jitter: bool, d_uniform: bool) -> Params:
    n = np.arange(d_state, dtype=np.float64)
    a_log = np.broadcast_to(np.log(n + 1.0), (d_inner, d_state)).copy()
    if a_jitter:
        a_log += rng.normal(0.0, 0.1, size=(d_inner, d_state))
    A = (-np.exp(a_log)).astype(np.float32)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=d_inner))
    bias = np.log(np.expm1(dt)).astype(np.float32)
    if d_uniform:
        Dv = rng.uniform(0.5, 1.5, size=d_inner).astype(np.float32)
    else:
        Dv = np.ones(d_inner, dtype=np.float32)
    return Params(A=A, D=Dv, bias=bias)


def _normal(seed: int, key: tuple, shape, dtype: str) -> np.ndarray:
    """Standard normal float32 draws for tensor `key`, stored as `dtype`."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == BF16 else np.float32)

    def fill(j):
        lo, hi = j * BLOCK, min(n, (j + 1) * BLOCK)
        ss = np.random.SeedSequence(seed, spawn_key=tuple(key) + (j,))
        g = np.random.Generator(np.random.PCG64(ss))
        x = g.standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = f32_to_bf16_bits(x) if dtype == BF16 else x

    nblocks = (n + BLOCK - 1) // BLOCK
    if nblocks <= 1:
        for j in range(nblocks):
            fill(j)
    else:
        list(_pool().map(fill, range(nblocks)))
    return out.reshape(shape)


_executor = None


def _pool() -> concurrent.futures.ThreadPoolExecutor:
    global _executor
    if _executor is None:
        _executor = concurrent.futures.ThreadPoolExecutor(_THREADS)
    return _executor


def make_scan_inputs(cfg: ScanConfig, *, batch: Optional[int] = None,
                     seqlen: Optional[int] = None, d_inner: Optional[int] = None,
                     seed: Optional[int] = None) -> ScanInputs:
    """Draw one workload.  Shape overrides give smaller cases with the same recipe."""
    if batch is not None or seqlen is not None or d_inner is not None:
        cfg = dataclasses.replace(cfg, batch=batch or cfg.batch,
                                  seqlen=cfg.seqlen if seqlen is None else seqlen,
                                  d_inner=d_inner or cfg.d_inner)
    if seed is not None:
        cfg = dataclasses.replace(cfg, seed=seed)
    rng = np.random.default_rng(cfg.seed)
    p = draw_params(rng, cfg.d_inner, cfg.d_state, cfg.a_jitter, cfg.d_uniform)
    bld = (cfg.batch, cfg.seqlen, cfg.d_inner)
    bln = (cfg.batch, cfg.seqlen, cfg.d_state)
    sd = cfg.seed
    u = _normal(sd, (0,), bld, cfg.dtype)
    delta = _normal(sd, (1,), bld, cfg.dtype)
    z = _normal(sd, (2,), bld, cfg.dtype) if cfg.gate else None
    B = _normal(sd, (3,), bln, cfg.dtype)
    C = _normal(sd, (4,), bln, cfg.dtype)
    h0 = (_normal(sd, (5,), (cfg.batch, cfg.d_inner, cfg.d_state), F32) if cfg.h0 else None)
    return ScanInputs(cfg=cfg, params=p, u=u, delta=delta, z=z, B=B, C=C, h0=h0)


# ----------------------------------------------------------------------------
# recurrent decode
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class DecodeStep:
    u: np.ndarray       # (batch, d_inner)
    delta: np.ndarray   # (batch, d_inner)
    z: np.ndarray       # (batch, d_inner)
    B: np.ndarray       # (batch, d_state)
    C: np.ndarray       # (batch, d_state)


def make_decode_state(batch: int = DECODE["batch"], d_inner: int = DECODE["d_inner"],
                      d_state: int = DECODE["d_state"], seed: int = DECODE["seed"]):
    """Parameters (drawn exactly as the large-model prefill config) and h ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    p = draw_params(rng, d_inner, d_state, a_jitter=True, d_uniform=True)
    h = _normal(seed, (5,), (batch, d_inner, d_state), F32)
    return p, h


def make_decode_step(step: int, batch: int = DECODE["batch"], d_inner: int = DECODE["d_inner"],
                     d_state: int = DECODE["d_state"], dtype: str = DECODE["dtype"],
                     seed: int = DECODE["seed"]) -> DecodeStep:
    """Fresh one-token inputs for one step (spawn keys (1000 + step, k))."""
    bd = (batch, d_inner)
    bn = (batch, d_state)
    k = 1000 + step
    return DecodeStep(u=_normal(seed, (k, 0), bd, dtype), delta=_normal(seed, (k, 1), bd, dtype),
                      z=_normal(seed, (k, 2), bd, dtype), B=_normal(seed, (k, 3), bn, dtype),
                      C=_normal(seed, (k, 4), bn, dtype))


# ----------------------------------------------------------------------------
# causal depthwise conv1d + SiLU (the Mamba block's conv, upstream of the scan)
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class ConvInputs:
    x: np.ndarray                  # (batch, L, d_inner), stored dtype
    w: np.ndarray                  # (d_inner, d_conv) float32
    bias: np.ndarray               # (d_inner,) float32
    state: Optional[np.ndarray]    # (batch, d_inner, d_conv - 1), stored dtype
    dtype: str


def make_conv_inputs(batch: int, seqlen: int, d_inner: int, d_conv: int = 4,
                     dtype: str = BF16, with_state: bool = True, seed: int = 7206) -> ConvInputs:
    """x ~ N(0, 1) like the scan's activations; weights and bias drawn as nn.Conv1d
    initialises them (uniform in +-1/sqrt(fan_in), fan_in = d_conv for a depthwise
    filter), in float64 and rounded once; the carried state ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    bound = 1.0 / np.sqrt(d_conv)
    w = rng.uniform(-bound, bound, size=(d_inner, d_conv)).astype(np.float32)
    bias = rng.uniform(-bound, bound, size=d_inner).astype(np.float32)
    x = _normal(seed, (10,), (batch, seqlen, d_inner), dtype)
    st = _normal(seed, (11,), (batch, d_inner, d_conv - 1), dtype) if with_state else None
    return ConvInputs(x=x, w=w, bias=bias, state=st, dtype=dtype)


def make_conv_step(step: int, batch: int, d_inner: int, dtype: str = BF16,
                   seed: int = 7206) -> np.ndarray:
    """One decode token's x (spawn keys (2000 + step, 10))."""
    return _normal(seed, (2000 + step, 10), (batch, d_inner), dtype)


# ----------------------------------------------------------------------------
# upstream gradients for the backward pass
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class UpstreamGrads:
    dy: np.ndarray                  # (batch, L, d_inner), stored dtype
    dh_last: Optional[np.ndarray]   # (batch, d_inner, d_state) float32


def make_upstream_grads(cfg: ScanConfig, with_dh_last: bool = True) -> UpstreamGrads:
    """dy ~ N(0, 1) in the config's dtype (tensor id 6) and dh_last ~ N(0, 1) float32
    (id 7), drawn like the activations of the same config (pass the config of the
    ScanInputs, which carries any shape overrides)."""
    dy = _normal(cfg.seed, (6,), (cfg.batch, cfg.seqlen, cfg.d_inner), cfg.dtype)
    dhl = (_normal(cfg.seed, (7,), (cfg.batch, cfg.d_inner, cfg.d_state), F32)
           if with_dh_last else None)
    return UpstreamGrads(dy=dy, dh_last=dhl)


# ----------------------------------------------------------------------------
# inputs of the Mamba-3 options (exponential-trapezoidal rule, rotation)
# ----------------------------------------------------------------------------

def _uniform01(seed: int, key: tuple, shape, dtype: str) -> np.ndarray:
    """U(0, 1) float32 draws for tensor `key`, blocked and seeded like _normal."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == BF16 else np.float32)
    for j in range((n + BLOCK - 1) // BLOCK):
        lo, hi = j * BLOCK, min(n, (j + 1) * BLOCK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key) + (j,))))
        x = g.random(hi - lo, dtype=np.float32)
        out[lo:hi] = f32_to_bf16_bits(x) if dtype == BF16 else x
    return out.reshape(shape)


@dataclasses.dataclass
class Mamba3Inputs:
    lam: np.ndarray      # (batch, L, d_inner) stored dtype: trapezoid mixing, U(0, 1)
    theta: np.ndarray    # (batch, L, d_state // 2) stored dtype: rotation rates, N(0, 1)
    u_prev: np.ndarray   # (batch, d_inner) stored dtype: input before t = 0, N(0, 1)
    B_prev: np.ndarray   # (batch, d_state) stored dtype: its B, N(0, 1)


def make_mamba3_inputs(cfg: ScanConfig) -> Mamba3Inputs:
    """Tensor ids 8 (lam), 9 (theta), 10 (u_prev), 11 (B_prev) of the config's seed.  The
    page gives lam in [0, 1] (initial value 0.5) and no scale for theta; theta is drawn
    like the other projections (standard normal), so Delta * theta spans small and large
    angles over the configs' Delta range."""
    sd = cfg.seed
    return Mamba3Inputs(
        lam=_uniform01(sd, (8,), (cfg.batch, cfg.seqlen, cfg.d_inner), cfg.dtype),
        theta=_normal(sd, (9,), (cfg.batch, cfg.seqlen, cfg.d_state // 2), cfg.dtype),
        u_prev=_normal(sd, (10,), (cfg.batch, cfg.d_inner), cfg.dtype),
        B_prev=_normal(sd, (11,), (cfg.batch, cfg.d_state), cfg.dtype))


# ----------------------------------------------------------------------------
# Mamba-2 SSD workloads (scalar A per head, one step size per token and head)
# ----------------------------------------------------------------------------

# large SSD prefill: the large prefill's tokens and channels as 80 heads of 64, d_state 128
# (the Mamba-2 block of "State Space Models and Mamba" uses d_state 128)
SSD_LARGE = dict(batch=8, seqlen=4096, n_heads=80, head_dim=64, d_state=128, dtype=BF16,
                 gate=True, h0=False, seed=7210)


@dataclasses.dataclass
class SsdInputs:
    x: np.ndarray          # (batch, L, H * P) stored dtype
    dt: np.ndarray         # (batch, L, H) stored dtype
    B: np.ndarray          # (batch, L, N)
    C: np.ndarray          # (batch, L, N)
    z: Optional[np.ndarray]
    h0: Optional[np.ndarray]   # (batch, H * P, N) float32
    A: np.ndarray          # (H,) float32
    D: np.ndarray          # (H,) float32
    dt_bias: np.ndarray    # (H,) float32
    head_dim: int
    dtype: str


def make_ssd_inputs(batch: int, seqlen: int, n_heads: int, head_dim: int = 64,
                    d_state: int = 128, dtype: str = BF16, gate: bool = True, h0: bool = False,
                    seed: int = 7210) -> SsdInputs:
    """Activations x, dt, B, C, z ~ N(0, 1) (tensor ids 20..24), h0 ~ N(0, 1) fp32 (25);
    per head: A = -exp(A_log), A_log ~ U(log 1, log 16) (the 1..16 range of the Mamba-1
    recipe's A = -(n + 1)), dt bias = inverse softplus of dt log-uniform in [1e-3, 1e-1],
    D ~ U(0.5, 1.5); drawn in float64 from default_rng(seed) in that order, rounded once."""
    rng = np.random.default_rng(seed)
    A = (-np.exp(rng.uniform(0.0, np.log(16.0), size=n_heads))).astype(np.float32)
    dtv = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=n_heads))
    dt_bias = np.log(np.expm1(dtv)).astype(np.float32)
    D = rng.uniform(0.5, 1.5, size=n_heads).astype(np.float32)
    d_inner = n_heads * head_dim
    x = _normal(seed, (20,), (batch, seqlen, d_inner), dtype)
    dt = _normal(seed, (21,), (batch, seqlen, n_heads), dtype)
    Bm = _normal(seed, (22,), (batch, seqlen, d_state), dtype)
    Cm = _normal(seed, (23,), (batch, seqlen, d_state), dtype)
    z = _normal(seed, (24,), (batch, seqlen, d_inner), dtype) if gate else None
    hz = _normal(seed, (25,), (batch, d_inner, d_state), F32) if h0 else None
    return SsdInputs(x=x, dt=dt, B=Bm, C=Cm, z=z, h0=hz, A=A, D=D, dt_bias=dt_bias,
                     head_dim=head_dim, dtype=dtype)
