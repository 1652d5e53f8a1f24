"""Seeded synthetic inputs for the Mesa layer (forward and decode).

This module only draws random numbers and lays them out.  It holds none of
the layer's arithmetic, so both the GPU path's tests/bench and the fp64
oracle can take their inputs from here.

Workload laws follow the MesaNet summary page (gist.science, paper
2506.05233), section "A Camada Mesa": queries/keys arrive already
normalised (section "Arquitetura (MesaNet)", bullet on pre-processing), values
are unconstrained, the forget gate gamma in (0, 1] and the regulariser Lambda
is symmetric positive definite (taken diagonal here).

Layout (row-major, contiguous):
  q, k : [B, H, T, d]     v : [B, H, T, d]
  gamma: [B, H, T] float32
  lam  : [H, d]    float32
bf16 tensors are carried as uint16 bit patterns (round-to-nearest-even from
float32), so that the exact stored value is known on the host.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "forward_inputs", "decode_lambda", "decode_prefix", "decode_steps",
    "decode_queries_windowed", "DecodeDeviceStream", "bf16_bits", "bf16_bits_to_f32", "as_f64",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtypes and the laws of every input."""
    name: str
    B: int                 # batch (decode: sequences N)
    H: int                 # heads
    T: int                 # tokens (decode: prefix length)
    d: int                 # d_k = d_v
    chunk: int
    dtype: str             # storage dtype of q, k, v: "f32" or "bf16"
    gamma_lo: float        # gamma ~ U[gamma_lo, 1)
    lam_law: str           # "const", "uniform" or "loguniform"
    lam_a: float
    lam_b: float
    max_iters: int
    tol: float
    seed: int
    steps: int = 0         # decode steps (decode workloads only)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_f32_d16_T256", 1, 1, 256, 16, 64, "f32", 0.9,
                 "const", 1.0, 1.0, 10, 0.0, 1000),
        Workload("mid_bf16_d64_T2048", 2, 4, 2048, 64, 64, "bf16", 0.95,
                 "uniform", 0.5, 2.0, 15, 0.0, 1001),
        Workload("layer_bf16_d128_T4096_k30", 8, 16, 4096, 128, 64, "bf16", 0.97,
                 "uniform", 0.5, 2.0, 30, 0.0, 1002),
        Workload("dynamic_f32_d128_T8192_tol1e-4", 4, 16, 8192, 128, 64, "f32", 0.99,
                 "loguniform", 0.25, 4.0, 30, 1e-4, 1003),
        Workload("decode_f32_d128_N256_prefix4096", 256, 16, 4096, 128, 64, "f32", 0.97,
                 "uniform", 0.5, 2.0, 30, 1e-4, 1004, steps=1024),
    ]
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> the exact float32 values they encode."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """The exact stored value of a q/k/v array as float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _unit_rows(rng: np.random.Generator, shape) -> np.ndarray:
    """Gaussian rows scaled to unit L2 norm over the last axis (float64)."""
    x = rng.standard_normal(shape)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    n[n == 0] = 1.0
    return x / n


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return bf16_bits(x32) if dtype == "bf16" else x32


def _lam(rng: np.random.Generator, H: int, d: int, law: str, a: float, b: float) -> np.ndarray:
    if law == "const":
        return np.full((H, d), a, dtype=np.float32)
    if law == "uniform":
        return rng.uniform(a, b, size=(H, d)).astype(np.float32)
    if law == "loguniform":
        return np.exp(rng.uniform(np.log(a), np.log(b), size=(H, d))).astype(np.float32)
    raise ValueError(f"unknown lambda law {law!r}")


def forward_inputs(w: Workload, B=None, H=None, T=None, seed=None):
    """Inputs of a forward workload (optionally with overridden sizes).

    Draw order from one PCG64 stream: q, k, v, gamma, lambda.
    Returns dict(q, k, v, gamma, lam) with q/k/v in the storage dtype.
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    T = w.T if T is None else T
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    shape = (B, H, T, w.d)
    q = _store(_unit_rows(rng, shape), w.dtype)
    k = _store(_unit_rows(rng, shape), w.dtype)
    v = _store(rng.standard_normal(shape), w.dtype)
    gamma = rng.uniform(w.gamma_lo, 1.0, size=(B, H, T)).astype(np.float32)
    lam = _lam(rng, H, w.d, w.lam_law, w.lam_a, w.lam_b)
    return dict(q=q, k=k, v=v, gamma=gamma, lam=lam)


def decode_lambda(w: Workload, H=None) -> np.ndarray:
    """Per-head regulariser of a decode workload ([H, d] float32)."""
    H = w.H if H is None else H
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 0x1A])))
    return _lam(rng, H, w.d, w.lam_law, w.lam_a, w.lam_b)


def decode_prefix(w: Workload, n: int, h: int, prefix: int = None):
    """Prefix tokens of one decode head (n, h): dict(k [P,d], v [P,d], gamma [P]).

    Each head has its own stream (SeedSequence([seed, n, h])), so any subset
    of heads can be drawn alone.  Draw order: k, v, gamma.  Keys are unit
    Gaussian rows, values N(0, 1), gamma ~ U[gamma_lo, 1); all float32.
    """
    P = w.T if prefix is None else prefix
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, n, h])))
    k = _unit_rows(rng, (P, w.d)).astype(np.float32)
    v = rng.standard_normal((P, w.d)).astype(np.float32)
    g = rng.uniform(w.gamma_lo, 1.0, size=P).astype(np.float32)
    return dict(k=k, v=v, gamma=g)


def decode_steps(w: Workload, steps: int, N: int = None, H: int = None, stream: int = 0):
    """Per-step decode inputs for N x H heads from one stream.

    Returns dict(q, k [steps,N,H,d] unit Gaussian rows, v [steps,N,H,d]
    N(0, 1), gamma [steps,N,H] U[gamma_lo, 1)); all float32.  Draw order:
    q, k, v, gamma.
    """
    N = w.B if N is None else N
    H = w.H if H is None else H
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 0x57E9, stream])))
    shape = (steps, N, H, w.d)
    q = _unit_rows(rng, shape).astype(np.float32)
    k = _unit_rows(rng, shape).astype(np.float32)
    v = rng.standard_normal(shape).astype(np.float32)
    g = rng.uniform(w.gamma_lo, 1.0, size=(steps, N, H)).astype(np.float32)
    return dict(q=q, k=k, v=v, gamma=g)


def decode_queries_windowed(w: Workload, steps: int, window: int, N: int = None, H: int = None,
                            stream: int = 0):
    """Decode queries [steps,N,H,d] whose neighbours overlap: each is the
    unit-normalised sum of `window` consecutive i.i.d. N(0, 1) rows, the way a
    short causal convolution over the token axis mixes neighbouring inputs
    before the layer.  Consecutive queries then share window - 1 of their
    terms.  window = 1 gives independent unit Gaussian rows.  float32.
    """
    N = w.B if N is None else N
    H = w.H if H is None else H
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 0xC0E, window, stream])))
    z = rng.standard_normal((steps + window - 1, N, H, w.d))
    s = np.zeros((steps, N, H, w.d))
    for j in range(window):
        s += z[j:j + steps]
    return (s / np.linalg.norm(s, axis=-1, keepdims=True)).astype(np.float32)


def preprocess_inputs(B: int, H: int, T: int, d: int, W: int, dtype: str, seed: int, with_hist: bool = False):
    """Raw (not yet normalised) query or key rows for the pre-processing step.

    x [B,H,T,d]: N(0, 1) rows, each scaled by a factor drawn from U(0.5, 2) so
    that row norms differ; conv_w [H,W,d] float32 ~ N(0, 1/W); hist
    [B,H,W-1,d] N(0, 1) rows (or None).  x and hist in the storage dtype.
    Draw order: x, row scales, conv_w, hist.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((B, H, T, d)) * rng.uniform(0.5, 2.0, (B, H, T, 1))
    w = (rng.standard_normal((H, W, d)) / np.sqrt(W)).astype(np.float32)
    hist = rng.standard_normal((B, H, W - 1, d)) if with_hist else None
    return dict(x=_store(x, dtype), w=w, hist=None if hist is None else _store(hist, dtype))


def hawk_inputs(B: int, T: int, D: int, dtype: str, seed: int, c: float = 8.0, with_h0: bool = False):
    """Inputs of the Hawk layer's recurrence: x, ga, gx [B,T,D] ~ N(0, 1) in the
    storage dtype; lam [D] float32 with sigmoid(lam)^c ~ U(0.9, 0.999) (slow to
    moderate decays); h0 [B,D] N(0, 1) or None.  Draw order: x, ga, gx, lam, h0.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((B, T, D))
    ga = rng.standard_normal((B, T, D))
    gx = rng.standard_normal((B, T, D))
    s = rng.uniform(0.9, 0.999, size=D) ** (1.0 / c)
    lam = np.log(s / (1.0 - s)).astype(np.float32)
    h0 = rng.standard_normal((B, D)).astype(np.float32) if with_h0 else None
    return dict(x=_store(x, dtype), ga=_store(ga, dtype), gx=_store(gx, dtype), lam=lam, h0=h0)


class DecodeDeviceStream:
    """The decode workload drawn on the device from one seeded torch generator,
    for sizes too large to draw on the host (256 x 16 heads with 4096-token
    prefixes are 4.3 G normals).  Same laws as decode_prefix / decode_steps:
    unit Gaussian key and query rows, N(0, 1) values, gamma ~ U[gamma_lo, 1).

    Draw order: the prefix tokens of `batch` sequences at a time (keys,
    values, gammas [nb, H, P]), then the per-step inputs of all steps
    (queries, keys, values [S, N, H, d], gammas [S, N, H]), then the
    i.i.d. rows of the windowed queries.  Callers draw in that order, so a
    test and the benchmark that follow it see the same numbers.
    """

    def __init__(self, torch, w: Workload, dev):
        self.torch, self.w, self.dev = torch, w, dev
        self.g = torch.Generator(device=dev)
        self.g.manual_seed(w.seed)

    def _unit(self, shape):
        x = self.torch.randn(shape, generator=self.g, device=self.dev)
        return x / x.norm(dim=-1, keepdim=True)

    def _gamma(self, shape):
        lo = self.w.gamma_lo
        return lo + (1 - lo) * self.torch.rand(shape, generator=self.g, device=self.dev)

    def prefix_batches(self, batch: int = 64):
        """Yields (n0, k, v, gamma) for sequences n0 .. n0 + nb - 1 of the
        prefix ([nb, H, P, d] float32 and [nb, H, P])."""
        w = self.w
        for n0 in range(0, w.B, batch):
            nb = min(batch, w.B - n0)
            k = self._unit((nb, w.H, w.T, w.d))
            v = self.torch.randn((nb, w.H, w.T, w.d), generator=self.g, device=self.dev)
            yield n0, k, v, self._gamma((nb, w.H, w.T))

    def steps(self, S: int):
        """Per-step inputs of S steps: (q, k, v [S, N, H, d], gamma [S, N, H])."""
        w = self.w
        q = self._unit((S, w.B, w.H, w.d))
        k = self._unit((S, w.B, w.H, w.d))
        v = self.torch.randn((S, w.B, w.H, w.d), generator=self.g, device=self.dev)
        return q, k, v, self._gamma((S, w.B, w.H))

    def windowed_queries(self, S: int, window: int = 4):
        """Queries [S, N, H, d], each the unit-normalised sum of `window`
        consecutive i.i.d. N(0, 1) rows (see decode_queries_windowed)."""
        w = self.w
        z = self.torch.randn((S + window - 1, w.B, w.H, w.d), generator=self.g, device=self.dev)
        s = z[0:S].clone()
        for j in range(1, window):
            s += z[j:j + S]
        return s / s.norm(dim=-1, keepdim=True)
