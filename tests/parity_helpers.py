"""Shared pieces of the GPU parity tests: moving seeded inputs to the device,
running the oracle on the same inputs, and the comparison rules.

Comparison rules (tolerances are the ones the layer is held to):
  - outputs: relative L2 error |o_gpu - o_ref| / |o_ref| over the compared
    tensor, <= 2e-3 for float32 q/k/v and <= 1e-2 for bfloat16 q/k/v;
  - iteration counts: a token is *decidable* when the oracle's stop decision
    is far from the threshold, i.e. every residual ratio checked before the
    stop is >= tol (1 + EPS) and the ratio that stopped it is < tol (1 - EPS)
    (a token at the cap only needs the first condition).  Decidable tokens
    must match exactly; the others may differ by one step and are counted.
  - a token the oracle solved to a residual ratio below CONVERGED (far below
    float32 resolution) has converged exactly; the float32 path may then see
    r^T r underflow to 0 and stop earlier through the breakdown guard, so its
    count may be anything from 1 up to the oracle's.
"""
from __future__ import annotations

import numpy as np

import oracle
from test_regression_amd import inputs

EPS = 1e-5
CONVERGED = 1e-10
RTOL = {"f32": 2e-3, "bf16": 1e-2}


def torch_mod():
    import torch
    return torch


def to_dev(x, dtype: str):
    """numpy input (float32 or bf16 bit patterns) -> contiguous CUDA tensor."""
    torch = torch_mod()
    if dtype == "bf16" and x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def gpu_forward(x, dtype, max_iters, tol, chunk=64, return_final=False):
    from test_regression_amd import mesa
    torch = torch_mod()
    q, k, v = (to_dev(x[n], dtype) for n in ("q", "k", "v"))
    g = to_dev(x["gamma"], "f32")
    lam = to_dev(x["lam"], "f32")
    out, it, fH, fG = mesa.mesa_forward(q, k, v, g, lam, max_iters, tol, chunk, return_final=return_final)
    torch.cuda.synchronize()
    res = dict(out=out.cpu().numpy().astype(np.float64), iters=it.cpu().numpy())
    if return_final:
        res["final_H"] = fH.cpu().numpy().astype(np.float64)
        res["final_G"] = fG.cpu().numpy().astype(np.float64)
    return res


def oracle_forward(x, dtype, max_iters, tol, want=None, final_state=False):
    q, k, v = (inputs.as_f64(x[n], dtype) for n in ("q", "k", "v"))
    return oracle.forward(q, k, v, x["gamma"], x["lam"], max_iters, tol, want=want,
                          final_state=final_state)


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def decidable(ref, cap: int, tol: float, eps: float = EPS):
    """Boolean mask of tokens whose oracle stop decision is away from tol."""
    it = ref["iters"]
    if tol == 0.0:
        return it >= 0
    rm = ref["rho_min_prev"]
    rs = ref["rho_stop"]
    reason = ref["reason"]
    far_before = rm >= tol * (1 + eps)
    by_tol = (reason == oracle.STOP_TOL) & (rs < tol * (1 - eps)) & far_before
    by_cap = (reason == oracle.STOP_CAP) & (it == cap) & far_before
    qzero = reason == oracle.STOP_Q_ZERO
    return by_tol | by_cap | qzero


def compare_counts(gpu_iters, ref, cap, tol, eps=EPS):
    """Returns (n_decidable, n_undecidable, n_undecidable_mismatch); asserts the rules."""
    it_ref = ref["iters"]
    sel = it_ref >= 0
    conv = sel & (ref["rho_stop"] < CONVERGED) & (it_ref > 0)
    early = conv & (gpu_iters >= 1) & (gpu_iters <= it_ref)
    dmask = decidable(ref, cap, tol, eps) & sel & ~early
    umask = sel & ~dmask & ~early
    bad = dmask & (gpu_iters != it_ref)
    assert not bad.any(), (
        f"{int(bad.sum())} decidable tokens differ; first: gpu={gpu_iters[bad][:5]} ref={it_ref[bad][:5]}")
    diff = np.abs(gpu_iters[umask].astype(np.int64) - it_ref[umask])
    assert (diff <= 1).all(), f"undecidable tokens differ by more than one step: {diff.max()}"
    return int(dmask.sum()), int(umask.sum()), int((diff > 0).sum())
