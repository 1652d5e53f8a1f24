"""GPU parity of the backward pass (mesa_forward_train + mesa_backward)
against the fp64 oracle's backward.

The page says the layer trains in parallel but gives no gradient (MesaNet
summary, section "A Camada Mesa", bullet "Paralelizacao"); the reading is
implicit differentiation with a k-step adjoint CG (oracle/mesa_oracle.c,
oracle_backward).  Each gradient (q, k, v, gamma, lambda) must match within
relative L2 2e-3 for float32 q/k/v and 1e-2 for bfloat16; adjoint iteration
counts follow the forward's rule (exact for decidable tokens).
"""
import sys

import numpy as np
import pytest

import oracle
from test_regression_amd import inputs
from tests.parity_helpers import RTOL, compare_counts, rel_l2, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dgamma", "dlam")
GPU_NAMES = dict(dq="grad_q", dk="grad_k", dv="grad_v", dgamma="grad_gamma", dlam="grad_lambda")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small_inputs(seed, B, H, T, d, dtype, glo=0.9):
    w = inputs.Workload("t", B, H, T, d, 64, dtype, glo, "uniform", 0.5, 2.0, 0, 0.0, seed)
    x = inputs.forward_inputs(w)
    x["gout"] = np.random.default_rng(seed + 7).standard_normal((B, H, T, d)).astype(np.float32)
    return x


def gpu_backward(x, dtype, max_iters, tol, chunk):
    import torch
    from test_regression_amd import mesa
    q, k, v = (to_dev(x[n], dtype) for n in ("q", "k", "v"))
    g, lam, gout = to_dev(x["gamma"], "f32"), to_dev(x["lam"], "f32"), to_dev(x["gout"], "f32")
    out, _, xs = mesa.mesa_forward_train(q, k, v, g, lam, max_iters, tol, chunk)
    r = mesa.mesa_backward(k, v, g, lam, xs, out, gout, max_iters, tol, chunk)
    torch.cuda.synchronize()
    res = {n: r[GPU_NAMES[n]].cpu().numpy().astype(np.float64) for n in NAMES}
    res["z_iters"] = r["z_iters"].cpu().numpy()
    return res


def oracle_backward(x, dtype, max_iters, tol, heads=None):
    q, k, v = (inputs.as_f64(x[n], dtype) for n in ("q", "k", "v"))
    g, lam, gout = x["gamma"], x["lam"], x["gout"]
    if heads is not None:
        b, h = heads
        q, k, v, g, gout = (a[b:b + 1, h:h + 1] for a in (q, k, v, g, gout))
        lam = lam[h:h + 1]
    return oracle.backward(q, k, v, g, lam, gout, max_iters, tol)


def check(gpu, ref, dtype, max_iters, tol, what=""):
    # gamma at a sequence's first token has no effect: its gradient is exactly
    # zero, reached on the GPU as the difference of two equal fp32 totals, so
    # it is held to an absolute bound and left out of the relative error.
    g0 = np.abs(gpu["dgamma"][:, :, 0]).max()
    assert g0 <= 1e-4 * (1.0 + np.abs(ref["dgamma"]).max()), g0
    errs = {}
    for n in NAMES:
        if n == "dgamma":
            if gpu[n].shape[2] > 1:
                errs[n] = rel_l2(gpu[n][:, :, 1:], ref[n][:, :, 1:])
        else:
            errs[n] = rel_l2(gpu[n], ref[n])
    say(f"  {what} " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= RTOL[dtype], (n, e)
    zref = dict(iters=ref["z_iters"], rho_stop=ref["z_rho_stop"], rho_min_prev=ref["z_rho_min_prev"],
                reason=ref["z_reason"])
    compare_counts(gpu["z_iters"], zref, max_iters, tol)


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_dims_chunks_dtypes(d, chunk, dtype):
    B, H = 1, 2
    T = 3 * chunk + chunk // 2 + 3
    seed = 5000 + d + chunk
    say("case backward", dict(d=d, chunk=chunk, dtype=dtype, B=B, H=H, T=T, seed=seed))
    x = small_inputs(seed, B, H, T, d, dtype)
    for max_iters, tol in ((8, 0.0), (30, 1e-4)):
        gpu = gpu_backward(x, dtype, max_iters, tol, chunk)
        ref = oracle_backward(x, dtype, max_iters, tol)
        check(gpu, ref, dtype, max_iters, tol, f"k={max_iters} tol={tol}")


@pytest.mark.parametrize("case", ["small_keys", "large_keys", "strong_decay"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_far_from_unit_and_strong_decay(dtype, d, case):
    """Keys, queries, values and lambda scaled by powers of two far from 1
    (keys x sk with lambda x sk^2: the fp16 split products and the stored
    fp16 reverse states rescale each group by its own exponent), and
    gamma ~ U(0.5, 1), whose decays span many orders of magnitude."""
    B, H, T = 1, 2, 150
    say("case backward", case, dtype, d)
    x = small_inputs(5400 + d, B, H, T, d, "f32", glo=0.5 if case == "strong_decay" else 0.9)
    if case != "strong_decay":
        sk, sq, sv = (2.0 ** -10, 2.0 ** -20, 2.0 ** 15) if case == "small_keys" else (2.0 ** 10, 2.0 ** 8, 2.0 ** -12)
        x["k"] = x["k"] * np.float32(sk)
        x["q"] = x["q"] * np.float32(sq)
        x["v"] = x["v"] * np.float32(sv)
        x["lam"] = (x["lam"] * np.float32(sk * sk)).astype(np.float32)
    if dtype == "bf16":
        x = {n: (inputs.bf16_bits(x[n]) if n in ("q", "k", "v") else x[n]) for n in x}
    for max_iters, tol in ((8, 0.0), (30, 1e-4)):
        gpu = gpu_backward(x, dtype, max_iters, tol, 64)
        ref = oracle_backward(x, dtype, max_iters, tol)
        check(gpu, ref, dtype, max_iters, tol, f"{case} k={max_iters} tol={tol}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_edge_cases(dtype):
    """bf16 runs the split-product adjoint kernel, chunk 16 its masked second
    key block."""
    import torch
    from test_regression_amd import mesa
    d = 32
    for chunk in (16, 64):
        for T in (1, 5, 64, 65):
            say("case backward edge", dtype, "chunk", chunk, "T", T)
            x = small_inputs(5200 + T, 2, 1, T, d, dtype)
            gpu = gpu_backward(x, dtype, 10, 0.0, chunk)
            ref = oracle_backward(x, dtype, 10, 0.0)
            check(gpu, ref, dtype, 10, 0.0, f"chunk={chunk} T={T}")
    chunk = 64
    say("case backward zero grad_out and max_iters=0")
    x = small_inputs(5300, 1, 2, 70, d, dtype)
    x["gout"][:] = 0.0
    gpu = gpu_backward(x, dtype, 10, 0.0, chunk)
    assert all(not gpu[n].any() for n in NAMES)
    x = small_inputs(5301, 1, 2, 70, d, dtype)
    gpu = gpu_backward(x, dtype, 0, 0.0, chunk)
    assert all(not gpu[n].any() for n in NAMES)
    say("case backward T=0")
    lam = torch.ones((2, d), dtype=torch.float32, device="cuda")
    e = torch.empty((1, 2, 0, d), dtype=torch.float32, device="cuda")
    g0 = torch.empty((1, 2, 0), dtype=torch.float32, device="cuda")
    r = mesa.mesa_backward(e, e, g0, lam, e, e, e, 10, 0.0, 64)
    torch.cuda.synchronize()
    assert not r["grad_lambda"].any()


@pytest.mark.timeout(600)
def test_backward_layer_shape_full():
    """The headline layer (8 x 16 x 4096, d=128, bf16, k=30) backward at full
    size against the oracle on every head: dq, dk, dv, dgamma per head and
    dlambda, which sums each head over the batch, compared whole."""
    w = inputs.WORKLOADS["layer_bf16_d128_T4096_k30"]
    say("case backward layer", w.name)
    x = inputs.forward_inputs(w)
    x["gout"] = np.random.default_rng(w.seed + 9).standard_normal((w.B, w.H, w.T, w.d)).astype(np.float32)
    gpu = gpu_backward(x, w.dtype, w.max_iters, w.tol, w.chunk)
    say("  gpu done, oracle on all heads")
    ref = oracle_backward(x, w.dtype, w.max_iters, w.tol)
    errs = {n: rel_l2(gpu[n], ref[n]) for n in ("dq", "dk", "dv", "dlam")}
    errs["dgamma"] = rel_l2(gpu["dgamma"][:, :, 1:], ref["dgamma"][:, :, 1:])
    worst = {n: max(rel_l2(gpu[n][:, h], ref[n][:, h]) for h in range(w.H)) for n in ("dq", "dk", "dv")}
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items())
        + " | worst head " + " ".join(f"{n}={e:.2e}" for n, e in worst.items()))
    for n, e in errs.items():
        assert e <= RTOL[w.dtype], (n, e)
    g0 = np.abs(gpu["dgamma"][:, :, 0]).max()
    assert g0 <= 1e-4 * (1.0 + np.abs(ref["dgamma"]).max()), g0
    assert (gpu["z_iters"] == w.max_iters).all() and (ref["z_iters"] == w.max_iters).all()


def test_backward_garbage_workspace_and_reuse():
    """The adjoint kernel's chunk-claim counter lives in the backward
    workspace tail and is reset by the library: garbage in the workspace,
    reused for a second call, changes nothing."""
    import torch
    from test_regression_amd import mesa
    B, H, T, d, C = 2, 3, 320, 64, 64
    x = small_inputs(11, B, H, T, d, "f32")
    q, k, v = (to_dev(x[n], "f32") for n in ("q", "k", "v"))
    g, lam, gout = to_dev(x["gamma"], "f32"), to_dev(x["lam"], "f32"), to_dev(x["gout"], "f32")
    out, _, xs = mesa.mesa_forward_train(q, k, v, g, lam, 12, 1e-4, C)
    ref = mesa.mesa_backward(k, v, g, lam, xs, out, gout, 12, 1e-4, C)
    ws = torch.full((mesa.mesa_backward_workspace_bytes(B, H, T, d, d, C),), 0x7f, dtype=torch.uint8,
                    device=q.device)
    for _ in range(2):
        r = mesa.mesa_backward(k, v, g, lam, xs, out, gout, 12, 1e-4, C, workspace=ws)
        torch.cuda.synchronize()
        for name in ref:
            assert torch.equal(r[name], ref[name]), name
