"""mesa_forward_noalloc -- the forward for callers that cannot allocate --
through the C ABI against mesa_forward on the same inputs.

Both run the same kernels, so out, iters and the final states must agree bit
for bit; the first result is also held to the oracle.  Two calls in a row
share the library's device array, the second with a smaller input, so the
second must not see anything the first left there.  Sizes whose chunk
states exceed the array are refused before anything is enqueued.
"""
import sys

import numpy as np
import pytest

import oracle
from test_regression_amd import inputs
from tests.parity_helpers import RTOL, compare_counts, oracle_forward, rel_l2, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _both(x, dtype, cap, tol, chunk):
    import torch
    from test_regression_amd import mesa
    q, k, v = (to_dev(x[n], dtype) for n in ("q", "k", "v"))
    g, lam = to_dev(x["gamma"], "f32"), to_dev(x["lam"], "f32")
    B, H, T, d = q.shape
    ref = mesa.mesa_forward(q, k, v, g, lam, cap, tol, chunk, return_final=True)
    out = torch.full((B, H, T, d), float("nan"), device="cuda")
    it = torch.full((B, H, T), -7, dtype=torch.int32, device="cuda")
    fH = torch.full((B, H, d, d), float("nan"), device="cuda")
    fG = torch.full((B, H, d, d), float("nan"), device="cuda")
    mesa.mesa_forward_noalloc(q, k, v, g, lam, cap, tol, chunk, out=out, iters=it, final_H=fH, final_G=fG)
    torch.cuda.synchronize()
    for a, b, n in ((out, ref[0], "out"), (it, ref[1], "iters"), (fH, ref[2], "final_H"), (fG, ref[3], "final_G")):
        assert torch.equal(a, b), f"{n} differs from mesa_forward's"
    return out.cpu().numpy().astype(np.float64), it.cpu().numpy()


def test_noalloc_matches_forward_twice_then_smaller():
    w = inputs.WORKLOADS["mid_bf16_d64_T2048"]
    say("case noalloc 1:", w.name)
    x = inputs.forward_inputs(w)
    o, it = _both(x, w.dtype, w.max_iters, 1e-3, w.chunk)
    r = oracle_forward(x, w.dtype, w.max_iters, 1e-3)
    e = rel_l2(o, r["out"])
    say(f"noalloc 1: rel_l2 vs oracle {e:.2e}")
    assert e <= RTOL[w.dtype]
    compare_counts(it, r, w.max_iters, 1e-3)
    say("case noalloc 2: 1x3x300, d=128, fp32, tol 1e-4, cap 30, chunk 32")
    w2 = inputs.Workload("t", 1, 3, 300, 128, 32, "f32", 0.97, "uniform", 0.5, 2.0, 30, 1e-4, 77)
    x2 = inputs.forward_inputs(w2)
    o2, it2 = _both(x2, "f32", 30, 1e-4, 32)
    r2 = oracle_forward(x2, "f32", 30, 1e-4)
    e2 = rel_l2(o2, r2["out"])
    say(f"noalloc 2: rel_l2 vs oracle {e2:.2e}")
    assert e2 <= RTOL["f32"]
    compare_counts(it2, r2, 30, 1e-4)


def test_noalloc_refuses_sizes_beyond_its_array():
    import torch
    from test_regression_amd import mesa
    B, H, T, d = 1, 16, 4096, 128
    say("case noalloc too large", (B, H, T, d))
    assert mesa.mesa_forward_workspace_bytes(B, H, T, d, d, 64) > (64 << 20)
    q = torch.zeros((B, H, T, d), dtype=torch.bfloat16, device="cuda")
    g = torch.ones((B, H, T), device="cuda")
    lam = torch.ones((H, d), device="cuda")
    out = torch.full((B, H, T, d), 3.0, device="cuda")
    with pytest.raises(ValueError, match="built-in scratch"):
        mesa.mesa_forward_noalloc(q, q, q, g, lam, 5, 0.0, 64, out=out)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())      # nothing was enqueued
    # zero iterations need no chunk states, so any size is accepted
    mesa.mesa_forward_noalloc(q, q, q, g, lam, 0, 0.0, 64, out=out)
    torch.cuda.synchronize()
    assert bool((out == 0).all())
