"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Each test prints the case it runs (name, shape, seed) before touching the
GPU.  Tolerances: relative L2 <= 2e-3 (float32 q/k/v) or <= 1e-2 (bfloat16),
iteration counts exact for every token whose stop decision is decidable
(see parity_helpers).  Full-size workloads are compared on sampled heads and
tokens the oracle computes one by one, in the launch configuration the
benchmark times (chunk 64).
"""
import sys

import numpy as np
import pytest

import oracle
from test_regression_amd import inputs
from tests.parity_helpers import (RTOL, compare_counts, gpu_forward, oracle_forward, rel_l2,
                                  to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def small_inputs(seed, B, H, T, d, dtype, glo=0.9, lam=(0.5, 2.0)):
    w = inputs.Workload("t", B, H, T, d, 64, dtype, glo, "uniform", lam[0], lam[1], 0, 0.0, seed)
    return inputs.forward_inputs(w)


def sub(x, b, h):
    """One (b, h) head of a forward input dict, kept 4-D."""
    return dict(q=x["q"][b:b + 1, h:h + 1], k=x["k"][b:b + 1, h:h + 1], v=x["v"][b:b + 1, h:h + 1],
                gamma=x["gamma"][b:b + 1, h:h + 1], lam=x["lam"][h:h + 1])


# ---------------------------------------------------------------- workloads
def test_tiny_workload_full():
    w = inputs.WORKLOADS["tiny_f32_d16_T256"]
    say("case", w)
    x = inputs.forward_inputs(w)
    g = gpu_forward(x, w.dtype, w.max_iters, w.tol, w.chunk)
    r = oracle_forward(x, w.dtype, w.max_iters, w.tol)
    e = rel_l2(g["out"], r["out"])
    say(f"tiny rel_l2={e:.3e}")
    assert e <= RTOL[w.dtype]
    compare_counts(g["iters"], r, w.max_iters, w.tol)


def test_mid_workload_full():
    w = inputs.WORKLOADS["mid_bf16_d64_T2048"]
    say("case", w)
    x = inputs.forward_inputs(w)
    g = gpu_forward(x, w.dtype, w.max_iters, w.tol, w.chunk)
    r = oracle_forward(x, w.dtype, w.max_iters, w.tol)
    e = rel_l2(g["out"], r["out"])
    worst = max(rel_l2(g["out"][b, h], r["out"][b, h]) for b in range(w.B) for h in range(w.H))
    say(f"mid rel_l2={e:.3e} worst head={worst:.3e}")
    assert e <= RTOL[w.dtype] and worst <= RTOL[w.dtype]
    compare_counts(g["iters"], r, w.max_iters, w.tol)


def _sample_mask(T, rng, n=96):
    idx = np.unique(np.concatenate([np.arange(3), np.arange(T - 3, T), rng.choice(T, n, replace=False)]))
    m = np.zeros(T, bool)
    m[idx] = True
    return m


def test_layer_workload_sampled():
    """Full layer size (8x16x4096, d=128, bf16, k=30) on the GPU; oracle on sampled tokens."""
    w = inputs.WORKLOADS["layer_bf16_d128_T4096_k30"]
    say("case", w)
    x = inputs.forward_inputs(w)
    g = gpu_forward(x, w.dtype, w.max_iters, w.tol, w.chunk)
    assert np.isfinite(g["out"]).all()
    assert (g["iters"] == w.max_iters).all()
    rng = np.random.default_rng(5)
    heads = [(0, 0), (7, 15), (3, 9), (5, 2)]
    errs = []
    for b, h in heads:
        want = _sample_mask(w.T, rng)[None, None]
        r = oracle_forward(sub(x, b, h), w.dtype, w.max_iters, w.tol, want=want)
        sel = want[0, 0]
        e = rel_l2(g["out"][b, h][sel], r["out"][0, 0][sel])
        errs.append(e)
        assert (r["iters"][0, 0][sel] == w.max_iters).all()
    say(f"layer sampled rel_l2 per head={['%.2e' % e for e in errs]}")
    assert max(errs) <= RTOL[w.dtype]


def test_dynamic_workload_sampled():
    """Full dynamic-stopping size (4x16x8192, fp32, tol 1e-4, cap 30); oracle on whole heads."""
    w = inputs.WORKLOADS["dynamic_f32_d128_T8192_tol1e-4"]
    say("case", w)
    x = inputs.forward_inputs(w)
    g = gpu_forward(x, w.dtype, w.max_iters, w.tol, w.chunk)
    heads = [(0, 0), (3, 15), (1, 7), (2, 11)]
    tot_d = tot_u = tot_m = 0
    for b, h in heads:
        r = oracle_forward(sub(x, b, h), w.dtype, w.max_iters, w.tol)
        e = rel_l2(g["out"][b, h], r["out"][0, 0])
        assert e <= RTOL[w.dtype], (b, h, e)
        nd, nu, nm = compare_counts(g["iters"][b:b + 1, h:h + 1], r, w.max_iters, w.tol)
        tot_d += nd
        tot_u += nu
        tot_m += nm
    it = g["iters"]
    say(f"dynamic: iters min/mean/max={it.min()}/{it.mean():.2f}/{it.max()} "
        f"decidable={tot_d} undecidable={tot_u} (mismatched {tot_m})")
    assert it.min() < it.max()          # counts vary per token
    assert tot_d > 0.99 * (tot_d + tot_u)


def _decode_case(w, steps, S, prefix):
    """States from S distinct oracle-built prefixes (fp64 -> fp32), tiled over N x H heads."""
    N, H, d = w.B, w.H, w.d
    pk = np.zeros((1, S, prefix, d), np.float32)
    pv = np.zeros_like(pk)
    pg = np.zeros((1, S, prefix), np.float32)
    for i in range(S):
        p = inputs.decode_prefix(w, i, i % H, prefix)
        pk[0, i], pv[0, i], pg[0, i] = p["k"], p["v"], p["gamma"]
    r = oracle.forward(pk, pk, pv, pg, np.ones((S, d)), 0, 0.0,
                       want=np.zeros((1, S, prefix), bool), final_state=True)
    idx = (np.arange(N * H) % S).reshape(N, H)
    H0 = r["final_H"][0][idx].astype(np.float32)
    G0 = r["final_G"][0][idx].astype(np.float32)
    return H0, G0, inputs.decode_steps(w, steps), inputs.decode_lambda(w)


def test_decode_workload_full_launch_shape():
    """256 x 16 heads, d=128, states from 4096-token prefixes; a few steps vs the oracle."""
    import torch
    from test_regression_amd import mesa
    w = inputs.WORKLOADS["decode_f32_d128_N256_prefix4096"]
    steps = 3
    say("case", w, "steps", steps)
    H0, G0, st, lam = _decode_case(w, steps, S=16, prefix=w.T)
    SH, SG = to_dev(H0, "f32"), to_dev(G0, "f32")
    lam_d = to_dev(lam, "f32")
    RH, RG = H0.astype(np.float64), G0.astype(np.float64)
    for s in range(steps):
        q, k, v, g = (to_dev(st[n][s], "f32") for n in ("q", "k", "v", "gamma"))
        out, it = mesa.mesa_decode_step(q, k, v, g, lam_d, SH, SG, w.max_iters, w.tol)
        torch.cuda.synchronize()
        r = oracle.decode_step(st["q"][s], st["k"][s], st["v"][s], st["gamma"][s], lam, RH, RG,
                               w.max_iters, w.tol)
        e = rel_l2(out.cpu().numpy(), r["out"])
        nd, nu, nm = compare_counts(it.cpu().numpy(), r, w.max_iters, w.tol)
        say(f"decode step {s}: rel_l2={e:.3e} iters mean={r['iters'].mean():.2f} "
            f"decidable={nd} undecidable={nu} mismatched={nm}")
        assert e <= RTOL["f32"]
    assert rel_l2(SH.cpu().numpy(), RH) < 1e-5 and rel_l2(SG.cpu().numpy(), RG) < 1e-5


@pytest.mark.parametrize("mode", [1, 2])
def test_warm_decode_full_launch_shape(mode):
    """Warm-started decode (x0 from each head's previous solution) at 256 x 16
    heads, d=128, chained over steps with queries that overlap their
    neighbours (window 4); the solution carried in state_x is compared too."""
    import torch
    from test_regression_amd import mesa
    w = inputs.WORKLOADS["decode_f32_d128_N256_prefix4096"]
    steps = 4
    say("case warm decode", w.name, "mode", mode, "steps", steps)
    H0, G0, st, lam = _decode_case(w, steps, S=16, prefix=w.T)
    st["q"] = inputs.decode_queries_windowed(w, steps, 4)
    SH, SG = to_dev(H0, "f32"), to_dev(G0, "f32")
    SX = torch.zeros((w.B, w.H, w.d), dtype=torch.float32, device="cuda")
    lam_d = to_dev(lam, "f32")
    RH, RG = H0.astype(np.float64), G0.astype(np.float64)
    RX = np.zeros((w.B, w.H, w.d))
    for s in range(steps):
        q, k, v, g = (to_dev(st[n][s], "f32") for n in ("q", "k", "v", "gamma"))
        out, it = mesa.mesa_decode_step_warm(q, k, v, g, lam_d, SH, SG, SX, w.max_iters, w.tol, mode)
        torch.cuda.synchronize()
        r = oracle.decode_step_warm(st["q"][s], st["k"][s], st["v"][s], st["gamma"][s], lam, RH, RG, RX,
                                    w.max_iters, w.tol, mode)
        e = rel_l2(out.cpu().numpy(), r["out"])
        ex = rel_l2(SX.cpu().numpy(), RX)
        nd, nu, nm = compare_counts(it.cpu().numpy(), r, w.max_iters, w.tol)
        say(f"warm decode step {s}: rel_l2={e:.3e} x rel_l2={ex:.3e} iters mean={r['iters'].mean():.2f} "
            f"decidable={nd} undecidable={nu} mismatched={nm}")
        assert e <= RTOL["f32"] and ex <= RTOL["f32"]


@pytest.mark.parametrize("d", [16, 32, 64])
def test_warm_decode_small_dims_and_zero_query(d):
    import torch
    from test_regression_amd import mesa
    N, H, P, cap, tol = 3, 2, 40, 30, 1e-5
    say("case warm decode dims", d)
    x = small_inputs(90 + d, N, H, P + 3, d, "f32")
    x["q"][1, 0, P + 1] = 0.0            # a zero query: x = 0 and no update, whatever x_prev is
    pre = oracle.forward(x["k"][:, :, :P], x["k"][:, :, :P], x["v"][:, :, :P], x["gamma"][:, :, :P],
                         x["lam"], 0, 0.0, want=np.zeros((N, H, P), bool), final_state=True)
    H0 = pre["final_H"].astype(np.float32)
    G0 = pre["final_G"].astype(np.float32)
    for mode in (0, 1, 2):
        SH, SG = to_dev(H0, "f32"), to_dev(G0, "f32")
        RH, RG = H0.astype(np.float64), G0.astype(np.float64)
        X0 = np.random.default_rng(d).standard_normal((N, H, d)).astype(np.float32)
        SX, RX = to_dev(X0, "f32"), X0.astype(np.float64)
        lam = to_dev(x["lam"], "f32")
        for s in (P, P + 1, P + 2):
            args = [np.ascontiguousarray(x[n][:, :, s]) for n in ("q", "k", "v", "gamma")]
            out, it = mesa.mesa_decode_step_warm(*(to_dev(a, "f32") for a in args), lam, SH, SG, SX,
                                                 cap, tol, mode)
            torch.cuda.synchronize()
            r = oracle.decode_step_warm(*args, x["lam"], RH, RG, RX, cap, tol, mode)
            assert rel_l2(out.cpu().numpy(), r["out"]) <= 2e-3, (mode, s)
            assert rel_l2(SX.cpu().numpy(), RX) <= 2e-3, (mode, s)
            compare_counts(it.cpu().numpy(), r, cap, tol)
            if s == P + 1:
                assert not SX.cpu().numpy()[1, 0].any() and int(it[1, 0]) == 0


# ---------------------------------------------------------------- structure
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dims_chunks_dtypes_ragged(d, chunk, dtype):
    """Every built (d, chunk, dtype) kernel variant, several chunks with a ragged tail."""
    B, H, T = 1, 2, 3 * chunk + chunk // 2 + 3
    say("case grid", d, chunk, dtype, (B, H, T))
    x = small_inputs(100 + d + chunk, B, H, T, d, dtype)
    for cap, tol in [(1, 0.0), (8, 0.0), (25, 1e-3)]:
        g = gpu_forward(x, dtype, cap, tol, chunk)
        r = oracle_forward(x, dtype, cap, tol)
        e = rel_l2(g["out"], r["out"])
        worst = np.max(np.linalg.norm(g["out"] - r["out"], axis=-1) /
                       np.maximum(np.linalg.norm(r["out"], axis=-1), 1e-30))
        assert e <= 1e-4 and worst <= 1e-3, (cap, tol, e, worst)
        compare_counts(g["iters"], r, cap, tol)


def test_chunk_size_invariance():
    B, H, T, d = 1, 3, 300, 64
    say("case chunk invariance", (B, H, T, d))
    x = small_inputs(7, B, H, T, d, "f32")
    r = oracle_forward(x, "f32", 12, 0.0)
    outs = {}
    for c in (16, 32, 64):
        g = gpu_forward(x, "f32", 12, 0.0, c)
        outs[c] = g["out"]
        assert rel_l2(g["out"], r["out"]) <= 1e-4, c
        assert (g["iters"] == 12).all()
    assert rel_l2(outs[16], outs[64]) <= 1e-5 and rel_l2(outs[32], outs[64]) <= 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("k", [1, 2])
def test_one_and_two_iterations(dtype, k):
    """max_iters = 1: x_1 = (q.q / q.Aq) q, so every output checks one chunked
    matvec; 2 checks the direction update too.  With bf16 keys this is the
    split-product kernel, whose loop issues the next matvec's first step
    before it finishes the update (discarded after the last iteration)."""
    B, H, T, d = 2, 2, 130, 128
    say("case one/two matvecs", (B, H, T, d, dtype, k))
    x = small_inputs(11, B, H, T, d, dtype)
    for chunk in (16, 32, 64):
        g = gpu_forward(x, dtype, k, 0.0, chunk)
        r = oracle_forward(x, dtype, k, 0.0)
        e = rel_l2(g["out"], r["out"])
        say(f"chunk {chunk} rel_l2={e:.2e}")
        assert e <= 1e-5, chunk
        assert (g["iters"] == k).all()


@pytest.mark.parametrize("d", [16, 128])
def test_iterating_far_past_convergence_stays_finite(d):
    """Lambda = I and a fixed cap far above d: every token's CG converges
    exactly and then keeps iterating on a residual that shrinks into the
    denormal range, where the hardware reciprocal would flush it to zero.
    alpha and beta must stay finite and the output must still match."""
    B, H, T = 1, 2, 96
    say("case past convergence", (B, H, T, d))
    x = small_inputs(41, B, H, T, d, "f32", lam=(1.0, 1.0))
    g = gpu_forward(x, "f32", 4 * d + 40, 0.0, 64)
    r = oracle_forward(x, "f32", 4 * d + 40, 0.0)
    assert np.isfinite(g["out"]).all()
    assert rel_l2(g["out"], r["out"]) <= 1e-4
    compare_counts(g["iters"], r, 4 * d + 40, 0.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_cases(dtype):
    """Short sequences inside one chunk, zero queries, no forgetting, zero
    iterations; bf16 runs the split-product kernel (chunk 16 its masked
    second key block)."""
    d = 32
    say("case edges", dtype)
    for chunk in (16, 64):
        for T in (1, 5, 16, 17, 64, 65):
            x = small_inputs(20 + T, 1, 2, T, d, dtype)
            x["q"][0, 0, T // 2] = 0
            x["gamma"][0, 1] = 1.0
            g = gpu_forward(x, dtype, 10, 1e-4, chunk)
            r = oracle_forward(x, dtype, 10, 1e-4)
            assert rel_l2(g["out"], r["out"]) <= 1e-4, (chunk, T)
            assert g["iters"][0, 0, T // 2] == 0 and np.all(g["out"][0, 0, T // 2] == 0)
            compare_counts(g["iters"], r, 10, 1e-4)
    # zero iterations: out = 0, counts 0, final states still exported
    x = small_inputs(31, 1, 2, 70, d, dtype)
    g = gpu_forward(x, dtype, 0, 0.0, 64, return_final=True)
    r = oracle_forward(x, dtype, 0, 0.0, final_state=True)
    assert np.all(g["out"] == 0) and np.all(g["iters"] == 0)
    assert rel_l2(g["final_H"], r["final_H"]) < 1e-5 and rel_l2(g["final_G"], r["final_G"]) < 1e-5


def test_empty_sequence_exports_zero_state():
    import torch
    from test_regression_amd import mesa
    say("case T=0")
    q = torch.zeros((1, 2, 0, 16), device="cuda")
    g = torch.zeros((1, 2, 0), device="cuda")
    lam = torch.ones((2, 16), device="cuda")
    fH = torch.full((1, 2, 16, 16), 7.0, device="cuda")
    fG = torch.full((1, 2, 16, 16), 7.0, device="cuda")
    out, it, fH, fG = mesa.mesa_forward(q, q, q, g, lam, 5, 0.0, 64, return_final=True,
                                        final_H=fH, final_G=fG)
    torch.cuda.synchronize()
    assert out.numel() == 0 and bool((fH == 0).all()) and bool((fG == 0).all())


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("d", [16, 128])
def test_bf16_states_at_float_accuracy(d, chunk):
    """bf16 keys and values: the chunk states come from bf16 MFMAs on an
    exact three-part split of the weighted keys, so the exported states must
    keep float accuracy (a two-part split would leave errors near 2^-17)."""
    B, H, T = 1, 2, 200
    say("case bf16 states", (B, H, T, d, chunk))
    x = small_inputs(43, B, H, T, d, "bf16")
    g = gpu_forward(x, "bf16", 0, 0.0, chunk, return_final=True)
    r = oracle_forward(x, "bf16", 0, 0.0, final_state=True)
    eh, eg = rel_l2(g["final_H"], r["final_H"]), rel_l2(g["final_G"], r["final_G"])
    say(f"final_H rel_l2={eh:.2e} final_G rel_l2={eg:.2e}")
    assert eh <= 5e-7 and eg <= 5e-7


def test_final_states_and_decode_continue_forward():
    import torch
    from test_regression_amd import mesa
    B, H, T, d, S, cap, tol = 2, 2, 150, 32, 6, 20, 1e-4
    say("case prefill->decode", (B, H, T, d))
    x = small_inputs(41, B, H, T, d, "f32")
    full = gpu_forward(x, "f32", cap, tol, 64, return_final=True)
    ref = oracle_forward(x, "f32", cap, tol, final_state=True)
    assert rel_l2(full["final_H"], ref["final_H"]) < 1e-5
    assert rel_l2(full["final_G"], ref["final_G"]) < 1e-5
    pre = {n: (x[n][:, :, :T - S] if n != "lam" else x[n]) for n in x}
    p = gpu_forward(pre, "f32", cap, tol, 64, return_final=True)
    SH = to_dev(p["final_H"].astype(np.float32), "f32")
    SG = to_dev(p["final_G"].astype(np.float32), "f32")
    lam = to_dev(x["lam"], "f32")
    for s in range(T - S, T):
        q, k, v = (to_dev(np.ascontiguousarray(x[n][:, :, s]), "f32") for n in ("q", "k", "v"))
        g = to_dev(np.ascontiguousarray(x["gamma"][:, :, s]), "f32")
        out, it = mesa.mesa_decode_step(q, k, v, g, lam, SH, SG, cap, tol)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert rel_l2(o, full["out"][:, :, s]) <= 1e-4, s
        assert rel_l2(o, ref["out"][:, :, s]) <= 1e-4, s
        sub_ref = {kname: ref[kname][:, :, s] for kname in ("iters", "rho_stop", "rho_min_prev", "reason")}
        compare_counts(it.cpu().numpy(), sub_ref, cap, tol)


@pytest.mark.parametrize("d", [16, 32, 64])
def test_decode_small_dims(d):
    import torch
    from test_regression_amd import mesa
    N, H, P, cap, tol = 3, 2, 40, 30, 1e-5
    say("case decode dims", d)
    x = small_inputs(50 + d, N, H, P + 2, d, "f32")
    pre = oracle.forward(x["k"][:, :, :P], x["k"][:, :, :P], x["v"][:, :, :P], x["gamma"][:, :, :P],
                         x["lam"], 0, 0.0, want=np.zeros((N, H, P), bool), final_state=True)
    H0 = pre["final_H"].astype(np.float32)
    G0 = pre["final_G"].astype(np.float32)
    SH, SG = to_dev(H0, "f32"), to_dev(G0, "f32")
    RH, RG = H0.astype(np.float64), G0.astype(np.float64)
    lam = to_dev(x["lam"], "f32")
    for s in (P, P + 1):
        args = [np.ascontiguousarray(x[n][:, :, s]) for n in ("q", "k", "v", "gamma")]
        out, it = mesa.mesa_decode_step(*(to_dev(a, "f32") for a in args), lam, SH, SG, cap, tol)
        torch.cuda.synchronize()
        r = oracle.decode_step(*args, x["lam"], RH, RG, cap, tol)
        assert rel_l2(out.cpu().numpy(), r["out"]) <= 2e-3
        compare_counts(it.cpu().numpy(), r, cap, tol)


def test_run_twice_bitwise_identical():
    w = inputs.WORKLOADS["mid_bf16_d64_T2048"]
    say("case determinism", w.name)
    x = inputs.forward_inputs(w, B=1)
    a = gpu_forward(x, w.dtype, w.max_iters, 1e-3, w.chunk)
    b = gpu_forward(x, w.dtype, w.max_iters, 1e-3, w.chunk)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["iters"], b["iters"])


def test_garbage_workspace_and_reuse():
    """The CG kernel's chunk-claim counter lives in the workspace tail and is
    reset by the chunk-state kernel: a workspace full of garbage, reused for
    a second call, gives the same bits as a fresh one."""
    import torch
    from test_regression_amd import mesa
    w = inputs.WORKLOADS["mid_bf16_d64_T2048"]
    say("case garbage workspace", w.name)
    x = inputs.forward_inputs(w, B=2)
    q, k, v = (to_dev(x[n], w.dtype) for n in ("q", "k", "v"))
    g, lam = to_dev(x["gamma"], "f32"), to_dev(x["lam"], "f32")
    B, H, T, d = q.shape
    ref_out, ref_it, _, _ = mesa.mesa_forward(q, k, v, g, lam, w.max_iters, 1e-3, w.chunk)
    ws = torch.full((mesa.mesa_forward_workspace_bytes(B, H, T, d, d, w.chunk),), 0x7f, dtype=torch.uint8,
                    device=q.device)
    for _ in range(2):
        out, it, _, _ = mesa.mesa_forward(q, k, v, g, lam, w.max_iters, 1e-3, w.chunk, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(it, ref_it)
