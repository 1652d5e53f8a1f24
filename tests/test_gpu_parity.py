"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Each test prints the case it runs (name, shape, seed) before touching the
GPU.  Tolerances: relative L2 <= 2e-3 (float32 q/k/v) or <= 1e-2 (bfloat16),
iteration counts exact for every token whose stop decision is decidable
(see parity_helpers).  The layer and dynamic-stopping workloads are compared
on every token of every head, in the launch configuration the benchmark
times (chunk 64); the decode workload on all heads for its first steps and
on sampled heads over the benchmark's whole run.
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


def test_layer_workload_full():
    """Full layer size (8x16x4096, d=128, bf16, k=30) in the launch
    configuration the benchmark times; the oracle solves every token of all
    128 heads."""
    w = inputs.WORKLOADS["layer_bf16_d128_T4096_k30"]
    say("case", w)
    x = inputs.forward_inputs(w)
    g = gpu_forward(x, w.dtype, w.max_iters, w.tol, w.chunk)
    assert np.isfinite(g["out"]).all()
    assert (g["iters"] == w.max_iters).all()
    r = oracle_forward(x, w.dtype, w.max_iters, w.tol)
    assert (r["iters"] == w.max_iters).all()
    e = rel_l2(g["out"], r["out"])
    per_head = [rel_l2(g["out"][b, h], r["out"][b, h]) for b in range(w.B) for h in range(w.H)]
    tok = np.linalg.norm(g["out"] - r["out"], axis=-1) / np.maximum(np.linalg.norm(r["out"], axis=-1), 1e-30)
    say(f"layer full: rel_l2={e:.3e} worst head={max(per_head):.3e} worst token={tok.max():.3e} "
        f"({w.B * w.H * w.T} token-heads)")
    assert e <= RTOL[w.dtype] and max(per_head) <= RTOL[w.dtype]


def test_dynamic_workload_full():
    """Full dynamic-stopping size (4x16x8192, fp32, tol 1e-4, cap 30); the
    oracle solves every token of all 64 heads and the iteration counts of
    every decidable token must match exactly."""
    w = inputs.WORKLOADS["dynamic_f32_d128_T8192_tol1e-4"]
    say("case", w)
    x = inputs.forward_inputs(w)
    g = gpu_forward(x, w.dtype, w.max_iters, w.tol, w.chunk)
    r = oracle_forward(x, w.dtype, w.max_iters, w.tol)
    e = rel_l2(g["out"], r["out"])
    worst = max(rel_l2(g["out"][b, h], r["out"][b, h]) for b in range(w.B) for h in range(w.H))
    nd, nu, nm = compare_counts(g["iters"], r, w.max_iters, w.tol)
    it = g["iters"]
    hist = np.bincount(it.ravel(), minlength=w.max_iters + 1)
    say(f"dynamic full: rel_l2={e:.3e} worst head={worst:.3e} iters min/mean/max="
        f"{it.min()}/{it.mean():.3f}/{it.max()} decidable={nd} undecidable={nu} (mismatched {nm}); "
        f"histogram {dict((i, int(c)) for i, c in enumerate(hist) if c)}")
    assert e <= RTOL[w.dtype] and worst <= RTOL[w.dtype]
    assert it.min() < it.max()          # counts vary per token
    assert nd > 0.99 * (nd + nu)


# Sampled decode heads (n, h): every head index and spread sequence indices.
DECODE_SAMPLE = [((37 * i + 5) % 256, i % 16) for i in range(32)]


@pytest.fixture(scope="module")
def decode_ws():
    """The decode workload as the benchmark draws it: start states of all
    256 x 16 heads built on the device from seeded 4096-token prefixes by the
    forward path (zero CG iterations, final states exported; distinct for
    every (n, h)), the per-step inputs of the benchmark's 8 warmup + 1024
    timed steps, and the prefix tokens of the sampled heads on the host."""
    import torch
    from test_regression_amd import mesa
    w = inputs.WORKLOADS["decode_f32_d128_N256_prefix4096"]
    N, H, d = w.B, w.H, w.d
    gen = inputs.DecodeDeviceStream(torch, w, torch.device("cuda"))
    lam = inputs.decode_lambda(w)
    lam_d = to_dev(lam, "f32")
    SH = torch.empty((N, H, d, d), dtype=torch.float32, device="cuda")
    SG = torch.empty_like(SH)
    pre = {}
    for n0, pk, pv, pg in gen.prefix_batches(64):
        nb = pk.shape[0]
        mesa.mesa_forward(pk, pk, pv, pg, lam_d, 0, 0.0, w.chunk, return_iters=False,
                          final_H=SH[n0:n0 + nb], final_G=SG[n0:n0 + nb], return_final=True)
        for n, h in DECODE_SAMPLE:
            if n0 <= n < n0 + nb:
                pre[(n, h)] = tuple(a[n - n0, h].cpu().numpy() for a in (pk, pv, pg))
        del pk, pv, pg
    steps = gen.steps(8 + w.steps)
    torch.cuda.synchronize()
    return dict(w=w, lam=lam, lam_d=lam_d, SH=SH, SG=SG, pre=pre, steps=steps)


def test_decode_workload_full(decode_ws):
    """The decode workload at full size: 256 x 16 heads (d=128), distinct
    start states from 4096-token prefixes, the benchmark's 1032 steps.
      1. the device-built start states of 32 sampled heads against the
         oracle run over the same prefix tokens;
      2. the first 16 steps of all 4096 heads against the oracle from the same
         fp32 start states (outputs, counts, and the states after them);
      3. every later step of the sampled heads against the oracle continuing
         from its own states, and their final states."""
    import torch
    from test_regression_amd import mesa
    ws = decode_ws
    w, lam = ws["w"], ws["lam"]
    N, H, d = w.B, w.H, w.d
    ns = np.array([n for n, _ in DECODE_SAMPLE])
    hs = np.array([h for _, h in DECODE_SAMPLE])
    say("case decode full", w.name, "sampled heads", len(DECODE_SAMPLE))
    # 1. start states against the oracle over the sampled heads' prefixes
    pk = np.stack([ws["pre"][nh][0] for nh in DECODE_SAMPLE])[None]
    pv = np.stack([ws["pre"][nh][1] for nh in DECODE_SAMPLE])[None]
    pg = np.stack([ws["pre"][nh][2] for nh in DECODE_SAMPLE])[None]
    rp = oracle.forward(pk, pk, pv, pg, lam[hs], 0, 0.0, want=np.zeros(pg.shape, bool), final_state=True)
    SH0 = ws["SH"].cpu().numpy()
    SG0 = ws["SG"].cpu().numpy()
    eh, eg = rel_l2(SH0[ns, hs], rp["final_H"][0]), rel_l2(SG0[ns, hs], rp["final_G"][0])
    say(f"decode start states (device-built) vs oracle: H rel_l2={eh:.2e} G rel_l2={eg:.2e}")
    assert eh < 1e-5 and eg < 1e-5
    # 2. all heads for the first steps
    SH, SG = ws["SH"].clone(), ws["SG"].clone()
    RH, RG = SH0.astype(np.float64), SG0.astype(np.float64)
    del SH0, SG0
    q, k, v, ga = ws["steps"]
    S_all, S = 16, q.shape[0]
    out = torch.empty((N, H, d), dtype=torch.float32, device="cuda")
    its = torch.empty((N, H), dtype=torch.int32, device="cuda")
    tot = np.zeros(3, np.int64)
    worst = 0.0
    for s in range(S_all):
        mesa.mesa_decode_step(q[s], k[s], v[s], ga[s], ws["lam_d"], SH, SG, w.max_iters, w.tol, out=out, iters=its)
        a = [t[s].cpu().numpy() for t in (q, k, v, ga)]
        r = oracle.decode_step(*a, lam, RH, RG, w.max_iters, w.tol)
        o = out.cpu().numpy()
        e = rel_l2(o, r["out"])
        wh = np.max(np.linalg.norm(o - r["out"], axis=-1) / np.linalg.norm(r["out"], axis=-1))
        worst = max(worst, wh)
        tot += compare_counts(its.cpu().numpy(), r, w.max_iters, w.tol)
        assert e <= RTOL["f32"] and wh <= RTOL["f32"], (s, e, wh)
    eh, eg = rel_l2(SH.cpu().numpy(), RH), rel_l2(SG.cpu().numpy(), RG)
    say(f"decode all {N * H} heads, {S_all} steps: worst head rel_l2={worst:.2e}; states H {eh:.2e} G {eg:.2e}; "
        f"decidable={tot[0]} undecidable={tot[1]} mismatched={tot[2]}")
    assert eh < 1e-5 and eg < 1e-5
    # 3. the rest of the run on the sampled heads
    RHs, RGs = np.ascontiguousarray(RH[ns, hs][None]), np.ascontiguousarray(RG[ns, hs][None])
    del RH, RG
    nsd, hsd = torch.from_numpy(ns).cuda(), torch.from_numpy(hs).cuda()
    outs = torch.empty((S, len(ns), d), dtype=torch.float32, device="cuda")
    itss = torch.empty((S, len(ns)), dtype=torch.int32, device="cuda")
    for s in range(S_all, S):
        mesa.mesa_decode_step(q[s], k[s], v[s], ga[s], ws["lam_d"], SH, SG, w.max_iters, w.tol, out=out, iters=its)
        outs[s] = out[nsd, hsd]
        itss[s] = its[nsd, hsd]
    sel = [t[:, nsd, hsd][:, None].cpu().numpy() for t in (q, k, v, ga)]
    outs, itss = outs.cpu().numpy(), itss.cpu().numpy()
    lam_s = np.ascontiguousarray(lam[hs])
    tot = np.zeros(3, np.int64)
    worst = 0.0
    hist = np.zeros(w.max_iters + 1, np.int64)
    for s in range(S_all, S):
        r = oracle.decode_step(sel[0][s], sel[1][s], sel[2][s], sel[3][s], lam_s, RHs, RGs, w.max_iters, w.tol)
        o = outs[s][None]
        wh = np.max(np.linalg.norm(o - r["out"], axis=-1) / np.linalg.norm(r["out"], axis=-1))
        worst = max(worst, wh)
        assert wh <= RTOL["f32"], (s, wh)
        tot += compare_counts(itss[s][None], r, w.max_iters, w.tol)
        hist += np.bincount(r["iters"].ravel(), minlength=w.max_iters + 1)
    eh = rel_l2(SH[nsd, hsd].cpu().numpy(), RHs[0])
    eg = rel_l2(SG[nsd, hsd].cpu().numpy(), RGs[0])
    say(f"decode sampled heads, steps {S_all}..{S - 1}: worst head rel_l2={worst:.2e}; final states H {eh:.2e} "
        f"G {eg:.2e}; decidable={tot[0]} undecidable={tot[1]} mismatched={tot[2]}; oracle iteration histogram "
        f"{dict((i, int(c)) for i, c in enumerate(hist) if c)}")
    assert eh < 1e-5 and eg < 1e-5
    assert tot[0] > 0.99 * (tot[0] + tot[1])


@pytest.mark.parametrize("mode", [1, 2])
def test_warm_decode_full_launch_shape(decode_ws, mode):
    """Warm-started decode (x0 from each head's previous solution) at 256 x 16
    heads, d=128, from the distinct device-built start states, chained over
    steps with queries that overlap their neighbours (window 4); the
    solution carried in state_x is compared too."""
    import torch
    from test_regression_amd import mesa
    w = decode_ws["w"]
    steps = 4
    say("case warm decode", w.name, "mode", mode, "steps", steps)
    st = inputs.decode_steps(w, steps)
    st["q"] = inputs.decode_queries_windowed(w, steps, 4)
    SH, SG = decode_ws["SH"].clone(), decode_ws["SG"].clone()
    RH, RG = SH.cpu().numpy().astype(np.float64), SG.cpu().numpy().astype(np.float64)
    SX = torch.zeros((w.B, w.H, w.d), dtype=torch.float32, device="cuda")
    lam, lam_d = decode_ws["lam"], decode_ws["lam_d"]
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


@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_decode_bf16_inputs(d):
    """mesa_decode_step and mesa_decode_step_warm with bf16 q, k, v (fp32
    states): against the oracle run on the bf16-rounded inputs."""
    import torch
    from test_regression_amd import mesa
    N, H, P, cap, tol = 5, 3, 48, 30, 1e-4
    say("case decode bf16", d)
    x = small_inputs(70 + d, N, H, P + 3, d, "bf16")
    xf = {n: (inputs.as_f64(x[n], "bf16") if n in ("q", "k", "v") else x[n]) for n in x}
    xf["q"][2, 1, P + 1] = 0.0
    x["q"][2, 1, P + 1] = 0
    pre = oracle.forward(xf["k"][:, :, :P], xf["k"][:, :, :P], xf["v"][:, :, :P], x["gamma"][:, :, :P],
                         x["lam"], 0, 0.0, want=np.zeros((N, H, P), bool), final_state=True)
    H0 = pre["final_H"].astype(np.float32)
    G0 = pre["final_G"].astype(np.float32)
    lam = to_dev(x["lam"], "f32")
    for mode in (None, 1, 2):
        SH, SG = to_dev(H0, "f32"), to_dev(G0, "f32")
        RH, RG = H0.astype(np.float64), G0.astype(np.float64)
        SX = torch.zeros((N, H, d), dtype=torch.float32, device="cuda")
        RX = np.zeros((N, H, d))
        for s in (P, P + 1, P + 2):
            dev_args = [to_dev(np.ascontiguousarray(x[n][:, :, s]), "bf16") for n in ("q", "k", "v")]
            g = to_dev(np.ascontiguousarray(x["gamma"][:, :, s]), "f32")
            ref_args = [np.ascontiguousarray(xf[n][:, :, s]) for n in ("q", "k", "v", "gamma")]
            if mode is None:
                out, it = mesa.mesa_decode_step(*dev_args, g, lam, SH, SG, cap, tol)
                r = oracle.decode_step(*ref_args, x["lam"], RH, RG, cap, tol)
            else:
                out, it = mesa.mesa_decode_step_warm(*dev_args, g, lam, SH, SG, SX, cap, tol, mode)
                r = oracle.decode_step_warm(*ref_args, x["lam"], RH, RG, RX, cap, tol, mode)
            torch.cuda.synchronize()
            e = rel_l2(out.cpu().numpy(), r["out"])
            assert e <= 1e-4, (mode, s, e)
            compare_counts(it.cpu().numpy(), r, cap, tol)
            if s == P + 1:
                assert int(it[2, 1]) == 0 and not out[2, 1].any()
        assert rel_l2(SH.cpu().numpy(), RH) < 1e-5 and rel_l2(SG.cpu().numpy(), RG) < 1e-5


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


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("scale", [(2.0 ** -10, 2.0 ** -20, 2.0 ** 15), (2.0 ** 10, 2.0 ** 8, 2.0 ** -12)])
def test_inputs_far_from_unit_size(dtype, scale, d):
    """Keys, queries, values and lambda scaled by powers of two far from 1
    (the fp16 split products rescale every group by its own exponent, so the
    result must keep its accuracy): keys x sk with lambda x sk^2 is the same
    system up to the scale of x, so the outputs are compared with the oracle
    at the same bar as unit inputs.  d = 128 with bf16 keys includes the
    mid-chunk state that the CG kernel forms from the chunk state and keys."""
    sk, sq, sv = scale
    B, H, T = 1, 2, 150
    say("case scaled inputs", dtype, scale, d)
    x = small_inputs(61, B, H, T, d, "f32")
    x["k"] = x["k"] * np.float32(sk)
    x["q"] = x["q"] * np.float32(sq)
    x["v"] = x["v"] * np.float32(sv)
    x["lam"] = (x["lam"] * np.float32(sk * sk)).astype(np.float32)
    if dtype == "bf16":
        x = {n: (inputs.bf16_bits(x[n]) if n in ("q", "k", "v") else x[n]) for n in x}
    for cap, tol in ((2, 0.0), (12, 0.0), (30, 1e-4)):
        g = gpu_forward(x, dtype, cap, tol, 64)
        r = oracle_forward(x, dtype, cap, tol)
        e = rel_l2(g["out"], r["out"])
        say(f"scaled {dtype} cap {cap} tol {tol}: rel_l2={e:.2e}")
        assert np.isfinite(g["out"]).all() and e <= 1e-5, (cap, tol, e)
        compare_counts(g["iters"], r, cap, tol)


@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_strong_decay(dtype, d):
    """gamma ~ U(0.5, 1): within a chunk the decays e^{l_t - l_i} span many
    orders of magnitude, the chunk states forget most of their history, and
    (d = 128, bf16) the mid-chunk state's key weights reach far below 1."""
    B, H, T = 1, 2, 200
    say("case strong decay", dtype, d)
    x = small_inputs(67, B, H, T, d, dtype, glo=0.5)
    for cap, tol in ((2, 0.0), (12, 0.0), (30, 1e-4)):
        g = gpu_forward(x, dtype, cap, tol, 64)
        r = oracle_forward(x, dtype, cap, tol)
        e = rel_l2(g["out"], r["out"])
        say(f"strong decay {dtype} d {d} cap {cap}: rel_l2={e:.2e}")
        assert np.isfinite(g["out"]).all() and e <= 1e-5, (cap, tol, e)
        compare_counts(g["iters"], r, cap, tol)


@pytest.mark.parametrize("T", [33, 96, 104, 127])
def test_mid_state_partial_last_chunk(T):
    """d = 128, bf16 keys, 64-token chunks: the waves that start from the
    mid-chunk state (tokens 32..63 of a chunk), with the layer ending at
    token 33, 32, 40 or 63 of its last chunk.  That state is formed by three
    waves and handed over through LDS counters whatever the chunk's length;
    192 heads, so that with two chunks per head some workgroups take two."""
    B, H, d = 8, 24, 128
    say("case mid-chunk state, ragged last chunk", T)
    x = small_inputs(90 + T, B, H, T, d, "bf16")
    for cap, tol in ((30, 0.0), (30, 1e-4)):
        g = gpu_forward(x, "bf16", cap, tol, 64)
        r = oracle_forward(x, "bf16", cap, tol)
        e = rel_l2(g["out"], r["out"])
        say(f"T {T} tol {tol}: rel_l2={e:.2e}")
        assert np.isfinite(g["out"]).all() and e <= 1e-5, (T, tol, e)
        compare_counts(g["iters"], r, cap, tol)


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


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunk_states_many_heads(dtype):
    """d = 128 with many heads: bf16 takes the chunk-state kernel's unsplit
    column sets (one G workgroup per row half, B*H >= 171), fp32 the
    eight-wave kernel; outputs, iteration counts and both final states
    against the oracle, with a ragged last chunk."""
    B, H, T, d = 12, 16, 130, 128
    say("case many heads", dtype, (B, H, T, d))
    x = small_inputs(47, B, H, T, d, dtype)
    g = gpu_forward(x, dtype, 3, 0.0, 64, return_final=True)
    r = oracle_forward(x, dtype, 3, 0.0, final_state=True)
    eo, eh, eg = rel_l2(g["out"], r["out"]), rel_l2(g["final_H"], r["final_H"]), rel_l2(g["final_G"], r["final_G"])
    say(f"out={eo:.2e} final_H={eh:.2e} final_G={eg:.2e}")
    assert eo <= 1e-5 and eh <= 5e-7 and eg <= 5e-7
    assert (g["iters"] == 3).all()


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
