"""GPU parity of the q/k pre-processing kernel against the fp64 oracle.

Section "Arquitetura (MesaNet)", bullet "Pre-processamento" of the MesaNet
summary page: keys and queries are normalised and convolved with a small
window before the Mesa layer (reading: causal depthwise convolution of width
W over the tokens, then L2 normalisation per token).  float32 outputs must
match within relative L2 2e-3 (bfloat16 inputs: 1e-2) and, element by
element, within the rounding of the fp32 arithmetic; bfloat16 outputs within
one bfloat16 step of the oracle's value (plus 1e-6 for sums that cancel);
carried history rows bit for bit.
"""
import sys

import numpy as np
import pytest

import oracle
from test_regression_amd import inputs
from tests.parity_helpers import RTOL, rel_l2, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_pre(x, w, dtype, out_dtype, hist=None, want_hist=False):
    import torch
    from test_regression_amd import mesa
    xd = to_dev(x, dtype)
    wd = to_dev(w, "f32")
    hd = None if hist is None else to_dev(hist, dtype)
    od = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    r = mesa.mesa_qk_preprocess(xd, wd, hd, out_dtype=od, return_hist=want_hist)
    torch.cuda.synchronize()
    y, ho = (r if want_hist else (r, None))
    y = y.float().cpu().numpy().astype(np.float64)
    if ho is not None:
        ho = ho.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" else ho.cpu().numpy()
    return y, ho


def check(y, ref, in_dtype, out_dtype):
    e = rel_l2(y, ref)
    assert e <= RTOL[in_dtype], e
    if out_dtype == "f32":
        assert np.abs(y - ref).max() <= 1e-5, np.abs(y - ref).max()
    else:
        # one bfloat16 step of the reference value (8 significant bits), plus
        # the fp32 error of a convolution sum that cancels (the rows have unit
        # norm, so that error is absolute: a few 2^-24 per term; 1e-6 allows
        # for it with room)
        step = np.where(ref != 0, 2.0 ** (np.floor(np.log2(np.abs(np.where(ref != 0, ref, 1)))) - 7), 0.0)
        assert (np.abs(y - ref) <= step * 1.0001 + 1e-6).all(), np.abs(y - ref).max()
    return e


@pytest.mark.parametrize("W", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("dtypes", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16")])
def test_preprocess_dims_widths_dtypes(d, W, dtypes):
    in_dt, out_dt = dtypes
    B, H, T = 2, 3, 37
    seed = 4000 + 10 * d + W
    say("case preprocess", dict(d=d, W=W, dtypes=dtypes, B=B, H=H, T=T, seed=seed))
    x = inputs.preprocess_inputs(B, H, T, d, W, in_dt, seed, with_hist=True)
    xf = inputs.as_f64(x["x"], in_dt)
    hf = None if x["hist"] is None else inputs.as_f64(x["hist"], in_dt)
    for hist, hist_f in ((None, None), (x["hist"], hf)):
        y, ho = gpu_pre(x["x"], x["w"], in_dt, out_dt, hist=hist, want_hist=W > 1)
        ref = oracle.qk_preprocess(xf, x["w"], hist=hist_f)
        check(y, ref, in_dt, out_dt)
        if W > 1:
            np.testing.assert_array_equal(ho, x["x"][:, :, T - (W - 1):])


@pytest.mark.parametrize("in_dt", ["f32", "bf16"])
def test_preprocess_in_pieces_with_carried_history(in_dt):
    """Prefill in pieces shorter and longer than the window, then single
    tokens as in decode; each piece's output and carried rows vs the oracle."""
    import torch
    B, H, d, W = 2, 2, 64, 4
    cuts = (2, 1, 9, 1, 1, 0, 5)
    T = sum(cuts)
    say("case preprocess pieces", in_dt, cuts)
    x = inputs.preprocess_inputs(B, H, T, d, W, in_dt, 4100)
    xf = inputs.as_f64(x["x"], in_dt)
    whole = oracle.qk_preprocess(xf, x["w"])
    hist, t0 = None, 0
    for n in cuts:
        piece = np.ascontiguousarray(x["x"][:, :, t0:t0 + n])
        y, ho = gpu_pre(piece, x["w"], in_dt, "f32", hist=hist, want_hist=True)
        ref_hist = None if hist is None else inputs.as_f64(hist, in_dt)
        ref, ref_ho = oracle.qk_preprocess(inputs.as_f64(piece, in_dt), x["w"], hist=ref_hist, want_hist=True)
        if n:
            check(y, ref, in_dt, "f32")
            check(y, whole[:, :, t0:t0 + n], in_dt, "f32")
        got_ho = inputs.as_f64(ho, in_dt)
        np.testing.assert_array_equal(got_ho, ref_ho)
        hist, t0 = ho, t0 + n


def test_preprocess_zero_rows_and_zero_weights():
    B, H, T, d, W = 1, 2, 12, 32, 3
    say("case preprocess zeros")
    x = inputs.preprocess_inputs(B, H, T, d, W, "f32", 4200)
    x["x"][0, 0, 3:6] = 0.0      # three zero rows: token 5 sees only zeros
    x["w"][1] = 0.0              # head 1: every output is zero
    y, _ = gpu_pre(x["x"], x["w"], "f32", "f32")
    ref = oracle.qk_preprocess(x["x"].astype(np.float64), x["w"])
    check(y, ref, "f32", "f32")
    assert not y[0, 0, 5].any() and not y[0, 1].any()


def test_preprocess_layer_shape_sampled_heads():
    """The headline layer's q at full size (8 x 16 x 4096, d=128, bf16 -> bf16,
    window 4), in the launch the benchmark times; four heads vs the oracle."""
    B, H, T, d, W = 8, 16, 4096, 128, 4
    say("case preprocess layer shape", (B, H, T, d, W))
    x = inputs.preprocess_inputs(B, H, T, d, W, "bf16", 4300)
    y, _ = gpu_pre(x["x"], x["w"], "bf16", "bf16")
    for (b, h) in ((0, 0), (3, 7), (5, 12), (7, 15)):
        xs = inputs.as_f64(x["x"][b:b + 1, h:h + 1], "bf16")
        ref = oracle.qk_preprocess(xs, x["w"][h:h + 1])
        e = check(y[b:b + 1, h:h + 1], ref, "bf16", "bf16")
        say(f"  head ({b},{h}) rel_l2={e:.2e}")
    n = np.linalg.norm(y, axis=-1)
    assert np.abs(n - 1).max() < 1e-2
