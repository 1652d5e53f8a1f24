"""GPU parity of the Hawk layer's recurrence (mesa_hawk_scan) against the
fp64 oracle.  Section "Arquitetura (MesaNet)", bullet "Variante Hibrida" of
the MesaNet summary page: the hybrid alternates LRU (Hawk) layers with Mesa
layers; the recurrence is Hawk's published real-gated LRU.  Outputs and final
states must match within relative L2 2e-3 (float32 inputs) or 1e-2
(bfloat16 inputs, compared on their rounded values)."""
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


def run(xin, dtype, c=8.0):
    import torch
    from test_regression_amd import mesa
    x, ga, gx = (to_dev(xin[n], dtype) for n in ("x", "ga", "gx"))
    lam = to_dev(xin["lam"], "f32")
    h0 = None if xin["h0"] is None else to_dev(xin["h0"], "f32")
    y, hf = mesa.mesa_hawk_scan(x, ga, gx, lam, c, h0, return_final=True)
    torch.cuda.synchronize()
    ref_y, ref_h = oracle.hawk_scan(*(inputs.as_f64(xin[n], dtype) for n in ("x", "ga", "gx")), xin["lam"], c,
                                    xin["h0"])
    return y.cpu().numpy(), hf.cpu().numpy(), ref_y, ref_h


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 100, 256, 257, 1000])
@pytest.mark.parametrize("D", [1, 7, 64, 300])
def test_hawk_shapes(D, T, dtype):
    seed = 6000 + D + T
    say("case hawk", dict(D=D, T=T, dtype=dtype, seed=seed))
    for with_h0 in (False, True):
        xin = inputs.hawk_inputs(2, T, D, dtype, seed, with_h0=with_h0)
        y, hf, ry, rh = run(xin, dtype)
        assert rel_l2(y, ry) <= RTOL[dtype] and rel_l2(hf, rh) <= RTOL[dtype]
        assert np.abs(y - ry).max() <= 1e-4 * max(1.0, np.abs(ry).max())


# Shapes with at least 128 blocks of 64 channels take the one-pass schedule
# (a workgroup per block, rounds of 16 x 8 tokens); the ones above take the
# two-pass chunked scan.  Ragged D leaves lanes of the last block idle, and
# ragged T ends inside a round and inside a wave's segment.
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,D", [(2, 1, 4096), (2, 127, 4039), (2, 300, 4096), (2, 1000, 4039), (128, 257, 64),
                                   (130, 129, 70)])
def test_hawk_one_pass_shapes(B, T, D, dtype):
    seed = 6300 + B + T + D
    say("case hawk one pass", dict(B=B, D=D, T=T, dtype=dtype, seed=seed))
    for with_h0 in (False, True):
        xin = inputs.hawk_inputs(B, T, D, dtype, seed, with_h0=with_h0)
        y, hf, ry, rh = run(xin, dtype)
        e, eh = rel_l2(y, ry), rel_l2(hf, rh)
        say(f"  h0={with_h0} rel_l2 y={e:.2e} h_final={eh:.2e}")
        assert e <= RTOL[dtype] and eh <= RTOL[dtype]
        assert np.abs(y - ry).max() <= 1e-4 * max(1.0, np.abs(ry).max())


def test_hawk_one_pass_closed_gates_keep_the_state():
    say("case hawk one pass closed gates")
    xin = inputs.hawk_inputs(2, 300, 4096, "f32", 6400, with_h0=True)
    xin["ga"][:] = -60.0
    y, hf, ry, rh = run(xin, "f32")
    np.testing.assert_allclose(y, np.broadcast_to(xin["h0"][:, None, :], y.shape), rtol=1e-6)
    np.testing.assert_allclose(hf, xin["h0"], rtol=1e-6)


def test_hawk_closed_gates_keep_the_state_and_empty_sequence():
    import torch
    from test_regression_amd import mesa
    say("case hawk closed gates")
    xin = inputs.hawk_inputs(2, 300, 16, "f32", 6100, with_h0=True)
    xin["ga"][:] = -60.0
    y, hf, ry, rh = run(xin, "f32")
    np.testing.assert_allclose(y, np.broadcast_to(xin["h0"][:, None, :], y.shape), rtol=1e-6)
    say("case hawk T=0")
    h0 = torch.randn((2, 16), device="cuda")
    e = torch.empty((2, 0, 16), dtype=torch.float32, device="cuda")
    _, hf = mesa.mesa_hawk_scan(e, e, e, torch.zeros(16, device="cuda"), 8.0, h0, return_final=True)
    torch.cuda.synchronize()
    assert torch.equal(hf, h0)


def test_hawk_layer_workload_full():
    """8 sequences x 4096 tokens x 2048 channels, bf16 inputs (the width of the
    headline Mesa layer, 16 heads x 128), every output against the oracle."""
    say("case hawk layer (8, 4096, 2048) bf16")
    xin = inputs.hawk_inputs(8, 4096, 2048, "bf16", 6200, with_h0=True)
    y, hf, ry, rh = run(xin, "bf16")
    e, eh = rel_l2(y, ry), rel_l2(hf, rh)
    say(f"  rel_l2 y={e:.2e} h_final={eh:.2e}")
    assert e <= RTOL["bf16"] and eh <= RTOL["bf16"]
