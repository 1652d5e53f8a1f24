"""The C ABI of libmesa on the CPU: it loads, exports every symbol the header
declares, and rejects bad arguments on the host before touching the device.

The pointers passed here are fake (never dereferenced): every call below
fails validation, so no HIP call is made and no GPU is needed.
"""
import ctypes
import os
import re

import pytest

from test_regression_amd import mesa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("mesa.h", "mesa_probe.h")]

OK, INVALID, UNSUPPORTED, WS_SMALL, HIPERR = range(5)
FAKE = 0x10000          # 16-byte aligned, never dereferenced


def header_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(mesa_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = mesa.lib()
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
        assert n in mesa.SIGNATURES, f"binding lacks {n}"
    assert set(mesa.SIGNATURES) == set(names)


def test_version_and_status_strings():
    L = mesa.lib()
    assert L.mesa_abi_version() == 1
    for s, name in [(OK, b"MESA_OK"), (INVALID, b"MESA_ERR_INVALID_ARGUMENT"),
                    (UNSUPPORTED, b"MESA_ERR_UNSUPPORTED"), (WS_SMALL, b"MESA_ERR_WORKSPACE_TOO_SMALL"),
                    (HIPERR, b"MESA_ERR_HIP")]:
        assert L.mesa_status_string(s) == name
    assert L.mesa_status_string(99) == b"MESA_ERR_UNKNOWN"
    assert [mesa.kernel_name(i) for i in range(8)] == [
        "chunk_states_kernel", "cg_output_kernel", "decode_kernel", "qk_preprocess_kernel", "bwd_adjoint_kernel",
        "bwd_states_kernel", "bwd_kv_kernel", "bwd_gate_kernel"]
    assert mesa.kernel_name(8) == "hawk_kernels"


def test_workspace_bytes():
    f = mesa.mesa_forward_workspace_bytes
    per_chunk = lambda d: d * (d + 16) // 2 + d * d   # packed upper H blocks + full G
    tail = 256                                         # chunk-claim counter of the CG kernel
    assert f(8, 16, 4096, 128, 128, 64) == 8 * 16 * 64 * per_chunk(128) * 4 + tail
    assert f(1, 1, 65, 16, 16, 64) == 2 * per_chunk(16) * 4 + tail   # ragged: 2 chunks
    assert f(1, 1, 0, 16, 16, 64) == 0
    assert f(0, 1, 10, 16, 16, 64) == 0 and f(1, 1, 10, 16, 16, 0) == 0


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=0, gamma=FAKE, lam=FAKE, B=1, H=2, T=128, dk=64, dv=64,
             chunk=64, max_iters=5, tol=0.0, out=FAKE, iters=FAKE, fH=None, fG=None, ws=FAKE,
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    L = mesa.lib()
    st = L.mesa_forward(a["q"], a["k"], a["v"], a["dtype"], a["gamma"], a["lam"], a["B"], a["H"],
                        a["T"], a["dk"], a["dv"], a["chunk"], a["max_iters"], ctypes.c_float(a["tol"]),
                        a["out"], a["iters"], a["fH"], a["fG"], a["ws"], a["ws_bytes"], a["stream"])
    return st, L.mesa_last_error_message().decode()


def dec(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=0, gamma=FAKE, lam=FAKE, SH=FAKE, SG=FAKE, N=4, H=2,
             dk=64, dv=64, max_iters=5, tol=1e-4, out=FAKE, iters=FAKE, stream=None)
    a.update(kw)
    L = mesa.lib()
    st = L.mesa_decode_step(a["q"], a["k"], a["v"], a["dtype"], a["gamma"], a["lam"], a["SH"], a["SG"],
                            a["N"], a["H"], a["dk"], a["dv"], a["max_iters"], ctypes.c_float(a["tol"]),
                            a["out"], a["iters"], a["stream"])
    return st, L.mesa_last_error_message().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), INVALID, "non-null"),
    (dict(v=None), INVALID, "non-null"),
    (dict(gamma=None), INVALID, "non-null"),
    (dict(lam=None), INVALID, "lambda"),
    (dict(out=None), INVALID, "non-null"),
    (dict(ws=None), INVALID, "workspace"),
    (dict(dtype=7), INVALID, "qkv_dtype"),
    (dict(B=0), INVALID, "positive"),
    (dict(H=-1), INVALID, "positive"),
    (dict(T=-5), INVALID, "positive"),
    (dict(chunk=0), INVALID, "positive"),
    (dict(max_iters=-1), INVALID, "max_iters"),
    (dict(max_iters=5000), INVALID, "max_iters"),
    (dict(tol=-1e-3), INVALID, "tol"),
    (dict(tol=float("nan")), INVALID, "tol"),
    (dict(tol=float("inf")), INVALID, "tol"),
    (dict(q=FAKE + 4), INVALID, "misaligned"),
    (dict(ws=FAKE + 8), INVALID, "misaligned"),
    (dict(gamma=FAKE + 2), INVALID, "misaligned"),
    (dict(dk=64, dv=32), UNSUPPORTED, "dv"),
    (dict(dk=48, dv=48), UNSUPPORTED, "d=48"),
    (dict(dk=256, dv=256), UNSUPPORTED, "d=256"),
    (dict(chunk=128), UNSUPPORTED, "chunk"),
    (dict(chunk=8), UNSUPPORTED, "chunk"),
    (dict(ws_bytes=1000), WS_SMALL, "workspace"),
])
def test_forward_rejects_bad_arguments(kw, status, needle):
    st, msg = fwd(**kw)
    assert st == status, (st, msg)
    assert needle in msg


def test_forward_workspace_optional_without_iterations():
    # max_iters == 0 needs no workspace; with a bad dtype it still fails in validation
    st, msg = fwd(ws=None, ws_bytes=0, max_iters=0, dtype=9)
    assert st == INVALID and "qkv_dtype" in msg
    st, msg = fwd(ws=None, ws_bytes=0, max_iters=0, dk=48, dv=48)
    assert st == UNSUPPORTED


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), INVALID, "non-null"),
    (dict(SH=None), INVALID, "non-null"),
    (dict(SG=None), INVALID, "non-null"),
    (dict(lam=None), INVALID, "non-null"),
    (dict(dtype=3), INVALID, "qkv_dtype"),
    (dict(N=0), INVALID, "positive"),
    (dict(max_iters=-2), INVALID, "max_iters"),
    (dict(tol=float("nan")), INVALID, "tol"),
    (dict(SH=FAKE + 4), INVALID, "misaligned"),
    (dict(iters=FAKE + 1), INVALID, "misaligned"),
    (dict(dk=128, dv=64), UNSUPPORTED, "dv"),
    (dict(dk=8, dv=8), UNSUPPORTED, "d=8"),
])
def test_decode_rejects_bad_arguments(kw, status, needle):
    st, msg = dec(**kw)
    assert st == status, (st, msg)
    assert needle in msg


def dec_warm(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=0, gamma=FAKE, lam=FAKE, SH=FAKE, SG=FAKE, SX=FAKE, N=4, H=2,
             dk=64, dv=64, max_iters=5, tol=1e-4, mode=2, out=FAKE, iters=FAKE, stream=None)
    a.update(kw)
    L = mesa.lib()
    st = L.mesa_decode_step_warm(a["q"], a["k"], a["v"], a["dtype"], a["gamma"], a["lam"], a["SH"], a["SG"],
                                 a["SX"], a["N"], a["H"], a["dk"], a["dv"], a["max_iters"],
                                 ctypes.c_float(a["tol"]), a["mode"], a["out"], a["iters"], a["stream"])
    return st, L.mesa_last_error_message().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(SX=None), INVALID, "state_x"),
    (dict(mode=3), INVALID, "warm_mode"),
    (dict(mode=-1), INVALID, "warm_mode"),
    (dict(SX=FAKE + 4), INVALID, "misaligned"),
    (dict(SH=None), INVALID, "non-null"),
    (dict(N=0), INVALID, "positive"),
    (dict(tol=-1.0), INVALID, "tol"),
    (dict(dk=48, dv=48), UNSUPPORTED, "d=48"),
])
def test_warm_decode_rejects_bad_arguments(kw, status, needle):
    st, msg = dec_warm(**kw)
    assert st == status, (st, msg)
    assert needle in msg


def pre(**kw):
    a = dict(x=FAKE, dt=0, w=FAKE, W=4, hist=None, hist_out=None, B=2, H=2, T=10, d=64, y=FAKE + 4096,
             odt=0, stream=None)
    a.update(kw)
    L = mesa.lib()
    st = L.mesa_qk_preprocess(a["x"], a["dt"], a["w"], a["W"], a["hist"], a["hist_out"], a["B"], a["H"], a["T"],
                              a["d"], a["y"], a["odt"], a["stream"])
    return st, L.mesa_last_error_message().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(w=None), INVALID, "conv_w"),
    (dict(x=None), INVALID, "non-null"),
    (dict(y=None), INVALID, "non-null"),
    (dict(W=0), INVALID, "width"),
    (dict(W=9), INVALID, "width"),
    (dict(dt=2), INVALID, "dtype"),
    (dict(odt=-1), INVALID, "dtype"),
    (dict(B=0), INVALID, "positive"),
    (dict(T=-1), INVALID, "T >= 0"),
    (dict(x=FAKE + 8), INVALID, "misaligned"),
    (dict(hist=FAKE + 4), INVALID, "misaligned"),
    (dict(y=FAKE), INVALID, "alias"),
    (dict(hist=FAKE + 8192, hist_out=FAKE + 8192), INVALID, "alias"),
    (dict(d=48), UNSUPPORTED, "d=48"),
    (dict(W=5), UNSUPPORTED, "width=5"),
])
def test_preprocess_rejects_bad_arguments(kw, status, needle):
    st, msg = pre(**kw)
    assert st == status, (st, msg)
    assert needle in msg


def test_preprocess_empty_piece_is_a_no_op():
    # T = 0 with no history to carry launches nothing; x and y may be NULL
    st, msg = pre(x=None, y=None, T=0)
    assert st == 0, msg


def bwd(**kw):
    a = dict(k=FAKE, v=FAKE, dt=0, gamma=FAKE, lam=FAKE, x=FAKE, out=FAKE, gout=FAKE, B=1, H=2, T=128, dk=64,
             dv=64, chunk=64, max_iters=5, tol=0.0, gq=FAKE, gk=FAKE, gv=FAKE, gg=FAKE, gl=FAKE, zi=None, ws=FAKE,
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    L = mesa.lib()
    st = L.mesa_backward(a["k"], a["v"], a["dt"], a["gamma"], a["lam"], a["x"], a["out"], a["gout"], a["B"], a["H"],
                         a["T"], a["dk"], a["dv"], a["chunk"], a["max_iters"], ctypes.c_float(a["tol"]), a["gq"],
                         a["gk"], a["gv"], a["gg"], a["gl"], a["zi"], a["ws"], a["ws_bytes"], a["stream"])
    return st, L.mesa_last_error_message().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(x=None), INVALID, "non-null"),
    (dict(gout=None), INVALID, "non-null"),
    (dict(gl=None), INVALID, "grad_lambda"),
    (dict(ws=None), INVALID, "workspace"),
    (dict(dt=5), INVALID, "qkv_dtype"),
    (dict(T=-1), INVALID, "positive"),
    (dict(max_iters=-1), INVALID, "max_iters"),
    (dict(tol=float("nan")), INVALID, "tol"),
    (dict(x=FAKE + 4), INVALID, "misaligned"),
    (dict(gg=FAKE + 2), INVALID, "misaligned"),
    (dict(dk=64, dv=32), UNSUPPORTED, "dv"),
    (dict(dk=48, dv=48), UNSUPPORTED, "d=48"),
    (dict(chunk=128), UNSUPPORTED, "chunk"),
    (dict(ws_bytes=1000), WS_SMALL, "workspace"),
])
def test_backward_rejects_bad_arguments(kw, status, needle):
    st, msg = bwd(**kw)
    assert st == status, (st, msg)
    assert needle in msg


def test_backward_workspace_bytes():
    f = mesa.lib().mesa_backward_workspace_bytes
    r4 = lambda n: (n + 3) // 4 * 4
    B, H, T, d, C = 2, 3, 130, 64, 64
    nc = 3
    waves = C // 16   # per-wave partial sums of z (.) x per chunk
    want = (r4(B * H * nc * d * (d + 16) // 2) + 3 * r4(B * H * nc * d * d)
            + 2 * r4(B * H * nc * (d // 16))   # the reverse states' exponents per 16-row block
            + 2 * r4(B * H * T)
            + r4(B * H * nc * waves * d) + 64) * 4   # + the 256-byte chunk-claim counter
    assert f(B, H, T, d, d, C) == want
    assert f(0, H, T, d, d, C) == 0 and f(B, H, T, d, d, 0) == 0


def test_forward_train_requires_x_out():
    L = mesa.lib()
    st = L.mesa_forward_train(FAKE, FAKE, FAKE, 0, FAKE, FAKE, 1, 2, 128, 64, 64, 64, 5, ctypes.c_float(0.0),
                              FAKE, None, None, FAKE, 1 << 40, None)
    assert st == INVALID and "x_out" in L.mesa_last_error_message().decode()


def hawk(**kw):
    a = dict(x=FAKE, ga=FAKE, gx=FAKE, dt=0, lam=FAKE, c=8.0, h0=None, B=2, T=100, D=64, y=FAKE + 65536, hf=None,
             ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    L = mesa.lib()
    st = L.mesa_hawk_scan(a["x"], a["ga"], a["gx"], a["dt"], a["lam"], ctypes.c_float(a["c"]), a["h0"], a["B"],
                          a["T"], a["D"], a["y"], a["hf"], a["ws"], a["ws_bytes"], a["stream"])
    return st, L.mesa_last_error_message().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(x=None), INVALID, "non-null"),
    (dict(lam=None), INVALID, "non-null"),
    (dict(ws=None), INVALID, "non-null"),
    (dict(dt=3), INVALID, "in_dtype"),
    (dict(B=0), INVALID, "positive"),
    (dict(T=-2), INVALID, "T >= 0"),
    (dict(c=-1.0), INVALID, "c must"),
    (dict(c=float("nan")), INVALID, "c must"),
    (dict(x=FAKE + 2), INVALID, "misaligned"),
    (dict(y=FAKE), INVALID, "alias"),
    (dict(ws_bytes=16), WS_SMALL, "workspace"),
])
def test_hawk_rejects_bad_arguments(kw, status, needle):
    st, msg = hawk(**kw)
    assert st == status, (st, msg)
    assert needle in msg


def test_hawk_workspace_bytes():
    f = mesa.lib().mesa_hawk_workspace_bytes
    assert f(2, 257, 64) == 2 * 2 * 3 * 64 * 4     # three chunks of 128 tokens
    assert f(1, 0, 8) == 0 and f(0, 5, 8) == 0


def test_probe_argument_validation():
    L = mesa.lib()
    assert L.mesa_probe_mfma_f32(0, 10, FAKE, None) == INVALID
    assert L.mesa_probe_mfma_bf16(4, 0, FAKE, None) == INVALID
    assert L.mesa_probe_mfma_f32(4, 10, None, None) == INVALID
    assert L.mesa_probe_copy(FAKE, FAKE, 100, None) == INVALID          # not a multiple of 16
    assert L.mesa_probe_copy(FAKE + 4, FAKE, 160, None) == INVALID      # misaligned
    assert L.mesa_probe_copy(None, FAKE, 160, None) == INVALID


def test_profile_api_host_paths():
    L = mesa.lib()
    ms = ctypes.c_double(-1)
    n = ctypes.c_int64(-1)
    assert L.mesa_profile_read(9, ctypes.byref(ms), ctypes.byref(n)) == INVALID
    assert L.mesa_profile_read(-1, ctypes.byref(ms), ctypes.byref(n)) == INVALID
    assert L.mesa_profile_read(0, None, ctypes.byref(n)) == INVALID
    assert L.mesa_profile_reset() == OK
    assert L.mesa_profile_read(1, ctypes.byref(ms), ctypes.byref(n)) == OK
    assert ms.value == 0.0 and n.value == 0


def test_error_message_is_thread_local_and_cleared():
    import threading
    st, msg = fwd(q=None)
    assert st == INVALID and msg
    seen = []
    t = threading.Thread(target=lambda: seen.append(mesa.lib().mesa_last_error_message()))
    t.start()
    t.join()
    assert seen == [b""]
    st, msg = dec(dtype=5)
    assert st == INVALID and "qkv_dtype" in msg


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(mesa, "_lib", None)
    monkeypatch.setattr(mesa, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        mesa.lib()


def test_status_mapping():
    with pytest.raises(ValueError):
        mesa._check(INVALID, "x")
    with pytest.raises(NotImplementedError):
        mesa._check(UNSUPPORTED, "x")
    with pytest.raises(ValueError):
        mesa._check(WS_SMALL, "x")
    with pytest.raises(mesa.MesaError):
        mesa._check(HIPERR, "x")


def _cpu(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=torch.float32 if dtype is None else dtype)


@pytest.mark.parametrize("case", [
    "forward_lambda", "forward_gamma", "forward_k", "forward_out", "train_v", "train_x_out",
    "backward_x", "backward_grad_out", "backward_lambda", "decode_lambda", "decode_k", "decode_gamma",
    "decode_state", "warm_state_x", "preprocess_w", "preprocess_hist", "hawk_lam", "hawk_ga", "hawk_h0",
])
def test_binding_rejects_mis_shaped_tensors(case):
    """Every wrapper checks the shape of every tensor against the sizes it
    passes to the library (which only sees raw pointers), before anything
    else: a mis-shaped tensor is a ValueError and never reaches a kernel."""
    import torch
    from test_regression_amd import mesa
    B, H, T, d = 2, 3, 5, 16
    q = _cpu(B, H, T, d)
    g = _cpu(B, H, T)
    lam = _cpu(H, d)
    calls = {
        "forward_lambda": lambda: mesa.mesa_forward(q, q, q, g, _cpu(d), 3),
        "forward_gamma": lambda: mesa.mesa_forward(q, q, q, _cpu(B, H, T + 1), lam, 3),
        "forward_k": lambda: mesa.mesa_forward(q, _cpu(B, H, T, 2 * d), q, g, lam, 3),
        "forward_out": lambda: mesa.mesa_forward(q, q, q, g, lam, 3, out=_cpu(B, H, T, d + 1)),
        "train_v": lambda: mesa.mesa_forward_train(q, q, _cpu(B, H, T - 1, d), g, lam, 3),
        "train_x_out": lambda: mesa.mesa_forward_train(q, q, q, g, lam, 3, x_out=_cpu(B, H, d)),
        "backward_x": lambda: mesa.mesa_backward(q, q, g, lam, _cpu(B, H, T, d + 2), q, q, 3),
        "backward_grad_out": lambda: mesa.mesa_backward(q, q, g, lam, q, q, _cpu(B, 1, T, d), 3),
        "backward_lambda": lambda: mesa.mesa_backward(q, q, g, _cpu(1, d), q, q, q, 3),
        "decode_lambda": lambda: mesa.mesa_decode_step(_cpu(B, H, d), _cpu(B, H, d), _cpu(B, H, d), _cpu(B, H),
                                                       _cpu(d), _cpu(B, H, d, d), _cpu(B, H, d, d), 3),
        "decode_k": lambda: mesa.mesa_decode_step(_cpu(B, H, d), _cpu(B, 1, d), _cpu(B, H, d), _cpu(B, H),
                                                  lam, _cpu(B, H, d, d), _cpu(B, H, d, d), 3),
        "decode_gamma": lambda: mesa.mesa_decode_step(_cpu(B, H, d), _cpu(B, H, d), _cpu(B, H, d), _cpu(B),
                                                      lam, _cpu(B, H, d, d), _cpu(B, H, d, d), 3),
        "decode_state": lambda: mesa.mesa_decode_step(_cpu(B, H, d), _cpu(B, H, d), _cpu(B, H, d), _cpu(B, H),
                                                      lam, _cpu(H, B, d, d), _cpu(B, H, d, d), 3),
        "warm_state_x": lambda: mesa.mesa_decode_step_warm(_cpu(B, H, d), _cpu(B, H, d), _cpu(B, H, d),
                                                           _cpu(B, H), lam, _cpu(B, H, d, d), _cpu(B, H, d, d),
                                                           _cpu(B, d), 3),
        "preprocess_w": lambda: mesa.mesa_qk_preprocess(q, _cpu(1, 4, d)),
        "preprocess_hist": lambda: mesa.mesa_qk_preprocess(q, _cpu(H, 4, d), hist=_cpu(B, H, 4, d)),
        "hawk_lam": lambda: mesa.mesa_hawk_scan(_cpu(B, T, d), _cpu(B, T, d), _cpu(B, T, d), _cpu(d + 1)),
        "hawk_ga": lambda: mesa.mesa_hawk_scan(_cpu(B, T, d), _cpu(B, T + 1, d), _cpu(B, T, d), _cpu(d)),
        "hawk_h0": lambda: mesa.mesa_hawk_scan(_cpu(B, T, d), _cpu(B, T, d), _cpu(B, T, d), _cpu(d),
                                               h0=_cpu(1, d)),
    }
    with pytest.raises(ValueError, match="must have shape"):
        calls[case]()
    del torch
