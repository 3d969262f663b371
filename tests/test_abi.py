"""The C ABI of libgsa on the host: every declared symbol is exported, and the
argument checks return the documented status codes before any HIP call.

These tests never hand the library a pointer that a kernel could dereference:
every call either fails validation, or (only on a host without a GPU) stops at
the device check with GSA_ERR_NO_DEVICE.
"""
import ctypes
import os
import re

import pytest

from gated_softmax_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gsa.h")

FAKE = 0x100000  # 16-byte aligned, never dereferenced (validation fails first)
MIS = FAKE + 4   # misaligned


def have_gpu():
    import torch
    return torch.cuda.is_available()


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from gated_softmax_attention_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gsa_[a-z_0-9]+)\s*\(", src)))


def test_header_declarations_match_binding():
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.gsa_version() == 100
    for code, name in [(0, b"GSA_OK"), (1, b"GSA_ERR_INVALID_ARG"), (2, b"GSA_ERR_UNSUPPORTED"),
                       (3, b"GSA_ERR_MISALIGNED"), (4, b"GSA_ERR_WORKSPACE"),
                       (5, b"GSA_ERR_NO_DEVICE"), (6, b"GSA_ERR_HIP"), (99, b"GSA_ERR_UNKNOWN")]:
        assert lib.gsa_status_string(code) == name


def fwd(lib, Q=FAKE, K=FAKE, V=FAKE, G=FAKE, Y=FAKE, B=1, S=8, Hq=4, Hkv=2, D=128, mode=1, dtype=1):
    return lib.gsa_forward(Q, K, V, G, Y, B, S, Hq, Hkv, D, mode, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), _lib.GSA_ERR_INVALID_ARG),
    (dict(Y=None), _lib.GSA_ERR_INVALID_ARG),
    (dict(B=0), _lib.GSA_ERR_INVALID_ARG),
    (dict(S=-3), _lib.GSA_ERR_INVALID_ARG),
    (dict(Hkv=3), _lib.GSA_ERR_INVALID_ARG),
    (dict(mode=7), _lib.GSA_ERR_INVALID_ARG),
    (dict(mode=0), _lib.GSA_ERR_INVALID_ARG),       # G given with mode NONE
    (dict(G=None, mode=1), _lib.GSA_ERR_INVALID_ARG),
    (dict(G=None, mode=2), _lib.GSA_ERR_INVALID_ARG),
    (dict(D=96), _lib.GSA_ERR_UNSUPPORTED),
    (dict(D=256), _lib.GSA_ERR_UNSUPPORTED),
    (dict(dtype=5), _lib.GSA_ERR_UNSUPPORTED),
    (dict(K=MIS), _lib.GSA_ERR_MISALIGNED),
    (dict(G=MIS), _lib.GSA_ERR_MISALIGNED),
])
def test_forward_argument_checks(lib, kw, code):
    assert fwd(lib, **kw) == code
    assert lib.gsa_last_error_message().decode().startswith("gsa_forward")


def test_gate_logits_argument_checks(lib):
    gl = lambda X=FAKE, W=FAKE, G=FAKE, M=4, dm=64, N=8, dt=1, sig=1: lib.gsa_gate_logits(
        X, W, G, M, dm, N, dt, sig, None)
    assert gl(X=None) == _lib.GSA_ERR_INVALID_ARG
    assert gl(M=0) == _lib.GSA_ERR_INVALID_ARG
    assert gl(N=-1) == _lib.GSA_ERR_INVALID_ARG
    assert gl(sig=4) == _lib.GSA_ERR_INVALID_ARG          # not a gsa_activation
    assert gl(sig=-1) == _lib.GSA_ERR_INVALID_ARG
    assert gl(dt=3) == _lib.GSA_ERR_UNSUPPORTED
    assert gl(dm=60) == _lib.GSA_ERR_UNSUPPORTED
    assert gl(W=MIS) == _lib.GSA_ERR_MISALIGNED


def test_decode_argument_checks(lib):
    def dec(Q=FAKE, G=FAKE, B=2, L=100, Hq=8, Hkv=2, D=128, mode=1, dtype=1, ns=0, ws=FAKE, wsb=1 << 30):
        return lib.gsa_decode(Q, FAKE, FAKE, G, FAKE, B, L, Hq, Hkv, D, mode, dtype, ns, ws, wsb, None)
    assert dec(Q=None) == _lib.GSA_ERR_INVALID_ARG
    assert dec(L=0) == _lib.GSA_ERR_INVALID_ARG
    assert dec(Hkv=3) == _lib.GSA_ERR_INVALID_ARG
    assert dec(ns=-1) == _lib.GSA_ERR_INVALID_ARG
    assert dec(G=None) == _lib.GSA_ERR_INVALID_ARG
    assert dec(D=32) == _lib.GSA_ERR_UNSUPPORTED
    assert dec(wsb=16) == _lib.GSA_ERR_WORKSPACE
    assert dec(ws=None) == _lib.GSA_ERR_WORKSPACE
    assert dec(ws=MIS) == _lib.GSA_ERR_MISALIGNED


def test_decode_noalloc_argument_checks(lib):
    def dec(Q=FAKE, G=FAKE, B=2, L=100, Hq=8, Hkv=2, D=128, mode=1, dtype=1, ns=0):
        return lib.gsa_decode_noalloc(Q, FAKE, FAKE, G, FAKE, B, L, Hq, Hkv, D, mode, dtype, ns, None)
    assert lib.gsa_noalloc_scratch_bytes() == 8 << 20
    assert dec(Q=None) == _lib.GSA_ERR_INVALID_ARG
    assert dec(L=0) == _lib.GSA_ERR_INVALID_ARG
    assert dec(Hkv=3) == _lib.GSA_ERR_INVALID_ARG
    assert dec(ns=-1) == _lib.GSA_ERR_INVALID_ARG
    assert dec(G=None) == _lib.GSA_ERR_INVALID_ARG
    assert dec(D=32) == _lib.GSA_ERR_UNSUPPORTED
    assert dec(Q=MIS) == _lib.GSA_ERR_MISALIGNED
    # partials beyond the 8 MiB device scratch are refused before any device call:
    # 64 x 32 heads x 7 splits x 132 floats fit, 8 splits do not
    assert lib.gsa_decode_workspace_bytes(64, 16384, 32, 8, 128, 7) <= 8 << 20
    assert dec(B=64, L=16384, Hq=32, Hkv=8, ns=8) == _lib.GSA_ERR_WORKSPACE
    assert b"scratch" in lib.gsa_last_error_message()
    if not have_gpu():
        assert dec(B=64, L=16384, Hq=32, Hkv=8, ns=7) == _lib.GSA_ERR_NO_DEVICE
        assert dec(dtype=0, B=64, L=16384, Hq=32, Hkv=8, ns=64) == _lib.GSA_ERR_NO_DEVICE  # fp32: no scratch


def test_size_limits(lib):
    # one batch of Q (prefill) above 2 GiB at the float32 size
    assert fwd(lib, S=1 << 20, Hq=8, Hkv=8, D=128) == _lib.GSA_ERR_UNSUPPORTED
    # decode: the limit is the cache's own size (L x Hkv x D), not L x Hq
    dec = lambda L, Hkv: lib.gsa_decode(FAKE, FAKE, FAKE, FAKE, FAKE, 1, L, 32, Hkv, 128, 1, 1, 0, FAKE,
                                        1 << 40, None)
    assert dec(1 << 21, 8) == _lib.GSA_ERR_UNSUPPORTED               # 2M x 8 x 128 x 4 B > 2 GiB
    if not have_gpu():
        assert dec(1 << 18, 8) == _lib.GSA_ERR_NO_DEVICE             # 256k x 32 query heads passes


def test_decode_split_arithmetic(lib):
    # requested counts are honoured up to the chunk rounding; every split is non-empty
    for L, ns in [(16384, 16), (1, 0), (1, 4), (63, 0), (1025, 3), (100, 7), (16384, 0)]:
        eff = lib.gsa_decode_num_splits(64, L, 32, 8, 128, ns)
        assert 1 <= eff <= max(ns, eff)
        chunk = -(-L // eff)
        chunk = -(-chunk // 16) * 16
        assert (eff - 1) * chunk < L <= eff * chunk or eff == 1
        assert lib.gsa_decode_workspace_bytes(64, L, 32, 8, 128, ns) == 64 * 32 * eff * (128 + 4) * 4
    assert lib.gsa_decode_num_splits(0, 10, 4, 4, 128, 0) == 0
    assert lib.gsa_decode_workspace_bytes(2, 10, 4, 3, 128, 0) == 0


def bwd(lib, X=FAKE, W=FAKE, G=FAKE, Q=FAKE, LSE=FAKE, dX=FAKE, dW=FAKE, dQ=FAKE, B=1, S=8, Hq=8, Hkv=2,
        D=128, dm=64, mode=1, dtype=1, ws=FAKE, wsb=1 << 30):
    return lib.gsa_backward(X, W, G, Q, FAKE, FAKE, FAKE, LSE, FAKE, dX, dW, dQ, FAKE, FAKE,
                            B, S, Hq, Hkv, D, dm, mode, dtype, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), _lib.GSA_ERR_INVALID_ARG),
    (dict(LSE=None), _lib.GSA_ERR_INVALID_ARG),
    (dict(dQ=None), _lib.GSA_ERR_INVALID_ARG),
    (dict(X=None), _lib.GSA_ERR_INVALID_ARG),          # gate without X
    (dict(dW=None), _lib.GSA_ERR_INVALID_ARG),
    (dict(G=None, mode=0), _lib.GSA_ERR_INVALID_ARG),  # no gate but X, W, dX, dW given
    (dict(Hkv=3), _lib.GSA_ERR_INVALID_ARG),
    (dict(dm=0), _lib.GSA_ERR_INVALID_ARG),
    (dict(dtype=0), _lib.GSA_ERR_UNSUPPORTED),         # fp32 backward
    (dict(D=96), _lib.GSA_ERR_UNSUPPORTED),
    (dict(dm=60), _lib.GSA_ERR_UNSUPPORTED),
    (dict(Hq=4, Hkv=4, mode=2), _lib.GSA_ERR_UNSUPPORTED),   # headwise gate width 4
    (dict(dX=MIS), _lib.GSA_ERR_MISALIGNED),
    (dict(ws=MIS), _lib.GSA_ERR_MISALIGNED),
    (dict(LSE=FAKE + 2), _lib.GSA_ERR_MISALIGNED),
    (dict(wsb=16), _lib.GSA_ERR_WORKSPACE),
    (dict(ws=None), _lib.GSA_ERR_WORKSPACE),
])
def test_backward_argument_checks(lib, kw, code):
    assert bwd(lib, **kw) == code
    assert lib.gsa_last_error_message().decode().startswith("gsa_backward")


@pytest.mark.skipif("have_gpu()", reason="a GPU is visible: valid-looking fake pointers must not be launched")
def test_backward_no_gate_takes_no_gate_tensors(lib):
    st = lib.gsa_backward(None, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE,
                          FAKE, 1, 8, 8, 2, 128, 0, 0, 1, FAKE, 1 << 30, None)
    assert st == _lib.GSA_ERR_NO_DEVICE


def test_backward_workspace_arithmetic(lib):
    al = lambda x: -(-x // 256) * 256
    B, S, Hq, Hkv, D = 2, 100, 8, 8, 64      # Hkv == Hq: no split GQA groups
    Sp = 128                                 # rows of the statistics: S rounded up to 64
    # no gate: only the per-row statistics (base-2 LSE and D)
    assert lib.gsa_backward_workspace_bytes(B, S, Hq, Hkv, D, 0, 0) == al(2 * B * Hq * Sp * 4)
    # gate: dY (bf16), statistics, dZ (bf16), then dW partials
    for mode, N, dm in [(1, Hq * D, 64), (2, Hq, 4096)]:
        got = lib.gsa_backward_workspace_bytes(B, S, Hq, Hkv, D, dm, mode)
        base = al(B * S * Hq * D * 2) + al(2 * B * Hq * Sp * 4) + al(B * S * N * 2)
        extra = got - base          # 0, or the 256-aligned partial sums of k > 1 token chunks
        assert extra == 0 or any(extra == al(k * dm * N * 4) for k in range(2, 1025)), extra
    # a GQA group split across workgroups adds float32 partial dK and dV
    stat1 = al(2 * 8 * Sp * 4)
    ws1 = lib.gsa_backward_workspace_bytes(1, 100, 8, 1, 64, 0, 0)
    assert ws1 > stat1 and (ws1 - stat1) % (2 * 100 * 64 * 4) == 0
    assert lib.gsa_backward_workspace_bytes(0, S, Hq, Hkv, D, 64, 1) == 0
    assert lib.gsa_backward_workspace_bytes(B, S, Hq, 3, D, 64, 1) == 0
    assert lib.gsa_backward_workspace_bytes(B, S, Hq, Hkv, D, 0, 1) == 0
    assert lib.gsa_backward_workspace_bytes(B, S, Hq, Hkv, D, 64, 9) == 0


def test_forward_variant_argument_checks(lib):
    def fv(Q=FAKE, G=FAKE, Y=FAKE, LSE=None, B=1, S=8, Hq=4, Hkv=2, D=128, layout=3, comb=0, norm=1, dtype=1):
        return lib.gsa_forward_variant(Q, FAKE, FAKE, G, Y, LSE, B, S, Hq, Hkv, D, layout, comb, norm, dtype, None)
    assert fv(Q=None) == _lib.GSA_ERR_INVALID_ARG
    assert fv(layout=4) == _lib.GSA_ERR_INVALID_ARG
    assert fv(comb=2) == _lib.GSA_ERR_INVALID_ARG
    assert fv(norm=3) == _lib.GSA_ERR_INVALID_ARG
    assert fv(G=None) == _lib.GSA_ERR_INVALID_ARG           # a gate layout needs G
    assert fv(layout=0) == _lib.GSA_ERR_INVALID_ARG         # no gate but G given
    assert fv(Hkv=3) == _lib.GSA_ERR_INVALID_ARG
    assert fv(D=96) == _lib.GSA_ERR_UNSUPPORTED
    assert fv(Y=MIS) == _lib.GSA_ERR_MISALIGNED
    assert fv(LSE=FAKE + 2) == _lib.GSA_ERR_MISALIGNED
    assert lib.gsa_last_error_message().decode().startswith("gsa_forward_variant")


def test_decode_variant_argument_checks(lib):
    need = lib.gsa_decode_workspace_bytes(2, 64, 4, 2, 128, 0)

    def dv(Q=FAKE, G=FAKE, Y=FAKE, B=2, L=64, Hq=4, Hkv=2, D=128, layout=3, comb=1, norm=1, dtype=1, ns=0,
           ws=FAKE, wsb=None):
        return lib.gsa_decode_variant(Q, FAKE, FAKE, G, Y, B, L, Hq, Hkv, D, layout, comb, norm, dtype, ns, ws,
                                      need if wsb is None else wsb, None)
    assert dv(Q=None) == _lib.GSA_ERR_INVALID_ARG
    assert dv(layout=-1) == _lib.GSA_ERR_INVALID_ARG
    assert dv(comb=7) == _lib.GSA_ERR_INVALID_ARG
    assert dv(norm=2) == _lib.GSA_ERR_INVALID_ARG
    assert dv(G=None) == _lib.GSA_ERR_INVALID_ARG           # a gate layout needs G
    assert dv(layout=0) == _lib.GSA_ERR_INVALID_ARG         # no gate but G given
    assert dv(L=0) == _lib.GSA_ERR_INVALID_ARG
    assert dv(Hkv=3) == _lib.GSA_ERR_INVALID_ARG
    assert dv(ns=-1) == _lib.GSA_ERR_INVALID_ARG
    assert dv(D=32) == _lib.GSA_ERR_UNSUPPORTED
    assert dv(dtype=5) == _lib.GSA_ERR_UNSUPPORTED
    assert dv(wsb=need - 1) == _lib.GSA_ERR_WORKSPACE      # bf16 needs the split workspace
    assert dv(ws=None) == _lib.GSA_ERR_WORKSPACE
    assert dv(Y=MIS) == _lib.GSA_ERR_MISALIGNED
    assert dv(ws=MIS) == _lib.GSA_ERR_MISALIGNED
    assert lib.gsa_last_error_message().decode().startswith("gsa_decode_variant")
    # float32 takes no workspace: with valid arguments only the device check
    # remains (asked only where no GPU is visible, so the fake pointers are never launched)
    if not have_gpu():
        assert dv(dtype=0, ws=None, wsb=0) == _lib.GSA_ERR_NO_DEVICE


def test_value_gate_argument_checks(lib):
    def vg(V=FAKE, G=FAKE, Vo=FAKE, B=1, S=8, Hkv=2, D=128, layout=1, dtype=1):
        return lib.gsa_value_gate(V, G, Vo, B, S, Hkv, D, layout, dtype, None)
    assert vg(V=None) == _lib.GSA_ERR_INVALID_ARG
    assert vg(S=0) == _lib.GSA_ERR_INVALID_ARG
    assert vg(layout=0) == _lib.GSA_ERR_INVALID_ARG
    assert vg(layout=3) == _lib.GSA_ERR_INVALID_ARG
    assert vg(D=32) == _lib.GSA_ERR_UNSUPPORTED
    assert vg(dtype=9) == _lib.GSA_ERR_UNSUPPORTED
    assert vg(G=MIS) == _lib.GSA_ERR_MISALIGNED
    assert lib.gsa_last_error_message().decode().startswith("gsa_value_gate")


def test_project_qkvg_argument_checks(lib):
    def pj(X=FAKE, W=FAKE, Q=FAKE, G=FAKE, M=16, dm=64, Hq=4, Hkv=2, D=128, ng=512, dtype=1):
        return lib.gsa_project_qkvg(X, W, Q, FAKE, FAKE, G, M, dm, Hq, Hkv, D, ng, dtype, None)
    assert pj(X=None) == _lib.GSA_ERR_INVALID_ARG
    assert pj(Q=None) == _lib.GSA_ERR_INVALID_ARG
    assert pj(M=0) == _lib.GSA_ERR_INVALID_ARG
    assert pj(ng=-8) == _lib.GSA_ERR_INVALID_ARG
    assert pj(Hkv=3) == _lib.GSA_ERR_INVALID_ARG
    assert pj(G=None) == _lib.GSA_ERR_INVALID_ARG            # gate columns but no G
    assert pj(ng=0) == _lib.GSA_ERR_INVALID_ARG              # G given without gate columns
    assert pj(dtype=0) == _lib.GSA_ERR_UNSUPPORTED
    assert pj(dm=60) == _lib.GSA_ERR_UNSUPPORTED
    assert pj(ng=4) == _lib.GSA_ERR_UNSUPPORTED
    assert pj(W=MIS) == _lib.GSA_ERR_MISALIGNED
    assert lib.gsa_last_error_message().decode().startswith("gsa_project_qkvg")


def test_gate_head_mean_argument_checks(lib):
    def hm(G=FAKE, Gs=FAKE + (1 << 24), M=8, Hq=4, D=64):
        return lib.gsa_gate_head_mean(G, Gs, M, Hq, D, None)
    assert hm(G=None) == _lib.GSA_ERR_INVALID_ARG
    assert hm(M=0) == _lib.GSA_ERR_INVALID_ARG
    assert hm(Hq=-1) == _lib.GSA_ERR_INVALID_ARG
    assert hm(D=6) == _lib.GSA_ERR_UNSUPPORTED
    assert hm(Hq=5000) == _lib.GSA_ERR_UNSUPPORTED
    assert hm(Gs=FAKE + (1 << 24) + 4) == _lib.GSA_ERR_MISALIGNED
    assert hm(Gs=FAKE + 16) == _lib.GSA_ERR_INVALID_ARG          # overlaps G
    assert hm(Gs=FAKE) == _lib.GSA_ERR_INVALID_ARG
    if not have_gpu():
        assert hm() == _lib.GSA_ERR_NO_DEVICE
        assert hm(Gs=FAKE + 8 * 4 * 64 * 4) == _lib.GSA_ERR_NO_DEVICE   # right after G


def test_first_token_attention_argument_checks(lib):
    def fa(Q=FAKE, K=FAKE, LSE=FAKE, F=FAKE, hm=None, B=1, S=8, Hq=4, Hkv=2, D=128, dtype=1):
        return lib.gsa_first_token_attention(Q, K, LSE, F, hm, B, S, Hq, Hkv, D, dtype, None)
    assert fa(Q=None) == _lib.GSA_ERR_INVALID_ARG
    assert fa(LSE=None) == _lib.GSA_ERR_INVALID_ARG
    assert fa(F=None) == _lib.GSA_ERR_INVALID_ARG
    assert fa(S=0) == _lib.GSA_ERR_INVALID_ARG
    assert fa(Hkv=3) == _lib.GSA_ERR_INVALID_ARG
    assert fa(D=32) == _lib.GSA_ERR_UNSUPPORTED
    assert fa(dtype=4) == _lib.GSA_ERR_UNSUPPORTED
    assert fa(K=MIS) == _lib.GSA_ERR_MISALIGNED
    assert fa(F=FAKE + 2) == _lib.GSA_ERR_MISALIGNED
    assert fa(hm=FAKE + 1) == _lib.GSA_ERR_MISALIGNED
    assert lib.gsa_last_error_message().decode().startswith("gsa_first_token_attention")


@pytest.mark.skipif("have_gpu()", reason="a GPU is visible: valid-looking fake pointers must not be launched")
def test_valid_arguments_without_a_gpu_report_no_device(lib):
    assert fwd(lib) == _lib.GSA_ERR_NO_DEVICE
    assert lib.gsa_gate_logits(FAKE, FAKE, FAKE, 4, 64, 8, 1, 1, None) == _lib.GSA_ERR_NO_DEVICE
    assert "device" in lib.gsa_last_error_message().decode()


def test_python_binding_refuses_cpu_tensors():
    import torch
    import gated_softmax_attention_amd as gsa
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    w = torch.zeros(64, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        gsa.gate_logits(x, w, G=torch.zeros(4, 8))


def test_error_messages_are_per_thread(lib):
    """Calls are thread-safe and the last-error message is per thread: threads
    making different invalid calls each read back their own message."""
    import threading
    results = {}

    def work(i):
        msgs = []
        for _ in range(200):
            if i % 3 == 0:
                st = fwd(lib, D=96)                                   # unsupported head dim
                want = "gsa_forward"
            elif i % 3 == 1:
                st = lib.gsa_gate_logits(FAKE, FAKE, FAKE, 4, 60, 8, 1, 1, None)   # d_model % 8
                want = "gsa_gate_logits"
            else:
                st = bwd(lib, dtype=0)                                # fp32 backward
                want = "gsa_backward"
            msgs.append((st, lib.gsa_last_error_message().decode().startswith(want)))
        results[i] = msgs

    threads = [threading.Thread(target=work, args=(i,)) for i in range(9)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for i, msgs in results.items():
        assert all(st == _lib.GSA_ERR_UNSUPPORTED and ok for st, ok in msgs), i


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    # the binding has no fallback path: without libgsa.so every call raises
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not found"):
        _lib.load(str(tmp_path / "libgsa.so"))


def test_gate_logits_ws_argument_checks(lib):
    def gw(X=FAKE, G=FAKE, M=64, dm=4096, N=4096, dt=1, act=1, ws=FAKE, wsb=1 << 30):
        return lib.gsa_gate_logits_ws(X, FAKE, G, M, dm, N, dt, act, ws, wsb, None)
    need = lib.gsa_gate_logits_workspace_bytes(64, 4096, 4096, 1)
    assert need == 4 * 64 * 4096 * 4
    assert lib.gsa_gate_logits_workspace_bytes(64, 4096, 4096, 0) == 0        # float32: one pass
    assert lib.gsa_gate_logits_workspace_bytes(0, 4096, 4096, 1) == 0
    assert gw(X=None) == _lib.GSA_ERR_INVALID_ARG
    assert gw(act=9) == _lib.GSA_ERR_INVALID_ARG
    assert gw(ws=None) == _lib.GSA_ERR_WORKSPACE
    assert gw(wsb=need - 1) == _lib.GSA_ERR_WORKSPACE
    assert gw(ws=MIS) == _lib.GSA_ERR_MISALIGNED
    # no split-K for this shape: the call is gsa_gate_logits (its checks apply)
    assert gw(M=8192, dm=60) == _lib.GSA_ERR_UNSUPPORTED
    if not have_gpu():
        assert gw() == _lib.GSA_ERR_NO_DEVICE
        assert gw(M=8192, dm=2048, N=2048, ws=None, wsb=0) == _lib.GSA_ERR_NO_DEVICE


def test_forward_value_gated_argument_checks(lib):
    def fv(Gv=FAKE, layout=1, D=128, dt=1, Hkv=2, lse=None):
        return lib.gsa_forward_value_gated(FAKE, FAKE, FAKE, Gv, FAKE, lse, 1, 64, 4, Hkv, D, layout, dt, None)
    assert fv(Gv=None) == _lib.GSA_ERR_INVALID_ARG
    assert fv(layout=0) == _lib.GSA_ERR_INVALID_ARG
    assert fv(layout=3) == _lib.GSA_ERR_INVALID_ARG
    assert fv(Hkv=3) == _lib.GSA_ERR_INVALID_ARG
    assert fv(D=96) == _lib.GSA_ERR_UNSUPPORTED
    assert fv(dt=5) == _lib.GSA_ERR_UNSUPPORTED
    assert fv(Gv=MIS) == _lib.GSA_ERR_MISALIGNED
    assert fv(lse=FAKE + 2) == _lib.GSA_ERR_MISALIGNED
    if not have_gpu():
        assert fv() == _lib.GSA_ERR_NO_DEVICE
        assert fv(layout=2, D=64, dt=0, lse=FAKE) == _lib.GSA_ERR_NO_DEVICE


def test_gated_decode_argument_checks(lib):
    def gd(X=FAKE, W=FAKE, Q=FAKE, mode=1, D=128, dt=1, dm=4096, ns=0, ws=FAKE, wsb=1 << 30, B=64, L=16384):
        return lib.gsa_gated_decode(X, W, Q, FAKE, FAKE, FAKE, B, L, 32, 8, D, dm, mode, dt, ns, ws, wsb, None)
    ws = lambda **k: lib.gsa_gated_decode_workspace_bytes(
        k.get("B", 64), k.get("L", 16384), 32, 8, k.get("D", 128), k.get("dm", 4096), k.get("mode", 1),
        k.get("dt", 1), 0)
    dec = lib.gsa_decode_workspace_bytes(64, 16384, 32, 8, 128, 0)
    base = (dec + 255) // 256 * 256
    # the split-K gate parts (4 parts of 64 x 4096 floats), then G, after the decode partials
    assert ws() == base + 4 * 64 * 4096 * 4 + 64 * 4096 * 4
    # headwise, float32: one G after the decode partials (float32 decode has none)
    assert ws(mode=2) == base + 64 * 32 * 4
    assert ws(dt=0) == 64 * 4096 * 4
    assert ws(mode=0) == dec
    assert ws(mode=7) == 0 and ws(B=0) == 0
    assert gd(X=None) == _lib.GSA_ERR_INVALID_ARG
    assert gd(mode=0) == _lib.GSA_ERR_INVALID_ARG              # X and W given without a gate
    assert gd(Q=None) == _lib.GSA_ERR_INVALID_ARG
    assert gd(ns=-1) == _lib.GSA_ERR_INVALID_ARG
    assert gd(dm=0) == _lib.GSA_ERR_INVALID_ARG
    assert gd(dm=4100) == _lib.GSA_ERR_UNSUPPORTED
    assert gd(dm=1 << 40) == _lib.GSA_ERR_INVALID_ARG
    assert gd(D=96) == _lib.GSA_ERR_UNSUPPORTED
    assert gd(ws=None) == _lib.GSA_ERR_WORKSPACE
    assert gd(wsb=ws() - 1) == _lib.GSA_ERR_WORKSPACE
    assert gd(ws=MIS) == _lib.GSA_ERR_MISALIGNED
    assert gd(X=MIS) == _lib.GSA_ERR_MISALIGNED
    if not have_gpu():
        assert gd() == _lib.GSA_ERR_NO_DEVICE
        assert gd(X=None, W=None, mode=0) == _lib.GSA_ERR_NO_DEVICE
        assert gd(mode=2, D=64, dt=0, B=2, L=100) == _lib.GSA_ERR_NO_DEVICE
