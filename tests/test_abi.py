"""The C-ABI library without a GPU: it loads next to torch's HIP runtime,
exports every function include/ssmdec.h declares, and rejects bad arguments
on the host with the documented status codes before any HIP call. None of
these calls launches anything.
"""
import ctypes
import os
import re

import pytest
import torch

import ssm_recurrent_decode_gated_amd as S
from ssm_recurrent_decode_gated_amd import _binding as Bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssmdec.h")

OK, NULL_ARG, BAD_SHAPE, BAD_DTYPE, UNSUPPORTED = 0, -1, -2, -3, -4


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|int64_t|const char\*)\s+(\w+)\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(Bd.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = S.load_library()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_single_hip_runtime_in_process():
    S.load_library()
    maps = open("/proc/self/maps").read()
    hip = {m for m in re.findall(r"\S*libamdhip64\S*", maps)}
    assert len(hip) == 1, hip


def _gdn(L, **kw):
    """Call gdn_decode_step with fake (never dereferenced) pointers."""
    a = dict(qkv=0x10000, stride=8192, a=0x20000, b=0x30000, A_log=0x40000, dt_bias=0x50000,
             state=0x60000, num_slots=16, idx=0x70000, out=0x80000, B=16, H=16, HV=32, K=128, V=128,
             act=1, odt=1, scale=0.088, l2=1, l2eps=1e-6, ng=None, nw=None, neps=1e-5, nact=0)
    a.update(kw)
    return L.gdn_decode_step(a["qkv"], a["stride"], a["a"], a["b"], a["A_log"], a["dt_bias"], a["state"],
                             a["num_slots"], a["idx"], a["out"], a["B"], a["H"], a["HV"], a["K"], a["V"],
                             a["act"], a["odt"], a["scale"], a["l2"], a["l2eps"], a["ng"], a["nw"],
                             a["neps"], a["nact"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(qkv=None), NULL_ARG),
    (dict(state=None), NULL_ARG),
    (dict(idx=None), NULL_ARG),
    (dict(HV=24, H=16), BAD_SHAPE),
    (dict(H=0), BAD_SHAPE),
    (dict(K=48), UNSUPPORTED),
    (dict(K=512), UNSUPPORTED),
    (dict(V=0), BAD_SHAPE),
    (dict(V=2048), BAD_SHAPE),
    (dict(num_slots=0), BAD_SHAPE),
    (dict(B=-1), BAD_SHAPE),
    (dict(act=7), BAD_DTYPE),
    (dict(odt=-1), BAD_DTYPE),
    (dict(nact=3), BAD_DTYPE),
    (dict(stride=8191), BAD_SHAPE),      # below 2*H*K + HV*V
    (dict(state=0x60004), BAD_SHAPE),
])
def test_gdn_host_validation(kw, code):
    L = S.load_library()
    assert _gdn(L, **kw) == code
    assert S.ssmd_last_error() != ""


def test_gdn_empty_batch_is_a_noop():
    L = S.load_library()
    assert _gdn(L, B=0, qkv=None, state=None, idx=None, out=None) == OK
    assert S.ssmd_last_error() == ""


def test_buffered_host_validation():
    L = S.load_library()

    def call(L_=8, d=0x90000, wp=0xA0000, K=128, B=4, V=128, gate=None):
        return L.gdn_decode_step_buffered(0x10000, 1 << 16, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000, 16,
                                          0x70000, 0x80000, B, 16, 32, K, V, 1, 1, 0.088, 1, 1e-6, gate,
                                          None, 1e-5, 0, d, 0xB0000, 0xC0000, wp, L_, None)
    assert call(L_=0) == BAD_SHAPE
    assert call(L_=65) == BAD_SHAPE
    assert call(d=None) == NULL_ARG
    assert call(wp=None) == NULL_ARG
    assert call(K=48) == UNSUPPORTED
    assert call(B=0, d=None, wp=None) == OK
    # the ring staging's shared-memory bound, 4 ((L-1)(K + R + 4) + 1 + 2R) <= 61440 bytes
    # (R: 128-row tiles at K = 128, 64 at K = 256, V with the gated norm), checked
    # before anything runs (B = 0 launches nothing either way)
    for K, V, gate, last in ((128, 128, None, 59), (256, 128, None, 48), (128, 1024, 0xD0000, 12)):
        assert call(B=0, L_=last, K=K, V=V, gate=gate) == OK, (K, V, last)
        assert call(B=0, L_=last + 1, K=K, V=V, gate=gate) == UNSUPPORTED, (K, V, last + 1)


def test_kda_host_validation():
    L = S.load_library()

    def call(T=64, H=96, D=128, W=4, x=0x10000, cs=(216 * 128 * 3, 1, 36864), act=1, state=0x60000,
             A_log=None, dt_bias=None):
        return L.kda_decode_step(x, 0x20000, None, 0x30000, cs[0], cs[1], cs[2], 0x40000, 0x50000, A_log,
                                 dt_bias, -5.0, state, 72, 0x70000, 0x80000, 0x90000, None, 1e-5, T, H, D, W,
                                 act, 1, 0.088, 1, 1e-6, None)
    assert call(D=96) == UNSUPPORTED
    assert call(W=1) == BAD_SHAPE
    assert call(W=9) == BAD_SHAPE
    assert call(H=0) == BAD_SHAPE
    assert call(T=-1) == BAD_SHAPE
    assert call(x=None) == NULL_ARG
    assert call(act=5) == BAD_DTYPE
    assert call(cs=(0, 1, 1)) == BAD_SHAPE
    assert call(state=0x60008) == BAD_SHAPE
    assert call(T=0, x=None) == OK
    # A_log / dt_bias have no formula on the pages: refused, also for an empty call
    assert call(A_log=0xA0000) == UNSUPPORTED
    assert "A_log" in S.ssmd_last_error()
    assert call(dt_bias=0xB0000) == UNSUPPORTED
    assert call(A_log=0xA0000, dt_bias=0xB0000, T=0) == UNSUPPORTED


def test_stream_copy_host_validation():
    L = S.load_library()
    assert L.ssmd_stream_copy(None, 0x1000, 16, None) == NULL_ARG
    assert L.ssmd_stream_copy(0x1000, 0x2000, 15, None) == BAD_SHAPE
    assert L.ssmd_stream_copy(0x1008, 0x2000, 16, None) == BAD_SHAPE
    assert L.ssmd_stream_copy(0x1000, 0x2000, 0, None) == OK


def test_binding_rejects_host_tensors():
    import torch
    t = torch.zeros(4, 4)
    with pytest.raises(ValueError, match="device"):
        S.gdn_decode_step(t, t, t, t, t, torch.zeros(1, 1, 4, 4), t, t)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(Bd, "_LIB", None)
    monkeypatch.setattr(Bd, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not built"):
        Bd.load_library()


def test_mamba_host_validation():
    L = S.load_library()

    def call(B=8, Dm=1536, N=16, x=0x10000, A=0x20000, state=0x30000, act=0, slots=8):
        return L.mamba_decode_step(x, 0x11000, A, 0x12000, 0x13000, None, None, state, slots, 0x14000, 0x15000,
                                   B, Dm, N, act, 0, None)
    assert call(N=12) == UNSUPPORTED
    assert call(Dm=0) == BAD_SHAPE
    assert call(B=-1) == BAD_SHAPE
    assert call(slots=0) == BAD_SHAPE
    assert call(act=9) == BAD_DTYPE
    assert call(x=None) == NULL_ARG
    assert call(A=0x20004) == BAD_SHAPE
    assert call(state=0x30008) == BAD_SHAPE
    assert call(B=0, x=None) == OK


def test_gdn_conv_host_validation():
    L = S.load_library()

    def call(W=4, cw=0x90000, cst=0xA0000, cs=(8192 * 3, 3, 1), H=16, HV=32, V=128, B=4, x=0x10000):
        stride = 2 * H * 128 + HV * V
        return L.gdn_decode_step_conv(x, stride, cw, None, cst, cs[0], cs[1], cs[2], W, 0x20000, 0x30000,
                                      0x40000, 0x50000, 0x60000, 16, 0x70000, 0x80000, B, H, HV, 128, V, 1, 1,
                                      0.088, 1, 1e-6, None, None, 1e-5, 0, None)
    assert call(W=1) == BAD_SHAPE
    assert call(W=9) == BAD_SHAPE
    assert call(cw=None) == NULL_ARG
    assert call(cst=None) == NULL_ARG
    assert call(x=None) == NULL_ARG
    assert call(cs=(1, 0, 1)) == BAD_SHAPE
    assert call(H=1, HV=32) == UNSUPPORTED        # a q/k group of 32 value heads
    assert call(H=4, HV=64, V=512) == UNSUPPORTED  # (HV/H) V = 8192 outputs in one group
    assert call(HV=24) == BAD_SHAPE
    assert call(B=0, x=None, cw=None, cst=None) == OK


def test_mamba_scan_host_validation():
    L = S.load_library()

    def call(B=2, T=64, Dm=256, N=16, x=0x10000, A=0x20000, state=0x30000, act=1, slots=2, ws=None, wsb=0):
        return L.mamba_scan(x, 0x11000, A, 0x12000, 0x13000, None, None, state, slots, 0x14000, None, 0, 0x15000,
                            ws, wsb, B, T, Dm, N, act, 1, None)
    assert call(N=12) == UNSUPPORTED
    assert call(Dm=0) == BAD_SHAPE
    assert call(B=-1) == BAD_SHAPE
    assert call(B=70000) == BAD_SHAPE
    assert call(T=-1) == BAD_SHAPE
    assert call(slots=0) == BAD_SHAPE
    assert call(act=9) == BAD_DTYPE
    assert call(x=None) == NULL_ARG
    assert call(state=None) == NULL_ARG
    assert call(A=0x20004) == BAD_SHAPE
    assert call(wsb=-1) == BAD_SHAPE
    assert call(ws=0x40008, wsb=4096) == BAD_SHAPE  # misaligned workspace
    assert call(B=0, x=None, state=None) == OK
    assert L.mamba_scan_workspace_bytes(1, 64, 256, 12) == UNSUPPORTED
    assert L.mamba_scan_workspace_bytes(-1, 64, 256, 16) == BAD_SHAPE


def test_gdn_fused_recurrent_host_validation():
    L = S.load_library()

    def call(T=4, V=128, K=128, ng=None, B=8, qkv=0x10000, lengths=None):
        return L.gdn_fused_recurrent(qkv, 2 * 16 * K + 32 * V, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000, 16, 0x70000, lengths,
                                     0x80000, B, T, 16, 32, K, V, 1, 1, 0.088, 1, 1e-6, ng, None, 1e-5, 0, None)
    assert call(T=-1) == BAD_SHAPE
    assert call(B=-1) == BAD_SHAPE
    assert call(K=48) == UNSUPPORTED
    assert call(qkv=None) == NULL_ARG
    assert call(ng=0x90000, V=512) == UNSUPPORTED   # the norm needs the head in one block
    assert call(ng=0x90000, K=256, V=192) == UNSUPPORTED
    assert call(T=0, qkv=None) == OK
    assert call(B=0, qkv=None) == OK


def test_gdn_chunk_prefill_host_validation():
    L = S.load_library()

    def call(K=128, V=128, ws=0x90000, wsb=1 << 30, T=128, B=2):
        return L.gdn_chunk_prefill(0x10000, 2 * 16 * K + 32 * V, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000, 16,
                                   0x70000, None, 0x80000, B, T, 16, 32, K, V, 1, 1, 0.088, 1, 1e-6, None, None, 1e-5,
                                   0, ws, wsb, None)
    assert call(K=32) == UNSUPPORTED
    assert call(V=120) == UNSUPPORTED
    assert call(V=512) == BAD_SHAPE or call(V=512) == UNSUPPORTED
    assert call(ws=None) == BAD_SHAPE
    assert call(wsb=1024) == BAD_SHAPE
    assert call(ws=0x90004) == BAD_SHAPE
    assert call(T=0, ws=None) == OK
    need = L.gdn_chunk_workspace_bytes(2, 128, 32, 128, 128, 0)
    assert need == 4 * 2 * 32 * 2 * (2 * 64 * 64 + 4 * 64 + 4)  # per chunk: M, P, four token factors, gamma_C
    assert L.gdn_chunk_workspace_bytes(2, 128, 32, 128, 128, 1) == need + 4 * 2 * 128 * 32 * 128


def test_check_slot_indices_host_validation():
    L = S.load_library()
    f = L.ssmd_check_slot_indices
    assert f(0x1000, -1, 4, 0, 0x2000, None) == BAD_SHAPE
    assert f(0x1000, 65537, 4, 0, 0x2000, None) == BAD_SHAPE
    assert f(0x1000, 4, 0, 0, 0x2000, None) == BAD_SHAPE
    assert f(0x1000, 4, 4, 0, None, None) == NULL_ARG
    assert f(None, 4, 4, 0, 0x2000, None) == NULL_ARG
    assert f(0x1001, 4, 4, 0, 0x2000, None) == BAD_SHAPE


def test_error_message_is_per_thread():
    """Validation failures on several host threads at once: each thread reads
    back its own message from ssmd_last_error (the error string is the only
    mutable state, and it is thread-local)."""
    import threading
    L = S.load_library()
    cases = {"H": (dict(HV=24, H=16), b"HV % H"), "K": (dict(K=48), b"K = 48"), "V": (dict(V=0), b"V = 0"),
             "stride": (dict(stride=8191), b"qkv_row_stride")}
    got, barrier = {}, threading.Barrier(len(cases))

    def run(name, kw, needle):
        barrier.wait()
        ok = True
        for _ in range(200):
            rc = _gdn(L, **kw)
            ok &= rc < 0 and needle in L.ssmd_last_error()
        got[name] = ok

    threads = [threading.Thread(target=run, args=(n, kw, nd)) for n, (kw, nd) in cases.items()]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert got == {n: True for n in cases}, got


def test_binding_rejects_tensors_on_several_devices():
    """The binding refuses a call whose tensors live on different devices
    before anything reaches the library (host and meta tensors stand in for
    two devices here)."""
    src, dst = torch.zeros(4), torch.empty(4, device="meta")
    with pytest.raises(ValueError, match="several devices"):
        S.ssmd_stream_copy(src, dst)
    with pytest.raises(ValueError, match="several devices"):
        S.ssmd_check_slot_indices(torch.zeros(4, dtype=torch.int32), 4,
                                  dup_count=torch.empty(1, dtype=torch.int32, device="meta"))


def test_product_path_is_independent_of_the_oracle():
    """The package imports nothing from oracle/ (in a fresh interpreter, after
    importing it and loading the library, no oracle module is loaded), none of
    its sources names it, and a missing library fails loudly instead of
    falling back to anything."""
    import subprocess
    import sys
    code = ("import sys, ssm_recurrent_decode_gated_amd as S; S.load_library(); "
            "print(sorted(m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().splitlines()[-1] == "[]", r.stdout
    pkg = os.path.join(ROOT, "ssm_recurrent_decode_gated_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "liboracle" not in text, f
    code = ("import ssm_recurrent_decode_gated_amd._binding as B; B.LIB_PATH = '/nonexistent/libssmdec.so'; "
            "B._LIB = None\ntry:\n    B.load_library()\nexcept RuntimeError as e:\n    print('raised', e)")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert "raised" in r.stdout and "no non-HIP fallback" in r.stdout, r.stdout + r.stderr


def test_chunk_prefill_noalloc_host_validation():
    """The static-workspace prefill refuses a call whose records would not fit
    its SSMD_CHUNK_SCRATCH_BYTES array (checked before any HIP call), and
    otherwise validates like gdn_chunk_prefill."""
    L = S.load_library()

    def call(B=1, T=8192, H=1, HV=32, K=64, V=64):
        return L.gdn_chunk_prefill_noalloc(0x10000, 2 * H * K + HV * V, 0x20000, 0x30000, 0x40000, 0x50000,
                                           0x60000, 4, 0x70000, None, 0x80000, B, T, H, HV, K, V, 1, 0, 0.125, 1,
                                           1e-6, None, None, 1e-5, 0, None)
    assert S.gdn_chunk_workspace_bytes(1, 8192, 32, 64, 64) > S.SSMD_CHUNK_SCRATCH_BYTES
    assert call() == BAD_SHAPE
    assert "static" in S.ssmd_last_error()
    assert call(K=32) == UNSUPPORTED
    assert call(T=0) == OK
