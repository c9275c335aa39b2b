"""C-ABI checks that need no GPU: the library loads, exports every function
include/gattn.h declares, and rejects bad arguments before any HIP call (so
no compute is enqueued; the fake pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

import causal_self_attention_sdpa_amd as ga

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, 1, 2, 3, 4


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "gattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gattn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return ga.load_library()


def test_exports_every_declared_function(lib):
    names = _declared_functions()
    assert "gattn_fwd" in names and "gattn_bwd" in names
    raw = ctypes.CDLL(ga.library_path())
    for n in names:
        assert hasattr(raw, n), n


def test_status_strings(lib):
    assert ga.gattn_status_string(OK) == "GATTN_OK"
    assert ga.gattn_status_string(INVALID) == "GATTN_ERR_INVALID_ARG"
    assert ga.gattn_status_string(UNSUPPORTED) == "GATTN_ERR_UNSUPPORTED"
    assert ga.gattn_status_string(WORKSPACE) == "GATTN_ERR_WORKSPACE"
    assert ga.gattn_status_string(HIP) == "GATTN_ERR_HIP"
    assert ga.gattn_status_string(99) == "GATTN_UNKNOWN_STATUS"


def test_workspace_bytes(lib):
    B, H, T, hs = 12, 12, 1024, 64
    n = ga.gattn_bwd_workspace_bytes(B, H, T, hs, ga.BF16)
    assert n == 2 * B * H * T * 4  # D and lse*log2(e)
    assert ga.gattn_bwd_workspace_bytes(4, 4, 8, 8, ga.F32) == 1024  # 2 x 4*4*8 floats, 256-aligned
    assert ga.gattn_bwd_workspace_bytes(1, 1, 3, 64, ga.BF16) == 512
    assert ga.gattn_bwd_workspace_bytes(1, 1, 65, 32, ga.BF16) == 1024
    assert ga.gattn_bwd_workspace_bytes(0, 1, 1, 64, ga.BF16) == 0
    assert ga.gattn_bwd_workspace_bytes(1, 1, 1, 48, ga.BF16) == 0  # unsupported hs
    assert ga.gattn_bwd_workspace_bytes(1, 1, 1, 8, 7) == 0


P = 0x10000  # fake, 256-aligned "device" address, never touched


def _fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, T=8, hs=64, scale=0.125, dtype=1):
    return lib.gattn_fwd(q, k, v, o, lse, B, H, T, hs, scale, dtype, None)


def test_fwd_validation(lib):
    assert _fwd(lib, q=None) == INVALID
    assert _fwd(lib, o=None) == INVALID
    assert _fwd(lib, k=P + 2) == INVALID      # misaligned
    assert _fwd(lib, lse=P + 4) == INVALID    # misaligned lse
    for bad in (dict(B=0), dict(H=-1), dict(T=0), dict(hs=0)):
        assert _fwd(lib, **bad) == INVALID, bad
    for s in (0.0, -1.0, float("inf"), float("nan")):
        assert _fwd(lib, scale=s) == INVALID, s
    assert _fwd(lib, dtype=5) == INVALID
    assert _fwd(lib, B=1 << 11, H=1 << 10, T=1 << 10, hs=64) == INVALID  # >= 2^31 elements
    assert _fwd(lib, hs=48) == UNSUPPORTED
    assert _fwd(lib, hs=128) == UNSUPPORTED
    assert _fwd(lib, hs=129, dtype=0) == UNSUPPORTED


def _bwd(lib, ptrs=None, B=1, H=1, T=8, hs=64, scale=0.125, dtype=1, ws=P, wsb=1 << 20):
    p = ptrs or [P] * 9
    return lib.gattn_bwd(*p, B, H, T, hs, scale, dtype, ws, wsb, None)


def test_bwd_validation(lib):
    for i in range(9):
        p = [P] * 9
        p[i] = None
        assert _bwd(lib, p) == INVALID, i
        p[i] = P + 8
        assert _bwd(lib, p) == INVALID, i
    assert _bwd(lib, scale=float("nan")) == INVALID
    assert _bwd(lib, hs=16) == UNSUPPORTED
    assert _bwd(lib, ws=None) == WORKSPACE
    assert _bwd(lib, ws=P + 16) == WORKSPACE  # not 256-aligned
    need = ga.gattn_bwd_workspace_bytes(1, 1, 8, 64, 1)
    assert _bwd(lib, wsb=need - 1) == WORKSPACE


def test_stage_validation(lib):
    # preprocess: o, dO, lse
    assert lib.gattn_bwd_preprocess(None, P, P, 1, 1, 8, 64, 1, P, 1 << 20, None) == INVALID
    assert lib.gattn_bwd_preprocess(P, P, None, 1, 1, 8, 64, 1, P, 1 << 20, None) == INVALID
    assert lib.gattn_bwd_preprocess(P, P, P, 1, 1, 8, 64, 1, P, 1, None) == WORKSPACE
    assert lib.gattn_bwd_preprocess(P, P, P, 1, 1, 8, 48, 1, P, 1 << 20, None) == UNSUPPORTED
    # dq: q, k, v, o, dO, lse, dq
    for i in range(7):
        p = [P] * 7
        p[i] = None
        assert lib.gattn_bwd_dq(*p, 1, 1, 8, 64, 0.125, 1, P, 1 << 20, None) == INVALID, i
        p[i] = P + 4
        assert lib.gattn_bwd_dq(*p, 1, 1, 8, 64, 0.125, 1, P, 1 << 20, None) == INVALID, i
    assert lib.gattn_bwd_dq(*([P] * 7), 1, 1, 8, 64, 0.0, 1, P, 1 << 20, None) == INVALID
    assert lib.gattn_bwd_dq(*([P] * 7), 1, 1, 8, 200, 0.125, 0, P, 1 << 20, None) == UNSUPPORTED
    assert lib.gattn_bwd_dq(*([P] * 7), 1, 1, 8, 64, 0.125, 1, None, 1 << 20, None) == WORKSPACE
    # dkdv: q, k, v, dO, dk, dv
    for i in range(6):
        p = [P] * 6
        p[i] = None
        assert lib.gattn_bwd_dkdv(*p, 1, 1, 8, 64, 0.125, 1, P, 1 << 20, None) == INVALID, i
    assert lib.gattn_bwd_dkdv(*([P] * 6), 1, 1, 8, 64, float("inf"), 1, P, 1 << 20,
                              None) == INVALID
    assert lib.gattn_bwd_dkdv(*([P] * 6), 1, 1, 8, 64, 0.125, 1, P, 4, None) == WORKSPACE
    assert lib.gattn_bwd_dkdv(*([P] * 6), 1, 1, 8, 64, 0.125, 1, P + 64, 1 << 20,
                              None) == WORKSPACE


def _st(*s):
    return (ctypes.c_int64 * 3)(*s)


def test_fwd_strided_validation(lib):
    B, H, T, hs = 2, 3, 8, 64
    good = _st(T * 3 * H * hs, hs, 3 * H * hs)  # fused (B, T, 3C) projection output

    def f(qkv=good, o=None, dtype=1, **kw):
        a = dict(q=P, k=P, v=P, o=P, lse=P, B=B, H=H, T=T, hs=hs, scale=0.125)
        a.update(kw)
        return lib.gattn_fwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                     a["T"], a["hs"], a["scale"], dtype, qkv, o, None)

    # the checks shared with gattn_fwd
    assert f(q=None) == INVALID
    assert f(v=P + 2) == INVALID
    assert f(scale=-1.0) == INVALID
    assert f(hs=48) == UNSUPPORTED
    # stride checks: negative, overlapping rows, rows off 16-byte boundaries, span
    assert f(qkv=_st(-8, hs, 3 * H * hs)) == INVALID
    assert f(qkv=_st(T * 3 * H * hs, -hs, 3 * H * hs)) == INVALID
    assert f(qkv=_st(T * 3 * H * hs, hs, hs - 8)) == INVALID   # row stride < hs
    assert f(qkv=_st(T * 3 * H * hs, hs, 3 * H * hs + 4)) == INVALID  # 8-byte rows
    assert f(o=_st(4, hs, H * hs)) == INVALID                  # batch stride of 8 bytes
    assert f(o=_st(T * H * hs, 12, H * hs)) == INVALID         # head stride of 24 bytes
    assert f(qkv=_st(0, 0, 1 << 22), T=1 << 8) == INVALID       # (T + 256) rows >= 2^31 bytes
    assert f(qkv=_st(0, 0, 1 << 20), T=1 << 8, dtype=0) == INVALID  # same for float32
    # float32 strides count 4-byte elements: 4 elements = 16 bytes is fine for
    # alignment, but not below hs
    assert f(qkv=_st(4, 4, 4), hs=8, dtype=0) == INVALID


def test_bwd_strided_validation(lib):
    B, H, T, hs = 2, 3, 8, 64
    qkv = _st(T * 3 * H * hs, hs, 3 * H * hs)
    out = _st(T * H * hs, hs, H * hs)

    def f(ptrs=None, s_qkv=qkv, s_o=out, s_g=qkv, ws=P, wsb=1 << 20, **kw):
        p = ptrs or [P] * 9
        a = dict(B=B, H=H, T=T, hs=hs, scale=0.125, dtype=1)
        a.update(kw)
        return lib.gattn_bwd_strided(*p, a["B"], a["H"], a["T"], a["hs"], a["scale"], a["dtype"],
                                     ws, wsb, s_qkv, s_o, s_g, None)

    for i in range(9):
        p = [P] * 9
        p[i] = None
        assert f(p) == INVALID, i
    assert f(ws=None) == WORKSPACE
    assert f(wsb=16) == WORKSPACE
    assert f(s_o=_st(T * H * hs, hs, hs - 1)) == INVALID
    assert f(s_g=_st(T * H * hs, hs + 1, H * hs)) == INVALID
    assert f(s_qkv=_st(-1, hs, 3 * H * hs)) == INVALID


def test_f16_dtype_code(lib):
    assert ga.F16 == 2
    assert ga.gattn_bwd_workspace_bytes(2, 3, 100, 64, ga.F16) == \
        ga.gattn_bwd_workspace_bytes(2, 3, 100, 64, ga.BF16)
    assert _fwd(lib, dtype=2, hs=48) == UNSUPPORTED
    assert _fwd(lib, dtype=2, hs=128) == UNSUPPORTED
    assert _fwd(lib, dtype=3) == INVALID
    assert _bwd(lib, dtype=2, hs=16) == UNSUPPORTED
    assert _bwd(lib, dtype=2, ws=None) == WORKSPACE


def test_decode_validation(lib):
    def f(q=P, k=P, v=P, o=P, lse=P, B=2, H=3, Tq=1, Tk=1000, hs=64, scale=0.125, dtype=1,
          sq=None, skv=None, so=None, ws=P, wsb=1 << 24):
        return lib.gattn_fwd_decode(q, k, v, o, lse, B, H, Tq, Tk, hs, scale, dtype, sq, skv, so,
                                    ws, wsb, None)
    assert f(q=None) == INVALID
    assert f(o=P + 2) == INVALID
    assert f(lse=P + 4) == INVALID
    assert f(Tq=0) == INVALID
    assert f(Tq=1001) == INVALID             # more queries than keys
    assert f(scale=float("nan")) == INVALID
    assert f(hs=48) == UNSUPPORTED
    assert f(dtype=2, hs=16) == UNSUPPORTED
    assert f(skv=_st(3 * 1000 * 64, 1000 * 64, 32)) == INVALID  # row stride < hs
    assert f(ws=None) == WORKSPACE            # 1000 keys: split, partials need a workspace
    assert f(ws=P + 128) == WORKSPACE         # not 256-aligned
    need = ga.gattn_fwd_decode_workspace_bytes(2, 3, 1, 1000, 64, 1)
    assert need > 0
    assert f(wsb=need - 4) == WORKSPACE
    assert ga.gattn_fwd_decode_workspace_bytes(2, 3, 1, 1000, 64, 0) == 0  # float32: none
    assert ga.gattn_fwd_decode_workspace_bytes(2, 3, 1, 256, 64, 1) == 0   # 4 tiles: no split
    assert ga.gattn_fwd_decode_workspace_bytes(2, 3, 5, 4, 64, 1) == 0     # Tq > Tk rejected
    assert ga.gattn_fwd_decode_workspace_bytes(2, 3, 1, 100, 48, 1) == 0   # unsupported hs


def test_dropout_validation(lib):
    def fwd(p=0.1, q=P, o=P, lse=P, hs=64, dtype=1, sqkv=None, so=None, keep=None, T=100):
        return lib.gattn_fwd_dropout(q, P, P, o, lse, 2, 3, T, hs, 0.125, dtype, p, 7, 1, keep,
                                     sqkv, so, None)

    def bwd(p=0.1, lse=P, ws=P, wsb=1 << 20, dtype=1, sg=None, keep=None):
        return lib.gattn_bwd_dropout(P, P, P, P, P, lse, P, P, P, 2, 3, 100, 64, 0.125, dtype, p, 7,
                                     1, keep, ws, wsb, None, None, sg, None)

    def mask(keep=P, B=2, H=3, T=100, p=0.1):
        return lib.gattn_dropout_mask(keep, B, H, T, p, 7, 1, None)

    for bad in (-0.1, 1.0, 2.0, float("nan"), float("inf"), 1.0 - 2.0 ** -18):
        assert fwd(p=bad) == INVALID, bad
        assert bwd(p=bad) == INVALID, bad
        assert mask(p=bad) == INVALID, bad
    assert fwd(q=None) == INVALID
    assert fwd(lse=P + 4) == INVALID
    assert fwd(hs=48) == UNSUPPORTED
    assert fwd(so=_st(3 * 100 * 64, 100 * 64, 8)) == INVALID  # row stride < hs
    assert bwd(lse=None) == INVALID                              # the backward needs lse
    assert bwd(ws=None) == WORKSPACE
    assert bwd(wsb=16) == WORKSPACE
    # The 16-bit backward with dropout also needs room for the keep bits.
    base = ga.gattn_bwd_workspace_bytes(2, 3, 100, 64, ga.BF16)
    assert bwd(wsb=base) == WORKSPACE
    assert bwd(wsb=ga.gattn_bwd_dropout_workspace_bytes(2, 3, 100, 64, ga.BF16, 0.1) - 1) == WORKSPACE
    big_t = 8 * 16383 + 1   # ceil(T / 8) past the keep-bit addressing limit
    assert lib.gattn_bwd_dropout(P, P, P, P, P, P, P, P, P, 1, 1, big_t, 64, 0.125, 1, 0.1, 7, 1,
                                 None, P, 1 << 40, None, None, None, None) == INVALID
    # A keep buffer must be 16-byte aligned and its shape must have a keep size.
    assert fwd(keep=P + 8) == INVALID
    assert bwd(keep=P + 8) == INVALID
    assert fwd(keep=P, T=big_t) == INVALID
    assert fwd(keep=P, p=1.0) == INVALID
    assert bwd(sg=_st(-1, 64, 64)) == INVALID
    assert mask(keep=None) == INVALID
    assert mask(T=0) == INVALID
    assert mask(B=1 << 10, H=1 << 10, T=1 << 10) == INVALID     # 2^40 bytes


def test_dropout_workspace_bytes(lib):
    """The dropout backward's workspace: the plain backward's, plus for bf16
    and fp16 one bit per query-key pair of every slice (ceil(T/8)^2 blocks of
    8 bytes per (b, h), 256-byte rounded)."""
    def need(B=2, H=3, T=100, hs=64, dt=ga.BF16, p=0.1):
        return ga.gattn_bwd_dropout_workspace_bytes(B, H, T, hs, dt, p)

    base = ga.gattn_bwd_workspace_bytes(2, 3, 100, 64, ga.BF16)
    keep = -(-(2 * 3 * 13 * 13 * 8) // 256) * 256  # ceil(100 / 8) = 13 groups
    assert need() == base + keep
    assert need(dt=ga.F16) == base + keep
    assert need(dt=ga.F32) == ga.gattn_bwd_workspace_bytes(2, 3, 100, 64, ga.F32)
    assert need(p=0.0) == base
    assert need(p=2.0 ** -18) == base             # rounds to threshold 0: no dropout
    assert need(T=8, B=1, H=1) == ga.gattn_bwd_workspace_bytes(1, 1, 8, 64, ga.BF16) + 256
    for bad in (-0.1, 1.0, float("nan")):
        assert need(p=bad) == 0
    assert need(hs=48) == 0 and need(B=0) == 0
    assert need(B=1, H=1, T=8 * 16383) > 0
    assert need(B=1, H=1, T=8 * 16383 + 1) == 0
    assert need(B=1, H=1, T=8 * 16383 + 1, dt=ga.F32) > 0


def test_dropout_keep_bytes(lib):
    """The keep buffer: ceil(T/8)^2 blocks of 8 bytes per (b, h), 256-byte
    rounded, for any dtype; 0 past the addressing limit."""
    assert ga.gattn_dropout_keep_bytes(2, 3, 100) == -(-(2 * 3 * 13 * 13 * 8) // 256) * 256
    assert ga.gattn_dropout_keep_bytes(12, 12, 1024) == 12 * 12 * 128 * 128 * 8
    assert ga.gattn_dropout_keep_bytes(1, 1, 1) == 256
    assert ga.gattn_dropout_keep_bytes(0, 1, 8) == 0 and ga.gattn_dropout_keep_bytes(1, 1, 0) == 0
    assert ga.gattn_dropout_keep_bytes(1, 1, 8 * 16383) > 0
    assert ga.gattn_dropout_keep_bytes(1, 1, 8 * 16383 + 1) == 0
    assert ga.gattn_dropout_keep_bytes(1 << 20, 1 << 10, 1024) == 0   # past 2^40 bytes


def test_probe_validation(lib):
    assert lib.gattn_probe_mfma_bf16(None, 4, 4, None) == INVALID
    assert lib.gattn_probe_mfma_bf16(P, 0, 4, None) == INVALID
    assert lib.gattn_probe_mfma_bf16(P, 4, 0, None) == INVALID
    assert lib.gattn_probe_issue(None, 4, 4, 4, 0, 1, None) == INVALID
    assert lib.gattn_probe_issue(P, 0, 4, 4, 0, 1, None) == INVALID
    assert lib.gattn_probe_issue(P, 4, -1, 4, 0, 1, None) == INVALID
    assert lib.gattn_probe_issue(P, 4, 4, -1, 0, 1, None) == INVALID
    for kind in (-1, 3):
        assert lib.gattn_probe_issue(P, 4, 4, 4, kind, 1, None) == INVALID
    for roles in (0, 16):
        assert lib.gattn_probe_issue(P, 4, 4, 4, 0, roles, None) == INVALID


def test_header_is_plain_c_and_the_c_caller_links(tmp_path):
    """include/gattn.h compiles as C11 with warnings as errors, and the plain-C
    caller of the GPU tests (tests/c_abi) links against libgattn.so, the
    oracle library and the HIP runtime (built here into a scratch path)."""
    import importlib.util
    path = os.path.join(ROOT, "tests", "c_abi", "build.py")
    spec = importlib.util.spec_from_file_location("gattn_c_abi_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    exe = mod.build(out=str(tmp_path / "gattn_c_roundtrip"))
    assert os.access(exe, os.X_OK)


def test_noalloc_rejects_before_any_hip_call(lib):
    """gattn_bwd_noalloc validates like gattn_bwd, and rejects a problem whose
    row terms do not fit its static scratch, before touching the GPU."""
    cap = ga.gattn_bwd_noalloc_max_bytes()
    assert cap == 8 << 20
    f = lib.gattn_bwd_noalloc
    s = ctypes.c_float(0.125)
    assert f(*([P] * 9), 1, 1, 1 << 21, 32, s, 1, None) == WORKSPACE  # 2^21 rows: 16 MiB
    rows_max = cap // 8  # D and lse*log2(e), 4 bytes each per row
    assert ga.gattn_bwd_workspace_bytes(1, 1, rows_max, 32, ga.BF16) <= cap
    assert ga.gattn_bwd_workspace_bytes(1, 1, rows_max + 64, 32, ga.BF16) > cap
    assert f(*([P] * 9), 1, 1, rows_max + 64, 32, s, 1, None) == WORKSPACE
    assert f(None, *([P] * 8), 1, 1, 8, 64, s, 1, None) == INVALID
    assert f(*([P] * 9), 1, 1, 8, 48, s, 1, None) == UNSUPPORTED
    assert f(*([P] * 9), 1, 1, 8, 64, ctypes.c_float(-1.0), 1, None) == INVALID


def test_contiguous_16bit_slice_byte_limit(lib):
    """A bf16/fp16 slice whose T + 256 rows reach 2^31 bytes is rejected on the
    contiguous path as on the strided one (the kernels address a slice with
    32-bit byte offsets); B*H*T*hs alone stays below 2^31 there."""
    limit = (1 << 24) - 256  # (limit + 256) * 64 * 2 == 2^31
    assert (limit + 256) * 64 * 2 == 1 << 31 and limit * 64 < 1 << 31
    for dt in (ga.BF16, ga.F16):
        assert ga.gattn_bwd_workspace_bytes(1, 1, limit, 64, dt) == 0
        assert ga.gattn_bwd_workspace_bytes(1, 1, limit - 1, 64, dt) > 0
        assert _fwd(lib, T=limit, hs=64, dtype=dt) == INVALID
        assert _fwd(lib, T=2 * limit + 256, hs=32, dtype=dt) == INVALID
    # float32 addresses rows with 64-bit offsets: only B*H*T*hs < 2^31 applies
    assert ga.gattn_bwd_workspace_bytes(1, 1, limit, 64, ga.F32) > 0


def test_binding_keeps_a_call_on_one_device():
    """The binding's stream choice: tensors of one call on two devices, or a
    stream of another device, are rejected before anything reaches the
    library (stand-ins carrying only a device, so no GPU is touched)."""
    import types
    import torch
    from causal_self_attention_sdpa_amd import _binding as b
    t0 = types.SimpleNamespace(device=torch.device("cuda", 0))
    t1 = types.SimpleNamespace(device=torch.device("cuda", 1))
    with pytest.raises(ValueError, match="one device"):
        b._on(None, t0, t1)
    s1 = types.SimpleNamespace(device=torch.device("cuda", 1), cuda_stream=1234)
    with pytest.raises(ValueError, match="stream is on"):
        b._on(s1, t0, None, t0)
    assert b._on(s1, t1, None).value == 1234


def test_binding_canonical_strides_for_size_one_dimensions():
    """Strides of size-1 dimensions are arbitrary in torch (0 for a view of a
    broadcast array): the binding passes canonical ones, so views of one
    layout compare equal (stand-ins carrying shape and strides only)."""
    import torch
    from causal_self_attention_sdpa_amd import _binding as b

    class View:
        def __init__(self, shape, stride, contiguous):
            self.shape, self._st, self._c = shape, stride, contiguous
            self.is_cuda, self.dtype = True, torch.bfloat16

        def stride(self, i=None):
            return self._st if i is None else self._st[i]

        def is_contiguous(self):
            return self._c

        def data_ptr(self):
            return 4096

    shape = (1, 1, 300, 64)
    a = b._view(View(shape, (0, 0, 64, 1), True), "a", shape, torch.bfloat16)[1]
    c = b._view(View(shape, (19200, 19200, 64, 1), True), "c", shape, torch.bfloat16)[1]
    assert a == c == (19200, 19200, 64)
    # a strided view (rows 3*C apart) with one batch and one head
    d = b._view(View(shape, (7, 0, 192, 1), False), "d", shape, torch.bfloat16)[1]
    assert d == (0, 0, 192)
    one = (2, 3, 1, 64)
    e = b._view(View(one, (64 * 5, 64, 0, 1), False), "e", one, torch.bfloat16)[1]
    assert e == (320, 64, 64)
