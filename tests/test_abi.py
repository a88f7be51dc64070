"""C-ABI checks that run without a GPU: the library loads, exports every
function the header declares, and rejects bad arguments on the host before
any HIP call (so nothing here touches a device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "int8lin.h")
LIB = os.path.join(ROOT, "int8_quantized_linear_rowwise_amd", "libint8lin.so")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_i8l_build", os.path.join(ROOT, "int8_quantized_linear_rowwise_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build(verbose=False)
    from int8_quantized_linear_rowwise_amd import _lib
    return _lib


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(int8_\w+)\s*\(", src)))


def test_header_declares_the_three_entry_points():
    names = _declared()
    for n in ("int8_quantize_rowwise", "int8_linear_forward", "int8_linear_backward_input"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    cdll = ctypes.CDLL(LIB)
    for n in _declared():
        assert hasattr(cdll, n), n
    # the binding describes exactly the declared set
    assert set(L.SIGNATURES) == set(_declared())


def test_exports_are_plain_c(L):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in _declared():
        assert n in syms, n          # unmangled


def test_strerror(L):
    for c in (0, -1, -2, -3, -4, -5, -6, -7, -99):
        assert isinstance(L.lib.int8_linear_strerror(c), bytes)
    assert L.lib.int8_linear_strerror(-4).startswith(b"workspace")


FAKE = 1 << 20   # a non-NULL, 256-aligned address that is never dereferenced


def test_quantize_host_errors(L):
    f = L.lib.int8_quantize_rowwise
    ws = L.lib.int8_quantize_rowwise_workspace_bytes(4, 64)
    args = dict(X=FAKE, dt=1, R=4, C=64, tau=6.0, codes=FAKE, scale=FAKE, idx=FAKE, cnt=FAKE, sub=FAKE, cap=64,
                ws=FAKE, wsb=ws, st=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["X"], a["dt"], a["R"], a["C"], a["tau"], a["codes"], a["scale"], a["idx"], a["cnt"], a["sub"],
                 a["cap"], a["ws"], a["wsb"], a["st"])

    assert call(dt=3) == L.I8L_EDTYPE
    assert call(dt=-1) == L.I8L_EDTYPE
    assert call(R=-1) == L.I8L_EINVAL
    assert call(C=-5) == L.I8L_EINVAL
    assert call(cap=-1) == L.I8L_EINVAL
    assert call(X=0) == L.I8L_EINVAL
    assert call(codes=0) == L.I8L_EINVAL
    assert call(scale=0) == L.I8L_EINVAL
    assert call(cnt=0) == L.I8L_EINVAL
    assert call(idx=0) == L.I8L_EINVAL
    assert call(sub=0) == L.I8L_EINVAL
    assert call(ws=0) == L.I8L_EWORKSPACE
    assert call(wsb=ws - 1) == L.I8L_EWORKSPACE
    assert call(ws=FAKE + 8) == L.I8L_EINVAL
    assert call(R=1 << 33) == L.I8L_ESHAPE
    assert call(C=L.I8L_MAX_COLS + 1, wsb=1 << 30) == L.I8L_ESHAPE


def test_forward_host_errors(L):
    f = L.lib.int8_linear_forward
    M, K, N, cap = 8, 64, 32, 64
    ws = L.lib.int8_linear_forward_workspace_bytes(M, K, N, cap)
    base = dict(A=FAKE, dt=1, M=M, K=K, CB=FAKE, SCB=FAKE, N=N, bias=0, tau=6.0, cap=cap, out=FAKE, c32=0, ws=FAKE,
                wsb=ws, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["A"], a["dt"], a["M"], a["K"], a["CB"], a["SCB"], a["N"], a["bias"], a["tau"], a["cap"],
                 a["out"], a["c32"], a["ws"], a["wsb"], a["st"])

    assert call(dt=7) == L.I8L_EDTYPE
    assert call(M=-1) == L.I8L_EINVAL
    assert call(K=-1) == L.I8L_EINVAL
    assert call(N=-1) == L.I8L_EINVAL
    assert call(cap=-1) == L.I8L_EINVAL
    assert call(A=0) == L.I8L_EINVAL
    assert call(CB=0) == L.I8L_EINVAL
    assert call(SCB=0) == L.I8L_EINVAL
    assert call(out=0) == L.I8L_EINVAL
    assert call(K=L.I8L_MAX_K + 1) == L.I8L_ESHAPE
    assert call(ws=0) == L.I8L_EWORKSPACE
    assert call(wsb=ws - 1) == L.I8L_EWORKSPACE
    assert call(ws=FAKE + 16) == L.I8L_EINVAL
    # empty problems succeed without touching the device
    assert call(M=0, wsb=L.lib.int8_linear_forward_workspace_bytes(0, K, N, cap)) == L.I8L_OK
    assert call(N=0) == L.I8L_OK


def test_backward_host_errors(L):
    f = L.lib.int8_linear_backward_input
    M, N, K = 8, 32, 64
    ws = L.lib.int8_linear_backward_workspace_bytes(M, N, 1)
    base = dict(G=FAKE, dt=2, M=M, N=N, CB=FAKE, SCB=FAKE, K=K, gA=FAKE, gb=FAKE, ws=FAKE, wsb=ws, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["G"], a["dt"], a["M"], a["N"], a["CB"], a["SCB"], a["K"], a["gA"], a["gb"], a["ws"], a["wsb"],
                 a["st"])

    assert call(dt=5) == L.I8L_EDTYPE
    assert call(M=-2) == L.I8L_EINVAL
    assert call(G=0) == L.I8L_EINVAL
    assert call(CB=0) == L.I8L_EINVAL
    assert call(SCB=0) == L.I8L_EINVAL
    assert call(gA=0) == L.I8L_EINVAL
    assert call(ws=0) == L.I8L_EWORKSPACE
    assert call(wsb=ws - 1) == L.I8L_EWORKSPACE
    assert call(M=1 << 32) == L.I8L_ESHAPE
    assert L.lib.int8_linear_backward_workspace_bytes(M, N, 0) == 0


def test_backward_int8_host_errors(L):
    f = L.lib.int8_linear_backward_input_int8
    M, N, K = 8, 32, 64
    ws = L.lib.int8_linear_backward_int8_workspace_bytes(M, N, 1)
    assert ws >= M * N + 4 * M
    base = dict(G=FAKE, dt=1, M=M, N=N, CB=FAKE, SCB=FAKE, K=K, gA=FAKE, gb=FAKE, c32=None, ws=FAKE, wsb=ws,
                st=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["G"], a["dt"], a["M"], a["N"], a["CB"], a["SCB"], a["K"], a["gA"], a["gb"], a["c32"], a["ws"],
                 a["wsb"], a["st"])

    assert call(dt=3) == L.I8L_EDTYPE
    assert call(N=-1) == L.I8L_EINVAL
    assert call(G=0) == L.I8L_EINVAL
    assert call(CB=0) == L.I8L_EINVAL
    assert call(SCB=0) == L.I8L_EINVAL
    assert call(gA=0) == L.I8L_EINVAL
    assert call(ws=0) == L.I8L_EWORKSPACE
    assert call(wsb=ws - 1) == L.I8L_EWORKSPACE
    assert call(ws=FAKE + 8) == L.I8L_EINVAL
    # the contraction runs over the output features: the forward GEMM's limit applies to N
    assert call(N=L.I8L_MAX_K + 1) == L.I8L_ESHAPE
    assert call(M=1 << 32) == L.I8L_ESHAPE
    assert (L.lib.int8_linear_backward_int8_workspace_bytes(M, N, 0)
            < L.lib.int8_linear_backward_int8_workspace_bytes(M, N, 1))
    assert L.lib.int8_linear_backward_int8_workspace_bytes(-1, N, 1) == 0


def test_backward_weight_host_errors(L):
    f = L.lib.int8_linear_backward_weight
    base = dict(G=FAKE, A=FAKE, dt=2, M=64, N=32, K=16, gW=FAKE, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["G"], a["A"], a["dt"], a["M"], a["N"], a["K"], a["gW"], a["st"])

    assert call(dt=7) == L.I8L_EDTYPE
    assert call(M=-1) == L.I8L_EINVAL
    assert call(G=0) == L.I8L_EINVAL
    assert call(A=0) == L.I8L_EINVAL
    assert call(gW=0) == L.I8L_EINVAL
    assert call(N=1 << 31) == L.I8L_ESHAPE
    assert call(M=1 << 21, N=1 << 20) == L.I8L_ESHAPE
    # nothing to write: no pointer is needed and nothing is launched
    assert call(N=0, G=0, A=0, gW=0) == L.I8L_OK
    assert call(K=0, G=0, A=0, gW=0) == L.I8L_OK


def test_producer_flags_host_errors(L):
    f = L.lib.int8_silu_outlier_flags
    words = L.lib.int8_outlier_flags_words
    nw = words(4, 8)
    assert f(FAKE, 9, 4, 8, 6.0, FAKE, FAKE, nw, None) == L.I8L_EDTYPE
    assert f(FAKE, 1, -1, 8, 6.0, FAKE, FAKE, nw, None) == L.I8L_EINVAL
    assert f(0, 1, 4, 8, 6.0, FAKE, FAKE, nw, None) == L.I8L_EINVAL
    assert f(FAKE, 1, 4, 8, 6.0, 0, FAKE, nw, None) == L.I8L_EINVAL
    assert f(FAKE, 1, 4, 8, 6.0, FAKE, 0, nw, None) == L.I8L_EINVAL
    assert f(FAKE, 1, 4, 8, 6.0, FAKE, FAKE, nw - 1, None) == L.I8L_EWORKSPACE
    assert f(FAKE, 1, 4, L.I8L_MAX_COLS + 1, 6.0, FAKE, FAKE, 1 << 30, None) == L.I8L_ESHAPE
    assert f(0, 1, 0, 8, 6.0, 0, 0, 0, None) == L.I8L_OK            # nothing to do
    assert words(4096, 4096) >= 4096 // 32 and words(4096, 4096) % (4096 // 32) == 0
    assert words(-1, 8) == 0
    g = L.lib.int8_linear_forward_flagged
    M, K, N = 8, 64, 32
    wsb = L.lib.int8_linear_forward_workspace_bytes(M, K, N, K)
    base = dict(A=FAKE, dt=2, M=M, K=K, fl=FAKE, fw=words(M, K), CB=FAKE, SCB=FAKE, N=N, b=None, cap=K, out=FAKE,
                c32=None, ws=FAKE, wsb=wsb, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return g(a["A"], a["dt"], a["M"], a["K"], a["fl"], a["fw"], a["CB"], a["SCB"], a["N"], a["b"], a["cap"],
                 a["out"], a["c32"], a["ws"], a["wsb"], a["st"])

    assert call(fl=0) == L.I8L_EINVAL
    assert call(fw=words(M, K) - 1) == L.I8L_EWORKSPACE
    assert call(dt=4) == L.I8L_EDTYPE
    assert call(wsb=wsb - 1) == L.I8L_EWORKSPACE
    assert call(K=L.I8L_MAX_K + 1, wsb=1 << 40) == L.I8L_ESHAPE


def wsub_width(cap):
    """Columns of the weight's dequantized outlier slice for staging width cap:
    cap rounded up to a multiple of 8, at most 256."""
    return 0 if cap <= 0 else min((cap + 7) // 8 * 8, 256)


def test_forward_layout(L):
    for (M, K, N, cap) in [(1, 1, 1, 0), (600, 4, 9, 4), (2048, 4096, 11008, 4096), (16384, 28672, 8192, 28672),
                           (5, 70, 3, 3), (7, 64, 0, 17)]:
        lay = L.ForwardLayout()
        assert L.lib.int8_linear_forward_workspace_layout(M, K, N, cap, lay) == 0
        offs = [lay.count, lay.idx, lay.scale, lay.codes, lay.sub, lay.wsub]
        sizes = [4, 4 * K, 4 * M, M * K, 2 * M * cap, 2 * N * wsub_width(cap)]
        assert all(o % 256 == 0 for o in offs)
        for (o, s), o2 in zip(zip(offs, sizes), offs[1:] + [lay.total]):
            assert o + s <= o2
        assert lay.total == L.lib.int8_linear_forward_workspace_bytes(M, K, N, cap)
    assert [wsub_width(c) for c in (0, 1, 8, 9, 16, 17, 255, 256, 257, 4096)] == [0, 8, 8, 16, 16, 24, 256, 256,
                                                                                   256, 256]
    assert L.lib.int8_linear_forward_workspace_layout(-1, 4, 4, 4, L.ForwardLayout()) == L.I8L_EINVAL
    assert L.lib.int8_linear_forward_workspace_layout(4, 4, -1, 4, L.ForwardLayout()) == L.I8L_EINVAL
    assert L.lib.int8_linear_forward_workspace_bytes(4, 4, -1, 4) == 0
    # the outlier list always has room for every column; only the staging widths follow cap
    small, big = L.ForwardLayout(), L.ForwardLayout()
    L.lib.int8_linear_forward_workspace_layout(16384, 28672, 8192, 256, small)
    L.lib.int8_linear_forward_workspace_layout(16384, 28672, 8192, 28672, big)
    assert small.sub - small.idx >= 4 * 28672
    assert small.total < 16384 * 28672 + 2 * (16384 + 8192) * 256 + (1 << 20)
    assert big.total - small.total >= 2 * 16384 * (28672 - 256)
    assert big.total - big.wsub < 2 * 8192 * 256 + (1 << 16)   # the weight slice stays at 256 columns


def test_gemm_dispatch(L):
    """Kernel choice by shape (host only), including the degenerate shapes:
    the large backward kernel reads two weight steps before its loop, so an
    empty contraction (N = 0) must never reach it."""
    fp, bp = L.lib.int8_linear_forward_plan, L.lib.int8_linear_backward_plan
    BF16, F16, F32 = L.I8L_BF16, L.I8L_F16, L.I8L_F32
    # forward: (dtype, M, K, N)
    assert fp(BF16, 4096, 4096, 4096) == 2          # 256 tiles of 256 x 256
    assert fp(BF16, 4096, 4096, 11008) == 2
    assert fp(F16, 2048, 4096, 4096) == 3           # 128 such tiles: half-width tiles
    assert fp(F32, 600, 4, 16) == 1
    assert fp(BF16, 4096, 4100, 4096) == 1          # K not a multiple of 16
    assert fp(BF16, 0, 4096, 4096) == 0 and fp(BF16, 4096, 4096, 0) == 0
    assert fp(BF16, 4096, 0, 4096) == 2             # K = 0: buffer loads past the end read zero
    assert fp(7, 1, 1, 1) == L.I8L_EDTYPE and fp(BF16, -1, 1, 1) == L.I8L_EINVAL
    assert fp(BF16, 8, L.I8L_MAX_K + 1, 8) == L.I8L_ESHAPE
    # backward: (dtype, M, N, K)
    assert bp(BF16, 4096, 4096, 4096) == 2
    assert bp(BF16, 4096, 11008, 4096) == 2
    assert bp(F16, 2048, 4096, 4096) == 3
    assert bp(F32, 4096, 4096, 4096) == 1           # fp32 gradients: generic kernel
    assert bp(BF16, 4096, 4100, 4096) == 1          # N % 8 != 0
    assert bp(BF16, 2048, 0, 2048) == 1             # empty contraction: the generic kernel writes zeros
    assert bp(F16, 2048, 0, 2048) == 1
    assert bp(BF16, 0, 4096, 4096) == 0 and bp(BF16, 4096, 4096, 0) == 0
    assert bp(BF16, 16384, 28672, 8192) == 2 and bp(BF16, 16384, 8192, 28672) == 2
    assert bp(BF16, 4096, 1 << 20, 4096) == 1       # beyond the 32-bit buffer offsets


def test_binding_rejects_mis_sized_results(L):
    """Result tensors passed in by the caller are checked for shape and dtype
    before any pointer reaches the library (a short buffer would be written
    past its end by the kernels)."""
    import torch
    import int8_quantized_linear_rowwise_amd as I8
    M, K, N = 4, 16, 8
    A = torch.zeros((M, K), dtype=torch.float16)
    G = torch.zeros((M, N), dtype=torch.float16)
    CB, SCB = torch.zeros((N, K), dtype=torch.int8), torch.zeros(N)
    CBt, SCBt = torch.zeros((K, N), dtype=torch.int8), torch.zeros(K)
    bad = [
        lambda: I8.int8_linear_forward(A, CB, SCB, out=torch.zeros((M, N - 1), dtype=torch.float16)),
        lambda: I8.int8_linear_forward(A, CB, SCB, c32=torch.zeros((M, N), dtype=torch.float32)),
        lambda: I8.int8_linear_backward_input(G, CB, SCB, grad_A=torch.zeros((M, K + 1), dtype=torch.float16)),
        lambda: I8.int8_linear_backward_input(G, CB.float(), SCB),
        lambda: I8.int8_linear_backward_input_int8(G, CBt, SCBt, c32=torch.zeros((M + 1, K), dtype=torch.int32)),
        lambda: I8.int8_linear_backward_input_int8(G, CBt, SCBt, grad_bias=torch.zeros(N, dtype=torch.float32)),
        lambda: I8.int8_linear_backward_input_int8(G, CB, SCB),
        lambda: I8.int8_linear_backward_weight(G, A, grad_W=torch.zeros((K, N), dtype=torch.float16)),
        lambda: I8.int8_linear_backward_weight(G, A[:3]),
        lambda: I8.int8_linear_backward_weight(G, A.float()),
    ]
    for f in bad:
        with pytest.raises(ValueError):
            f()


def test_noalloc_forward_host_errors(L):
    """The allocation-free forward validates like the forward and rejects a
    problem beyond its static scratch on the host, before any HIP call."""
    f = L.lib.int8_linear_forward_noalloc
    cap_max = L.lib.int8_linear_forward_noalloc_max_bytes()
    assert cap_max == L.I8L_NOALLOC_SCRATCH_BYTES == 64 << 20
    need = L.lib.int8_linear_forward_noalloc_bytes
    assert need(4096, 11008, 4096) <= cap_max         # the 7B block's widest input fits
    assert need(16384, 28672, 8192) > cap_max         # the 70B down layer does not
    assert need(300, 1040, 77) == L.lib.int8_linear_forward_workspace_bytes(300, 1040, 77, 64)
    assert need(5, 16, 3) == L.lib.int8_linear_forward_workspace_bytes(5, 16, 3, 16)
    assert need(-1, 4, 4) == 0 and need(4, 4, -1) == 0
    base = dict(A=FAKE, dt=2, M=8, K=64, CB=FAKE, SCB=FAKE, N=32, b=None, tau=6.0, out=FAKE, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["A"], a["dt"], a["M"], a["K"], a["CB"], a["SCB"], a["N"], a["b"], a["tau"], a["out"], a["st"])

    assert call(dt=9) == L.I8L_EDTYPE
    assert call(M=-1) == L.I8L_EINVAL
    assert call(A=0) == L.I8L_EINVAL
    assert call(out=0) == L.I8L_EINVAL
    assert call(K=L.I8L_MAX_K + 1) == L.I8L_ESHAPE
    assert call(M=16384, K=28672, N=8192) == L.I8L_ESCRATCH
    assert call(M=8192, K=8192) == L.I8L_ESCRATCH     # 64 MiB of codes alone
    assert call(M=0) == L.I8L_OK and call(N=0) == L.I8L_OK
    assert b"static scratch" in L.lib.int8_linear_strerror(L.I8L_ESCRATCH)


def test_header_compiles_as_c99_and_links(L, tmp_path):
    """include/int8lin.h is plain C: the C caller (tests/c_abi_main.c) compiles
    with gcc -std=c99 -Wall -Wextra -Werror and links against the library."""
    from tests import c_abi_build
    out = str(tmp_path / "c_abi_main")
    assert c_abi_build.build(out) == out and os.path.exists(out)
