"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Integer results (codes, row scales as bits, outlier lists and counts, the
fp16 outlier sub-matrix, int32 accumulators, int8 weights) must match bit
for bit; float results must meet bitsandbytes PR #33's test bounds against
the oracle's float64 value plus a tight ulp bound. Sizes here span several
tiles with ragged tails; the full workload sizes are in test_gpu_workloads.py.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu import TORCH, assert_bits_equal, assert_float_gate, dev, host

pytestmark = pytest.mark.gpu

DTS = ["f16", "bf16", "f32"]


@pytest.fixture(scope="module")
def I8():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import int8_quantized_linear_rowwise_amd as I8
    return I8


def _quant_case(dt, R, C, seed, n_out=3, scale=20.0):
    g = np.random.default_rng(np.random.SeedSequence([7, R, C, seed]))
    x = g.standard_normal((R, C)).astype(np.float32)
    if n_out and C:
        cols = g.choice(C, min(n_out, C), replace=False)
        x[:, cols] *= np.float32(scale)
    return workloads._store(x, dt)


def _check_quant(I8, X, dt, tau, cap=None):
    """Two calls on one workspace that starts as arbitrary bytes (workspaces
    need no initialisation and are reused across calls)."""
    R, C = X.shape
    q = oracle.quantize_rowwise(X, dt, tau)
    capn = C if cap is None else cap
    wsb = I8.lib.int8_quantize_rowwise_workspace_bytes(R, C)
    ws = torch.full((max(wsb, 1),), 0xA7, dtype=torch.uint8, device="cuda:0")
    Xd = dev(X, dt)
    for call in range(2):
        codes, scale, idx, cnt, sub = I8.int8_quantize_rowwise(Xd, tau, cap, workspace=ws)
        torch.cuda.synchronize()
        n = int(host(cnt)[0])
        assert n == q["outliers"].size, (call, n, q["outliers"].size)
        k = min(n, capn)
        assert_bits_equal(host(codes), q["codes"], f"codes (call {call})")
        assert_bits_equal(host(scale), q["scale"], f"row scale (call {call})")
        assert_bits_equal(host(idx)[:k], q["outliers"][:k], f"outlier index list (call {call})")
        assert_bits_equal(host(sub)[:, :k], q["sub"][:, :k], f"outlier sub-matrix (call {call})")
    return q


# rows of up to 4096 16-bit values stay in a wave's registers (several rows per
# wave past 4096 rows), rows of up to 32768 in a workgroup's (4, 8 or 16
# chunks per thread; several rows per workgroup past 1024 rows); wider,
# ragged or fp32 rows stream through the cache twice
QSHAPES = [(1, 1), (3, 7), (17, 70), (64, 4096), (4100, 2048), (129, 4104), (4100, 4104), (5, 8200),
           (1100, 8200), (33, 11008), (3, 20000), (1030, 16392), (2, 40000), (600, 4), (600, 16), (1000, 64)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("R,C", QSHAPES)
def test_quantize_bit_exact(I8, dt, R, C):
    X = _quant_case(dt, R, C, 0)
    for tau in (6.0, 0.0, float("inf")):
        _check_quant(I8, X, dt, tau)


@pytest.mark.parametrize("dt", DTS)
def test_quantize_edge_cases(I8, dt):
    # ties at the threshold (6.0 is not an outlier), zero rows, rows with only outliers
    X = np.zeros((6, 40), np.float32)
    X[1, 3] = 6.0
    X[2, :] = 1.0
    X[2, 5] = 6.0078125
    X[3, 5] = 7.0
    X[4, 10] = -6.5
    X[4, 11] = 0.25
    X = workloads._store(X, dt)
    q = _check_quant(I8, X, dt, 6.0)
    assert q["outliers"].tolist() == [5, 10]
    # all-outlier input (tiny threshold), and a threshold below every value
    Y = _quant_case(dt, 9, 33, 1, n_out=0)
    q = _check_quant(I8, Y, dt, 1e-6)
    assert q["outliers"].size == 33
    # fp16-subnormal magnitudes
    g = np.random.default_rng(9)
    z = g.standard_normal((8, 48)).astype(np.float32) * np.float32(2.0 ** -20)
    _check_quant(I8, workloads._store(z, dt), dt, 6.0)


@pytest.mark.parametrize("dt", DTS)
def test_quantize_cap_overflow_visible(I8, dt):
    X = _quant_case(dt, 20, 64, 3, n_out=5)
    q = _check_quant(I8, X, dt, 6.0, cap=2)
    assert q["outliers"].size >= 5


# --------------------------------------------------------------------------
# forward / backward at sizes spanning several tiles


LSHAPES = [(1, 64, 1), (33, 70, 45), (130, 200, 260), (257, 4096, 300), (64, 16, 4), (600, 4, 16),
           (300, 1040, 520), (513, 256, 1031)]


def _layer(dt, M, K, N, seed, n_out=4, bias=True):
    c = workloads.small_case(dt, M, K, N, seed, n_outliers=min(n_out, K), has_bias=bias)
    return c["A"], c["W"], c["bias"], c["G"]


def _gpu_weights(I8, W):
    CB, SCB = I8.quantize_weight(dev(W))
    return CB, SCB


def _check_weights(I8, W):
    CB, SCB = _gpu_weights(I8, W)
    torch.cuda.synchronize()
    cb, scb = oracle.quantize_weight(W)
    assert_bits_equal(host(CB), cb, "CB")
    assert_bits_equal(host(SCB), scb, "SCB")
    return CB, SCB, cb, scb


def wsub_width(cap):
    """Columns of the weight's outlier slice for staging width cap (a multiple of 8, at most 256)."""
    return 0 if cap <= 0 else min((cap + 7) // 8 * 8, 256)


def _forward_and_check(I8, A, dt, CB, SCB, cb, scb, bias, tau, cap=None, rows=None):
    M, K = A.shape
    N = cb.shape[0]
    capn = K if cap is None else cap
    ws = I8.forward_workspace(M, K, N, capn, "cuda:0")
    ws.fill_(0x5C)                   # arbitrary bytes: workspaces need no initialisation
    c32 = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    Ad, bd = dev(A, dt), (dev(bias, dt) if bias is not None else None)
    out0 = I8.int8_linear_forward(Ad, CB, SCB, bd, tau, capn, workspace=ws)
    out = I8.int8_linear_forward(Ad, CB, SCB, bd, tau, capn, c32=c32, workspace=ws)
    torch.cuda.synchronize()
    assert_bits_equal(host(out0), host(out), "out of two calls on one workspace")
    f = oracle.linear_forward(A, dt, cb, scb, bias, tau, rows=rows)
    q = f["q"]
    # the forward's own quantization, read back from its workspace
    L = I8.forward_layout(M, K, N, capn)
    wsh = host(ws)
    cnt = int(wsh[L.count:L.count + 4].view(np.int32)[0])
    assert cnt == q["outliers"].size
    k = min(cnt, capn)
    # the list holds every outlier column; the first cap of them are staged
    assert_bits_equal(wsh[L.idx:L.idx + 4 * cnt].view(np.int32), q["outliers"], "forward outlier list")
    assert_bits_equal(wsh[L.scale:L.scale + 4 * M].view(np.float32), q["scale"], "SCA")
    assert_bits_equal(wsh[L.codes:L.codes + M * K].view(np.int8).reshape(M, K), q["codes"], "CA")
    if capn:
        subw = wsh[L.sub:L.sub + 2 * M * capn].view(np.float16).reshape(M, capn)[:, :k]
        assert_bits_equal(subw, q["sub"][:, :k], "subA")
    # the weight's dequantized outlier slice written by the row pass
    wcap = wsub_width(capn)
    kw = min(cnt, wcap)
    if kw:
        wsw = wsh[L.wsub:L.wsub + 2 * N * wcap].view(np.float16).reshape(N, wcap)[:, :kw]
        assert_bits_equal(wsw, oracle.dequant_weight(cb, scb, cols=q["outliers"][:kw]), "weight outlier slice")
    idx = f["rows"]
    assert_bits_equal(host(c32)[idx], f["c32"].astype(np.int32), "C32")
    assert_float_gate(host(out)[idx], dt, f["y"], "out")
    return out, f


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("M,K,N", LSHAPES)
def test_forward_parity(I8, dt, M, K, N):
    A, W, b, _ = _layer(dt, M, K, N, 1)
    CB, SCB, cb, scb = _check_weights(I8, W)
    _forward_and_check(I8, A, dt, CB, SCB, cb, scb, b, 6.0)
    _forward_and_check(I8, A, dt, CB, SCB, cb, scb, None, float("inf"))


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("M,K,N", LSHAPES)
def test_backward_parity(I8, dt, M, K, N):
    _, W, _, G = _layer(dt, M, K, N, 2)
    CB, SCB, cb, scb = _check_weights(I8, W)
    gA, gb = I8.int8_linear_backward_input(dev(G, dt), CB, SCB, with_grad_bias=True)
    torch.cuda.synchronize()
    r = oracle.linear_backward_input(G, dt, cb, scb)
    assert_float_gate(host(gA), dt, r["y"], "grad_A")
    gb64, _ = oracle.grad_bias(G, dt)
    assert_float_gate(host(gb), dt, gb64, "grad_bias", tight_rel=2.0 ** -16)


# shapes with at least 64 output tiles of 256 x 256, which select the
# large-tile pipelined kernels (with half-width tiles up to 128 such tiles);
# ragged in every dimension (partial tiles and a contraction tail that is not
# a multiple of the k step)
BIG_FWD = [(2100, 1040, 2090), (2048, 4096, 2048), (1030, 528, 4100), (2304, 16, 2304), (2100, 1040, 4200),
           (4100, 528, 2090)]
BIG_BWD = [(2100, 2088, 1044), (2048, 2048, 2048), (2060, 1000, 4100), (2304, 8, 2304), (2100, 1000, 2092),
           (4100, 1000, 2092)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("M,K,N", BIG_FWD)
def test_forward_parity_large_tiles(I8, dt, M, K, N):
    A, W, b, _ = _layer(dt, M, K, N, 7, n_out=5)
    CB, SCB, cb, scb = _check_weights(I8, W)
    rows = np.unique(np.concatenate([np.arange(0, M, 97), [M - 1, 255, 256, 257]]))
    _forward_and_check(I8, A, dt, CB, SCB, cb, scb, b, 6.0, rows=rows)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("M,N,K", BIG_BWD)
def test_backward_parity_large_tiles(I8, dt, M, N, K):
    _, W, _, G = _layer(dt, M, K, N, 8)
    CB, SCB, cb, scb = _check_weights(I8, W)
    gA, gb = I8.int8_linear_backward_input(dev(G, dt), CB, SCB, with_grad_bias=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, M, 97), [M - 1, 255, 256, 257]]))
    r = oracle.linear_backward_input(G, dt, cb, scb, rows=rows)
    assert_float_gate(host(gA)[rows], dt, r["y"], "grad_A")
    gb64, _ = oracle.grad_bias(G, dt)
    assert_float_gate(host(gb), dt, gb64, "grad_bias", tight_rel=2.0 ** -16)


@pytest.mark.parametrize("dt", DTS)
def test_forward_zero_input_is_bias_bitwise(I8, dt):
    M, K, N = 70, 96, 130
    _, W, b, _ = _layer(dt, M, K, N, 3)
    CB, SCB = _gpu_weights(I8, W)
    A = workloads._store(np.zeros((M, K), np.float32), dt)
    out = I8.int8_linear_forward(dev(A, dt), CB, SCB, dev(b, dt), 6.0)
    assert_bits_equal(host(out), np.broadcast_to(b, (M, N)).copy(), "out == bias")


def _int_weights(g, N, K):
    W = g.integers(-127, 128, (N, K)).astype(np.float32)
    W[np.arange(N), g.integers(0, K, N)] = np.where(g.random(N) < 0.5, -127, 127)
    return W


def test_forward_integer_case_exact(I8):
    g = np.random.default_rng(50)
    M, K, N = 150, 320, 140
    A = _int_weights(g, M, K)
    W = _int_weights(g, N, K)
    CB, SCB = _gpu_weights(I8, W)
    c32 = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    out = I8.int8_linear_forward(dev(A), CB, SCB, None, float("inf"), c32=c32)
    ref = A.astype(np.int64) @ W.astype(np.int64).T
    assert_bits_equal(host(c32), ref.astype(np.int32), "C32 textbook")
    assert np.array_equal(host(out).astype(np.float64), ref.astype(np.float64))


def test_forward_all_outliers(I8):
    g = np.random.default_rng(51)
    M, K, N = 90, 72, 50
    A = (g.uniform(0.5, 2, (M, K)) * np.where(g.random((M, K)) < .5, -1, 1)).astype(np.float16)
    W = _int_weights(g, N, K)
    CB, SCB = _gpu_weights(I8, W)
    b = (g.standard_normal(N) * 0.01).astype(np.float16)
    out = I8.int8_linear_forward(dev(A), CB, SCB, dev(b), 1e-3)
    ref = A.astype(np.float64) @ W.astype(np.float64).T + b.astype(np.float64)
    assert_float_gate(host(out), "f16", ref, "all-outlier out")


def test_backward_integer_case_exact(I8):
    g = np.random.default_rng(52)
    M, N, K = 200, 300, 260
    W = _int_weights(g, N, K)
    CB, SCB = _gpu_weights(I8, W)
    G = g.integers(-1, 2, (M, N)).astype(np.float32)
    gA, _ = I8.int8_linear_backward_input(dev(G), CB, SCB, with_grad_bias=False)
    ref = G.astype(np.int64) @ W.astype(np.int64)
    assert np.array_equal(host(gA), ref.astype(np.float32))


# more outlier columns than the staging width: the epilogue reads the values
# of the columns past `cap` from the input itself. Shapes for the generic
# kernel and for both large-tile kernels (256 x 128 and 256 x 256 tiles);
# 21 seeded columns, so that the outlier product runs past the 16 columns the
# large kernels stage in LDS
OSHAPES = [(300, 1040, 520), (1024, 1024, 4096), (1040, 512, 8320)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("M,K,N", OSHAPES)
def test_forward_outliers_beyond_staging(I8, dt, M, K, N):
    A, W, b, _ = _layer(dt, M, K, N, 4, n_out=21)
    CB, SCB, cb, scb = _check_weights(I8, W)
    outs = {}
    for cap in (K, 0, 2, 16, 17):
        print(f"  [{dt} {M}x{K}x{N}] cap={cap}", flush=True)
        out, f = _forward_and_check(I8, A, dt, CB, SCB, cb, scb, b, 6.0, cap=cap)
        assert f["q"]["outliers"].size >= 21
        outs[cap] = host(out)
    for cap in (0, 2, 16, 17):       # identical bits whatever the staging width
        assert_bits_equal(outs[cap], outs[K], f"out with cap={cap} against cap=K")
    ws = I8.forward_workspace(M, K, N, 3, "cuda:0")
    I8.int8_linear_forward(dev(A, dt), CB, SCB, dev(b, dt), 6.0, cap=3, workspace=ws)
    assert I8.forward_check(ws, M, K, N, 3) == f["q"]["outliers"].size


# many outlier columns (150 and 300, beyond the 256-column staging): the
# generic kernel and both large-tile kernels, with the default staging width
# (16-byte staged reads up to 256 columns, gathered values beyond) and with a
# staging width that is not a multiple of 8 (every value gathered); the bits
# must not depend on it
MSHAPES = [(300, 1040, 520), (2100, 1040, 2090), (1040, 512, 8320)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("M,K,N", MSHAPES)
@pytest.mark.parametrize("n_out", [150, 300])
def test_forward_many_outliers(I8, dt, M, K, N, n_out):
    A, W, b, _ = _layer(dt, M, K, N, 9, n_out=n_out)
    CB, SCB, cb, scb = _check_weights(I8, W)
    rows = np.unique(np.concatenate([np.arange(0, M, 61), [M - 1, 255, 256, 257]]))
    outs = {}
    for cap in (None, 100):
        print(f"  [{dt} {M}x{K}x{N}] outliers={n_out} cap={cap}", flush=True)
        out, f = _forward_and_check(I8, A, dt, CB, SCB, cb, scb, b, 6.0, cap=I8.default_cap(K) if cap is None
                                    else cap, rows=rows)
        assert f["q"]["outliers"].size >= n_out
        outs[cap] = host(out)
    assert_bits_equal(outs[100], outs[None], "out with cap=100 against the default staging")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_backward_empty_contraction_is_zero(I8, dt):
    """N = 0 output features with M = K = 2048 (a shape whose non-empty
    version takes the large-tile kernel): grad_A is all zeros and grad_bias
    empty; the empty weight arrives as a NULL pointer."""
    M, K = 2048, 2048
    assert I8.lib.int8_linear_backward_plan(I8.DTYPE_CODE[TORCH[dt]], M, 0, K) == 1
    G = torch.empty((M, 0), dtype=TORCH[dt], device="cuda:0")
    CB = torch.empty((0, K), dtype=torch.int8, device="cuda:0")
    SCB = torch.empty((0,), dtype=torch.float32, device="cuda:0")
    gA = torch.full((M, K), 7.0, dtype=TORCH[dt], device="cuda:0")
    gA, gb = I8.int8_linear_backward_input(G, CB, SCB, with_grad_bias=True, grad_A=gA)
    torch.cuda.synchronize()
    assert gb.numel() == 0
    assert torch.count_nonzero(gA).item() == 0


def test_empty_and_degenerate(I8):
    CB, SCB = _gpu_weights(I8, np.ones((8, 16), np.float32))
    A = torch.zeros((0, 16), dtype=torch.float16, device="cuda:0")
    assert I8.int8_linear_forward(A, CB, SCB).shape == (0, 8)
    G = torch.zeros((0, 8), dtype=torch.float16, device="cuda:0")
    gA, gb = I8.int8_linear_backward_input(G, CB, SCB)
    torch.cuda.synchronize()
    assert gA.shape == (0, 16) and np.all(host(gb) == 0)
    # K = 0: out = bias
    CB0 = torch.zeros((8, 0), dtype=torch.int8, device="cuda:0")
    SCB0 = torch.zeros((8,), dtype=torch.float32, device="cuda:0")
    b = torch.arange(8, dtype=torch.float16, device="cuda:0")
    out = I8.int8_linear_forward(torch.zeros((5, 0), dtype=torch.float16, device="cuda:0"), CB0, SCB0, b)
    assert np.array_equal(host(out), np.broadcast_to(host(b), (5, 8)))


def test_rejects_cpu_tensors(I8):
    with pytest.raises(ValueError):
        I8.int8_linear_forward(torch.zeros((2, 16)), torch.zeros((4, 16), dtype=torch.int8),
                               torch.zeros(4))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_determinism_ten_runs(I8, dt):
    """bitsandbytes PR #33 ran every test ten times for stability: outputs must be bitwise identical."""
    M, K, N = 520, 1100, 700
    A, W, b, G = _layer(dt, M, K, N, 5)
    CB, SCB = _gpu_weights(I8, W)
    At, bt, Gt = dev(A, dt), dev(b, dt), dev(G, dt)
    ref = None
    for _ in range(10):
        out = I8.int8_linear_forward(At, CB, SCB, bt, 6.0)
        gA, gb = I8.int8_linear_backward_input(Gt, CB, SCB)
        cur = (host(out), host(gA), host(gb))
        if ref is None:
            ref = cur
        else:
            for a, r, w in zip(cur, ref, ("out", "grad_A", "grad_bias")):
                assert_bits_equal(a, r, w)


# --------------------------------------------------------------------------
# autograd glue and the residual MLP of the EasyDeL example


@pytest.mark.parametrize("dt", DTS)
def test_autograd_module_matches_c_calls(I8, dt):
    M, K, N = 96, 200, 72
    A, W, b, G = _layer(dt, M, K, N, 6)
    lin = I8.Int8Linear(dev(W), dev(b, dt).float()).cuda()
    x = dev(A, dt).reshape(2, 48, K).requires_grad_(True)
    y = lin(x)
    y.backward(dev(G, dt).reshape(2, 48, N))
    out = I8.int8_linear_forward(dev(A, dt), lin.CB, lin.SCB, lin.bias.detach().to(TORCH[dt]), 6.0)
    gA, gb = I8.int8_linear_backward_input(dev(G, dt), lin.CB, lin.SCB)
    assert_bits_equal(host(y.detach().reshape(M, N)), host(out), "module out")
    assert_bits_equal(host(x.grad.reshape(M, K)), host(gA), "module grad_A")
    assert_bits_equal(host(lin.bias.grad.to(TORCH[dt])), host(gb), "module grad_bias")


def test_mlp600_residual_example(I8):
    wl = workloads.WORKLOADS["mlp600"]
    x = workloads.make_activation(wl, 0)
    g = workloads.make_grad(wl, 1)
    Ws = [workloads.make_weight(wl, i) for i in range(2)]
    bs = [workloads.make_bias(wl, i) for i in range(2)]
    layers = []
    for W, b in zip(Ws, bs):
        cb, s = oracle.quantize_weight(W)
        layers.append((cb, s, b))
    r = oracle.mlp_forward_backward(x, g, "f32", layers, wl.threshold)
    # GPU: the int8 linears and the SiLU between them from the library (the
    # SiLU kernel also hands the second linear its input's outlier flags);
    # the residual add and SiLU's derivative as torch glue
    gw = [_gpu_weights(I8, W) for W in Ws]
    xt, gt = dev(x), dev(g)
    h = I8.int8_linear_forward(xt, gw[0][0], gw[0][1], dev(bs[0]), wl.threshold)
    a, flags = I8.silu_outlier_flags(h, wl.threshold)
    o = I8.int8_linear_forward_flagged(a, flags, gw[1][0], gw[1][1], dev(bs[1])) + xt
    ga, gb2 = I8.int8_linear_backward_input(gt, gw[1][0], gw[1][1])
    sg = torch.sigmoid(h)
    gh = ga * sg * (1 + h * (1 - sg))
    gx, gb1 = I8.int8_linear_backward_input(gh, gw[0][0], gw[0][1])
    gx = gx + gt
    torch.cuda.synchronize()
    assert_float_gate(host(a), "f32", oracle.to_f64(r["a"], "f32"), "mlp SiLU", tight_rel=2.0 ** -8)
    assert_float_gate(host(o), "f32", oracle.to_f64(r["out"], "f32"), "mlp out", tight_rel=2.0 ** -8)
    assert_float_gate(host(gx), "f32", oracle.to_f64(r["grad_x"], "f32"), "mlp grad_x", tight_rel=2.0 ** -8)
    assert_float_gate(host(gb2), "f32", oracle.grad_bias(g, "f32")[0], "mlp grad_bias 2", tight_rel=2.0 ** -16)
    assert_float_gate(host(gb1), "f32", oracle.grad_bias(r["g_h"], "f32")[0], "mlp grad_bias 1", tight_rel=2.0 ** -8)
    # the second layer's quantizer on the oracle's own SiLU output is bit-exact
    _check_quant(I8, r["a"], "f32", wl.threshold)
