"""GPU parity of the int8 backward variant (EasyDeL discussion #66, the
bwd_bits=8 choice): grad_output quantized row-wise, multiplied in int8 by a
second weight copy quantized along the input features, the int32 product
dequantized with both scales.

Bit-exact: the column-quantized weight copy (CBt, SCBt) and the int32
product C32. Float: grad_A against the oracle's float64 value (pages' bounds
plus the tight ulp bound), grad_bias as in the fp16 backward. The integer
case (G and the weight already on the int8 grid with a full-range entry in
every row) reduces to the textbook integer product, exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu import assert_bits_equal, assert_float_gate, dev, host, tile_rows

pytestmark = pytest.mark.gpu

DTS = ["f16", "bf16", "f32"]


@pytest.fixture(scope="module")
def I8():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import int8_quantized_linear_rowwise_amd as I8
    return I8


def _case(dt, M, K, N, seed):
    c = workloads.small_case(dt, M, K, N, seed, n_outliers=min(3, K), has_bias=True)
    return c["W"], c["G"]


def _weights_t(I8, W):
    CBt, SCBt = I8.quantize_weight_colwise(dev(W))
    torch.cuda.synchronize()
    cbt, scbt = oracle.quantize_weight_colwise(W)
    assert_bits_equal(host(CBt), cbt, "CBt")
    assert_bits_equal(host(SCBt), scbt, "SCBt")
    return CBt, SCBt, cbt, scbt


def _run_and_check(I8, G, dt, CBt, SCBt, cbt, scbt, rows=None):
    M, N = G.shape
    K = cbt.shape[0]
    c32 = torch.empty((M, K), dtype=torch.int32, device="cuda:0")
    gA, gb = I8.int8_linear_backward_input_int8(dev(G, dt), CBt, SCBt, with_grad_bias=True, c32=c32)
    torch.cuda.synchronize()
    r = oracle.linear_backward_input_int8(G, dt, cbt, scbt, rows=rows)
    if rows is None:
        assert_bits_equal(host(c32), r["c32"].astype(np.int32), "C32")
        assert_float_gate(host(gA), dt, r["y"], "grad_A")
    else:
        rt = torch.from_numpy(np.asarray(rows)).to("cuda:0")
        assert_bits_equal(host(c32.index_select(0, rt)), r["c32"].astype(np.int32), "C32 (sampled rows)")
        assert_float_gate(host(gA.index_select(0, rt)), dt, r["y"], "grad_A (sampled rows)")
    gb64, _ = oracle.grad_bias(G, dt)
    assert_float_gate(host(gb), dt, gb64, "grad_bias", tight_rel=2.0 ** -16)


# (M, K, N): M tokens, K input features (grad_A columns), N output features
# (the contraction); ragged against the 256 x 256 output tiles and the k step
SHAPES = [(1, 64, 1), (33, 70, 45), (130, 200, 260), (257, 300, 4096), (64, 4, 16), (600, 16, 4),
          (300, 520, 1040), (513, 1031, 256)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_backward_int8_parity(I8, dt, M, K, N):
    W, G = _case(dt, M, K, N, 21)
    CBt, SCBt, cbt, scbt = _weights_t(I8, W)
    _run_and_check(I8, G, dt, CBt, SCBt, cbt, scbt)


# at least 64 output tiles: the large-tile pipelined forward kernel
BIG = [(2100, 1044, 2088), (2048, 2048, 2048), (2060, 4100, 1000), (2304, 2304, 8)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("M,K,N", BIG)
def test_backward_int8_parity_large_tiles(I8, dt, M, K, N):
    W, G = _case(dt, M, K, N, 22)
    CBt, SCBt, cbt, scbt = _weights_t(I8, W)
    rows = np.unique(np.concatenate([np.arange(0, M, 97), [M - 1, 255, 256, 257]]))
    _run_and_check(I8, G, dt, CBt, SCBt, cbt, scbt, rows=rows)


def _int_matrix(g, R, C):
    X = g.integers(-127, 128, (R, C)).astype(np.float32)
    X[np.arange(R), g.integers(0, C, R)] = np.where(g.random(R) < 0.5, -127, 127)
    return X


def test_backward_int8_integer_case_exact(I8):
    # every row of G and every column of W already on the int8 grid with one
    # entry of magnitude 127: both quantizations are the identity, the scales
    # are 127 and 127 * 127 / 127^2 = 1, so grad_A = G @ W exactly
    g = np.random.default_rng(60)
    M, N, K = 200, 300, 260
    G = _int_matrix(g, M, N)
    W = np.ascontiguousarray(_int_matrix(g, K, N).T)
    CBt, SCBt = I8.quantize_weight_colwise(dev(W))
    c32 = torch.empty((M, K), dtype=torch.int32, device="cuda:0")
    gA, gb = I8.int8_linear_backward_input_int8(dev(G), CBt, SCBt, with_grad_bias=False, c32=c32)
    assert gb is None
    ref = G.astype(np.int64) @ W.astype(np.int64)
    assert_bits_equal(host(c32), ref.astype(np.int32), "C32 textbook")
    assert np.array_equal(host(gA), ref.astype(np.float32))


@pytest.mark.parametrize("dt", DTS)
def test_backward_int8_zero_grad_is_zero(I8, dt):
    M, K, N = 70, 96, 130
    W, _ = _case(dt, M, K, N, 23)
    CBt, SCBt = I8.quantize_weight_colwise(dev(W))
    G = workloads._store(np.zeros((M, N), np.float32), dt)
    gA, gb = I8.int8_linear_backward_input_int8(dev(G, dt), CBt, SCBt)
    torch.cuda.synchronize()
    assert not np.any(host(gA).astype(np.float64)), "grad_A of a zero G"
    assert not np.any(host(gb).astype(np.float64)), "grad_bias of a zero G"


def test_backward_int8_empty_and_degenerate(I8):
    W = np.ones((8, 16), np.float32)
    CBt, SCBt = I8.quantize_weight_colwise(dev(W))
    assert CBt.shape == (16, 8) and SCBt.shape == (16,)
    # M = 0: empty grad_A, grad_bias = 0
    gA, gb = I8.int8_linear_backward_input_int8(torch.zeros((0, 8), dtype=torch.float16, device="cuda:0"), CBt, SCBt)
    torch.cuda.synchronize()
    assert gA.shape == (0, 16) and np.all(host(gb) == 0)
    # N = 0 (no output features): grad_A = 0, grad_bias empty
    CBt0 = torch.zeros((16, 0), dtype=torch.int8, device="cuda:0")
    gA, gb = I8.int8_linear_backward_input_int8(torch.zeros((5, 0), dtype=torch.float16, device="cuda:0"), CBt0,
                                                SCBt)
    torch.cuda.synchronize()
    assert gA.shape == (5, 16) and gb.shape == (0,) and np.all(host(gA) == 0)
    # K = 0 (no input features): grad_A empty, grad_bias still the column sums
    Gs = np.arange(15, dtype=np.float32).reshape(5, 3).astype(np.float16)
    gA, gb = I8.int8_linear_backward_input_int8(dev(Gs), torch.zeros((0, 3), dtype=torch.int8, device="cuda:0"),
                                                torch.zeros((0,), dtype=torch.float32, device="cuda:0"))
    torch.cuda.synchronize()
    assert gA.shape == (5, 0)
    assert np.array_equal(host(gb), Gs.astype(np.float32).sum(0).astype(np.float16))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_backward_int8_deterministic_and_workspace_reuse(I8, dt):
    # a larger call, then a smaller one in the same workspace, each repeated:
    # bitwise identical results, and the second matches a fresh-workspace call
    shapes = [(520, 700, 1100), (130, 200, 260)]
    ws = I8.backward_int8_workspace(520, 1100, True, "cuda:0")
    for i, (M, K, N) in enumerate(shapes):
        W, G = _case(dt, M, K, N, 24 + i)
        CBt, SCBt = I8.quantize_weight_colwise(dev(W))
        Gt = dev(G, dt)
        ref = [host(t) for t in I8.int8_linear_backward_input_int8(Gt, CBt, SCBt)]
        for _ in range(5):
            cur = [host(t) for t in I8.int8_linear_backward_input_int8(Gt, CBt, SCBt, workspace=ws)]
            for a, r, w in zip(cur, ref, ("grad_A", "grad_bias")):
                assert_bits_equal(a, r, w)


def test_backward_int8_full_size_block(I8):
    """The 7B-class block's gate projection at its full size (M = 4096 tokens,
    K = 4096 input features, contraction over N = 11008 output features):
    bit-exact CBt / SCBt and C32, gated grad_A on sampled rows."""
    wl = workloads.WORKLOADS["llama7b_block"]
    li = [i for i, L in enumerate(wl.layers) if L.name == "gate"][0]
    L = wl.layers[li]
    dt = wl.dtype
    print(f"\n[llama7b_block/{L.name}] M={L.M} K={L.K} N={L.N} dt={dt}", flush=True)
    W = workloads.make_weight(wl, li)
    CBt, SCBt, cbt, scbt = _weights_t(I8, W)
    del W
    G = workloads.make_grad(wl, li)
    rows = tile_rows(L.M)
    _run_and_check(I8, G, dt, CBt, SCBt, cbt, scbt, rows=rows)
