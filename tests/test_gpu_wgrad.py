"""GPU parity of the weight gradient of the trainable-weight mode
(bitsandbytes PR #33's has_fp16_weights option): grad_W = D(fp16(G)^T fp16(A)),
fp32 accumulation, against the oracle's float64 value; the integer case
exactly against the textbook product.

No quantization is involved, so the gate is the arithmetic's own bound
rather than the pages' statistical one: one fp32 accumulation over M terms
and one rounding to D give |T - y| <= ulp_D(y) + M 2^-24 sum_m |g16 a16|.
Shapes cover the large-tile MFMA kernel (16-bit, N and K multiples of 8, at
least 16 output tiles of 256 x 256, ragged tiles and contraction tails) and
the general kernel (fp32, odd sizes, small outputs).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.formats import to_f64, to_half, ulp
from tests._gpu import assert_bits_equal, dev, host, tile_rows

pytestmark = pytest.mark.gpu

DTS = ["f16", "bf16", "f32"]


@pytest.fixture(scope="module")
def I8():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import int8_quantized_linear_rowwise_amd as I8
    return I8


def _case(dt, M, K, N, seed):
    c = workloads.small_case(dt, M, K, N, seed, n_outliers=min(3, K), has_bias=False)
    return c["A"], c["G"]


def assert_accum_gate(T, dt, y, G, A, rows, what):
    t = to_f64(T, dt)
    assert t.shape == y.shape, (what, t.shape, y.shape)
    if t.size == 0:
        return
    assert np.all(np.isfinite(t)), f"{what}: non-finite output"
    g16 = np.abs(to_half(G, dt).astype(np.float64))
    a16 = np.abs(to_half(A, dt).astype(np.float64))
    S = g16[:, rows].T @ a16
    lim = ulp(np.abs(y), dt) + G.shape[0] * 2.0 ** -24 * S
    err = np.abs(t - y)
    bad = err > lim
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {t.size} beyond the accumulation bound; worst "
                           f"{float((err / lim).max()):.3g}x")


def _check(I8, dt, M, K, N, seed, rows=None):
    A, G = _case(dt, M, K, N, seed)
    gW = I8.int8_linear_backward_weight(dev(G, dt), dev(A, dt))
    torch.cuda.synchronize()
    rows = np.arange(N) if rows is None else np.asarray(rows)
    r = oracle.linear_backward_weight(G, A, dt, rows=rows)
    got = host(gW.index_select(0, torch.from_numpy(rows).to("cuda:0")))
    assert_accum_gate(got, dt, r["y"], G, A, rows, "grad_W")


# (M, K, N): M tokens (the contraction), K input features, N output features
SMALL = [(1, 1, 1), (5, 7, 3), (70, 33, 45), (300, 130, 200), (129, 64, 1000), (1000, 8, 8), (64, 300, 40)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("M,K,N", SMALL)
def test_wgrad_parity_small(I8, dt, M, K, N):
    _check(I8, dt, M, K, N, 31)


# >= 16 output tiles of 256 x 256 with N % 8 == K % 8 == 0: the MFMA kernel
# (for 16-bit inputs); ragged output tiles and contraction tails
BIG = [(1000, 1024, 1024), (4096, 1288, 1032), (130, 2056, 1800), (63, 1024, 4104), (2049, 2048, 2048)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("M,K,N", BIG)
def test_wgrad_parity_large_tiles(I8, dt, M, K, N):
    rows = np.unique(np.concatenate([np.arange(0, N, 89), [N - 1, 255, 256, 257]]))
    _check(I8, dt, M, K, N, 32, rows=rows)


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_wgrad_integer_case_exact(I8, dt):
    g = np.random.default_rng(80)
    M, N, K = 1030, 1040, 1032
    G = g.integers(-4, 5, (M, N)).astype(np.float32)
    A = g.integers(-4, 5, (M, K)).astype(np.float32)
    ref = G.astype(np.int64).T @ A.astype(np.int64)
    gW = I8.int8_linear_backward_weight(dev(workloads._store(G, dt), dt), dev(workloads._store(A, dt), dt))
    torch.cuda.synchronize()
    # |ref| <= 16 M < 2^15: every partial sum is exact in fp32, so the output is
    # the exact product rounded once to the output type
    assert_bits_equal(host(gW), workloads._store(ref.astype(np.float32), dt), "grad_W textbook")


def test_wgrad_zero_tokens_and_empty(I8):
    G = torch.zeros((0, 300), dtype=torch.bfloat16, device="cuda:0")
    A = torch.zeros((0, 264), dtype=torch.bfloat16, device="cuda:0")
    gW = torch.full((300, 264), 7.0, dtype=torch.bfloat16, device="cuda:0")
    I8.int8_linear_backward_weight(G, A, grad_W=gW)
    torch.cuda.synchronize()
    assert not np.any(host(gW))
    assert I8.int8_linear_backward_weight(torch.zeros((5, 0), dtype=torch.float16, device="cuda:0"),
                                          torch.zeros((5, 3), dtype=torch.float16, device="cuda:0")).shape == (0, 3)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_wgrad_deterministic(I8, dt):
    A, G = _case(dt, 777, 1032, 1040, 33)
    At, Gt = dev(A, dt), dev(G, dt)
    ref = host(I8.int8_linear_backward_weight(Gt, At))
    for _ in range(5):
        assert_bits_equal(host(I8.int8_linear_backward_weight(Gt, At)), ref, "grad_W")


def test_wgrad_full_size_block(I8):
    """The 7B-class block's gate projection at its full size (M = 4096 tokens,
    K = 4096, N = 11008), gated on sampled weight rows."""
    wl = workloads.WORKLOADS["llama7b_block"]
    li = [i for i, L in enumerate(wl.layers) if L.name == "gate"][0]
    L = wl.layers[li]
    print(f"\n[llama7b_block/{L.name}] M={L.M} K={L.K} N={L.N} dt={wl.dtype}", flush=True)
    A = workloads.make_activation(wl, li)
    G = workloads.make_grad(wl, li)
    gW = I8.int8_linear_backward_weight(dev(G, wl.dtype), dev(A, wl.dtype))
    torch.cuda.synchronize()
    rows = tile_rows(L.N)          # one weight row in every 256-row output tile
    r = oracle.linear_backward_weight(G, A, wl.dtype, rows=rows)
    assert_accum_gate(host(gW.index_select(0, torch.from_numpy(rows).to("cuda:0"))), wl.dtype, r["y"], G, A,
                      rows, "grad_W (sampled rows)")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_trainable_module_matches_c_calls(I8, dt):
    """The trainable-weight module: output and all three gradients equal the
    C calls bit for bit, and after an update the forward uses the re-quantized
    weight."""
    M, K, N = 96, 264, 80
    c = workloads.small_case(dt, M, K, N, 34, n_outliers=3, has_bias=True)
    A, W, b, G = c["A"], workloads._store(c["W"], dt), c["bias"], c["G"]
    lin = I8.Int8LinearTrainable(dev(W, dt), dev(b, dt))
    x = dev(A, dt).reshape(2, 48, K).requires_grad_(True)
    y = lin(x)
    y.backward(dev(G, dt).reshape(2, 48, N))
    CB, SCB = I8.quantize_weight(dev(W, dt))
    out = I8.int8_linear_forward(dev(A, dt), CB, SCB, dev(b, dt), 6.0)
    gA, gb = I8.int8_linear_backward_input(dev(G, dt), CB, SCB)
    gW = I8.int8_linear_backward_weight(dev(G, dt), dev(A, dt))
    assert_bits_equal(host(y.detach().reshape(M, N)), host(out), "module out")
    assert_bits_equal(host(x.grad.reshape(M, K)), host(gA), "module grad_A")
    assert_bits_equal(host(lin.weight.grad), host(gW), "module grad_W")
    assert_bits_equal(host(lin.bias.grad), host(gb), "module grad_bias")
    with torch.no_grad():
        lin.weight -= 0.5 * lin.weight.grad
    y2 = lin(dev(A, dt))
    CB2, SCB2 = I8.quantize_weight(lin.weight.detach())
    assert not torch.equal(CB2, CB)
    assert_bits_equal(host(y2.detach()), host(I8.int8_linear_forward(dev(A, dt), CB2, SCB2, dev(b, dt), 6.0)),
                      "forward after the update")
