"""GPU parity of the producer-side outlier flags (EasyDeL discussion #66's
Dense -> SiLU -> Dense): the activation kernel writes A = D(SiLU(H)) and A's
outlier-column flags in one pass; the flagged forward uses those flags
instead of its own flagging read of A.

Checked: A against the oracle's float64 SiLU rounded once (at most one unit
in the last place of D off: the kernel evaluates SiLU in fp32); the flags
bit-exactly against the oracle's outlier columns of the kernel's own A; the
flagged forward bit-for-bit against the ordinary forward on the same A
(codes, scales, outlier list, int32 accumulators, output); and the two-layer
chain against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.formats import to_f64, to_half, ulp
from tests._gpu import assert_bits_equal, assert_float_gate, dev, host

pytestmark = pytest.mark.gpu

DTS = ["f16", "bf16", "f32"]


@pytest.fixture(scope="module")
def I8():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import int8_quantized_linear_rowwise_amd as I8
    return I8


def _H(dt, R, C, seed, hot=3):
    g = np.random.default_rng(np.random.SeedSequence([91, R, C, seed]))
    h = (g.standard_normal((R, C)) * 2).astype(np.float32)
    if hot and C:
        cols = g.choice(C, min(hot, C), replace=False)
        h[g.integers(0, R, len(cols)), cols] = 7.5      # SiLU(7.5) ~ 7.496 > 6: outlier columns of A
    return workloads._store(h, dt)


def _mask(I8, flags, R, C):
    words = I8.lib.int8_outlier_flags_words(R, C)
    nw = (C + 31) // 32
    w = host(flags)[:words].view(np.uint32).reshape(words // nw, nw)
    m = np.bitwise_or.reduce(w, axis=0)
    return np.array([c for c in range(C) if (m[c >> 5] >> (c & 31)) & 1], dtype=np.int32)


SHAPES = [(1, 1), (3, 7), (17, 70), (64, 4096), (129, 4104), (600, 16), (33, 11008), (1000, 64)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("R,C", SHAPES)
def test_silu_and_flags(I8, dt, R, C):
    H = _H(dt, R, C, 1)
    A, flags = I8.silu_outlier_flags(dev(H, dt), 6.0)
    torch.cuda.synchronize()
    r = oracle.silu_activation(H, dt)
    a = to_f64(host(A), dt)
    lim = ulp(np.abs(r["y"]), dt) * (1.0 if dt != "f32" else 4.0)
    assert np.all(np.abs(a - r["y"]) <= lim + 1e-300), "SiLU beyond one unit in the last place"
    want = oracle.outlier_columns(to_half(host(A), dt), 6.0)
    assert_bits_equal(_mask(I8, flags, R, C), want, "outlier columns of A")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_flags_off_flag_nothing(I8, dt):
    H = _H(dt, 50, 300, 2)
    for tau in (0.0, float("inf")):
        _, flags = I8.silu_outlier_flags(dev(H, dt), tau)
        torch.cuda.synchronize()
        assert _mask(I8, flags, 50, 300).size == 0


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("M,K,N", [(33, 70, 45), (257, 4096, 300), (600, 16, 4), (2100, 1040, 2090)])
def test_flagged_forward_equals_forward(I8, dt, M, K, N):
    H = _H(dt, M, K, 3, hot=5)
    c = workloads.small_case(dt, M, K, N, 4, has_bias=True)
    CB, SCB = I8.quantize_weight(dev(c["W"]))
    b = dev(c["bias"], dt)
    A, flags = I8.silu_outlier_flags(dev(H, dt), 6.0)
    ws1, ws2 = I8.forward_workspace(M, K, N, K, "cuda:0"), I8.forward_workspace(M, K, N, K, "cuda:0")
    c1 = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    c2 = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    o1 = I8.int8_linear_forward(A, CB, SCB, b, 6.0, K, c32=c1, workspace=ws1)
    o2 = I8.int8_linear_forward_flagged(A, flags, CB, SCB, b, K, c32=c2, workspace=ws2)
    torch.cuda.synchronize()
    assert_bits_equal(host(c2), host(c1), "C32")
    assert_bits_equal(host(o2), host(o1), "out")
    lay = I8.forward_layout(M, K, N, K)
    cnt = int(host(ws1[lay.count:lay.count + 4]).view(np.int32)[0])
    assert cnt >= 1
    # the outlier list holds `count` entries; the rest of its buffer is not written
    for name, off, n in (("count", lay.count, 4), ("outlier list", lay.idx, 4 * cnt), ("SCA", lay.scale, 4 * M),
                         ("CA", lay.codes, M * K)):
        assert_bits_equal(host(ws2[off:off + n]), host(ws1[off:off + n]), name)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_mlp_chain_through_producer_flags(I8, dt):
    """x -> linear 1 -> SiLU (+ flags) -> flagged linear 2: layer 2 against the
    oracle on the kernel's own activation (bit-exact int32 accumulators)."""
    M, K, Hd, N = 600, 64, 256, 48
    g = np.random.default_rng(92)
    x = workloads._store((g.standard_normal((M, K)) * 2).astype(np.float32), dt)
    W1 = (g.standard_normal((Hd, K)) * 0.3).astype(np.float32)
    W2 = (g.standard_normal((N, Hd)) * 0.1).astype(np.float32)
    CB1, SCB1 = I8.quantize_weight(dev(W1))
    CB2, SCB2 = I8.quantize_weight(dev(W2))
    h = I8.int8_linear_forward(dev(x, dt), CB1, SCB1, None, 6.0)
    a, flags = I8.silu_outlier_flags(h, 6.0)
    c32 = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    y = I8.int8_linear_forward_flagged(a, flags, CB2, SCB2, None, c32=c32)
    torch.cuda.synchronize()
    cb2, scb2 = oracle.quantize_weight(W2)
    f2 = oracle.linear_forward(host(a), dt, cb2, scb2, None, 6.0)
    assert f2["q"]["outliers"].size >= 1
    assert_bits_equal(host(c32), f2["c32"].astype(np.int32), "layer-2 C32")
    assert_float_gate(host(y), dt, f2["y"], "layer-2 out")


def test_full_size_down_projection_input(I8):
    """The 7B-class block's widest input (4096 tokens x 11008, bf16): the SiLU
    kernel's flags bit-exact against the oracle's outlier columns of its A,
    and the flagged forward bit-identical to the ordinary one."""
    wl = workloads.WORKLOADS["llama7b_block"]
    li = [i for i, L in enumerate(wl.layers) if L.name == "down"][0]
    L = wl.layers[li]
    print(f"\n[llama7b_block/{L.name} input] {L.M} x {L.K} bf16", flush=True)
    H = workloads.make_activation(wl, li)
    A, flags = I8.silu_outlier_flags(dev(H, "bf16"), wl.threshold)
    torch.cuda.synchronize()
    Ah = host(A)
    want = oracle.outlier_columns(to_half(Ah, "bf16"), wl.threshold)
    assert want.size >= 1
    assert_bits_equal(_mask(I8, flags, L.M, L.K), want, "outlier columns of A")
    rows = np.array([0, 1, 2047, L.M - 1])
    y = oracle.silu_activation(H[rows], "bf16")["y"]
    a = to_f64(Ah[rows], "bf16")
    assert np.all(np.abs(a - y) <= ulp(np.abs(y), "bf16") + 1e-300)
    W = workloads.make_weight(wl, li)
    CB, SCB = I8.quantize_weight(dev(W))
    del W
    o1 = I8.int8_linear_forward(A, CB, SCB, None, wl.threshold)
    o2 = I8.int8_linear_forward_flagged(A, flags, CB, SCB, None)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_flagged_forward_beyond_staging(I8):
    """More flagged columns than the outlier staging holds: the flagged forward
    reads the rest from its input, exactly as the ordinary forward does."""
    M, K, N = 40, 64, 32
    H = _H("f16", M, K, 5, hot=6)
    A, flags = I8.silu_outlier_flags(dev(H, "f16"), 6.0)
    CB, SCB = I8.quantize_weight(torch.randn(N, K, device="cuda:0") * 0.02)
    ws = I8.forward_workspace(M, K, N, 2, "cuda:0")
    o2 = I8.int8_linear_forward_flagged(A, flags, CB, SCB, None, cap=2, workspace=ws)
    assert I8.forward_check(ws, M, K, N, 2) >= 6
    oK = I8.int8_linear_forward_flagged(A, flags, CB, SCB, None, cap=K)
    oP = I8.int8_linear_forward(A, CB, SCB, None, 6.0, cap=K)
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), oK.view(torch.int16))
    assert torch.equal(o2.view(torch.int16), oP.view(torch.int16))
