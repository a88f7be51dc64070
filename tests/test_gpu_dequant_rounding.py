"""Dequantized weights at fp16 midpoints (GPU against the oracle, bit for bit).

Wdq[n, k] = fp16(fl32(CB[n, k] * fl32(SCB[n] * fl32(1/127)))) rounds twice
(the oracle's reading 9). Where the fp32 product lies exactly halfway between
two fp16 values, rounding the exact product once gives the other neighbour;
the weights here are built so that a quarter of their entries are such
cases (scales SCB that are not fp16 values, as a caller's own scales may be).

The inputs make the layer's outputs equal to Wdq itself, so every element is
compared exactly:
* forward: each activation row holds a single outlier value 8 (all other
  entries 0), so out[m, n] = 8 * Wdq[n, O[j(m)]]: the outlier product alone,
  through the staged weight slice and through the gathered columns past it;
* backward: G is one-hot per row, so grad_A[m, :] = Wdq[n(m), :].
"""
import numpy as np
import pytest
import torch

import oracle
from tests._gpu import assert_bits_equal, dev, host

C127 = np.float32(1.0) / np.float32(127.0)


def _midpoint_pairs():
    """(v, SCB) with 1 <= v <= 127 such that fl32(v * fl32(SCB * fl32(1/127)))
    is an fp16 midpoint that the exact product exceeds or falls short of in
    the direction where one rounding and two roundings disagree."""
    pairs = []
    for M in (1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 0.75 + 2.0 ** -12, 1.5 + 5 * 2.0 ** -11):
        for v in range(1, 128):
            base = np.array([M / v / float(C127)], np.float32).view(np.uint32)[0]
            cand = (np.arange(-40, 41, dtype=np.int64) + int(base)).astype(np.uint32).view(np.float32)
            sig = (cand.astype(np.float64) * float(C127)).astype(np.float32)      # one fp32 rounding
            p = v * sig.astype(np.float64)                                       # exact (31 bits)
            p32 = p.astype(np.float32)
            hit = (p32.astype(np.float64) == M) & (p != M) & \
                  (p32.astype(np.float16) != p.astype(np.float16))
            pairs += [(v, float(c)) for c in cand[hit]]
    return pairs


def midpoint_weights(N, K, seed):
    """CB (N x K int8), SCB (N fp32): row n takes a scale from the pairs and
    holds +-v (its pair's code) in a quarter of its entries."""
    pairs = _midpoint_pairs()
    g = np.random.default_rng(seed)
    pick = g.integers(0, len(pairs), N)
    CB = g.integers(-127, 128, (N, K)).astype(np.int8)
    SCB = np.array([pairs[i][1] for i in pick], np.float32)
    v = np.array([pairs[i][0] for i in pick], np.int64)
    sel = g.random((N, K)) < 0.25
    sgn = np.where(g.random((N, K)) < 0.5, -1, 1)
    CB = np.where(sel, sgn * v[:, None], CB).astype(np.int8)
    return CB, SCB


def _one_rounding(CB, SCB):
    sig = (SCB.astype(np.float64) * float(C127)).astype(np.float32).astype(np.float64)
    return (CB.astype(np.float64) * sig[:, None]).astype(np.float16)


def test_midpoint_weights_premise():
    """CPU: the constructed weights are full of midpoint cases (a quarter of
    the entries), where the oracle's Wdq and a single rounding disagree."""
    CB, SCB = midpoint_weights(64, 512, 1)
    d = oracle.dequant_weight(CB, SCB) != _one_rounding(CB, SCB)
    assert d.mean() > 0.2, d.mean()


FWD = [(300, 1040, 520), (2100, 1040, 2090), (1040, 1040, 8320)]


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,N", FWD)
def test_forward_outlier_product_midpoints(M, K, N):
    import int8_quantized_linear_rowwise_amd as I8
    CB, SCB = midpoint_weights(N, K, 2)
    g = np.random.default_rng(3)
    cols = np.sort(g.choice(K, 300, replace=False))          # more than the 256 staged columns
    A = np.zeros((M, K), np.float16)
    A[np.arange(M), cols[np.arange(M) % cols.size]] = 8.0
    Wdq = oracle.dequant_weight(CB, SCB)
    expect = (8.0 * Wdq[:, cols[np.arange(M) % cols.size]].T.astype(np.float32)).astype(np.float16)
    assert np.all(expect.astype(np.float64) == 8.0 * Wdq[:, cols[np.arange(M) % cols.size]].T)   # exact
    plan = I8.lib.int8_linear_forward_plan(1, M, K, N)
    print(f"\n  [{M}x{K}x{N}] forward plan {plan}", flush=True)
    Ad, CBd, SCBd = dev(A), dev(CB), dev(SCB)
    for cap in (I8.default_cap(K), 0, K):
        ws = I8.forward_workspace(M, K, N, cap, "cuda:0")
        out = I8.int8_linear_forward(Ad, CBd, SCBd, None, 6.0, cap=cap, workspace=ws)
        assert I8.forward_check(ws, M, K, N, cap) == cols.size
        assert_bits_equal(host(out), expect, f"8 * Wdq through the outlier product, cap={cap}")


BWD = [(600, 520, 1040), (2048, 1024, 2048), (4096, 512, 4096)]


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", BWD)
def test_backward_dequant_midpoints(M, N, K):
    import int8_quantized_linear_rowwise_amd as I8
    CB, SCB = midpoint_weights(N, K, 4)
    rows = np.arange(M) % N
    G = np.zeros((M, N), np.float16)
    G[np.arange(M), rows] = 1.0
    plan = I8.lib.int8_linear_backward_plan(1, M, N, K)
    print(f"\n  [{M}x{N}x{K}] backward plan {plan}", flush=True)
    gA, _ = I8.int8_linear_backward_input(dev(G), dev(CB), dev(SCB), with_grad_bias=False)
    assert_bits_equal(host(gA), oracle.dequant_weight(CB, SCB)[rows], "grad_A = Wdq rows")
