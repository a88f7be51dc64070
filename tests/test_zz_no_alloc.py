"""The allocation-free forward (static per-GPU scratch) through the C ABI:
its output equals the ordinary forward's bit for bit on consecutive calls,
each smaller than the one before, on the same GPU (the scratch keeps the
previous call's contents), and meets the oracle's gate."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu import TORCH, assert_bits_equal, assert_float_gate, dev, host, tile_rows

pytestmark = pytest.mark.gpu

# (M, K, N, dtype): the 7B block's widest input at its full size, then
# smaller inputs on other kernel paths (256 x 128 tiles, the generic kernel)
CALLS = [(4096, 11008, 4096, "bf16"), (1024, 4096, 4352, "bf16"), (300, 1040, 520, "f16"), (64, 16, 40, "f32")]


def test_noalloc_forward_matches_forward_on_consecutive_calls():
    assert torch.cuda.is_available()
    import int8_quantized_linear_rowwise_amd as I8
    lib = I8.lib
    stream = torch.cuda.current_stream().cuda_stream
    for i, (M, K, N, dt) in enumerate(CALLS):
        print(f"\n[noalloc call {i}] M={M} K={K} N={N} {dt}", flush=True)
        # more seeded outlier columns than the 64-column staging of this entry point
        c = workloads.small_case(dt, M, K, N, seed=70 + i, n_outliers=min(80, K), has_bias=True)
        A = dev(c["A"], dt)
        CB, SCB = I8.quantize_weight(dev(c["W"]))
        b = dev(c["bias"], dt)
        ref = I8.int8_linear_forward(A, CB, SCB, b, 6.0)
        out = torch.full((M, N), float("nan"), dtype=TORCH[dt], device="cuda:0")
        torch.cuda.synchronize()
        rc = lib.int8_linear_forward_noalloc(A.data_ptr(), I8.DTYPE_CODE[A.dtype], M, K, CB.data_ptr(),
                                             SCB.data_ptr(), N, b.data_ptr(), ctypes.c_float(6.0),
                                             out.data_ptr(), stream)
        assert rc == 0, lib.int8_linear_strerror(rc)
        torch.cuda.synchronize()
        assert_bits_equal(host(out), host(ref), "noalloc out against int8_linear_forward")
        # and the oracle's gate on a row of every 256-row tile
        cb, scb = oracle.quantize_weight(c["W"])
        rows = tile_rows(M)
        f = oracle.linear_forward(c["A"], dt, cb, scb, c["bias"], 6.0, rows=rows)
        assert f["q"]["outliers"].size > min(64, K - 1) or K <= 64
        assert_float_gate(host(out)[rows], dt, f["y"], "noalloc out (sampled rows)")
    # the binding's wrapper, and the host-side rejection of a problem beyond the scratch
    A = torch.zeros((16384, 28672), dtype=torch.bfloat16, device="cuda:0")
    CB = torch.zeros((16, 28672), dtype=torch.int8, device="cuda:0")
    SCB = torch.zeros((16,), dtype=torch.float32, device="cuda:0")
    with pytest.raises(I8.Int8LinError) as e:
        I8.int8_linear_forward_noalloc(A, CB, SCB)
    assert e.value.code == I8._lib.I8L_ESCRATCH
