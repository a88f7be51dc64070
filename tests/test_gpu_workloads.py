"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: every layer of every workload.

Bit-exact over the whole tensors: int8 weights and scales, the forward's
quantized activation (codes, row scales, outlier list and count, fp16
outlier sub-matrix). On sampled rows -- one in every 256-row tile of the
kernels, plus rows 0, 255, 256, 257 and M - 1 -- which the oracle computes one
by one: int32 accumulators (bit-exact), forward output and input gradient
(pages' bounds + tight ulp bound). grad_bias is checked whole. The forward
runs with the default outlier staging width (256 columns), as in the
benchmark.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu import assert_bits_equal, assert_float_gate, dev, host, tile_rows

pytestmark = pytest.mark.gpu

CASES = [(name, li) for name in workloads.WORKLOAD_ORDER if name != "mlp600"
         for li in range(len(workloads.WORKLOADS[name].layers))]


@pytest.fixture(scope="module")
def I8():
    assert torch.cuda.is_available()
    import int8_quantized_linear_rowwise_amd as I8
    return I8


@pytest.mark.parametrize("name,li", CASES, ids=[f"{n}-{workloads.WORKLOADS[n].layers[i].name}" for n, i in CASES])
def test_workload_layer(I8, name, li):
    wl = workloads.WORKLOADS[name]
    L = wl.layers[li]
    dt, tau = wl.dtype, wl.threshold
    print(f"\n[{name}/{L.name}] M={L.M} K={L.K} N={L.N} dt={dt}", flush=True)
    W = workloads.make_weight(wl, li)
    CB, SCB = I8.quantize_weight(dev(W))
    cb, scb = oracle.quantize_weight(W)
    assert_bits_equal(host(CB), cb, "CB")
    assert_bits_equal(host(SCB), scb, "SCB")
    del W
    print("  weights bit-exact", flush=True)
    A = workloads.make_activation(wl, li)
    b = workloads.make_bias(wl, li)
    M, K, N = L.M, L.K, L.N
    cap = I8.default_cap(K)
    ws = I8.forward_workspace(M, K, N, cap, "cuda:0")
    c32 = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    out = I8.int8_linear_forward(dev(A, dt), CB, SCB, dev(b, dt) if b is not None else None, tau, cap, c32=c32,
                                 workspace=ws)
    torch.cuda.synchronize()
    rows = tile_rows(M)
    print("  forward done on GPU; oracle ...", flush=True)
    f = oracle.linear_forward(A, dt, cb, scb, b, tau, rows=rows)
    q = f["q"]
    lay = I8.forward_layout(M, K, N, cap)
    cnt = int(host(ws[lay.count:lay.count + 4]).view(np.int32)[0])
    assert cnt == q["outliers"].size
    seeded = workloads.outlier_columns(wl.wid, li, K, L.n_outliers)
    assert set(seeded.tolist()) <= set(q["outliers"].tolist())
    assert_bits_equal(host(ws[lay.idx:lay.idx + 4 * cnt]).view(np.int32), q["outliers"], "outlier list")
    assert_bits_equal(host(ws[lay.scale:lay.scale + 4 * M]).view(np.float32), q["scale"], "SCA")
    assert_bits_equal(host(ws[lay.codes:lay.codes + M * K]).view(np.int8).reshape(M, K), q["codes"], "CA")
    k = min(cnt, cap)
    subw = host(ws[lay.sub:lay.sub + 2 * M * cap]).view(np.float16).reshape(M, cap)[:, :k]
    assert_bits_equal(subw, q["sub"][:, :k], "subA")
    rt = torch.from_numpy(rows).to("cuda:0")
    assert_bits_equal(host(c32.index_select(0, rt)), f["c32"].astype(np.int32), "C32 (sampled rows)")
    assert_float_gate(host(out.index_select(0, rt)), dt, f["y"], "out (sampled rows)")
    del A, c32, out, ws, f, q
    print(f"  forward parity ok (|O|={cnt})", flush=True)
    G = workloads.make_grad(wl, li)
    gA, gb = I8.int8_linear_backward_input(dev(G, dt), CB, SCB, with_grad_bias=b is not None)
    torch.cuda.synchronize()
    r = oracle.linear_backward_input(G, dt, cb, scb, rows=rows)
    assert_float_gate(host(gA.index_select(0, rt)), dt, r["y"], "grad_A (sampled rows)")
    if b is not None:
        gb64, _ = oracle.grad_bias(G, dt)
        assert_float_gate(host(gb), dt, gb64, "grad_bias", tight_rel=2.0 ** -16)
