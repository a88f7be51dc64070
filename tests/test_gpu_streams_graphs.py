"""The C entry points on a non-default stream and inside a captured HIP graph.

Apart from the outlier-count readback (int8_linear_forward_check), every entry
point only enqueues kernels on the caller's stream: no allocation, no memset,
no synchronisation. So the layer runs on any stream and can be captured into
a HIP graph and replayed. The results must be bit-identical to the same calls
made eagerly on the default stream (all kernels are deterministic), and the
eager results are checked against the oracle. Graph replays are separated by
eager work and synchronisations, and every replay is checked.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu import assert_bits_equal, dev, host

# a ragged shape on the generic kernels and one on the 256-row tile kernels
SHAPES = [(520, 1040, 2090), (2100, 2064, 4104)]
DT = "bf16"


def _weights(I8, M, K, N, seed):
    c = workloads.small_case(DT, M, K, N, seed=seed, n_outliers=5)
    CB, SCB = I8.quantize_weight(dev(c["W"]))
    return c, CB, SCB


def _check_oracle(c, CB, SCB, out, c32, gA, gb, what):
    cb, scb = host(CB), host(SCB)
    f = oracle.linear_forward(c["A"], DT, cb, scb, c["bias"], 6.0)
    assert np.array_equal(host(c32), f["c32"].astype(np.int32)), f"{what}: int32 accumulators differ"
    b = oracle.linear_backward_input(c["G"], DT, cb, scb)
    gb64, _ = oracle.grad_bias(c["G"], DT)
    for name, T, y in (("out", host(out), f["y"]), ("grad_A", host(gA), b["y"]), ("grad_bias", host(gb), gb64)):
        r = oracle.page_bounds(oracle.to_f64(T, DT), y)
        assert r["ok"], f"{what}: {name} outside the bounds: {r}"


def _eager(I8, c, CB, SCB, M, K, N):
    A, G, bias = dev(c["A"], DT), dev(c["G"], DT), dev(c["bias"], DT)
    c32 = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    out = I8.int8_linear_forward(A, CB, SCB, bias, 6.0, c32=c32)
    gA, gb = I8.int8_linear_backward_input(G, CB, SCB)
    return out, c32, gA, gb


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_side_stream_matches_default_stream(M, K, N):
    import int8_quantized_linear_rowwise_amd as I8
    print(f"\n  [{M}x{K}x{N} {DT}] default stream, then a side stream beside other work", flush=True)
    c, CB, SCB = _weights(I8, M, K, N, 31)
    ref = _eager(I8, c, CB, SCB, M, K, N)
    torch.cuda.synchronize()
    _check_oracle(c, CB, SCB, *ref, "default stream")

    other = workloads.small_case(DT, M, K, N, seed=32, n_outliers=7)
    A2 = dev(other["A"], DT)
    side = torch.cuda.Stream()            # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        res = _eager(I8, c, CB, SCB, M, K, N)
    # unrelated work on the default stream while the side stream runs
    for _ in range(3):
        I8.int8_linear_forward(A2, CB, SCB, None, 6.0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for name, a, b in zip(("out", "c32", "grad_A", "grad_bias"), res, ref):
        assert_bits_equal(host(a), host(b), f"side stream {name}")


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_graph_capture_and_replay(M, K, N):
    import int8_quantized_linear_rowwise_amd as I8
    print(f"\n  [{M}x{K}x{N} {DT}] forward, allocation-free forward and backward captured in one graph", flush=True)
    c0, CB, SCB = _weights(I8, M, K, N, 41)
    cap = I8.default_cap(K)
    sA, sG, bias = dev(c0["A"], DT), dev(c0["G"], DT), dev(c0["bias"], DT)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    out_na = torch.empty_like(out)
    c32 = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    gA = torch.empty((M, K), dtype=torch.bfloat16, device="cuda:0")
    gb = torch.empty((N,), dtype=torch.bfloat16, device="cuda:0")
    wsf = I8.forward_workspace(M, K, N, cap, "cuda:0")
    wsb = torch.empty((max(1, I8.lib.int8_linear_backward_workspace_bytes(M, N, 1)),), dtype=torch.uint8,
                      device="cuda:0")
    noalloc = I8.lib.int8_linear_forward_noalloc_bytes(M, K, N) <= I8.lib.int8_linear_forward_noalloc_max_bytes()

    def calls():
        I8.int8_linear_forward(sA, CB, SCB, bias, 6.0, cap, out=out, c32=c32, workspace=wsf)
        if noalloc:
            I8.int8_linear_forward_noalloc(sA, CB, SCB, bias, 6.0, out=out_na)
        I8.int8_linear_backward_input(sG, CB, SCB, grad_A=gA, grad_bias=gb, workspace=wsb)

    calls()                                # eager warm-up (kernel attributes set outside capture)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()

    for rep, seed in enumerate((42, 43, 44)):
        c = workloads.small_case(DT, M, K, N, seed=seed, n_outliers=3 + 2 * rep)
        c["bias"] = c0["bias"]
        sA.copy_(dev(c["A"], DT))
        sG.copy_(dev(c["G"], DT))
        torch.cuda.synchronize()
        print(f"  replay {rep} (seed {seed})", flush=True)
        g.replay()
        torch.cuda.synchronize()
        ref = _eager(I8, c, CB, SCB, M, K, N)
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "c32", "grad_A", "grad_bias"), (out, c32, gA, gb), ref):
            assert_bits_equal(host(a), host(b), f"replay {rep} {name}")
        if noalloc:
            assert_bits_equal(host(out_na), host(ref[0]), f"replay {rep} allocation-free out")
        if rep == 0:
            _check_oracle(c, CB, SCB, *ref, f"replay {rep}")


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_graph_capture_other_entry_points(M, K, N):
    """The quantizer, the SiLU producer with its flags, the flagged forward, the
    int8 backward variant and the weight gradient, captured in one graph:
    every replay bit-identical to the same calls made eagerly."""
    import int8_quantized_linear_rowwise_amd as I8
    print(f"\n  [{M}x{K}x{N} {DT}] quantizer, SiLU flags, flagged forward, int8 backward, grad_W in one graph",
          flush=True)
    c0, CB, SCB = _weights(I8, M, K, N, 51)
    W = dev(c0["W"])
    CBt, SCBt = I8.quantize_weight_colwise(W)
    cap = I8.default_cap(K)
    bias = dev(c0["bias"], DT)
    sX, sH, sG = dev(c0["A"], DT), dev(c0["A"], DT), dev(c0["G"], DT)
    bf = torch.bfloat16

    def buffers():
        return dict(codes=torch.empty((M, K), dtype=torch.int8, device="cuda:0"),
                    scale=torch.empty((M,), dtype=torch.float32, device="cuda:0"),
                    idx=torch.empty((cap,), dtype=torch.int32, device="cuda:0"),
                    cnt=torch.empty((1,), dtype=torch.int32, device="cuda:0"),
                    sub=torch.empty((M, cap), dtype=torch.float16, device="cuda:0"),
                    qws=torch.empty((max(1, I8.lib.int8_quantize_rowwise_workspace_bytes(M, K)),),
                                    dtype=torch.uint8, device="cuda:0"),
                    act=torch.empty((M, K), dtype=bf, device="cuda:0"),
                    flags=I8.outlier_flags_buffer(M, K, "cuda:0"),
                    out=torch.empty((M, N), dtype=bf, device="cuda:0"),
                    c32=torch.empty((M, N), dtype=torch.int32, device="cuda:0"),
                    wsf=I8.forward_workspace(M, K, N, cap, "cuda:0"),
                    gA8=torch.empty((M, K), dtype=bf, device="cuda:0"),
                    gb8=torch.empty((N,), dtype=bf, device="cuda:0"),
                    ws8=I8.backward_int8_workspace(M, N, True, "cuda:0"),
                    gW=torch.empty((N, K), dtype=bf, device="cuda:0"))

    def calls(X, H, G, b):
        I8.check(I8.lib.int8_quantize_rowwise(X.data_ptr(), I8.DTYPE_CODE[X.dtype], M, K, 6.0, b["codes"].data_ptr(),
                                              b["scale"].data_ptr(), b["idx"].data_ptr(), b["cnt"].data_ptr(),
                                              b["sub"].data_ptr(), cap, b["qws"].data_ptr(), b["qws"].numel(),
                                              torch.cuda.current_stream().cuda_stream), "int8_quantize_rowwise")
        I8.silu_outlier_flags(H, 6.0, A=b["act"], flags=b["flags"])
        I8.int8_linear_forward_flagged(b["act"], b["flags"], CB, SCB, bias, cap, out=b["out"], c32=b["c32"],
                                       workspace=b["wsf"])
        I8.int8_linear_backward_input_int8(G, CBt, SCBt, True, grad_A=b["gA8"], grad_bias=b["gb8"],
                                           workspace=b["ws8"])
        I8.int8_linear_backward_weight(G, X, grad_W=b["gW"])

    gbuf = buffers()
    calls(sX, sH, sG, gbuf)                 # eager warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(sX, sH, sG, gbuf)
    torch.cuda.synchronize()

    names = ("codes", "scale", "idx", "cnt", "sub", "act", "flags", "out", "c32", "gA8", "gb8", "gW")
    for rep, seed in enumerate((52, 53)):
        c = workloads.small_case(DT, M, K, N, seed=seed, n_outliers=4 + 3 * rep)
        h = workloads.small_case(DT, M, K, N, seed=seed + 100, n_outliers=0)
        sX.copy_(dev(c["A"], DT))
        sH.copy_(dev(h["A"], DT))
        sG.copy_(dev(c["G"], DT))
        torch.cuda.synchronize()
        print(f"  replay {rep} (seed {seed})", flush=True)
        g.replay()
        torch.cuda.synchronize()
        ebuf = buffers()
        calls(dev(c["A"], DT), dev(h["A"], DT), dev(c["G"], DT), ebuf)
        torch.cuda.synchronize()
        n = int(host(gbuf["cnt"])[0])
        assert n == int(host(ebuf["cnt"])[0])
        for name in names:
            a, b = host(gbuf[name]), host(ebuf[name])
            if name == "idx":
                a, b = a[:min(n, cap)], b[:min(n, cap)]
            elif name == "sub":
                a, b = a[:, :min(n, cap)], b[:, :min(n, cap)]
            elif name == "flags":
                w = I8.lib.int8_outlier_flags_words(M, K)
                a, b = a[:w], b[:w]
            assert_bits_equal(a, b, f"replay {rep} {name}")
