"""Pins of the CPU oracle of the int8 linear layer (CPU only).

Each check ties the oracle to something other than itself:
* brute force over exact rationals on tiny inputs (quantizer, forward,
  backward, grad_bias), written with Python loops;
* closed-form special cases that reduce to textbook integer or float matmuls;
* invariants of the quantizer on the workloads' own data;
* an implementation-free error bound against the unquantized product;
* the error bounds of bitsandbytes PR #33's module test at small shapes.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from oracle.formats import to_f64, to_half
from tests._exact import exact_round, fl32, round_half_even

# --------------------------------------------------------------------------
# brute force (exact rationals)

F127 = Fraction(127)
INV127 = fl32(Fraction(1, 127))


def bf_quantize(X16_vals, tau):
    """Exact-rational quantizer; X16_vals: R x C list of fp16 values as Fractions."""
    R = len(X16_vals)
    C = len(X16_vals[0]) if R else 0
    on = tau is not None and 0 < tau < float("inf")
    t = Fraction(float(np.float32(tau))) if on else None
    O = [c for c in range(C) if on and any(abs(X16_vals[r][c]) > t for r in range(R))]
    codes, codes_exact_real, scales = [], [], []
    for r in range(R):
        s = Fraction(0)
        for c in range(C):
            if c not in O:
                s = max(s, abs(X16_vals[r][c]))
        inv = fl32(F127 / s) if s > 0 else Fraction(0)
        row, row_real = [], []
        for c in range(C):
            if c in O or s == 0:
                row.append(0)
                row_real.append(0)
                continue
            v = fl32(X16_vals[r][c] * inv)                 # fp32 product, exactly rounded
            row.append(max(-127, min(127, round_half_even(v))))
            row_real.append(max(-127, min(127, round_half_even(F127 * X16_vals[r][c] / s))))
        codes.append(row)
        codes_exact_real.append(row_real)
        scales.append(s)
    sub = [[X16_vals[r][c] for c in O] for r in range(R)]
    return codes, codes_exact_real, scales, O, sub


def _tiny_fp16(g, R, C):
    kind = g.integers(0, 4)
    if kind == 0:
        x = g.standard_normal((R, C)) * 3
    elif kind == 1:
        x = g.integers(-8, 9, (R, C)).astype(np.float64)            # ties, repeats, zeros
    elif kind == 2:
        x = g.standard_normal((R, C)) * np.ldexp(1.0, g.integers(-20, 4))
    else:
        x = g.standard_normal((R, C))
        x[:, g.integers(0, C)] *= 20
    return x.astype(np.float16)


@pytest.mark.parametrize("dt", ["f16", "f32", "bf16"])
def test_quantizer_brute_force(dt):
    g = np.random.default_rng(100 + ["f16", "f32", "bf16"].index(dt))
    near_half = 0
    total = 0
    for case in range(700):
        R, C = int(g.integers(1, 7)), int(g.integers(1, 7))
        x16 = _tiny_fp16(g, R, C)
        if dt == "f16":
            X = x16
        elif dt == "f32":
            X = (x16.astype(np.float32) + g.standard_normal((R, C)).astype(np.float32) * 1e-4)
        else:
            X = workloads._store(x16.astype(np.float32), "bf16")
        tau = float(g.choice([6.0, 2.0, 0.0, np.inf, 1.5, 4.0]))
        X16 = to_half(X, dt)
        vals = [[Fraction(float(v)) for v in row] for row in X16]
        codes, real, scales, O, sub = bf_quantize(vals, tau)
        q = oracle.quantize_rowwise(X, dt, tau)
        assert q["outliers"].tolist() == O
        assert [Fraction(float(s)) for s in q["scale"]] == scales
        assert q["codes"].tolist() == codes
        assert [[Fraction(float(v)) for v in row] for row in q["sub"]] == sub
        total += R * C
        near_half += sum(a != b for ra, rb in zip(codes, real) for a, b in zip(ra, rb))
    # The fp32 formula equals exact rounding of 127*x/s except within ~2^-22
    # of a half-integer; such cases must be rare on these inputs.
    assert near_half <= total * 0.002


def test_threshold_is_strict_and_off_values():
    X = np.array([[6.0, 1.0, -6.0], [0.5, 6.0078125, 2.0]], dtype=np.float16)
    q = oracle.quantize_rowwise(X, "f16", 6.0)
    assert q["outliers"].tolist() == [1]                      # 6.0 is not > 6.0
    for off in (0.0, -1.0, float("inf"), float("nan")):
        assert oracle.quantize_rowwise(X, "f16", off)["outliers"].size == 0


def test_zero_rows_and_all_outlier_rows():
    X = np.array([[0, 0, 0], [7, 0, 0], [7, 1, -2]], dtype=np.float16)
    q = oracle.quantize_rowwise(X, "f16", 6.0)
    assert q["outliers"].tolist() == [0]
    assert q["scale"].tolist() == [0.0, 0.0, 2.0]
    assert q["codes"].tolist() == [[0, 0, 0], [0, 0, 0], [0, 64, -127]]
    assert q["sub"].astype(np.float64).ravel().tolist() == [0.0, 7.0, 7.0]


# --------------------------------------------------------------------------
# invariants on the workloads' data


def _wl_rows(name, li, rows):
    wl = workloads.WORKLOADS[name]
    return workloads.make_activation(wl, li, rows=rows), wl


# rows: every row of single4096 (2048, two of the oracle's 1024-row chunks),
# more than one chunk of the others
@pytest.mark.parametrize("name,li,rows", [("single4096", 0, None), ("llama7b_mlp", 2, 1100),
                                          ("llama7b_block", 4, 2048), ("mlp600", 0, None)])
def test_quantizer_invariants(name, li, rows):
    A, wl = _wl_rows(name, li, rows)
    dt, tau = wl.dtype, wl.threshold
    q = oracle.quantize_rowwise(A, dt, tau)
    X = to_half(A, dt).astype(np.float64)
    codes, s, O = q["codes"].astype(np.int64), q["scale"].astype(np.float64), q["outliers"]
    keep = np.ones(X.shape[1], bool)
    keep[O] = False
    # (i) range, never -128
    assert codes.min() >= -127 and codes.max() <= 127
    # (ii) absmax element maps to +-127
    for r in range(X.shape[0]):
        if s[r] > 0:
            c = np.argmax(np.where(keep, np.abs(X[r]), -1))
            assert abs(codes[r, c]) == 127
    # (iii) sign
    assert np.all((np.sign(codes) == np.sign(X)) | (codes == 0))
    # (iv) monotone within a row
    for r in range(0, X.shape[0], 17):
        o = np.argsort(X[r, keep], kind="stable")
        assert np.all(np.diff(codes[r, keep][o]) >= 0)
    # (v) outlier columns leave the int8 path and are copied bit for bit
    assert np.all(codes[:, O] == 0)
    assert np.array_equal(q["sub"].view(np.uint16), to_half(A, dt)[:, O].view(np.uint16))
    # (vi) remaining magnitudes are within tau
    assert np.all(s <= tau)
    # (vii) tau off => no outliers
    assert oracle.quantize_rowwise(A, dt, float("inf"))["outliers"].size == 0
    # seeded outlier columns are detected
    seeded = workloads.outlier_columns(wl.wid, li, wl.layers[li].K, wl.layers[li].n_outliers)
    assert set(seeded.tolist()) <= set(O.tolist())


def test_quantizer_scale_equivariance():
    A, wl = _wl_rows("single4096", 0, 64)
    q0 = oracle.quantize_rowwise(A, "f16", 0.0)
    for e in (-3, 2):
        A2 = (A.astype(np.float64) * 2.0 ** e).astype(np.float16)
        q1 = oracle.quantize_rowwise(A2, "f16", 0.0)
        assert np.array_equal(q1["codes"], q0["codes"])
        assert np.array_equal(q1["scale"].astype(np.float64), q0["scale"].astype(np.float64) * 2.0 ** e)


# --------------------------------------------------------------------------
# closed-form special cases


def _int_weights(g, N, K):
    """Integer weights in [-127, 127] with +-127 in every row: quantize to themselves."""
    W = g.integers(-127, 128, (N, K)).astype(np.float32)
    W[np.arange(N), g.integers(0, K, N)] = np.where(g.random(N) < 0.5, -127, 127)
    return W


def test_integer_forward_is_textbook_matmul():
    g = np.random.default_rng(20)
    M, K, N = 37, 70, 29
    A = _int_weights(g, M, K)          # same construction: every row has |127|
    W = _int_weights(g, N, K)
    CB, SCB = oracle.quantize_weight(W)
    assert np.array_equal(CB, W.astype(np.int8)) and np.all(SCB == 127)
    f = oracle.linear_forward(A, "f32", CB, SCB, None, float("inf"))
    assert np.array_equal(f["q"]["codes"], A.astype(np.int8))
    ref = A.astype(np.int64) @ W.astype(np.int64).T
    assert np.array_equal(f["c32"], ref)
    # y = C32 * 127 * 127 / 127^2 = C32 exactly
    assert np.array_equal(f["y"], ref.astype(np.float64))


def test_zero_input_gives_bias_bitwise():
    g = np.random.default_rng(21)
    for dt in ("f16", "bf16", "f32"):
        W = g.standard_normal((13, 40)).astype(np.float32) * 0.02
        CB, SCB = oracle.quantize_weight(W)
        b = workloads._store(g.standard_normal(13).astype(np.float32) * 0.01, dt)
        A = workloads._store(np.zeros((5, 40), np.float32), dt)
        f = oracle.linear_forward(A, dt, CB, SCB, b, 6.0)
        assert np.array_equal(np.asarray(f["out"]).view(np.uint8),
                              np.broadcast_to(b, (5, 13)).view(np.uint8))


def test_threshold_off_equals_dequantized_int8_product():
    g = np.random.default_rng(22)
    M, K, N = 50, 96, 40
    A = (g.standard_normal((M, K)) * 2).astype(np.float16)
    W = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    CB, SCB = oracle.quantize_weight(W)
    f = oracle.linear_forward(A, "f16", CB, SCB, None, float("inf"))
    q = f["q"]
    deqA = q["codes"].astype(np.float64) * (q["scale"].astype(np.float64)[:, None] / 127)
    deqW = CB.astype(np.float64) * (SCB.astype(np.float64)[:, None] / 127)
    assert np.allclose(f["y"], deqA @ deqW.T, rtol=1e-12, atol=1e-12)


def test_all_outlier_columns_is_textbook_float_matmul():
    g = np.random.default_rng(23)
    M, K, N = 40, 33, 21
    A = (g.uniform(0.5, 2, (M, K)) * np.where(g.random((M, K)) < .5, -1, 1)).astype(np.float16)
    W = _int_weights(g, N, K)                     # SCB = 127 -> Wdq = CB exactly
    CB, SCB = oracle.quantize_weight(W)
    b = (g.standard_normal(N) * 0.01).astype(np.float16)
    f = oracle.linear_forward(A, "f16", CB, SCB, b, 1e-3)
    q = f["q"]
    assert q["outliers"].tolist() == list(range(K))
    assert np.all(q["codes"] == 0) and np.all(q["scale"] == 0)
    ref = A.astype(np.float64) @ W.astype(np.float64).T + b.astype(np.float64)
    assert np.allclose(f["y"], ref, rtol=1e-13, atol=1e-12)


def test_integer_backward_is_textbook_matmul():
    g = np.random.default_rng(24)
    M, N, K = 45, 31, 66
    W = _int_weights(g, N, K)
    CB, SCB = oracle.quantize_weight(W)
    sig = (SCB * np.float32(1) / np.float32(127))
    assert np.all(oracle.dequant_weight(CB, SCB) == CB.astype(np.float16))
    G = g.integers(-1, 2, (M, N)).astype(np.float32)
    b = oracle.linear_backward_input(G, "f32", CB, SCB)
    ref = G.astype(np.int64) @ W.astype(np.int64)
    assert np.array_equal(b["grad_A"], ref.astype(np.float32))
    del sig


def test_dequant_constant_is_one_for_scale_127():
    assert np.float32(127) * (np.float32(1) / np.float32(127)) == np.float32(1.0)


def test_dequant_weight_rounds_twice_at_an_fp16_midpoint():
    """Reading 9 rounds CB * sigma to fp32, then to fp16. With SCB = 0x41cb4c9a
    (25.41240...), 5 * sigma = 1.00048832... exactly, 4.5e-8 above the fp16
    midpoint 1 + 2^-11; the fp32 spacing at 1 is 2^-23, so the fp32 product is
    that midpoint, which ties to the even neighbour 1.0 (0x3C00). Rounding the
    exact product once would give 1 + 2^-10 (0x3C01). Likewise 10 * sigma lands
    on 2 + 2^-10 and ties to 2.0 (0x4000)."""
    scb = np.array([0x41CB4C9A], np.uint32).view(np.float32)
    sig = fl32(Fraction(float(scb[0])) * INV127)
    exact = 5 * sig
    mid = 1 + Fraction(1, 2048)
    assert exact > mid and fl32(exact) == mid                       # the worked case holds
    assert exact_round(exact, "f16") == 1 + Fraction(1, 1024)       # one rounding: the other neighbour
    w = oracle.dequant_weight(np.array([[5, -5, 0, 10, -10]], np.int8), scb)
    assert w.view(np.uint16)[0].tolist() == [0x3C00, 0xBC00, 0x0000, 0x4000, 0xC000]


# --------------------------------------------------------------------------
# brute force of the whole forward / backward on tiny inputs


def _tiny_layer(g, M, K, N, dt):
    x = (g.standard_normal((M, K)) * 2).astype(np.float32)
    x[:, g.integers(0, K)] *= 8
    A = workloads._store(x, dt)
    W = (g.standard_normal((N, K)) * 0.05).astype(np.float32)
    b = workloads._store((g.standard_normal(N) * 0.1).astype(np.float32), dt)
    G = workloads._store((g.standard_normal((M, N)) * 0.5).astype(np.float32), dt)
    return A, W, b, G


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_forward_backward_brute_force(dt):
    g = np.random.default_rng(30 + ["f16", "bf16", "f32"].index(dt))
    for case in range(25):
        M, K, N = int(g.integers(1, 6)), int(g.integers(1, 7)), int(g.integers(1, 6))
        A, W, b, G = _tiny_layer(g, M, K, N, dt)
        tau = 6.0
        CB, SCB = oracle.quantize_weight(W)
        f = oracle.linear_forward(A, dt, CB, SCB, b, tau)
        X16 = [[Fraction(float(v)) for v in row] for row in to_half(A, dt)]
        codes, _, s, O, sub = bf_quantize(X16, tau)
        bvals = [Fraction(float(v)) for v in to_f64(b, dt)]
        # weights: exact quantization of W (tau off) by the same brute force
        W16 = [[Fraction(float(v)) for v in row] for row in W.astype(np.float16)]
        # (weights quantize from fp32 -> fp16 cast first, as activations do)
        cbs, _, sbs, _, _ = bf_quantize(W16, None)
        assert CB.tolist() == cbs and [Fraction(float(v)) for v in SCB] == sbs
        sig = [fl32(sb * INV127) for sb in sbs]
        wdq = [[exact_round(fl32(Fraction(cbs[n][k]) * sig[n]), "f16") for k in range(K)]
               for n in range(N)]
        for m in range(M):
            for n in range(N):
                acc = sum(Fraction(codes[m][k] * cbs[n][k]) for k in range(K))
                assert f["c32"][m, n] == acc
                terms = [acc * s[m] * sbs[n] / 16129]
                terms += [sub[m][j] * wdq[n][O[j]] for j in range(len(O))]
                terms += [bvals[n]]
                y = sum(terms)
                mag = sum(abs(t) for t in terms)
                # float64 evaluation: a few roundings, each within 2^-53 of the magnitudes
                assert abs(Fraction(float(f["y"][m, n])) - y) <= mag * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 200)
        bw = oracle.linear_backward_input(G, dt, CB, SCB)
        G16 = [[Fraction(float(v)) for v in row] for row in to_half(G, dt)]
        for m in range(M):
            for k in range(K):
                terms = [G16[m][n] * wdq[n][k] for n in range(N)]
                y = sum(terms)
                mag = sum(abs(t) for t in terms)
                assert abs(Fraction(float(bw["y"][m, k])) - y) <= mag * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 200)
        gb64, gbD = oracle.grad_bias(G, dt)
        Gv = to_f64(G, dt)
        for n in range(N):
            exact = sum(Fraction(float(Gv[m, n])) for m in range(M))
            mag = sum(abs(Fraction(float(Gv[m, n]))) for m in range(M))
            assert abs(Fraction(float(gb64[n])) - exact) <= mag * Fraction(1, 2 ** 48)


def test_rows_subset_matches_full():
    g = np.random.default_rng(40)
    A, W, b, G = _tiny_layer(g, 70, 40, 30, "bf16")
    CB, SCB = oracle.quantize_weight(W)
    full = oracle.linear_forward(A, "bf16", CB, SCB, b, 6.0)
    rows = np.array([3, 0, 69, 12])
    part = oracle.linear_forward(A, "bf16", CB, SCB, b, 6.0, rows=rows)
    assert np.array_equal(part["out"], full["out"][rows])
    bf = oracle.linear_backward_input(G, "bf16", CB, SCB)
    bp = oracle.linear_backward_input(G, "bf16", CB, SCB, rows=rows)
    assert np.array_equal(bp["grad_A"], bf["grad_A"][rows])


# --------------------------------------------------------------------------
# int8 backward variant (EasyDeL discussion #66, bwd_bits=8; oracle reading 13)


def test_int8_backward_integer_case_is_textbook_matmul():
    """Integer G with +-127 in every row and integer W with +-127 in every column:
    both quantize to themselves with scale 127, so grad_A = G @ W exactly."""
    g = np.random.default_rng(50)
    M, N, K = 33, 47, 58
    G = _int_weights(g, M, N)
    Wt = _int_weights(g, K, N)           # rows of W^T = columns of W
    W = np.ascontiguousarray(Wt.T)
    CBt, SCBt = oracle.quantize_weight_colwise(W)
    assert np.array_equal(CBt, Wt.astype(np.int8)) and np.all(SCBt == 127)
    b = oracle.linear_backward_input_int8(G, "f32", CBt, SCBt)
    ref = G.astype(np.int64) @ W.astype(np.int64)
    assert np.array_equal(b["c32"], ref)
    assert np.array_equal(b["grad_A"], ref.astype(np.float32))


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_int8_backward_brute_force(dt):
    g = np.random.default_rng(51 + ["f16", "bf16", "f32"].index(dt))
    for case in range(25):
        M, K, N = int(g.integers(1, 6)), int(g.integers(1, 7)), int(g.integers(1, 6))
        _, W, _, G = _tiny_layer(g, M, K, N, dt)
        CBt, SCBt = oracle.quantize_weight_colwise(W)
        b = oracle.linear_backward_input_int8(G, dt, CBt, SCBt)
        G16 = [[Fraction(float(v)) for v in row] for row in to_half(G, dt)]
        cg, _, sg, _, _ = bf_quantize(G16, None)
        Wt16 = [[Fraction(float(v)) for v in row] for row in np.ascontiguousarray(W.T).astype(np.float16)]
        cbt, _, sbt, _, _ = bf_quantize(Wt16, None)
        assert CBt.tolist() == cbt and [Fraction(float(v)) for v in SCBt] == sbt
        for m in range(M):
            for k in range(K):
                acc = sum(Fraction(cg[m][n] * cbt[k][n]) for n in range(N))
                assert b["c32"][m, k] == acc
                y = acc * sg[m] * sbt[k] / 16129
                assert abs(Fraction(float(b["y"][m, k])) - y) <= abs(y) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_int8_backward_error_bound_against_true_product():
    """|y - G16 W16| <= sum_n |g| e_w + |w| e_g + e_g e_w with e_g = (1/2 + 2^-20) SG/127
    per row and e_w = (1/2 + 2^-20) SCBt/127 per column of the result."""
    g = np.random.default_rng(52)
    M, N, K = 48, 256, 40
    G = (g.standard_normal((M, N)) * 0.01).astype(np.float16)
    W = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    CBt, SCBt = oracle.quantize_weight_colwise(W)
    b = oracle.linear_backward_input_int8(G, "f16", CBt, SCBt)
    gg = G.astype(np.float64)
    w = W.astype(np.float16).astype(np.float64)                       # N x K
    eg = (0.5 + 2 ** -20) * b["q"]["scale"].astype(np.float64) / 127
    ew = (0.5 + 2 ** -20) * SCBt.astype(np.float64) / 127
    bound = (np.abs(gg).sum(1)[:, None] * ew[None, :] + eg[:, None] * np.abs(w).sum(0)[None, :]
             + N * eg[:, None] * ew[None, :])
    err = np.abs(b["y"] - gg @ w)
    assert np.all(err <= bound * (1 + 1e-9))
    assert err.max() > 0.05 * bound.max()


# --------------------------------------------------------------------------
# error bounds against the unquantized product


def test_closed_form_error_bound_against_true_product():
    """|y - A16 W^T| <= sum_k |a| e_w + |w| e_a + e_a e_w (+ outlier-product rounding),
    e_a = (1/2 + 2^-20) SCA/127, e_w = (1/2 + 2^-20) SCB/127 (tau off)."""
    g = np.random.default_rng(41)
    M, K, N = 64, 256, 48
    A = g.standard_normal((M, K)).astype(np.float16)
    W = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    CB, SCB = oracle.quantize_weight(W)
    f = oracle.linear_forward(A, "f16", CB, SCB, None, float("inf"))
    a = A.astype(np.float64)
    w = W.astype(np.float16).astype(np.float64)
    ea = (0.5 + 2 ** -20) * f["q"]["scale"].astype(np.float64) / 127
    ew = (0.5 + 2 ** -20) * SCB.astype(np.float64) / 127
    bound = (np.abs(a).sum(1)[:, None] * ew[None, :] + ea[:, None] * np.abs(w).sum(1)[None, :]
             + K * ea[:, None] * ew[None, :])
    err = np.abs(f["y"] - a @ w.T)
    assert np.all(err <= bound * (1 + 1e-9))
    # and the bound is not vacuous
    assert err.max() > 0.05 * bound.max()


def test_page_bounds_two_stacked_layers_small_shape():
    """bitsandbytes PR #33 module-test design: the input gradient through two
    int8 layers (32 -> 64 -> 32, 128 tokens) against grad_proj @ W2 @ W1 with
    fp16 weights; max err <= 0.05*mean|ref| and <= 0.5 % of elements outside
    (atol 0.01*mean|ref|, rtol 0.1). Weights use torch.nn.Linear's default
    init U(-1/sqrt(fan_in), 1/sqrt(fan_in)) (reading: the page does not state it)."""
    g = np.random.default_rng(42)
    M, K, H, N = 128, 32, 64, 32
    for rep in range(6):
        W1 = g.uniform(-1 / np.sqrt(K), 1 / np.sqrt(K), (H, K)).astype(np.float32)
        W2 = g.uniform(-1 / np.sqrt(H), 1 / np.sqrt(H), (N, H)).astype(np.float32)
        gp = g.standard_normal((M, N)).astype(np.float16)
        cb1, s1 = oracle.quantize_weight(W1)
        cb2, s2 = oracle.quantize_weight(W2)
        g1 = oracle.linear_backward_input(gp, "f16", cb2, s2)["grad_A"]
        gx = oracle.linear_backward_input(g1, "f16", cb1, s1)["grad_A"]
        w1h = W1.astype(np.float16).astype(np.float64)
        w2h = W2.astype(np.float16).astype(np.float64)
        r = oracle.page_bounds(gx, gp.astype(np.float64) @ w2h @ w1h)
        assert r["ok"], r
    # a plausible slip (dequantizing with the wrong row's scale) breaks the bound
    bad = oracle.linear_backward_input(g1, "f16", cb1, np.roll(s1, 1))["grad_A"]
    assert not oracle.page_bounds(bad, g1.astype(np.float64) @ w1h)["ok"]


def test_page_bounds_detect_a_planted_error():
    ref = np.random.default_rng(43).standard_normal(10000)
    T = ref.copy()
    assert oracle.page_bounds(T, ref)["ok"]
    T[:100] += 0.5 * np.abs(ref).mean()        # 1% of elements off by half the scale
    assert not oracle.page_bounds(T, ref)["ok"]


# --------------------------------------------------------------------------
# the residual MLP of the EasyDeL example


def _mlp600_weights():
    wl = workloads.WORKLOADS["mlp600"]
    Ws = [workloads.make_weight(wl, i) for i in range(2)]
    bs = [workloads.make_bias(wl, i) for i in range(2)]
    return wl, Ws, bs


def test_silu_grad_finite_difference():
    h = np.linspace(-8, 8, 1001)
    fd = (oracle.silu(h + 1e-6) - oracle.silu(h - 1e-6)) / 2e-6
    assert np.allclose(oracle.silu_grad(h), fd, atol=1e-8)


def test_mlp600_magnitude_against_printed_example():
    """Parity unpinned (JAX streams / fjformer quantizer): magnitude check only.

    The printed int8-vs-float gap of the example is below 0.05*mean|out|; the
    oracle's int8 MLP must be in the same class against its float twin."""
    rows = np.loadtxt(__file__.replace("test_oracle_layer.py", "golden/easydel66_mlp_printed.txt"))
    fp, i8 = rows[:, 1:5], rows[:, 5:9]
    printed = oracle.page_bounds(i8, fp)
    assert printed["ok"]
    wl, Ws, bs = _mlp600_weights()
    x = workloads.make_activation(wl, 0)
    g = workloads.make_grad(wl, 1)
    layers = []
    for W, b in zip(Ws, bs):
        cb, s = oracle.quantize_weight(W)
        layers.append((cb, s, b))
    r = oracle.mlp_forward_backward(x, g, "f32", layers, wl.threshold)
    xf = x.astype(np.float64)
    h = xf @ Ws[0].astype(np.float64).T
    ref = oracle.silu(h) @ Ws[1].astype(np.float64).T + xf
    mine = oracle.page_bounds(r["out"], ref)
    assert mine["ok"], mine
    assert mine["max_rel"] < 5 * printed["max_rel"] + 0.02


# --------------------------------------------------------------------------
# weight gradient of the trainable-weight mode (oracle reading 14)


def _exact_value(x, dt):
    """Exact rational value of one stored element, decoded without the oracle's formats module."""
    if dt == "bf16":
        return Fraction(float(np.array([int(x) << 16], dtype=np.uint32).view(np.float32)[0]))
    return Fraction(float(x))


def test_wgrad_integer_case_is_textbook_matmul():
    """Small integers are exact in fp16 and bf16, so grad_W = G^T A exactly
    (non-square shapes: a transposed or swapped operand fails)."""
    g = np.random.default_rng(70)
    M, N, K = 37, 29, 23
    G = g.integers(-100, 101, (M, N)).astype(np.float32)
    A = g.integers(-100, 101, (M, K)).astype(np.float32)
    ref = G.astype(np.int64).T @ A.astype(np.int64)
    r = oracle.linear_backward_weight(G, A, "f32")
    assert r["grad_W"].shape == (N, K)
    assert np.array_equal(r["grad_W"], ref.astype(np.float32))
    rb = oracle.linear_backward_weight(workloads._store(G, "bf16"), workloads._store(A, "bf16"), "bf16")
    assert np.array_equal(rb["y"], ref.astype(np.float64))


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_wgrad_brute_force(dt):
    """Every element against the exact rational sum of exactly rounded fp16 casts."""
    g = np.random.default_rng(71 + ["f16", "bf16", "f32"].index(dt))
    for case in range(25):
        M, N, K = int(g.integers(1, 7)), int(g.integers(1, 6)), int(g.integers(1, 6))
        G = workloads._store((g.standard_normal((M, N)) * 0.01).astype(np.float32), dt)
        A = workloads._store((g.standard_normal((M, K)) * 3).astype(np.float32), dt)
        r = oracle.linear_backward_weight(G, A, dt)
        g16 = [[exact_round(_exact_value(v, dt), "f16") for v in row] for row in G]
        a16 = [[exact_round(_exact_value(v, dt), "f16") for v in row] for row in A]
        for n in range(N):
            for k in range(K):
                y = sum((g16[m][n] * a16[m][k] for m in range(M)), Fraction(0))
                assert abs(Fraction(float(r["y"][n, k])) - y) <= abs(y) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)
                got = _exact_value(r["grad_W"][n, k], dt) if dt != "f32" else Fraction(float(r["grad_W"][n, k]))
                assert got == exact_round(Fraction(float(r["y"][n, k])), dt)


def test_wgrad_casts_operands_to_fp16():
    """bf16 operands go through the fp16 cast: 3 * 2^-26 becomes the fp16
    subnormal 2^-24, and 2^17 (beyond fp16's range) becomes inf."""
    G = workloads._store(np.array([[3 * 2.0 ** -26, 1.0]], np.float32), "bf16")
    A = workloads._store(np.array([[1.0, 2.0 ** 17]], np.float32), "bf16")
    with np.errstate(over="ignore"):
        r = oracle.linear_backward_weight(G, A, "bf16")
    assert r["y"][0, 0] == 2.0 ** -24
    assert np.isinf(r["y"][0, 1]) and np.isinf(r["y"][1, 1])
    assert r["y"][1, 0] == 1.0


def test_wgrad_rows_subset_matches_full():
    g = np.random.default_rng(72)
    G = workloads._store((g.standard_normal((50, 40)) * 0.01).astype(np.float32), "bf16")
    A = workloads._store(g.standard_normal((50, 30)).astype(np.float32), "bf16")
    full = oracle.linear_backward_weight(G, A, "bf16")
    rows = np.array([7, 0, 39])
    part = oracle.linear_backward_weight(G, A, "bf16", rows=rows)
    assert np.array_equal(part["grad_W"], full["grad_W"][rows])


# --------------------------------------------------------------------------
# SiLU between the EasyDeL MLP's linears, with producer-side outlier flags (reading 15)


def test_silu_closed_forms():
    """SiLU(x) - SiLU(-x) = x for every x (x s(x) + x s(-x) = x), SiLU(0) = 0,
    SiLU(x) -> x and SiLU(-x) -> 0 for large x, and the well-known minimum
    near x = -1.2785 of about -0.2785 (the root of 1 + x (1 - s(x)) = 0)."""
    x = np.linspace(-30, 30, 6001)
    assert np.allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=0, atol=1e-12)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(oracle.silu(np.array([-40.0]))[0]) < 1e-15
    xm = x[np.argmin(oracle.silu(x))]
    assert abs(xm + 1.2785) < 0.01 and abs(oracle.silu(np.array([xm]))[0] + 0.2785) < 1e-3


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_silu_activation_rounds_once(dt):
    g = np.random.default_rng(90)
    H = workloads._store((g.standard_normal((40, 30)) * 4).astype(np.float32), dt)
    r = oracle.silu_activation(H, dt)
    h = to_f64(H, dt)
    assert np.array_equal(r["y"], h / (1.0 + np.exp(-h)))
    # one rounding: A is the stored value nearest to y
    a = to_f64(r["A"], dt)
    u = oracle.ulp(np.abs(r["y"]), dt)
    assert np.all(np.abs(a - r["y"]) <= 0.5 * u + 1e-300)


# --------------------------------------------------------------------------
# the oracle's row chunks (1024 rows bound its float64 temporaries): the
# chunked loops must equal the plain definitions on inputs of several chunks


def _chunk_case():
    g = np.random.default_rng(60)
    M, K, N = 1537, 72, 40
    x = g.standard_normal((M, K)).astype(np.float32)
    x[:, [5, 41]] *= 20                              # outlier columns spread over all rows
    x[1536, 63] = 9.0                                # a column flagged only by the very last row
    x[3, 17] = 7.5                                   # ... and one only by an early row
    A = workloads._store(x, "bf16")
    W = (g.standard_normal((N, K)) * 0.05).astype(np.float32)
    G = workloads._store((g.standard_normal((M, N)) * 0.1).astype(np.float32), "bf16")
    return A, W, G


def test_chunked_loops_equal_plain_definition():
    A, W, G = _chunk_case()
    X16 = to_half(A, "bf16")
    # plain definitions, no chunks
    plain_O = np.nonzero((np.abs(X16.astype(np.float32)) > np.float32(6.0)).any(axis=0))[0]
    assert plain_O.tolist() == [5, 17, 41, 63]
    CB, SCB = oracle.quantize_weight(W)
    for chunk in (7, 1024, 10 ** 9):
        assert oracle.outlier_columns(X16, 6.0, chunk=chunk).tolist() == plain_O.tolist()
    ref_q = oracle.quantize_rowwise(A, "bf16", 6.0, chunk=10 ** 9)
    for chunk in (7, 1024):
        q = oracle.quantize_rowwise(A, "bf16", 6.0, chunk=chunk)
        assert q["outliers"].tolist() == plain_O.tolist()
        assert np.array_equal(q["codes"], ref_q["codes"])
        assert np.array_equal(q["scale"].view(np.uint32), ref_q["scale"].view(np.uint32))
        assert np.array_equal(q["sub"].view(np.uint16), ref_q["sub"].view(np.uint16))
    # the row scale of every row, written out per row without any chunking
    keep = np.ones(X16.shape[1], bool)
    keep[plain_O] = False
    s_rows = np.array([np.abs(X16[r, keep].astype(np.float32)).max() for r in range(X16.shape[0])])
    assert np.array_equal(ref_q["scale"], s_rows.astype(np.float32))
    CA = ref_q["codes"]
    ref_c = CA.astype(np.int64) @ CB.astype(np.int64).T          # textbook integer product
    for chunk in (7, 1024, 10 ** 9):
        assert np.array_equal(oracle.int_matmul(CA, CB, chunk=chunk), ref_c)
    Wdq = oracle.dequant_weight(CB, SCB).astype(np.float64)
    ref_b = to_half(G, "bf16").astype(np.float64) @ Wdq
    for chunk in (7, 1024, 10 ** 9):
        b = oracle.linear_backward_input(G, "bf16", CB, SCB, chunk=chunk)
        assert np.array_equal(b["y"], ref_b)


def test_quantizer_rejects_non_finite_half_cast():
    """Reading 23: an input whose fp16 cast is not finite has no code."""
    base = np.ones((3, 4), np.float32)
    for bad in (70000.0, 65520.0, float("inf"), float("nan")):
        x = base.copy()
        x[1, 2] = bad
        for dt in ("f32", "bf16"):
            with pytest.raises(ValueError):
                oracle.quantize_rowwise(workloads._store(x, dt) if dt == "bf16" else x, dt, 6.0)
    x = base.copy()
    x[1, 2] = 65504.0                                # the largest finite fp16 value is accepted
    q = oracle.quantize_rowwise(x, "f32", 0.0)
    assert q["codes"][1, 2] == 127 and q["scale"][1] == np.float32(65504.0)


# --------------------------------------------------------------------------
# the EasyDeL residual MLP's backward half, pinned against the float64
# backward of the unquantized MLP (bitsandbytes PR #33 bounds)


def _mlp600_case():
    wl, Ws, bs = _mlp600_weights()
    x = workloads.make_activation(wl, 0)
    g = workloads.make_grad(wl, 1)
    layers = []
    for W, b in zip(Ws, bs):
        cb, s = oracle.quantize_weight(W)
        layers.append((cb, s, b))
    r = oracle.mlp_forward_backward(x, g, "f32", layers, wl.threshold)
    xf, gf = x.astype(np.float64), g.astype(np.float64)
    W1, W2 = Ws[0].astype(np.float64), Ws[1].astype(np.float64)
    b1 = bs[0].astype(np.float64) if bs[0] is not None else 0.0
    b2 = bs[1].astype(np.float64) if bs[1] is not None else 0.0
    h = xf @ W1.T + b1                               # unquantized float64 MLP
    # derivative of SiLU by complex-step differentiation (no closed form of it)
    hs = 1e-30
    dsilu = np.imag((h + 1j * hs) / (1.0 + np.exp(-(h + 1j * hs)))) / hs
    ref = {"h": h, "out": (h / (1.0 + np.exp(-h))) @ W2.T + b2 + xf}
    ref["g_a"] = gf @ W2
    ref["g_h"] = ref["g_a"] * dsilu
    ref["grad_x"] = ref["g_h"] @ W1 + gf
    ref["gb1"] = ref["g_h"].sum(axis=0)
    ref["gb2"] = gf.sum(axis=0)
    return r, ref, layers, (xf, gf, W1)


def test_mlp600_backward_against_float_mlp():
    r, ref, layers, (xf, gf, W1) = _mlp600_case()
    for name in ("out", "grad_x", "gb1", "gb2"):
        res = oracle.page_bounds(to_f64(r[name], "f32"), ref[name])
        assert res["ok"], (name, res)
    # two plausible slips in the composite backward break the grad_x bound:
    # (1) SiLU' taken at the activation a instead of at the pre-activation h
    g_a = to_f64(r["g_a"], "f32")
    h = to_f64(r["h"], "f32")
    cb1, s1, _ = layers[0]
    slip1 = oracle.from_f64(g_a * oracle.silu_grad(to_f64(r["a"], "f32")), "f32")
    gx1 = to_f64(oracle.linear_backward_input(slip1, "f32", cb1, s1)["grad_A"], "f32") + gf
    assert not oracle.page_bounds(gx1, ref["grad_x"])["ok"]
    assert not oracle.page_bounds(slip1.astype(np.float64).sum(axis=0), ref["gb1"])["ok"]
    # (2) the residual's gradient + g dropped
    gx2 = to_f64(oracle.linear_backward_input(r["g_h"], "f32", cb1, s1)["grad_A"], "f32")
    assert not oracle.page_bounds(gx2, ref["grad_x"])["ok"]
    # and the forward half without the residual input fails too
    assert not oracle.page_bounds(to_f64(r["out"], "f32") - xf, ref["out"])["ok"]
    # the un-slipped composition from the same pieces reproduces the oracle
    gh = oracle.from_f64(g_a * oracle.silu_grad(h), "f32")
    assert np.array_equal(gh, r["g_h"])


def test_mlp600_g_h_is_silu_derivative_at_stored_h():
    """g_h = D(g_a * SiLU'(h)) with h the first linear's stored output: SiLU'
    by complex-step differentiation, elementwise within one unit of f32."""
    r, ref, layers, _ = _mlp600_case()
    h = to_f64(r["h"], "f32")
    hs = 1e-30
    d = np.imag((h + 1j * hs) / (1.0 + np.exp(-(h + 1j * hs)))) / hs
    y = to_f64(r["g_a"], "f32") * d
    from oracle.formats import ulp
    err = np.abs(to_f64(r["g_h"], "f32") - y)
    assert np.all(err <= 0.5 * ulp(np.abs(y), "f32") * (1 + 1e-6) + 1e-300)
    # gb1 and gb2 are the column sums of g_h and g in f32 (one rounding of the exact sums)
    assert np.array_equal(r["gb1"], oracle.from_f64(to_f64(r["g_h"], "f32").sum(axis=0), "f32"))
    assert np.array_equal(r["gb2"], oracle.from_f64(to_f64(workloads.make_grad(workloads.WORKLOADS["mlp600"], 1),
                                                           "f32").sum(axis=0), "f32"))
