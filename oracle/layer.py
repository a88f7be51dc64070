"""CPU oracle of the int8 rowwise-quantized linear layer (test infrastructure).

TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this module. It is a plain, slow, obviously
correct definition of what the layer computes; it shares no code with the
HIP library and the library never calls it.

Sources (public web pages):

* bitsandbytes PR #33 "Memory efficient backward" (BNB33):
  - PR description: int8 weights stored row-major; the backward builds fp16
    weights on the fly from them and runs an fp16 matmul with the fp16
    output gradient, never storing fp16 weights; inputs are cast to fp16 and
    outputs back to the input dtype.
  - review on ``_functions.py`` ("Cast A to fp16"): the cast of A before
    quantization; commit "cast to half before double_quant".
  - review on ``_functions.py`` (bias add and "4. Mixed-precision
    decomposition matmul"): dequantized int8 product plus bias, plus the fp16
    product of the outlier sub-matrices; the ``addmm_`` discussion.
  - author notes: grad_bias from the un-cast output gradient; the weight is
    frozen (no weight gradient).
  - review on ``_functions.py`` (backward dequantization): CB cast, then
    multiplied by SCB * (1/127) (multiply instead of divide, "applied").
  - review on ``tests/test_modules.py``: the error bounds (max error below
    0.05 * mean|ref|; at most 0.5 % of elements outside atol 0.01 * mean|ref|,
    rtol 0.1).
* EasyDeL discussion #66, "Run and find Out" example: the residual MLP
  Dense -> SiLU -> Dense -> + input.

Notation: X16 is the fp16 cast of X; fl32(.) one correctly rounded fp32
operation; rint round-half-to-even; D the tensor's storage dtype.

Readings where the pages are silent (each also listed, with the same number,
in the design notes; 16-22 there concern the workloads, not this module):
  1. outlier columns: |X16| > tau strictly, tau compared in fp32;
  2. tau <= 0, tau = +inf or NaN disables the split (no outlier columns);
  3. a column is an outlier column if any row of the flattened batch exceeds tau;
  4. the row scale (absmax) is taken over non-outlier columns only;
  5. code = clamp(rint(fl32(X16 * fl32(127 / s))), -127, 127); never -128;
  6. a row with s = 0 (all zero, or only outlier columns) gets codes 0;
  7. the threshold applies to X16 (after the fp16 cast);
  8. the backward dequantizes to fp16;
  9. sigma = fl32(SCB * fl32(1/127)); Wdq = fp16(fl32(CB * sigma)); the same
     Wdq feeds the outlier product and the backward;
 10. the float result is exact (float64) up to one final rounding to D;
 11. the outlier weight slice comes from the int8 weights (no fp16 copy kept);
 12. grad_bias sums the un-cast gradient and is returned in D.
 13. int8 backward variant (EasyDeL discussion #66: fwd_bits=8, bwd_bits=8;
     the page only says the backward dot product is computed in 8 bits): both
     operands carry scales constant along the contraction N. G is quantized
     by Q with the split off (one scale per token row); the weight has a second
     offline int8 copy, W^T (K x N) quantized by Q with the split off (one
     scale per input feature k); grad_A = D(C32 * SG[m] * SCBt[k] / 127^2)
     with C32 = CG . CBt^T exact; grad_bias as in reading 12.
 14. trainable-weight mode (BNB33 PR description: the has_fp16_weights option
     beside the memory-efficient one; the pages give no formula): the weight
     gradient of y = A16 W^T is grad_W[n, k] = D(sum_m G16[m, n] * A16[m, k]),
     both operands cast to fp16 as in the rest of the layer (values beyond
     fp16's range become +-inf), exact products, one rounding to D.
 15. producer-side outlier flags (EasyDeL discussion #66's MLP: Dense -> SiLU
     -> Dense): the SiLU between the linears is applied to the first
     linear's output as stored in D and rounded to D once; the kernel that
     produces A = D(SiLU(H)) may also hand over A's outlier columns, which
     are by definition those the quantizer would find in A (readings 1-3, 7).
 23. the quantizer's domain is inputs whose fp16 cast is finite: the pages
     cast to fp16 before quantizing, and a value beyond fp16's range (or a
     non-finite input) has no int8 code; quantize_rowwise raises ValueError
     for such inputs instead of producing one.

Pins: tests/test_oracle_*.py (brute force with exact rationals, closed-form
special cases, invariants, the pages' error bounds).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .formats import from_f64, to_f64, to_half

F32_1_OVER_127 = np.float32(1.0) / np.float32(127.0)   # fl32(1/127)


def threshold_active(tau: float) -> bool:
    """Reading 2: the outlier split is on only for 0 < tau < inf."""
    t = float(tau)
    return (t == t) and 0.0 < t < float("inf")


def outlier_columns(X16: np.ndarray, tau: float, chunk: int = 1024) -> np.ndarray:
    """Ascending indices of feature columns with any |X16| > tau (readings 1, 3, 7).

    BNB33 "4. Mixed-precision decomposition matmul": outlier feature columns
    of A are taken out of the int8 product and multiplied in fp16.
    """
    R, C = X16.shape
    if not threshold_active(tau) or R == 0 or C == 0:
        return np.zeros(0, dtype=np.int32)
    t = np.float32(tau)
    flag = np.zeros(C, dtype=bool)
    for r0 in range(0, R, chunk):
        flag |= (np.abs(X16[r0:r0 + chunk].astype(np.float32)) > t).any(axis=0)
    return np.nonzero(flag)[0].astype(np.int32)


def quantize_rowwise(X: np.ndarray, dt: str, tau: float, chunk: int = 1024) -> dict:
    """Row-wise int8 quantization with outlier-column split.

    Steps (BNB33 "Cast A to fp16" review, commit "cast to half before
    double_quant"; the 127 scale of the dequantization review):
      Q1 X16 = fp16(X)
      Q2 O = outlier columns of X16
      Q3 s[r] = max over c not in O of |X16[r, c]|   (0 if none)
      Q4 inv[r] = fl32(127 / s[r])                    (0 if s[r] = 0)
      Q5 code[r, c] = clamp(rint(fl32(X16[r, c] * inv[r])), -127, 127); 0 on O
      Q6 sub[r, j] = X16[r, O[j]]
    Returns codes (int8, R x C), scale s (float32, R), outlier index list O
    (int32 ascending), sub (float16, R x |O|).
    """
    X16 = to_half(X, dt)
    if not np.all(np.isfinite(X16)):
        # reading 23: the method's domain is inputs whose fp16 cast is finite
        raise ValueError("quantize_rowwise: the fp16 cast of the input holds inf or NaN "
                         "(|x| beyond 65504 after rounding, or a non-finite input)")
    R, C = X16.shape
    O = outlier_columns(X16, tau, chunk)
    keep = np.ones(C, dtype=bool)
    keep[O] = False
    codes = np.zeros((R, C), dtype=np.int8)
    s = np.zeros(R, dtype=np.float32)
    for r0 in range(0, R, chunk):
        x = X16[r0:r0 + chunk].astype(np.float32)          # exact widening
        a = np.where(keep[None, :], np.abs(x), np.float32(0))
        sr = a.max(axis=1) if C else np.zeros(x.shape[0], np.float32)
        with np.errstate(divide="ignore"):
            inv = np.where(sr > 0, np.float32(127.0) / sr, np.float32(0)).astype(np.float32)
        v = x * inv[:, None]                                  # fl32 products
        q = np.clip(np.rint(v), -127, 127).astype(np.int8)
        q[:, ~keep] = 0
        codes[r0:r0 + chunk] = q
        s[r0:r0 + chunk] = sr
    sub = np.ascontiguousarray(X16[:, O])
    return {"codes": codes, "scale": s, "outliers": O, "sub": sub}


def dequant_weight(CB: np.ndarray, SCB: np.ndarray, cols=None) -> np.ndarray:
    """fp16 weights built from the int8 weights (reading 9).

    BNB33 backward-dequantization review: CB is cast and multiplied by
    SCB * (1/127), the reciprocal multiply being the version applied.
    Wdq[n, k] = fp16(fl32(CB[n, k] * fl32(SCB[n] * fl32(1/127)))).
    """
    sigma = (np.asarray(SCB, dtype=np.float32) * F32_1_OVER_127).astype(np.float32)
    cb = CB if cols is None else CB[:, cols]
    return (cb.astype(np.float32) * sigma[:, None]).astype(np.float16)


def int_matmul(CA: np.ndarray, CB: np.ndarray, rows=None, chunk: int = 1024) -> np.ndarray:
    """C32[m, n] = sum_k CA[m, k] * CB[n, k], exact (int64 result).

    Computed as a float64 matmul of integer-valued arrays: every partial sum
    is an integer below 127^2 * K < 2^53, so it is exact in any order.
    """
    if rows is not None:
        CA = CA[rows]
    B = CB.astype(np.float64).T
    out = np.empty((CA.shape[0], CB.shape[0]), dtype=np.int64)
    for r0 in range(0, CA.shape[0], chunk):
        out[r0:r0 + chunk] = (CA[r0:r0 + chunk].astype(np.float64) @ B).astype(np.int64)
    return out


def linear_forward(A: np.ndarray, dt: str, CB: np.ndarray, SCB: np.ndarray,
                   bias: Optional[np.ndarray], tau: float, rows=None, q: Optional[dict] = None) -> dict:
    """Forward of the int8 linear layer (BNB33 forward reviews).

    y[m, n] = C32[m, n] * SCA[m] * SCB[n] / 127^2
              + sum_j subA[m, j] * Wdq[n, O[j]]
              + bias[n]
    computed in float64; out = D(y), one rounding (reading 10).
    ``rows`` restricts y/out/C32 to a subset of rows (the quantization still
    sees every row, since the outlier columns depend on all of them).
    """
    if q is None:
        q = quantize_rowwise(A, dt, tau)
    CA, SCA, O, subA = q["codes"], q["scale"], q["outliers"], q["sub"]
    idx = np.arange(CA.shape[0]) if rows is None else np.asarray(rows)
    C32 = int_matmul(CA, CB, rows=idx)
    y = C32.astype(np.float64) * (SCA[idx].astype(np.float64)[:, None]
                                  * np.asarray(SCB, np.float64)[None, :]) / 16129.0
    if O.size:
        Wo = dequant_weight(CB, SCB, cols=O).astype(np.float64)       # N x |O|
        y = y + subA[idx].astype(np.float64) @ Wo.T
    if bias is not None:
        y = y + to_f64(bias, dt)[None, :]
    return {"y": y, "out": from_f64(y, dt), "c32": C32, "rows": idx, "q": q}


def grad_bias(G: np.ndarray, dt: str) -> tuple:
    """grad_bias[n] = sum over rows of the un-cast G (BNB33 author notes).

    Returns (float64 sum, value rounded to D)."""
    g = to_f64(G, dt).sum(axis=0)
    return g, from_f64(g, dt)


def linear_backward_input(G: np.ndarray, dt: str, CB: np.ndarray, SCB: np.ndarray,
                          rows=None, chunk: int = 1024) -> dict:
    """Memory-efficient backward: grad_A = D(fp16(G) @ Wdq) (BNB33 PR description).

    The weight gradient is not computed: the int8 weight is frozen (BNB33
    author notes). ``rows`` restricts grad_A to a subset of rows.
    """
    idx = np.arange(G.shape[0]) if rows is None else np.asarray(rows)
    W = dequant_weight(CB, SCB).astype(np.float64)                       # N x K
    ga = np.empty((idx.size, CB.shape[1]), dtype=np.float64)
    for r0 in range(0, idx.size, chunk):
        g16 = to_half(G[idx[r0:r0 + chunk]], dt).astype(np.float64)
        ga[r0:r0 + chunk] = g16 @ W
    return {"y": ga, "grad_A": from_f64(ga, dt), "rows": idx}


def linear_backward_weight(G: np.ndarray, A: np.ndarray, dt: str, rows=None) -> dict:
    """Weight gradient of the trainable-weight mode (reading 14).

    grad_W[n, k] = D(sum_m fp16(G[m, n]) * fp16(A[m, k])), the sum in float64
    (products of fp16 values are exact there). ``rows`` restricts the output
    to a subset of weight rows n.
    """
    idx = np.arange(G.shape[1]) if rows is None else np.asarray(rows)
    g16 = to_half(G, dt)[:, idx].astype(np.float64)                     # M x |rows|
    a16 = to_half(A, dt).astype(np.float64)                             # M x K
    y = g16.T @ a16
    return {"y": y, "grad_W": from_f64(y, dt), "rows": idx}


def quantize_weight(W: np.ndarray, dt: str = "f32") -> tuple:
    """Offline weight quantization: Q with the outlier split off -> (CB, SCB)."""
    q = quantize_rowwise(W, dt, 0.0)
    return q["codes"], q["scale"]


def quantize_weight_colwise(W: np.ndarray, dt: str = "f32") -> tuple:
    """Second offline int8 copy for the int8 backward (reading 13): W^T (K x N)
    quantized row-wise, i.e. one scale per input feature k -> (CBt, SCBt)."""
    return quantize_weight(np.ascontiguousarray(np.asarray(W).T), dt)


def linear_backward_input_int8(G: np.ndarray, dt: str, CBt: np.ndarray, SCBt: np.ndarray,
                               rows=None) -> dict:
    """int8 backward variant (EasyDeL discussion #66, bwd_bits=8; reading 13).

    (CG, SG) = Q(G, split off); C32[m, k] = sum_n CG[m, n] * CBt[k, n] (exact);
    grad_A[m, k] = D(C32 * SG[m] * SCBt[k] / 127^2), float64 then one rounding.
    ``rows`` restricts grad_A / C32 to a subset of rows.
    """
    q = quantize_rowwise(G, dt, 0.0)
    CG, SG = q["codes"], q["scale"]
    idx = np.arange(CG.shape[0]) if rows is None else np.asarray(rows)
    C32 = int_matmul(CG, CBt, rows=idx)
    y = C32.astype(np.float64) * (SG[idx].astype(np.float64)[:, None]
                                  * np.asarray(SCBt, np.float64)[None, :]) / 16129.0
    return {"y": y, "grad_A": from_f64(y, dt), "c32": C32, "rows": idx, "q": q}


# ----------------------------------------------------------------------------
# EasyDeL discussion #66 "Run and find Out": Dense -> SiLU -> Dense -> + input.


def silu(h: np.ndarray) -> np.ndarray:
    return h / (1.0 + np.exp(-h))


def silu_activation(H: np.ndarray, dt: str) -> dict:
    """The activation between the two linears of EasyDeL discussion #66's
    "Run and find Out" MLP, applied to the first linear's output H as stored
    in D: A = D(SiLU(H)), SiLU in float64 and one rounding (reading 15). The
    outlier columns of A (the second linear's input) are
    outlier_columns(fp16(A), tau), as the quantizer finds them."""
    y = silu(to_f64(H, dt))
    return {"y": y, "A": from_f64(y, dt)}


def silu_grad(h: np.ndarray) -> np.ndarray:
    s = 1.0 / (1.0 + np.exp(-h))
    return s * (1.0 + h * (1.0 - s))


def mlp_forward_backward(x: np.ndarray, g: np.ndarray, dt: str, layers: list, tau: float) -> dict:
    """Residual MLP with two int8 linears; layers = [(CB, SCB, bias), (CB, SCB, bias)].

    Each linear's output is stored in D (as the layer returns it); SiLU and
    the residual add are evaluated in float64 and rounded to D once.
    """
    (cb1, s1, b1), (cb2, s2, b2) = layers
    f1 = linear_forward(x, dt, cb1, s1, b1, tau)
    h = to_f64(f1["out"], dt)
    a = from_f64(silu(h), dt)
    f2 = linear_forward(a, dt, cb2, s2, b2, tau)
    out = from_f64(to_f64(f2["out"], dt) + to_f64(x, dt), dt)
    b2r = linear_backward_input(g, dt, cb2, s2)
    g_a = to_f64(b2r["grad_A"], dt)
    g_h = from_f64(g_a * silu_grad(h), dt)
    b1r = linear_backward_input(g_h, dt, cb1, s1)
    grad_x = from_f64(to_f64(b1r["grad_A"], dt) + to_f64(g, dt), dt)
    return {"h": f1["out"], "a": a, "out": out, "g_a": b2r["grad_A"], "g_h": g_h,
            "grad_x": grad_x, "gb1": grad_bias(g_h, dt)[1], "gb2": grad_bias(g, dt)[1],
            "f1": f1, "f2": f2}


# ----------------------------------------------------------------------------
# The pages' error bounds (BNB33 review on tests/test_modules.py).


def page_bounds(T: np.ndarray, ref: np.ndarray) -> dict:
    """Max error vs 0.05*mean|ref| and the share outside isclose(atol=0.01*mean|ref|, rtol=0.1)."""
    T = np.asarray(T, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = float(np.abs(ref).mean()) if ref.size else 0.0
    err = np.abs(T - ref)
    max_err = float(err.max()) if err.size else 0.0
    outside = int((err > 0.01 * scale + 0.1 * np.abs(ref)).sum())
    return {"scale": scale, "max_err": max_err, "max_rel": max_err / scale if scale else 0.0,
            "outside": outside, "frac_outside": outside / max(T.size, 1),
            "ok": (max_err <= 0.05 * scale) and (outside <= 0.005 * T.size)}
