"""Seeded synthetic inputs for the int8 rowwise-quantized linear layer.

This module is shared by the CPU oracle, the tests and the benchmark. It only
draws random numbers and lays them out; it holds none of the layer's
arithmetic (no quantization, no scaling, no products). Activations, weights,
biases and output gradients are drawn in float32 and then rounded once to the
tensor's storage dtype by torch's CPU conversion (round to nearest even).

Storage dtypes are named "f32", "f16" and "bf16". On the host, an "f32" tensor
is a numpy float32 array, an "f16" tensor a numpy float16 array and a "bf16"
tensor a numpy uint16 array holding the bfloat16 bit patterns.

Workloads (the shapes, distributions and outlier structure of the pages):

* ``mlp600``: the residual MLP of the EasyDeL discussion #66 example
  ("Run and find Out"): input (1, 600, 4) fp32 ~ N(0, 1), Dense 4->16, SiLU,
  Dense 16->4, plus the input; weights LeCun-normal (truncated at two standard
  deviations), bias zero, outlier threshold 6.0.
* ``single4096``: one 4096->4096 linear on 2048 tokens, fp16 activations
  ~ N(0, 1) with 8 seeded outlier feature columns scaled x20, weights
  ~ N(0, 0.02), bias ~ N(0, 0.01), output gradient ~ N(0, 0.01).
* ``llama7b_mlp``: gate/up 4096->11008 and down 11008->4096 on 4096 tokens,
  bf16, 0.1 % outlier columns x15, bias and output gradient ~ N(0, 0.01).
* ``llama7b_block``: q, k, v, o 4096->4096, gate/up 4096->11008,
  down 11008->4096 on 1 x 4096 tokens, bf16, 0.1 % outlier columns x20, no
  bias, output gradient ~ N(0, 0.01).
* ``llama70b_mlp``: 8192->28672 and 28672->8192 on 16384 tokens, bf16, 0.5 %
  outlier columns x25, weights ~ N(0, 0.015), bias and output gradient
  ~ N(0, 0.01).

Each linear layer gets independent inputs (the activation entering the down
projection is drawn, not produced by the layers above it), so that every
layer sees exactly the stated distribution. Random streams are numpy PCG64
seeded with SeedSequence([workload id, layer index, tensor id]); tensor ids:
0 activation, 1 outlier-column choice, 2 weight, 3 bias, 4 output gradient.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

DTYPES = ("f32", "f16", "bf16")
ITEMSIZE = {"f32": 4, "f16": 2, "bf16": 2}

T_ACT, T_OUTCOLS, T_WEIGHT, T_BIAS, T_GRAD = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class LinearShape:
    name: str
    M: int          # tokens (leading dims flattened)
    K: int          # in_features
    N: int          # out_features
    n_outliers: int  # seeded outlier feature columns of the activation
    has_bias: bool


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    dtype: str
    threshold: float
    outlier_scale: float
    w_std: float            # 0 => LeCun normal (std 1/sqrt(K), truncated at 2 sigma)
    bias_std: float         # 0 with has_bias => zero bias
    grad_std: float
    act_std: float
    layers: tuple

    def layer(self, name: str) -> LinearShape:
        for l in self.layers:
            if l.name == name:
                return l
        raise KeyError(name)


def _frac(K: int, f: float) -> int:
    return int(round(f * K))


def _mk_workloads() -> dict:
    w = {}
    w["mlp600"] = Workload(
        0, "mlp600", "f32", 6.0, 1.0, 0.0, 0.0, 1.0, 1.0,
        (LinearShape("dense1", 600, 4, 16, 0, True),
         LinearShape("dense2", 600, 16, 4, 0, True)))
    w["single4096"] = Workload(
        1, "single4096", "f16", 6.0, 20.0, 0.02, 0.01, 0.01, 1.0,
        (LinearShape("proj", 2048, 4096, 4096, 8, True),))
    w["llama7b_mlp"] = Workload(
        2, "llama7b_mlp", "bf16", 6.0, 15.0, 0.02, 0.01, 0.01, 1.0,
        (LinearShape("gate", 4096, 4096, 11008, _frac(4096, 1e-3), True),
         LinearShape("up", 4096, 4096, 11008, _frac(4096, 1e-3), True),
         LinearShape("down", 4096, 11008, 4096, _frac(11008, 1e-3), True)))
    w["llama7b_block"] = Workload(
        3, "llama7b_block", "bf16", 6.0, 20.0, 0.02, 0.0, 0.01, 1.0,
        tuple(LinearShape(n, 4096, 4096, 4096, _frac(4096, 1e-3), False)
              for n in ("q", "k", "v", "o"))
        + (LinearShape("gate", 4096, 4096, 11008, _frac(4096, 1e-3), False),
           LinearShape("up", 4096, 4096, 11008, _frac(4096, 1e-3), False),
           LinearShape("down", 4096, 11008, 4096, _frac(11008, 1e-3), False)))
    w["llama70b_mlp"] = Workload(
        4, "llama70b_mlp", "bf16", 6.0, 25.0, 0.015, 0.01, 0.01, 1.0,
        (LinearShape("up", 16384, 8192, 28672, _frac(8192, 5e-3), True),
         LinearShape("down", 16384, 28672, 8192, _frac(28672, 5e-3), True)))
    return w


WORKLOADS = _mk_workloads()
WORKLOAD_ORDER = ("mlp600", "single4096", "llama7b_mlp", "llama7b_block", "llama70b_mlp")


def rng(wid: int, layer: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([wid, layer, tensor]))


def _store(x32: np.ndarray, dt: str) -> np.ndarray:
    """Round float32 values to the storage dtype (torch CPU conversion, RNE)."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dt == "f32":
        return x32
    if dt == "f16":
        return x32.astype(np.float16)
    if dt == "bf16":
        import torch
        t = torch.from_numpy(x32).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dt)


def outlier_columns(wid: int, layer: int, K: int, n: int) -> np.ndarray:
    if n <= 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng(wid, layer, T_OUTCOLS).choice(K, n, replace=False))


def normal32(g: np.random.Generator, shape, std: float) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def truncated_normal32(g: np.random.Generator, shape, std: float, bound: float = 2.0) -> np.ndarray:
    """N(0,1) truncated to [-bound, bound] by resampling, times std."""
    x = g.standard_normal(size=shape, dtype=np.float32)
    bad = np.abs(x) > bound
    while bad.any():
        x[bad] = g.standard_normal(size=int(bad.sum()), dtype=np.float32)
        bad = np.abs(x) > bound
    return x * np.float32(std)


def make_activation(wl: Workload, li: int, rows: Optional[int] = None) -> np.ndarray:
    """Activation A (M x K) of layer li, in the workload's dtype."""
    L = wl.layers[li]
    M = L.M if rows is None else rows
    x = normal32(rng(wl.wid, li, T_ACT), (M, L.K), wl.act_std)
    cols = outlier_columns(wl.wid, li, L.K, L.n_outliers)
    if cols.size:
        x[:, cols] *= np.float32(wl.outlier_scale)
    return _store(x, wl.dtype)


def make_weight(wl: Workload, li: int) -> np.ndarray:
    """Float32 master weight W (N x K, out_features x in_features)."""
    L = wl.layers[li]
    g = rng(wl.wid, li, T_WEIGHT)
    if wl.w_std == 0.0:
        # LeCun normal: variance 1/fan_in, drawn from a normal truncated at
        # two standard deviations whose std is rescaled to keep that variance.
        return truncated_normal32(g, (L.N, L.K), (1.0 / np.sqrt(L.K)) / 0.87962566103423978)
    return normal32(g, (L.N, L.K), wl.w_std)


def make_bias(wl: Workload, li: int) -> Optional[np.ndarray]:
    L = wl.layers[li]
    if not L.has_bias:
        return None
    if wl.bias_std == 0.0:
        return _store(np.zeros(L.N, dtype=np.float32), wl.dtype)
    return _store(normal32(rng(wl.wid, li, T_BIAS), (L.N,), wl.bias_std), wl.dtype)


def make_grad(wl: Workload, li: int, rows: Optional[int] = None) -> np.ndarray:
    """Output gradient G (M x N) of layer li, in the workload's dtype."""
    L = wl.layers[li]
    M = L.M if rows is None else rows
    return _store(normal32(rng(wl.wid, li, T_GRAD), (M, L.N), wl.grad_std), wl.dtype)


def small_case(dtype: str, M: int, K: int, N: int, seed: int, n_outliers: int = 0,
               outlier_scale: float = 20.0, w_std: float = 0.02, bias_std: float = 0.01,
               grad_std: float = 0.01, act_std: float = 1.0, has_bias: bool = True) -> dict:
    """A self-contained random case (used for ragged/edge parity tests)."""
    g = np.random.default_rng(np.random.SeedSequence([1000 + seed, M, K, N]))
    x = normal32(g, (M, K), act_std)
    if n_outliers:
        cols = np.sort(g.choice(K, n_outliers, replace=False))
        x[:, cols] *= np.float32(outlier_scale)
    W = normal32(g, (N, K), w_std)
    b = _store(normal32(g, (N,), bias_std), dtype) if has_bias else None
    G = _store(normal32(g, (M, N), grad_std), dtype)
    return {"A": _store(x, dtype), "W": W, "bias": b, "G": G, "dtype": dtype}


def rotating_sets_bytes(shapes: Sequence[LinearShape], dt: str) -> int:
    """HBM bytes of one set of per-step inputs (A, G) for the listed layers."""
    s = ITEMSIZE[dt]
    return sum(L.M * L.K * s + L.M * L.N * s for L in shapes)
