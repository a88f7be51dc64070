"""Helpers for the GPU parity tests: host <-> device transfer in the storage
representation used by the workloads module, and the comparison gates."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle.formats import to_f64, ulp

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def dev(x: np.ndarray, dt: str | None = None, device="cuda:0") -> torch.Tensor:
    """numpy (float32 / float16 / uint16-as-bf16 / int8 / int32) -> contiguous GPU tensor."""
    if dt == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device).contiguous()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    return a.view({1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize])


def assert_bits_equal(a: np.ndarray, b: np.ndarray, what: str):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if a.size == 0:
        return
    eq = bits(a) == bits(b)
    if not eq.all():
        i = np.argwhere(~eq)[:5]
        raise AssertionError(f"{what}: {int((~eq).sum())} of {a.size} differ; first at {i.tolist()}: "
                             f"gpu={a[tuple(i[0])]!r} oracle={b[tuple(i[0])]!r}")


def assert_float_gate(T: np.ndarray, dt: str, y: np.ndarray, what: str, tight_ulps: float = 2.0,
                      tight_rel: float = 2.0 ** -12):
    """Pages' bounds (max err <= 0.05*mean|y|; <= 0.5% outside atol 0.01*mean|y|, rtol 0.1)
    against the oracle's float64 y, plus a tight check: |T - y| <= tight_ulps * ulp_D(y)
    + tight_rel * mean|y| elementwise."""
    t = to_f64(T, dt)
    y = np.asarray(y, dtype=np.float64)
    assert t.shape == y.shape, (what, t.shape, y.shape)
    if t.size == 0:
        return
    assert np.all(np.isfinite(t)), f"{what}: non-finite output"
    r = oracle.page_bounds(t, y)
    assert r["ok"], f"{what}: pages' bounds violated: {r}"
    scale = np.abs(y).mean()
    lim = tight_ulps * ulp(np.abs(y), dt) + tight_rel * scale
    err = np.abs(t - y)
    bad = err > lim
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond the tight bound; worst "
                           f"{float((err / lim).max()):.3g}x at {np.unravel_index(np.argmax(err / lim), err.shape)}")


def tile_rows(M: int, tile: int = 256, seed: int = 0) -> np.ndarray:
    """Rows for sampled full-size checks: one random row inside every tile of
    `tile` rows (so no row tile of the kernels goes unchecked), plus the first
    and last rows and the rows around the first tile boundary."""
    g = np.random.default_rng(seed)
    r = {int(t + g.integers(0, min(tile, M - t))) for t in range(0, M, tile)}
    r |= {x for x in (0, tile - 1, tile, tile + 1, M - 1) if 0 <= x < M}
    return np.array(sorted(r), dtype=np.int64)
