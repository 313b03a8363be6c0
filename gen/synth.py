"""Seeded synthetic attention inputs shared by the oracle-side tests and the GPU side.

This module only draws and stores numbers: it contains none of the method's arithmetic
(no pooling, no softmax, no selection). Both the float64 oracle and the GPU library
consume exactly the arrays produced here.

Storage: fp32 tensors are float32 numpy arrays; bf16 tensors are uint16 numpy arrays
holding bfloat16 bit patterns, rounded to nearest-even from the float32 draw.

Recipes (the design notes of the repository give the reasoning):
  sink     Q, K, V, dO ~ N(0, 1) (float32 draws, in that order). Per head, with
           mu = mean of the head's query rows, the rows of the first `n_sink` key blocks
           get (s * sqrt(d) / |mu|^2) * mu added. This raises the mean pooled logit of
           a sink block by about s, so sink blocks attract most of the pooled mass on
           many rows (attention sinks). Optional query temperature multiplies Q.
  uniform  the sink recipe with no sink and Q scaled by 0.1: near-uniform pooled rows.
  fourier  Q = gamma_i * g * Phi A + 0.5 eps, K = g * Phi A + 0.5 eps', where Phi holds
           16 random Fourier features cos(2 pi <w_m, c_t> + b_m) * sqrt(2/16) of the
           token's normalised (frame, y, x) position in raster order, w_m ~ N(0, sigma^2 I),
           b_m ~ U[0, 2 pi), A ~ N(0, 1)^{16 x d}; gamma_i in {1, 0.25} per query block
           (Bernoulli 1/2) mixes skewed and near-uniform rows; sinks as above.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field

import numpy as np


# ------------------------------------------------------------------ dtype handling
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def stored_to_f64(a: np.ndarray) -> np.ndarray:
    """Stored array (float32 or bf16 bits) -> float64 values (exact)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


@dataclass
class Inputs:
    """Stored tensors [B, H, N, d] plus the recipe that made them."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray | None
    do: np.ndarray | None
    dtype: str  # "f32" or "bf16"
    recipe: dict = field(default_factory=dict)

    def f64(self, name: str) -> np.ndarray:
        return stored_to_f64(getattr(self, name))

    def head_f64(self, name: str, b: int, h: int) -> np.ndarray:
        return stored_to_f64(getattr(self, name)[b, h])

    def hashes(self) -> dict:
        return {n: sha256(getattr(self, n)) for n in ("q", "k", "v", "do")
                if getattr(self, n) is not None}


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype}")


def _add_sinks(q32: np.ndarray, k32: np.ndarray, bkv: int, n_sink: int, s: float) -> None:
    """In place: shift the first n_sink key blocks of every head along its mean query."""
    if n_sink <= 0 or s == 0.0:
        return
    b_, h_, n, d = q32.shape
    rows = min(n, n_sink * bkv)
    for b in range(b_):
        for h in range(h_):
            mu = q32[b, h].astype(np.float64).mean(axis=0)
            shift = (s * math.sqrt(d) / float(mu @ mu)) * mu
            k32[b, h, :rows] += shift.astype(np.float32)


# ------------------------------------------------------------------ recipes
def sink_inputs(B: int, H: int, N: int, d: int, bkv: int, *, seed: int, dtype: str,
                n_sink: int = 1, sink_scale: float = 3.0, q_temp: float = 1.0,
                with_v: bool = True, with_do: bool = True) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    q32 = rng.standard_normal(shape, dtype=np.float32)
    k32 = rng.standard_normal(shape, dtype=np.float32)
    v32 = rng.standard_normal(shape, dtype=np.float32) if with_v else None
    do32 = rng.standard_normal(shape, dtype=np.float32) if with_do else None
    if q_temp != 1.0:
        q32 *= np.float32(q_temp)
    _add_sinks(q32, k32, bkv, n_sink, sink_scale)
    return Inputs(
        q=_store(q32, dtype), k=_store(k32, dtype),
        v=None if v32 is None else _store(v32, dtype),
        do=None if do32 is None else _store(do32, dtype),
        dtype=dtype,
        recipe=dict(kind="sink", B=B, H=H, N=N, d=d, bkv=bkv, seed=seed, n_sink=n_sink,
                    sink_scale=sink_scale, q_temp=q_temp))


def uniform_inputs(B: int, H: int, N: int, d: int, bkv: int, *, seed: int, dtype: str,
                   q_temp: float = 0.1, with_do: bool = False) -> Inputs:
    inp = sink_inputs(B, H, N, d, bkv, seed=seed, dtype=dtype, n_sink=0, sink_scale=0.0,
                      q_temp=q_temp, with_do=with_do)
    inp.recipe["kind"] = "uniform"
    return inp


def fourier_inputs(B: int, H: int, grid: tuple[int, int, int], d: int, bq: int, bkv: int, *,
                   seed: int, dtype: str, rank: int = 16, sigma: float = 1.0, g: float = 2.0,
                   noise: float = 0.5, gammas: tuple[float, float] = (1.0, 0.25),
                   n_sink: int = 2, sink_scale: float = 3.0, with_do: bool = True) -> Inputs:
    f_, y_, x_ = grid
    N = f_ * y_ * x_
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    eq = rng.standard_normal(shape, dtype=np.float32)
    ek = rng.standard_normal(shape, dtype=np.float32)
    v32 = rng.standard_normal(shape, dtype=np.float32)
    do32 = rng.standard_normal(shape, dtype=np.float32) if with_do else None
    w = rng.standard_normal((B, H, rank, 3)) * sigma
    bph = rng.uniform(0.0, 2.0 * math.pi, size=(B, H, rank))
    a = rng.standard_normal((B, H, rank, d))
    t_m = -(-N // bq)
    gam = np.where(rng.uniform(size=(B, H, t_m)) < 0.5, gammas[0], gammas[1])

    # token t -> (frame, y, x) in raster order, frame-major, each normalised to [0, 1)
    t = np.arange(N)
    coords = np.stack([(t // (y_ * x_)) / f_, ((t // x_) % y_) / y_, (t % x_) / x_], axis=1)
    q32 = np.empty(shape, dtype=np.float32)
    k32 = np.empty(shape, dtype=np.float32)
    for b in range(B):
        for h in range(H):
            phi = np.cos(2.0 * math.pi * coords @ w[b, h].T + bph[b, h]) * math.sqrt(2.0 / rank)
            base = g * (phi @ a[b, h])  # [N, d]
            gq = np.repeat(gam[b, h], bq)[:N][:, None]
            q32[b, h] = (gq * base + noise * eq[b, h]).astype(np.float32)
            k32[b, h] = (base + noise * ek[b, h]).astype(np.float32)
    del eq, ek
    _add_sinks(q32, k32, bkv, n_sink, sink_scale)
    return Inputs(
        q=_store(q32, dtype), k=_store(k32, dtype), v=_store(v32, dtype),
        do=None if do32 is None else _store(do32, dtype), dtype=dtype,
        recipe=dict(kind="fourier", B=B, H=H, grid=list(grid), N=N, d=d, bq=bq, bkv=bkv,
                    seed=seed, rank=rank, sigma=sigma, g=g, noise=noise,
                    gammas=list(gammas), n_sink=n_sink, sink_scale=sink_scale))
