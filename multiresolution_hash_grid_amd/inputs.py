"""Seeded synthetic inputs for the hash-grid encoder workloads.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark. It only draws random numbers and shapes them into points, tables and
upstream gradients; it contains none of the encoder's arithmetic (no scaling,
hashing, interpolation or scatter).

Random numbers come from one counter-based generator: element ``i`` of stream
``s`` under seed ``seed`` is SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014; the 64-bit finaliser constants
are the ones published with Vigna's reference implementation) evaluated at state
``key(seed, s) + (i + 1) * GAMMA``.  Streams: 0 points, 1 tables, 2 upstream
gradients, 3 MLP weights, 4 ray parameters, 5 ray-sample jitter.

Workloads (sizes of the Instant-NGP style grids used to test and measure the
encoder; page 1 "HashGridEncoder" constructor defaults give the standard grid):

* ``tiny``      L=4,  F=2, T=2^10, N_min=4,  N_max=32,   fp32, 4096 uniform points
* ``standard``  L=16, F=2, T=2^19, N_min=16, N_max=512,  fp32, 2^18 uniform points
* ``ray``       standard grid, 4096 rays x 256 stratified samples, ray-major
* ``large_f16`` L=32, F=2, T=2^21, N_min=16, N_max=4096, fp16 tables, 2^21 points
* ``fused_mlp`` standard grid with fp16 tables, 2^22 points, MLP 32->64->64->4
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22

STREAM_POINTS = 0
STREAM_TABLE = 1
STREAM_DOUT = 2
STREAM_MLP = 3
STREAM_RAYS = 4
STREAM_JITTER = 5


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _key(seed: int, stream: int) -> np.uint64:
    base = np.array([(seed * 0x100000001B3 + stream * 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF],
                    dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(base)[0]


_BLOCK = 1 << 18
_STEPS = np.arange(1, _BLOCK + 1, dtype=np.uint64) * GAMMA  # wraps mod 2^64


def splitmix64(seed: int, stream: int, count: int, offset: int = 0) -> np.ndarray:
    """Raw 64-bit draws ``offset .. offset+count-1`` of one stream
    (state_i = key + (i + 1) * GAMMA, output = the SplitMix64 finaliser)."""
    key = _key(seed, stream)
    out = np.empty(count, dtype=np.uint64)
    tmp = np.empty(_BLOCK, dtype=np.uint64)
    s30, s27, s31 = np.uint64(30), np.uint64(27), np.uint64(31)
    with np.errstate(over="ignore"):
        for s in range(0, count, _BLOCK):
            e = min(count, s + _BLOCK)
            z, t = out[s:e], tmp[:e - s]
            np.add(_STEPS[:e - s], key + np.uint64(offset + s) * GAMMA, out=z)
            np.right_shift(z, s30, out=t)
            np.bitwise_xor(z, t, out=z)
            np.multiply(z, _M1, out=z)
            np.right_shift(z, s27, out=t)
            np.bitwise_xor(z, t, out=z)
            np.multiply(z, _M2, out=z)
            np.right_shift(z, s31, out=t)
            np.bitwise_xor(z, t, out=z)
    return out


def uniform_f32(seed: int, stream: int, count: int, offset: int = 0) -> np.ndarray:
    """Uniform in [0, 1) on the 2^-24 lattice, hence exact in float32."""
    bits = splitmix64(seed, stream, count, offset)
    return ((bits >> np.uint64(40)).astype(np.float64) * 2.0 ** -24).astype(np.float32)


def uniform_f64(seed: int, stream: int, count: int, offset: int = 0) -> np.ndarray:
    """Uniform in [0, 1) on the 2^-53 lattice."""
    bits = splitmix64(seed, stream, count, offset)
    return (bits >> np.uint64(11)).astype(np.float64) * 2.0 ** -53


def _parallel_chunks(count: int, fill) -> None:
    """Run fill(start, end) over CHUNK-sized pieces on a few threads (numpy
    releases the GIL inside its loops); each piece depends only on its range."""
    spans = [(s, min(count, s + _CHUNK)) for s in range(0, count, _CHUNK)]
    if len(spans) <= 1:
        for s, e in spans:
            fill(s, e)
        return
    workers = max(1, min(8, os.cpu_count() or 1, len(spans)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda se: fill(*se), spans))


def normal_f32(seed: int, stream: int, count: int) -> np.ndarray:
    """N(0,1) by the Box-Muller transform, one normal per pair of uniforms."""
    out = np.empty(count, dtype=np.float32)

    def fill(s, e):
        u = uniform_f64(seed, stream, 2 * (e - s), offset=2 * s)
        r = np.sqrt(-2.0 * np.log1p(-u[0::2]))  # 1 - u1 lies in (0, 1]
        out[s:e] = (r * np.cos(2.0 * math.pi * u[1::2])).astype(np.float32)

    _parallel_chunks(count, fill)
    return out


# ----------------------------------------------------------------------------- shapes

def points_uniform(seed: int, n: int, dims: int = 3) -> np.ndarray:
    return uniform_f32(seed, STREAM_POINTS, dims * n).reshape(n, dims)


def table_uniform(seed: int, n_levels: int, table_size: int, n_features: int,
                  dtype: str = "f32", scale: float = 1e-4) -> np.ndarray:
    """Tables drawn uniform(-scale, scale) in float64, rounded to float32 and,
    for ``dtype == "f16"``, then rounded to IEEE binary16 (nearest-even,
    subnormals kept)."""
    count = n_levels * table_size * n_features
    out = np.empty(count, dtype=np.float32)

    def fill(s, e):
        u = uniform_f64(seed, STREAM_TABLE, e - s, offset=s)
        out[s:e] = ((2.0 * u - 1.0) * scale).astype(np.float32)

    _parallel_chunks(count, fill)
    if dtype == "f16":
        half = np.empty(count, dtype=np.float16)

        def narrow(s, e):
            half[s:e] = out[s:e].astype(np.float16)

        _parallel_chunks(count, narrow)
        return half.reshape(n_levels, table_size, n_features)
    out = out.reshape(n_levels, table_size, n_features)
    if dtype != "f32":
        raise ValueError(f"unknown table dtype {dtype!r}")
    return out


def dout_normal(seed: int, n: int, cols: int) -> np.ndarray:
    return normal_f32(seed, STREAM_DOUT, n * cols).reshape(n, cols)


def points_rays(seed: int, n_rays: int, samples: int,
                box_lo: float = 0.25, box_hi: float = 0.75, radius: float = 1.5) -> np.ndarray:
    """Ray-major stratified samples of rays that start on a sphere around the
    unit cube and aim at a random point of a head-sized box inside it.

    Each ray's segment inside [0,1]^3 (slab test) is split into ``samples``
    equal strata with one jittered sample per stratum; the samples are rounded
    to float32 and clamped to [0, 1 - 2^-24]."""
    u = uniform_f64(seed, STREAM_RAYS, 5 * n_rays).reshape(n_rays, 5)
    cz = 2.0 * u[:, 0] - 1.0
    phi = 2.0 * math.pi * u[:, 1]
    rr = np.sqrt(np.maximum(0.0, 1.0 - cz * cz))
    s = np.stack([rr * np.cos(phi), rr * np.sin(phi), cz], axis=1)
    o = 0.5 + radius * s
    p = box_lo + (box_hi - box_lo) * u[:, 2:5]
    d = p - o
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        t0 = (0.0 - o) / d
        t1 = (1.0 - o) / d
    t_in = np.max(np.minimum(t0, t1), axis=1)
    t_out = np.min(np.maximum(t0, t1), axis=1)
    assert np.all(t_out > t_in), "every ray must cross the unit cube"
    jit = uniform_f64(seed, STREAM_JITTER, n_rays * samples).reshape(n_rays, samples)
    frac = (np.arange(samples, dtype=np.float64)[None, :] + jit) / samples
    t = t_in[:, None] + frac * (t_out - t_in)[:, None]
    pts = o[:, None, :] + t[:, :, None] * d[:, None, :]
    pts = pts.reshape(-1, 3).astype(np.float32)
    return np.clip(pts, np.float32(0.0), np.float32(1.0 - 2.0 ** -24))


def xavier_uniform(seed: int, fan_in: int, fan_out: int, offset: int = 0) -> np.ndarray:
    """[fan_out, fan_in] weights drawn U(-a, a), a = sqrt(6 / (fan_in + fan_out))
    (Glorot and Bengio, 2010)."""
    a = math.sqrt(6.0 / (fan_in + fan_out))
    u = uniform_f64(seed, STREAM_MLP, fan_in * fan_out, offset=offset)
    return ((2.0 * u - 1.0) * a).astype(np.float32).reshape(fan_out, fan_in)


def mlp_params(seed: int, sizes=(32, 64, 64, 4), bias_scale="linear"):
    """Weights and biases of the MLP head: per layer W [out, in] Xavier-uniform,
    rounded to binary16 (the dtype the matrix cores read), and fp32 biases
    drawn U(-a, a) with a = bias_scale, or a = 1/sqrt(fan_in) for "linear"
    (torch.nn.Linear's own bias initialisation, the layer the NeRFace head is
    built from).  Returns [W1, b1, W2, b2, ...] as numpy arrays."""
    out, off = [], 0
    for fin, fout in zip(sizes[:-1], sizes[1:]):
        out.append(xavier_uniform(seed, fin, fout, offset=off).astype(np.float16))
        off += fin * fout
    for fin, fout in zip(sizes[:-1], sizes[1:]):
        u = uniform_f64(seed, STREAM_MLP, fout, offset=off)
        off += fout
        a = 1.0 / np.sqrt(fin) if isinstance(bias_scale, str) and bias_scale == "linear" else float(bias_scale)
        out.append(((2.0 * u - 1.0) * a).astype(np.float32))
    n = len(sizes) - 1
    return [v for i in range(n) for v in (out[i], out[n + i])]


# ----------------------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Workload:
    name: str
    n_levels: int
    n_features: int
    log2_table_size: int
    base_resolution: int
    finest_resolution: int
    table_dtype: str          # "f32" | "f16"
    n_points: int
    structure: str            # "uniform" | "rays"
    seed: int
    n_rays: int = 0
    samples_per_ray: int = 0
    mlp: tuple = field(default=())
    n_dims: int = 3

    @property
    def table_size(self) -> int:
        return 1 << self.log2_table_size

    @property
    def out_cols(self) -> int:
        return self.n_levels * self.n_features


WORKLOADS = {
    "tiny": Workload("tiny", 4, 2, 10, 4, 32, "f32", 4096, "uniform", seed=1000),
    "standard": Workload("standard", 16, 2, 19, 16, 512, "f32", 1 << 18, "uniform", seed=1001),
    "ray": Workload("ray", 16, 2, 19, 16, 512, "f32", 4096 * 256, "rays", seed=1002,
                    n_rays=4096, samples_per_ray=256),
    "large_f16": Workload("large_f16", 32, 2, 21, 16, 4096, "f16", 1 << 21, "uniform", seed=1003),
    "fused_mlp": Workload("fused_mlp", 16, 2, 19, 16, 512, "f16", 1 << 22, "uniform", seed=1004,
                          mlp=(32, 64, 64, 4)),
}


def resized(w: Workload, n_points: int | None = None, **kw) -> Workload:
    """The same grid with another point count (rays: another ray count)."""
    if n_points is not None:
        if w.structure == "rays":
            nr = max(1, n_points // w.samples_per_ray)
            kw.update(n_rays=nr, n_points=nr * w.samples_per_ray)
        else:
            kw["n_points"] = n_points
    return replace(w, **kw)


def make_points(w: Workload) -> np.ndarray:
    if w.structure == "rays":
        return points_rays(w.seed, w.n_rays, w.samples_per_ray)
    return points_uniform(w.seed, w.n_points, w.n_dims)


def make_table(w: Workload) -> np.ndarray:
    return table_uniform(w.seed, w.n_levels, w.table_size, w.n_features, w.table_dtype)


def make_dout(w: Workload, cols: int | None = None) -> np.ndarray:
    return dout_normal(w.seed, w.n_points, w.out_cols if cols is None else cols)
