"""Seeded synthetic inputs for the causal attention path.

This module is the only code shared by the CPU oracle side and the GPU side of
the tests and the bench.  It holds no attention arithmetic: it draws iid
standard normals from a counter-based generator, rounds them to the storage
precision, and hands out (B, H, T, hs) arrays.

Generator (published definitions, written out here):
  * splitmix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014; constants as in Vigna's public-domain
    splitmix64.c): output(c) = mix(seed + (c + 1) * 0x9E3779B97F4A7C15) with
    mix(z) = z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
    z *= 0x94D049BB133111EB; z ^= z >> 31.
  * Box-Muller (Box & Muller 1958) on pairs of 53-bit uniforms, in float64:
    u1 in (0, 1], u2 in [0, 1): z0 = r cos(2 pi u2), z1 = r sin(2 pi u2),
    r = sqrt(-2 ln u1).
Then float64 -> float32 (round to nearest even), times a power-of-two variant
scale (exact), then float32 -> bfloat16 (round to nearest even) when the
storage type is bf16.  bf16 values are carried as float32 arrays holding
exactly representable values, plus the raw uint16 bit patterns.
"""
from __future__ import annotations

import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 21  # elements per worker chunk


def _mix(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * _M1
    z = z ^ (z >> np.uint64(27))
    z = z * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(seed: int, counters: np.ndarray) -> np.ndarray:
    """splitmix64 output for each counter value (uint64 array)."""
    c = counters.astype(np.uint64, copy=False)
    with np.errstate(over="ignore"):
        state = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + (c + np.uint64(1)) * _GOLDEN
        return _mix(state)


def _normals_chunk(seed: int, start: int, n: int) -> np.ndarray:
    # pairs [start/2, (start+n)/2); start is even
    p0 = start // 2
    npairs = (n + 1) // 2
    idx = np.arange(p0, p0 + npairs, dtype=np.uint64)
    a = splitmix64(seed, idx * np.uint64(2))
    b = splitmix64(seed, idx * np.uint64(2) + np.uint64(1))
    u1 = ((a >> np.uint64(11)).astype(np.float64) + 1.0) * (1.0 / 9007199254740992.0)
    u2 = (b >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)
    r = np.sqrt(-2.0 * np.log(u1))
    t = 2.0 * np.pi * u2
    out = np.empty(2 * npairs, dtype=np.float64)
    out[0::2] = r * np.cos(t)
    out[1::2] = r * np.sin(t)
    return out[:n]


def normal_f64(seed: int, n: int, workers: int = 8) -> np.ndarray:
    """n iid N(0,1) float64 draws for `seed` (element c uses counters 2*(c//2), 2*(c//2)+1)."""
    if n <= _CHUNK:
        return _normals_chunk(seed, 0, n)
    out = np.empty(n, dtype=np.float64)
    starts = list(range(0, n, _CHUNK))

    def work(s: int) -> None:
        m = min(_CHUNK, n - s)
        out[s:s + m] = _normals_chunk(seed, s, m)

    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(work, starts))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even; NaN -> quiet NaN."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    with np.errstate(over="ignore"):
        rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    rounded = np.where(nan, (u >> np.uint32(16)) | np.uint32(0x0040), rounded)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded (RNE) to the nearest bfloat16, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def round_to_f16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest IEEE binary16 (numpy's conversion:
    round to nearest even, overflow to inf), returned as float32."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


TENSORS = ("q", "k", "v", "do")


def tensor_seed(base_seed: int, workload: str, layer: int, tensor: str) -> int:
    """Seed per (workload, layer, tensor): splitmix64 of a CRC32 of the label."""
    label = f"{workload}/{layer}/{tensor}".encode()
    key = (int(base_seed) << 32) ^ zlib.crc32(label)
    return int(splitmix64(key, np.zeros(1, dtype=np.uint64))[0])


def normal_tensor(seed: int, shape, scale: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    """iid N(0,1) * scale, rounded to the storage type; returned as float32.

    `scale` must be a power of two so the variant is an exact bit-scaling of the
    same draw (checked).
    """
    m, e = np.frexp(scale)
    if m != 0.5:
        raise ValueError("scale must be a power of two")
    n = int(np.prod(shape))
    x = normal_f64(seed, n).astype(np.float32) * np.float32(scale)
    if dtype == "bf16":
        x = round_to_bf16(x)
    elif dtype == "f16":
        x = round_to_f16(x)
    elif dtype != "f32":
        raise ValueError(dtype)
    return x.reshape(shape)


def attention_inputs(B: int, H: int, T: int, hs: int, dtype: str = "bf16", *, seed: int = 1234,
                     workload: str = "custom", layer: int = 0, qkv_scale: float = 1.0,
                     do_scale: float = 1.0) -> dict:
    """q, k, v (times qkv_scale) and dO (times do_scale), float32 arrays (B, H, T, hs)."""
    shape = (B, H, T, hs)
    out = {}
    for name in TENSORS:
        s = tensor_seed(seed, workload, layer, name)
        sc = do_scale if name == "do" else qkv_scale
        out[name] = normal_tensor(s, shape, sc, dtype)
    return out
