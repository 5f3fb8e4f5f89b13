"""Seeded synthetic inputs for block-sparse attention (test and benchmark infrastructure).

This module holds none of the attention method's arithmetic: it only draws random
numbers, builds positional codes and rounds to bf16.  The same bytes feed the HIP
path and the CPU oracle.

Random numbers: counter-based SplitMix64 (Steele, Lea, Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) keyed per (seed, tensor id), mapped to
uniforms with 53 bits and to normals with the Box-Muller transform (both members of
each pair are used).  Values are rounded fp64 -> fp32 (round to nearest even) and then
fp32 -> bf16 (round to nearest even) once.

Workloads (shapes follow Wan2.1-style video DiT attention layers):
  * ``tiny``: B=1 H=2 N=1024 d=64, iid N(0,1) plus a shared rank-4 component added to
    Q and K of 4 tokens; blocks 64x64.
  * ``video``: tokens on a (t, h, w) raster grid; Q = z_q + alpha*PE, K = z_k + alpha*PE,
    V = z_v, dO = z_do with z ~ N(0,1); PE holds sin/cos pairs of each axis coordinate
    with geometric periods from 2 tokens to 4x the axis length; a few sink keys are
    rescaled to ``sink_scale`` x the head's rms key norm (direction kept).
  * ``stress``: the video grid, heads split into near-uniform heads (Q scaled by 0.1)
    and sink-dominated heads (sink keys in key block 0 along a direction u that every
    query shares).
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "do": 4, "aux": 5}


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _stream_key(seed: int, tensor_id: int) -> np.uint64:
    with np.errstate(over="ignore"):
        a = np.array([np.uint64(seed) * _GOLDEN + np.uint64(tensor_id)], dtype=np.uint64)
        return _mix64(a + _GOLDEN)[0]


def splitmix64(seed: int, tensor_id: int, start: int, count: int) -> np.ndarray:
    """Counter-based SplitMix64: output i = mix(key + (start+i+1)*golden)."""
    key = _stream_key(seed, tensor_id)
    ctr = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(key + ctr * _GOLDEN)


def normals(seed: int, tensor_id: int, start: int, count: int) -> np.ndarray:
    """Standard normals for flat indices [start, start+count) (fp64); start must be even."""
    assert start % 2 == 0
    npair = (count + 1) // 2
    bits = splitmix64(seed, tensor_id, start, 2 * npair).reshape(npair, 2)
    u = (bits >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)
    r = np.sqrt(-2.0 * np.log1p(-u[:, 0]))
    th = 2.0 * math.pi * u[:, 1]
    out = np.empty((npair, 2), dtype=np.float64)
    out[:, 0] = r * np.cos(th)
    out[:, 1] = r * np.sin(th)
    return out.reshape(-1)[:count]


def normals_parallel(seed: int, tensor_id: int, count: int, threads: int = 8,
                     chunk: int = 1 << 22) -> np.ndarray:
    out = np.empty(count, dtype=np.float64)
    starts = list(range(0, count, chunk))

    def work(s):
        n = min(chunk, count - s)
        out[s:s + n] = normals(seed, tensor_id, s, n)

    if len(starts) == 1:
        work(0)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(work, starts))
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64/fp32 -> bf16 bit patterns (uint16): round to fp32, then round-to-nearest-even."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    blk_q: int
    blk_k: int
    k_frac: float
    p: float
    kind: str = "video"          # "tiny" | "video" | "stress"
    grid: tuple | None = None    # (T, Hg, Wg) for video/stress
    alpha: float = 0.5
    n_sinks: int = 8
    sink_scale: float = 6.0
    seed: int = 1

    @property
    def n_qblk(self) -> int:
        return -(-self.N // self.blk_q)

    @property
    def n_kblk(self) -> int:
        return -(-self.N // self.blk_k)

    def shape(self):
        return (self.B, self.H, self.N, self.d)


# alpha for the video recipe: amplitude of the positional code.  The literal recipe
# (alpha = 0.5) gives a nearly flat pooled map; ALPHA_* put the pooled map in the
# regime where k = 5 %, p = 0.9 keeps about 5 % of the key blocks (see the density test).
ALPHA_480P = 2.0
ALPHA_720P = 2.0
# stress workload: every query of a sink-dominated head gets this multiple of u added
STRESS_SINK_QUERY_GAIN = 8.0

WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 1024, 64, 64, 64, 0.10, 0.9, kind="tiny", seed=1),
    "tiny_sparse": Workload("tiny_sparse", 1, 2, 1024, 64, 64, 64, 0.10, 0.9, kind="video",
                            grid=(4, 16, 16), alpha=ALPHA_480P, n_sinks=2, seed=11),
    "wan13b_480p": Workload("wan13b_480p", 1, 12, 32760, 128, 128, 64, 0.05, 0.9, kind="video",
                            grid=(21, 30, 52), alpha=ALPHA_480P, n_sinks=8, sink_scale=6.0, seed=2),
    "wan13b_480p_literal": Workload("wan13b_480p_literal", 1, 12, 32760, 128, 128, 64, 0.05, 0.9,
                                    kind="video", grid=(21, 30, 52), alpha=0.5, n_sinks=8,
                                    sink_scale=6.0, seed=2),
    "wan14b_720p": Workload("wan14b_720p", 1, 40, 75600, 128, 128, 64, 0.05, 0.9, kind="video",
                            grid=(21, 45, 80), alpha=ALPHA_720P, n_sinks=16, sink_scale=6.0, seed=4),
    "stress": Workload("stress", 1, 12, 32760, 128, 128, 64, 0.05, 0.9, kind="stress",
                       grid=(21, 30, 52), alpha=ALPHA_480P, n_sinks=8, sink_scale=10.0, seed=5),
}


def axis_groups(d: int):
    """Split d into three even-sized groups for the (t, h, w) axes."""
    g = (d // 3) & ~1
    rest = d - 2 * g
    return (rest, g, g)


def positional_code(grid, d: int) -> np.ndarray:
    """[N, d] fp64 sin/cos code of the (t, h, w) coordinates of each token (raster order)."""
    T, Hg, Wg = grid
    n = np.arange(T * Hg * Wg)
    coords = (n // (Hg * Wg), (n // Wg) % Hg, n % Wg)
    lens = (T, Hg, Wg)
    pe = np.zeros((T * Hg * Wg, d), dtype=np.float64)
    col = 0
    for axis, width in enumerate(axis_groups(d)):
        npairs = width // 2
        lo, hi = 2.0, 4.0 * lens[axis]
        for f in range(npairs):
            period = lo * (hi / lo) ** (f / max(1, npairs - 1))
            ang = 2.0 * math.pi * coords[axis] / period
            pe[:, col] = np.sin(ang)
            pe[:, col + 1] = np.cos(ang)
            col += 2
    return pe


def _head_slice(x, b, h):
    return x[b, h]


def generate(w: Workload, with_do: bool = True, threads: int = 8):
    """Return dict of bf16 bit arrays (uint16, shape [B,H,N,d]) for q, k, v (and do)."""
    B, H, N, d = w.shape()
    total = B * H * N * d
    raw = {}
    names = ["q", "k", "v"] + (["do"] if with_do else [])
    for name in names:
        raw[name] = normals_parallel(w.seed, TENSOR_IDS[name], total, threads).reshape(B, H, N, d)
    rng = np.random.Generator(np.random.Philox(key=w.seed + 1000))
    if w.kind == "tiny":
        g = rng.standard_normal((d, 4))
        U, _ = np.linalg.qr(g)
        toks = rng.choice(N, size=4, replace=False)
        for r in range(4):
            raw["q"][:, :, toks[r], :] += 8.0 * U[:, r]
            raw["k"][:, :, toks[r], :] += 8.0 * U[:, r]
    else:
        pe = positional_code(w.grid, d)
        raw["q"] += w.alpha * pe
        raw["k"] += w.alpha * pe
        for b in range(B):
            for h in range(H):
                kk = raw["k"][b, h]
                rms = math.sqrt(float(np.mean(np.sum(kk * kk, axis=1))))
                stress_uniform = w.kind == "stress" and h < H // 2
                stress_sink = w.kind == "stress" and h >= H // 2
                if stress_uniform:
                    raw["q"][b, h] *= 0.1
                    sinks = rng.choice(N, size=w.n_sinks, replace=False)
                elif stress_sink:
                    # sink keys in key block 0 along a direction u that every query shares
                    u = rng.standard_normal(d)
                    u /= np.linalg.norm(u)
                    sinks = rng.choice(min(N, w.blk_k), size=w.n_sinks, replace=False)
                    kk[sinks] = w.sink_scale * rms * u
                    raw["q"][b, h] += STRESS_SINK_QUERY_GAIN * u
                    continue
                else:
                    sinks = rng.choice(N, size=w.n_sinks, replace=False)
                nrm = np.linalg.norm(kk[sinks], axis=1, keepdims=True)
                kk[sinks] *= (w.sink_scale * rms) / nrm
    return {name: to_bf16_bits(raw[name]) for name in names}
