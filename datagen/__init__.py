"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only *makes inputs*.  It holds none of the normalisation or
rotation arithmetic, imports neither the oracle nor the HIP library, and both
of those consume its arrays as plain data.

Random numbers: a counter-based SplitMix64 (Steele, Lea and Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014; the 64-bit finaliser
with constants 0xBF58476D1CE4E5B9 / 0x94D049BB133111EB and increment
0x9E3779B97F4A7C15).  Element i of stream (seed, stream_id) is
``mix(key + (i + 1) * golden)`` with ``key = mix(mix(seed) ^ stream_id *
0xD1B54A32D192ED03)``, so any element can be produced on its own and the
result does not depend on chunking.

 - uniform(0,1):  (z >> 11) * 2^-53, an exact 0 replaced by 2^-54;
 - normal(0,1):   Box-Muller on the uniform pair (2k, 2k+1):
                  r = sqrt(-2 ln u1); n[2k] = r cos(2 pi u2), n[2k+1] = r sin(2 pi u2);
 - bf16 values:   the double is rounded to binary32 and then to bf16 with
                  round-to-nearest-even, as a framework cast does; arrays
                  carry the bf16 bit patterns as uint16.

Workload recipes (shapes and distributions of the pages' micro-benchmark
shapes, see ``CONFIGS``) use base seed 1234 and stream ids x = 1, w = 2,
outlier mask = 3, each offset by ``config_id << 8``.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)
_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_C1 = np.uint64(0xBF58476D1CE4E5B9)
_C2 = np.uint64(0x94D049BB133111EB)
_STREAM_MUL = 0xD1B54A32D192ED03
_CHUNK = 1 << 22

BASE_SEED = 1234
STREAM_X, STREAM_W, STREAM_OUTLIER = 1, 2, 3


def _mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output finaliser on uint64 arrays (wrapping arithmetic)."""
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _C1
        z = (z ^ (z >> np.uint64(27))) * _C2
        return z ^ (z >> np.uint64(31))


def _mix_int(v: int) -> int:
    return int(_mix(np.array([v & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64))[0])


def stream_key(seed: int, stream: int) -> int:
    return _mix_int(_mix_int(seed) ^ ((stream * _STREAM_MUL) & 0xFFFFFFFFFFFFFFFF))


def raw_u64(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Elements start .. start+count-1 of the stream as uint64."""
    key = np.uint64(stream_key(seed, stream))
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(key + idx * _GOLDEN)


def uniform(seed: int, stream: int, n: int, start: int = 0) -> np.ndarray:
    """n doubles in (0, 1)."""
    out = np.empty(n, dtype=np.float64)
    for s in range(0, n, _CHUNK):
        c = min(_CHUNK, n - s)
        z = raw_u64(seed, stream, start + s, c)
        u = (z >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
        u[u == 0.0] = 2.0 ** -54
        out[s:s + c] = u
    return out


def normal(seed: int, stream: int, n: int) -> np.ndarray:
    """n standard normal doubles (Box-Muller on consecutive uniform pairs)."""
    pairs = (n + 1) // 2
    out = np.empty(2 * pairs, dtype=np.float64)
    step = _CHUNK // 2
    for k in range(0, pairs, step):
        c = min(step, pairs - k)
        u = uniform(seed, stream, 2 * c, start=2 * k)
        r = np.sqrt(-2.0 * np.log(u[0::2]))
        t = 2.0 * np.pi * u[1::2]
        out[2 * k:2 * (k + c):2] = r * np.cos(t)
        out[2 * k + 1:2 * (k + c):2] = r * np.sin(t)
    return out[:n]


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """double -> binary32 (numpy cast, round-to-nearest-even) -> bf16 bit
    pattern (round-to-nearest-even on the 16 dropped bits).  Inputs are finite
    synthetic values; no NaN handling is needed here."""
    v = np.asarray(v)
    flat = v.reshape(-1)
    out = np.empty(flat.size, dtype=np.uint16)
    for s in range(0, flat.size, _CHUNK):
        u = flat[s:s + _CHUNK].astype(np.float32).view(np.uint32)
        high = u >> np.uint32(16)
        low = u & np.uint32(0xFFFF)
        up = (low > 0x8000) | ((low == 0x8000) & ((high & np.uint32(1)) == 1))
        out[s:s + _CHUNK] = (high + up).astype(np.uint16)
    return out.reshape(v.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to binary32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def rope_tables(seq_len: int, head_dim: int, theta: float = 10000.0,
                positions: np.ndarray | None = None):
    """binary32 cos/sin tables [len(positions), head_dim/2] for positions
    0..seq_len-1 (or the given ones): angle = p * theta^(-2i/head_dim),
    evaluated in double and rounded once to binary32.  These tables are an
    input of the rotation, prepared here the way a model prepares them."""
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = np.exp(-(2.0 * i / head_dim) * np.log(theta))
    p = np.arange(seq_len, dtype=np.float64) if positions is None else np.asarray(positions, dtype=np.float64)
    ang = p[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rope_tables_3d(frames: int, height: int, width: int, head_dim: int, theta: float = 10000.0):
    """binary32 cos/sin tables with one row per video token of a
    [frames x height x width] grid, flattened t-major ([batch, t*h*w, heads,
    head_dim] layout).  The pages give the layout but not how the three
    coordinates share the head_dim/2 rotation slots; this synthetic recipe
    assigns slot i to axis i mod 3 (t, h, w) with frequency
    theta^(-2 * (i // 3) / head_dim) applied to that axis' coordinate.  The
    rotation kernels treat tables as data, so any recipe exercises them."""
    half = head_dim // 2
    i = np.arange(half)
    axis = i % 3
    inv_freq = np.exp(-(2.0 * (i // 3) / head_dim) * np.log(theta))
    t, h, w = np.meshgrid(np.arange(frames), np.arange(height), np.arange(width), indexing="ij")
    coords = np.stack([t.reshape(-1), h.reshape(-1), w.reshape(-1)], axis=1).astype(np.float64)
    ang = coords[:, axis] * inv_freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def fnv1a64(a: np.ndarray) -> str:
    """64-bit FNV-1a of the array's bytes (hex), recorded next to results."""
    data = np.ascontiguousarray(a).view(np.uint8)
    h = 0xCBF29CE484222325
    # FNV-1a on a digest keeps this fast for 100 MB tensors while still
    # depending on every byte: hash the SHA-256 of the bytes.
    for byte in hashlib.sha256(data.tobytes()).digest():
        h = ((h ^ byte) * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return "%016x" % h


@dataclass(frozen=True)
class Config:
    """One workload: x ~ N(0, sigma) [rows, hidden] (optionally with each
    element independently scaled by ``outlier_scale`` with probability
    ``outlier_p``), weight ~ U(0.5, 1.5) [hidden], eps, and for RoPE the head
    split, the table length and theta."""
    name: str
    config_id: int
    batch: int
    seq: int
    hidden: int
    sigma: float = 1.0
    outlier_p: float = 0.0
    outlier_scale: float = 1.0
    eps: float = 1e-6
    heads: int = 0
    head_dim: int = 0
    theta: float = 10000.0
    interleaved: bool = False  # RoPE pairing: rotate-half (False) or adjacent pairs
    adaln_sigma: float = 0.0   # > 0: per-sample scale and shift ~ N(0, adaln_sigma), [batch, hidden]

    @property
    def rows(self) -> int:
        return self.batch * self.seq

    @property
    def rope(self) -> bool:
        return self.heads > 0

    @property
    def adaln(self) -> bool:
        return self.adaln_sigma > 0

    def algorithmic_bytes(self, elem_bytes: int = 2) -> int:
        """Bytes the op must move at least once: read x, write y, read the
        weight once (elements of `elem_bytes`: 2 for bf16/fp16, 4 for fp32);
        for RoPE also both binary32 tables once; for AdaLN the per-sample
        scale and shift rows once."""
        e = elem_bytes
        b = 2 * self.rows * self.hidden * e + self.hidden * e
        if self.rope:
            b += 2 * self.seq * (self.head_dim // 2) * 4
        if self.adaln:
            b += 2 * self.batch * self.hidden * e
        return b


# The pages' micro-benchmark shapes ([B x S x H] bf16, Hugging Face cuda-kernels
# skill page, section "RMSNorm Micro-benchmarks") and the fused RMSNorm+RoPE
# workload (32 heads x 64, positions 0..4095, theta 10000).
CONFIGS = {
    "rms_1x1024x2048": Config("rms_1x1024x2048", 1, 1, 1024, 2048),
    "rms_2x1024x2048": Config("rms_2x1024x2048", 2, 2, 1024, 2048),
    "rms_4x1024x2048": Config("rms_4x1024x2048", 3, 4, 1024, 2048),
    "rms_2x4096x3072_outliers": Config("rms_2x4096x3072_outliers", 4, 2, 4096, 3072,
                                       sigma=2.0, outlier_p=0.01, outlier_scale=50.0),
    "rms_4x4096x3072": Config("rms_4x4096x3072", 5, 4, 4096, 3072),
    "rope_2x4096x2048_h32d64": Config("rope_2x4096x2048_h32d64", 6, 2, 4096, 2048,
                                      heads=32, head_dim=64, theta=10000.0),
    "ropei_2x4096x2048_h32d64": Config("ropei_2x4096x2048_h32d64", 7, 2, 4096, 2048,
                                       heads=32, head_dim=64, theta=10000.0, interleaved=True),
    "adaln_2x4096x2048": Config("adaln_2x4096x2048", 8, 2, 4096, 2048, adaln_sigma=0.25),
}
# Shapes outside the pages' set that exercise the kernels for rows of any
# length, with the same value recipe: a hidden size that is not a whole number
# of 16-byte vectors, a head size the vector kernels cannot pair (16 heads x
# 72, rotate-half), rows longer than the register budget, rows of one head
# (per-head normalisation), and AdaLN rows of 144 vectors.
GENERAL_CONFIGS = {
    "rms_4x4096x3076": Config("rms_4x4096x3076", 9, 4, 4096, 3076),
    "rope_2x4096x1152_h16d72": Config("rope_2x4096x1152_h16d72", 10, 2, 4096, 1152,
                                      heads=16, head_dim=72, theta=10000.0),
    # rows past the register budget in whole rounds of the two-pass kernel:
    # 512 rows of 131072 (8 chunks of 2048 vectors each)
    "rms_1x512x131072": Config("rms_1x512x131072", 11, 1, 512, 131072),
    # per-head normalisation (query/key norm): rows of one 128-element head,
    # [2 x 4096 x 24 heads] of them
    "rms_2x4096x24_d128": Config("rms_2x4096x24_d128", 12, 2, 4096 * 24, 128),
    # AdaLN at hidden 1152 (the PixArt size), rows of 144 vectors that
    # several rows share a wavefront for
    "adaln_8x4096x1152": Config("adaln_8x4096x1152", 16, 8, 4096, 1152, adaln_sigma=0.25),
    # a few very long rows: 64 rows of 2^20, each cut into 64 chunks
    "rms_1x64x1048576": Config("rms_1x64x1048576", 17, 1, 64, 1 << 20),
}
# The fused operations at the headline's size ([4 x 4096 x 3072]), large
# enough that the launch floor no longer sets their rate: RoPE with 24 heads
# of 128 in both pairings, and AdaLN with per-sample rows [4 x 3072].
LARGE_CONFIGS = {
    "rope_4x4096x3072_h24d128": Config("rope_4x4096x3072_h24d128", 13, 4, 4096, 3072,
                                       heads=24, head_dim=128, theta=10000.0),
    "ropei_4x4096x3072_h24d128": Config("ropei_4x4096x3072_h24d128", 14, 4, 4096, 3072,
                                        heads=24, head_dim=128, theta=10000.0, interleaved=True),
    "adaln_4x4096x3072": Config("adaln_4x4096x3072", 15, 4, 4096, 3072, adaln_sigma=0.25),
}
HEADLINE = "rms_4x4096x3072"
ROPE = "rope_2x4096x2048_h32d64"
ROPE_INTERLEAVED = "ropei_2x4096x2048_h32d64"
ADALN = "adaln_2x4096x2048"
STREAM_SCALE, STREAM_SHIFT = 4, 5


def encode(v: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """Doubles as inputs of the given type: bf16 bit patterns (uint16), or
    float16 / float32 arrays (numpy's round-to-nearest-even cast)."""
    if dtype == "bf16":
        return to_bf16_bits(v)
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return np.asarray(v).astype(np.float16)
    if dtype == "f32":
        return np.asarray(v).astype(np.float32)
    raise ValueError(dtype)


def make_x(rows: int, hidden: int, seed: int = BASE_SEED, stream: int = STREAM_X,
           sigma: float = 1.0, outlier_p: float = 0.0, outlier_scale: float = 1.0,
           outlier_stream: int = STREAM_OUTLIER, dtype: str = "bf16") -> np.ndarray:
    n = rows * hidden
    v = normal(seed, stream, n) * sigma
    if outlier_p > 0.0:
        mask = uniform(seed, outlier_stream, n) < outlier_p
        v[mask] *= outlier_scale
    return encode(v, dtype).reshape(rows, hidden)


def make_w(hidden: int, seed: int = BASE_SEED, stream: int = STREAM_W, dtype: str = "bf16") -> np.ndarray:
    return encode(0.5 + uniform(seed, stream, hidden), dtype)


def make_inputs(cfg: Config, seed: int = BASE_SEED, rows: int | None = None,
                dtype: str = "bf16") -> dict:
    """Inputs for a workload in the given I/O type ("bf16", "f16", "f32");
    ``rows`` < cfg.rows gives the leading rows only (the same values the
    full workload has there)."""
    off = cfg.config_id << 8
    r = cfg.rows if rows is None else rows
    x = make_x(r, cfg.hidden, seed, off | STREAM_X, cfg.sigma, cfg.outlier_p,
               cfg.outlier_scale, off | STREAM_OUTLIER, dtype=dtype)
    w = make_w(cfg.hidden, seed, off | STREAM_W, dtype=dtype)
    out = {"x": x, "w": w, "eps": cfg.eps}
    if cfg.adaln:
        out.update(scale=make_x(cfg.batch, cfg.hidden, seed, off | STREAM_SCALE, cfg.adaln_sigma,
                                dtype=dtype),
                   shift=make_x(cfg.batch, cfg.hidden, seed, off | STREAM_SHIFT, cfg.adaln_sigma,
                                dtype=dtype),
                   rows_per_sample=cfg.seq)
    if cfg.rope:
        cos_t, sin_t = rope_tables(cfg.seq, cfg.head_dim, cfg.theta)
        out.update(cos=cos_t, sin=sin_t, heads=cfg.heads, head_dim=cfg.head_dim,
                   interleaved=cfg.interleaved)
    return out
