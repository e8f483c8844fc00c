"""Seeded synthetic inputs shared by the GPU library's tests/bench and the CPU oracle.

Holds no arithmetic of the attention method: it draws counter-based normal
deviates (SplitMix64 + Box-Muller, defined in ``gen.c``) and rounds them to
bfloat16 bit patterns (``numpy.uint16``).  Tensor *stream ids* keep the
tensors independent: Q = 0, K = 1, V = 2, gate = 3 (further ids are free for
other tensors).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

STREAM_Q, STREAM_K, STREAM_V, STREAM_GATE = 0, 1, 2, 3
STREAM_X, STREAM_W0, STREAM_FIELD = 4, 5, 9   # hidden states; W_q..W_gate = 5..8; video noise
HEAD_DIM = 128


def build() -> str:
    """Compile gen.c into libsynth.so (always recompiles)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-o", _LIB_PATH, _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_double, ctypes.c_double,
                                          ctypes.c_void_p, ctypes.c_int]
        lib.synth_normal_bf16.restype = None
        lib.synth_normal_f64.argtypes = lib.synth_normal_bf16.argtypes
        lib.synth_normal_f64.restype = None
        lib.synth_smooth_field_bf16.argtypes = [
            ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
        lib.synth_smooth_field_bf16.restype = None
        lib.synth_splitmix64.argtypes = [ctypes.c_uint64]
        lib.synth_splitmix64.restype = ctypes.c_uint64
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


def normal_bf16(seed: int, stream: int, shape, mean: float = 0.0, std: float = 1.0,
                offset: int = 0, threads: int | None = None) -> np.ndarray:
    """Row-major array of bfloat16 bit patterns drawn from N(mean, std^2)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    if n:
        _load().synth_normal_bf16(seed, stream, offset, n, mean, std,
                                  out.ctypes.data, threads or default_threads())
    return out.reshape(shape)


def normal_f64(seed: int, stream: int, shape, mean: float = 0.0, std: float = 1.0,
               offset: int = 0, threads: int | None = None) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float64)
    if n:
        _load().synth_normal_f64(seed, stream, offset, n, mean, std,
                                 out.ctypes.data, threads or default_threads())
    return out.reshape(shape)


def splitmix64(x: int) -> int:
    return int(_load().synth_splitmix64(x))


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest even (finite values)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def vsa_inputs(seed: int, heads: int, text_len: int, video_len: int, audio_len: int,
               std: float = 1.0, threads: int | None = None) -> dict:
    """Q, K, V, gate as bfloat16 bits, token-major [S, heads, 128], iid N(0, std^2)."""
    s = text_len + video_len + audio_len
    shape = (s, heads, HEAD_DIM)
    return {
        "q": normal_bf16(seed, STREAM_Q, shape, std=std, threads=threads),
        "k": normal_bf16(seed, STREAM_K, shape, std=std, threads=threads),
        "v": normal_bf16(seed, STREAM_V, shape, std=std, threads=threads),
        "gate": normal_bf16(seed, STREAM_GATE, shape, std=std, threads=threads),
    }


def smooth_field_bf16(seed: int, grid, channels: int, sigma=(1.0, 2.0, 2.0), tile=(2, 8, 4),
                      out: np.ndarray | None = None, threads: int | None = None) -> np.ndarray:
    """Video rows of the full-layer workload: per channel, white noise over
    the (T, H, W) latent grid, a separable Gaussian blur (sigma in grid cells,
    half-sample symmetric boundary), scaled to unit root mean square, in
    tile-packed token order (gen.c states the exact definition).  Returns
    bfloat16 bits [T*H*W, channels], or fills `out` (rows of that shape)."""
    T, Hh, Ww = grid
    pt, ph, pw = tile
    if T % pt or Hh % ph or Ww % pw:
        raise ValueError("grid must be a whole number of tiles")
    n = T * Hh * Ww
    if out is None:
        out = np.empty((n, channels), dtype=np.uint16)
    if out.shape != (n, channels) or out.dtype != np.uint16 or not out.flags.c_contiguous:
        raise ValueError("out must be a contiguous uint16 [T*H*W, channels] array")
    _load().synth_smooth_field_bf16(seed, STREAM_FIELD, T, Hh, Ww, channels, *[float(x) for x in sigma],
                                    pt, ph, pw, out.ctypes.data, channels,
                                    threads or default_threads())
    return out


def full_layer_inputs(seed: int, text_len: int, grid, audio_len: int, hidden: int, heads: int,
                      sigma=(1.0, 2.0, 2.0), tile=(2, 8, 4), w_std: float = 0.02,
                      threads: int | None = None) -> dict:
    """Hidden states and projection weights of one attention layer:
    x [text | video | audio, hidden] with text and audio rows iid N(0, 1)
    (stream 4, element index row * hidden + c) and video rows the smooth field
    above; w [4, heads*128, hidden] iid N(0, w_std^2), projection p from
    stream 5 + p.  All bfloat16 bits."""
    T, Hh, Ww = grid
    s_v = T * Hh * Ww
    s = text_len + s_v + audio_len
    x = np.empty((s, hidden), dtype=np.uint16)
    if text_len:
        x[:text_len] = normal_bf16(seed, STREAM_X, (text_len, hidden), threads=threads)
    smooth_field_bf16(seed, grid, hidden, sigma, tile, out=x[text_len:text_len + s_v], threads=threads)
    if audio_len:
        off = (text_len + s_v) * hidden
        x[text_len + s_v:] = normal_bf16(seed, STREAM_X, (audio_len, hidden), offset=off,
                                         threads=threads)
    n_out = heads * HEAD_DIM
    w = np.empty((4, n_out, hidden), dtype=np.uint16)
    for p in range(4):
        w[p] = normal_bf16(seed, STREAM_W0 + p, (n_out, hidden), std=w_std, threads=threads)
    return {"x": x, "w": w}
