"""CPU oracle for the VSA forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never uses it.

Thin ctypes binding over ``vsa_oracle.c`` (plain C, float64 arithmetic;
tile means are rounded once to FP32, the pooled-statistics precision the page
fixes).  Arrays are
numpy: bfloat16 tensors travel as ``uint16`` bit patterns, token-major
``[S, H, 128]``.  The method follows the page "UniServe: serving FastH3 at its
fastest" (sections "The FastH3 workload", "Fused attention preprocessing",
"Fused output combination", "Setup"); each C function states the passage it
implements and the reading taken where the page is open.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_vsa.so")
_lib = None

HEAD_DIM = 128
TILE = 64

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F64 = ctypes.c_double


def build() -> str:
    """Compile vsa_oracle.c (always recompiles).  No fused multiply-add
    contraction and no fast-math: the C source's float64 operations are the
    ones executed."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-o", _LIB_PATH, _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.vsa_oracle_topk_count.argtypes = [_I64, _F64]
        lib.vsa_oracle_topk_count.restype = _I32
        lib.vsa_oracle_pool.argtypes = [_P, _I32, _I64, _I64, _P]
        lib.vsa_oracle_pool.restype = None
        lib.vsa_oracle_row_scores.argtypes = [_P, _P, _I32, _I64, _I64, _P]
        lib.vsa_oracle_row_scores.restype = None
        lib.vsa_oracle_select_coarse.argtypes = [_P, _P, _P, _I32, _I64, _I64, _I64, _F64,
                                                 _P, _P, _P, _P, _P, _P, _P, ctypes.c_int]
        lib.vsa_oracle_select_coarse.restype = _I32
        lib.vsa_oracle_fine.argtypes = [_P, _P, _P, _P, _I32, _I64, _I64, _I64, _P, _I32, _P,
                                        _P, _I64, _P, _P, ctypes.c_int]
        lib.vsa_oracle_fine.restype = _I32
        lib.vsa_oracle_select_coarse_valid.argtypes = [_P, _P, _P, _I32, _I64, _I64, _I64, _I64,
                                                       _F64, _P, _P, _P, _P, _P, _P, _P,
                                                       ctypes.c_int]
        lib.vsa_oracle_select_coarse_valid.restype = _I32
        lib.vsa_oracle_fine_valid.argtypes = [_P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, _I64,
                                              _I64, _P, _I32, _P, _P, _I64, _P, _P, ctypes.c_int]
        lib.vsa_oracle_fine_valid.restype = _I32
        lib.vsa_oracle_pool_valid.argtypes = [_P, _I32, _I64, _I64, _I64, _P, ctypes.c_int]
        lib.vsa_oracle_pool_valid.restype = None
        lib.vsa_oracle_subblock_count.argtypes = [_I64, _F64]
        lib.vsa_oracle_subblock_count.restype = _I32
        lib.vsa_oracle_subblock_select.argtypes = [_P, _P, _I32, _I64, _I64, _I64, _F64, _P, _P,
                                                   _P, _P, _P, ctypes.c_int]
        lib.vsa_oracle_subblock_select.restype = _I32
        lib.vsa_oracle_subblock_select_rows.argtypes = [_P, _P, _I32, _I64, _I64, _I64, _F64, _P,
                                                        _I64, _P, _P, _P, _P, _P, ctypes.c_int]
        lib.vsa_oracle_subblock_select_rows.restype = _I32
        lib.vsa_oracle_subblock_select_whole.argtypes = [_P, _P, _I32, _I64, _I64, _I64, _F64,
                                                         _P, _P, _P, _P, _P, ctypes.c_int]
        lib.vsa_oracle_subblock_select_whole.restype = _I32
        lib.vsa_oracle_subblock_select_whole_rows.argtypes = [_P, _P, _I32, _I64, _I64, _I64,
                                                              _F64, _P, _I64, _P, _P, _P, _P, _P,
                                                              ctypes.c_int]
        lib.vsa_oracle_subblock_select_whole_rows.restype = _I32
        lib.vsa_oracle_fine_lists.argtypes = [_P, _P, _P, _I32, _I64, _P, _I32, _P, _I64, _P, _P,
                                              ctypes.c_int]
        lib.vsa_oracle_fine_lists.restype = _I32
        lib.vsa_oracle_bf16_from_f64.argtypes = [_F64]
        lib.vsa_oracle_bf16_from_f64.restype = ctypes.c_uint16
        lib.vsa_oracle_default_threads.argtypes = []
        lib.vsa_oracle_default_threads.restype = _I32
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _check_tensor(x: np.ndarray, s: int, h: int) -> np.ndarray:
    if x.dtype != np.uint16 or x.shape != (s, h, HEAD_DIM):
        raise ValueError(f"expected uint16 [{s},{h},{HEAD_DIM}], got {x.dtype} {x.shape}")
    return np.ascontiguousarray(x)


def frac_as_passed(frac: float) -> float:
    """The library takes topk_frac as a C float; the oracle widens that float."""
    return float(np.float32(frac))


def default_threads() -> int:
    return int(_load().vsa_oracle_default_threads())


def topk_count(n_v: int, frac: float) -> int:
    return int(_load().vsa_oracle_topk_count(n_v, frac_as_passed(frac)))


def bf16_from_f64(x: float) -> int:
    return int(_load().vsa_oracle_bf16_from_f64(float(x)))


def pool(x: np.ndarray, row0: int, n_tiles: int) -> np.ndarray:
    """FP32 tile means [H][n_tiles][128] of tiles starting at token row0."""
    x = np.ascontiguousarray(x)
    h = x.shape[1]
    out = np.empty((h, n_tiles, HEAD_DIM), dtype=np.float32)
    _load().vsa_oracle_pool(_ptr(x), h, row0, n_tiles, _ptr(out))
    return out


def row_scores(qbar: np.ndarray, kbar: np.ndarray, h: int, u: int) -> np.ndarray:
    n_v = qbar.shape[1]
    s = np.empty(n_v, dtype=np.float64)
    _load().vsa_oracle_row_scores(_ptr(np.ascontiguousarray(qbar)), _ptr(np.ascontiguousarray(kbar)),
                                  h, n_v, u, _ptr(s))
    return s


def select_coarse(q, k, v, text_len, video_len, audio_len, frac, want_scores=False,
                  threads=None, video_valid=None) -> dict:
    """Pooling, ranking, exact top-k and coarse branch for every (head, video
    query tile).  video_valid: valid rows at the start of the video segment
    (default all); tile means then cover valid rows only."""
    s = text_len + video_len + audio_len
    h = q.shape[1]
    q, k, v = (_check_tensor(x, s, h) for x in (q, k, v))
    n_v = video_len // TILE
    kk = topk_count(n_v, frac) if video_len % TILE == 0 else -1
    if kk < 0:
        raise ValueError("bad arguments")
    qbar = np.empty((h, n_v, HEAD_DIM), np.float32)
    kbar = np.empty_like(qbar)
    vbar = np.empty_like(qbar)
    sel = np.empty((h, n_v, kk), np.int32)
    coarse = np.empty((h, n_v, HEAD_DIM), np.float64)
    kth = np.empty((h, n_v), np.float64)
    scores = np.empty((h, n_v, n_v), np.float64) if want_scores else None
    r = _load().vsa_oracle_select_coarse_valid(
        _ptr(q), _ptr(k), _ptr(v), h, text_len, video_len, audio_len,
        video_len if video_valid is None else video_valid, frac_as_passed(frac),
        _ptr(qbar), _ptr(kbar), _ptr(vbar), _ptr(sel), _ptr(coarse), _ptr(kth), _ptr(scores),
        threads or 0)
    if r < 0:
        raise ValueError("bad arguments")
    return {"k": kk, "qbar": qbar, "kbar": kbar, "vbar": vbar, "sel": sel, "coarse": coarse,
            "kth": kth, "scores": scores}


def fine(q, k, v, gate, text_len, video_len, audio_len, sel, coarse, rows, threads=None,
         valid=None):
    """Rows `rows` of every head, on the given selection.  valid = (text,
    video, audio) valid rows at the start of each segment (default: all);
    padding rows are never keys and output zeros.  Returns (bfloat16 bits
    [n_rows][H][128], float64 [n_rows][H][128])."""
    s = text_len + video_len + audio_len
    h = q.shape[1]
    q, k, v, gate = (_check_tensor(x, s, h) for x in (q, k, v, gate))
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n_v = video_len // TILE
    sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(h, n_v, -1) if n_v else \
        np.zeros((h, 0, 0), np.int32)
    kk = sel.shape[2] if n_v else 0
    coarse = np.ascontiguousarray(coarse, dtype=np.float64).reshape(h, n_v, HEAD_DIM) if n_v else \
        np.zeros((h, 0, HEAD_DIM))
    out_b = np.empty((len(rows), h, HEAD_DIM), np.uint16)
    out_d = np.empty((len(rows), h, HEAD_DIM), np.float64)
    vt, vv, va = (text_len, video_len, audio_len) if valid is None else valid
    r = _load().vsa_oracle_fine_valid(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), h, text_len,
                                      video_len, audio_len, vt, vv, va, _ptr(sel), kk,
                                      _ptr(coarse), _ptr(rows), len(rows), _ptr(out_b),
                                      _ptr(out_d), threads or 0)
    if r < 0:
        raise ValueError("bad arguments")
    return out_b, out_d


def forward(q, k, v, gate, text_len, video_len, audio_len, frac, rows=None, threads=None) -> dict:
    """The whole path: selection, coarse, fine and combination (all rows by default)."""
    sc = select_coarse(q, k, v, text_len, video_len, audio_len, frac, threads=threads)
    s = text_len + video_len + audio_len
    if rows is None:
        rows = np.arange(s, dtype=np.int64)
    out_b, out_d = fine(q, k, v, gate, text_len, video_len, audio_len, sc["sel"], sc["coarse"],
                        rows, threads=threads)
    sc.update({"rows": np.asarray(rows), "out": out_b, "out_f64": out_d})
    return sc


def project_rows(x: np.ndarray, w: np.ndarray, rows) -> np.ndarray:
    """The Q, K, V and gate projections of selected token rows, float64:
    out[p][i][n] = sum over c of x[rows[i]][c] * w[p][n][c].

    Page "UniServe: serving FastH3 at its fastest", section "The FastH3
    workload": hidden size 5,376 and 56 heads of 128, so each projection maps
    5,376 channels to 7,168 (weights stored out x in).  x is bfloat16 bits
    [tokens][hidden], w bfloat16 bits [4][out][hidden]; both are widened
    exactly to float64 and multiplied with numpy's matrix product (every
    product of two bfloat16 values is exact in float64).  Returns float64
    [4][len(rows)][out]; the GPU result is this value rounded to bfloat16
    after fp32 accumulation."""
    rows = np.asarray(rows, dtype=np.int64)
    xr = (x[rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    out = np.empty((4, len(rows), w.shape[1]), dtype=np.float64)
    for p in range(4):
        wp = (w[p].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        out[p] = xr @ wp.T
    return out


# ---------------------------------------------------------------------------
# Attention preprocessing: Q/K RMSNorm and partial 3D RoPE
# ---------------------------------------------------------------------------

RMS_EPS = 1e-6
ROPE_DIM = 96          # rotated dimensions per head (32 per grid axis)
ROPE_BASE = 10000.0


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bits, one rounding to nearest with ties to even.
    Values in the normal range are rounded in the float64 bit pattern (bit 45
    of the fraction is bfloat16's last kept bit); the rest (bfloat16
    subnormals, zero, non-finite) go through vsa_oracle_bf16_from_f64, which
    the pins also compare against on random values."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    u = x.view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    r = (u + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    out = (r.view(np.float64).astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    a = np.abs(x)
    odd = ~((a >= 2.0 ** -126) & (a < 2.0 ** 127))
    if odd.any():
        f = _load().vsa_oracle_bf16_from_f64
        idx = np.flatnonzero(odd)
        flat = out.reshape(-1)
        for i in idx:
            flat[i] = f(float(x.reshape(-1)[i]))
    return out


def _widen(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def video_positions(grid, tile, video_valid: int) -> np.ndarray:
    """(t, h, w) latent-grid coordinates of video tokens 0 .. video_valid-1 in
    tile-packed order: tiles of pt x ph x pw grid points in raster order over
    the tile grid, points in raster order inside a tile."""
    T_, Hh, Ww = grid
    pt, ph, pw = tile
    i = np.arange(video_valid, dtype=np.int64)
    pts = pt * ph * pw
    tile_id, off = i // pts, i % pts
    nth, ntw = Hh // ph, Ww // pw
    tt, th, tw = tile_id // (nth * ntw), (tile_id // ntw) % nth, tile_id % ntw
    ot, oh, ow = off // (ph * pw), (off // pw) % ph, off % pw
    return np.stack([tt * pt + ot, th * ph + oh, tw * pw + ow], axis=1)


def rms_norm_rope(x: np.ndarray, gamma: np.ndarray, text_len, video_len, audio_len, valid,
                  grid, tile, rows=None) -> np.ndarray:
    """Learned RMSNorm and partial 3D RoPE of Q or K, float64, as bfloat16 bits.

    Page "UniServe: serving FastH3 at its fastest", section "Fused attention
    preprocessing": the attention inputs go through a learned Q/K RMSNorm and
    a partial RoPE before tile pooling; the SGLang Diffusion benchmark page
    gives RoPE dimension 96 of the 128 and the exact-rounding order
    (normalised values rounded before RoPE).  Readings where the pages are
    silent: the norm is per head over its 128 dims,
        y = x / sqrt(mean(x^2) + 1e-6) * gamma[h],  rounded to bfloat16;
    RoPE rotates dims 0..95 of video tokens only (text and audio carry no
    latent-grid position): axis a in (t, h, w) owns dims 32a .. 32a+31 as 16
    interleaved pairs (2i, 2i+1) turned by pos_a * 10000^(-i/16),
        (y0, y1) -> (y0 cos - y1 sin, y0 sin + y1 cos),
    then rounded to bfloat16 again.  Padding rows (past each segment's valid
    count) become zeros.

    x: bfloat16 bits [S][H][128]; gamma: bfloat16 bits [H][128];
    valid = (text, video, audio) valid rows; grid, tile as in
    video_positions; rows: token rows to return (default all).  Returns
    bfloat16 bits [len(rows)][H][128]."""
    S, H, Dh = x.shape
    rows = np.arange(S, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    xf = _widen(x[rows])
    ms = (xf ** 2).mean(axis=2, keepdims=True)
    yb = _widen(bf16_round(xf / np.sqrt(ms + RMS_EPS) * _widen(gamma)[None, :, :]))
    vt, vv, va = valid
    is_video = (rows >= text_len) & (rows < text_len + vv)
    vid = np.flatnonzero(is_video)
    if len(vid):
        pos_all = video_positions(grid, tile, vv)
        pos = pos_all[rows[vid] - text_len]
        seg = yb[vid]
        per_axis = ROPE_DIM // 3
        half = per_axis // 2
        inv = ROPE_BASE ** (-np.arange(half, dtype=np.float64) / half)
        out = seg.copy()
        for a in range(3):
            ang = pos[:, a:a + 1].astype(np.float64) * inv[None, :]      # [n][16]
            c, s_ = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
            d0 = per_axis * a + 2 * np.arange(half)
            x0, x1 = seg[:, :, d0], seg[:, :, d0 + 1]
            out[:, :, d0] = x0 * c - x1 * s_
            out[:, :, d0 + 1] = x0 * s_ + x1 * c
        yb[vid] = out
    res = bf16_round(yb)
    tok = (rows < vt) | is_video | ((rows >= text_len + video_len) & (rows < text_len + video_len + va))
    res[~tok] = 0
    return res


# ---------------------------------------------------------------------------
# SubBlock router (the C functions state the passage and the readings)
# ---------------------------------------------------------------------------

def subblock_count(n_v: int, sparsity: float) -> int:
    """Kept video tiles per row: 8 * floor((1 - sparsity) * n_v / 8 + 1/2),
    clamped to [min(8, n_v), n_v]; -1 for sparsity outside [0, 1).  The
    sparsity is the C float the library receives, widened."""
    return int(_load().vsa_oracle_subblock_count(n_v, frac_as_passed(sparsity)))


def subblock_select(q, k, text_len, video_len, audio_len, sparsity, want_scores=False,
                    threads=None) -> dict:
    s = text_len + video_len + audio_len
    h = q.shape[1]
    q, k = (_check_tensor(x, s, h) for x in (q, k))
    n_v = video_len // TILE
    kk = subblock_count(n_v, sparsity)
    if kk < 0 or video_len % TILE:
        raise ValueError("bad arguments")
    qsub = np.empty((h, n_v, 4, HEAD_DIM), np.float32)
    ksub = np.empty_like(qsub)
    sel = np.empty((h, n_v, kk), np.int32)
    kth = np.empty((h, n_v), np.float64)
    scores = np.empty((h, n_v, n_v), np.float64) if want_scores else None
    r = _load().vsa_oracle_subblock_select(_ptr(q), _ptr(k), h, text_len, video_len, audio_len,
                                           frac_as_passed(sparsity), _ptr(qsub), _ptr(ksub),
                                           _ptr(sel), _ptr(kth), _ptr(scores), threads or 0)
    if r < 0:
        raise ValueError("bad arguments")
    return {"k": kk, "qsub": qsub, "ksub": ksub, "sel": sel, "kth": kth, "scores": scores}


def subblock_select_rows(q, k, text_len, video_len, audio_len, sparsity, rows, threads=None) -> dict:
    """subblock_select for the (head, video tile) rows listed as pairs; the
    sub-block means cover every tile.  Returns qsub, ksub [H][n_v][4][128],
    sel [n][k], kth [n], scores [n][n_v]."""
    s = text_len + video_len + audio_len
    h = q.shape[1]
    q, k = (_check_tensor(x, s, h) for x in (q, k))
    n_v = video_len // TILE
    kk = subblock_count(n_v, sparsity)
    if kk < 0 or video_len % TILE:
        raise ValueError("bad arguments")
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
    flat = np.ascontiguousarray(rows[:, 0] * n_v + rows[:, 1])
    n = len(flat)
    qsub = np.empty((h, n_v, 4, HEAD_DIM), np.float32)
    ksub = np.empty_like(qsub)
    sel = np.empty((n, kk), np.int32)
    kth = np.empty(n, np.float64)
    scores = np.empty((n, n_v), np.float64)
    r = _load().vsa_oracle_subblock_select_rows(_ptr(q), _ptr(k), h, text_len, video_len,
                                                audio_len, frac_as_passed(sparsity), _ptr(flat), n,
                                                _ptr(qsub), _ptr(ksub), _ptr(sel), _ptr(kth),
                                                _ptr(scores), threads or 0)
    if r < 0:
        raise ValueError("bad arguments")
    return {"k": kk, "qsub": qsub, "ksub": ksub, "sel": sel, "kth": kth, "scores": scores}


def subblock_select_whole(q, k, text_len, video_len, audio_len, sparsity, want_scores=False,
                          threads=None) -> dict:
    """The SubBlock router over the whole sequence: every one of the N tiles
    is a query tile and a candidate key tile.  Returns qsub, ksub [H][N][4][128],
    sel [H][N][k] (global tile indices, ascending), kth [H][N] and, when asked,
    scores [H][N][N]; k = subblock_count(N, sparsity)."""
    s = text_len + video_len + audio_len
    h = q.shape[1]
    q, k = (_check_tensor(x, s, h) for x in (q, k))
    n = s // TILE
    kk = subblock_count(n, sparsity)
    if kk < 0 or s % TILE or text_len % TILE or video_len % TILE:
        raise ValueError("bad arguments")
    qsub = np.empty((h, n, 4, HEAD_DIM), np.float32)
    ksub = np.empty_like(qsub)
    sel = np.empty((h, n, kk), np.int32)
    kth = np.empty((h, n), np.float64)
    scores = np.empty((h, n, n), np.float64) if want_scores else None
    r = _load().vsa_oracle_subblock_select_whole(_ptr(q), _ptr(k), h, text_len, video_len,
                                                 audio_len, frac_as_passed(sparsity), _ptr(qsub),
                                                 _ptr(ksub), _ptr(sel), _ptr(kth), _ptr(scores),
                                                 threads or 0)
    if r < 0:
        raise ValueError("bad arguments")
    return {"k": kk, "qsub": qsub, "ksub": ksub, "sel": sel, "kth": kth, "scores": scores}


def subblock_select_whole_rows(q, k, text_len, video_len, audio_len, sparsity, rows,
                               threads=None) -> dict:
    """subblock_select_whole for the (head, tile) rows listed as pairs."""
    s = text_len + video_len + audio_len
    h = q.shape[1]
    q, k = (_check_tensor(x, s, h) for x in (q, k))
    n = s // TILE
    kk = subblock_count(n, sparsity)
    if kk < 0 or s % TILE:
        raise ValueError("bad arguments")
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
    flat = np.ascontiguousarray(rows[:, 0] * n + rows[:, 1])
    m = len(flat)
    qsub = np.empty((h, n, 4, HEAD_DIM), np.float32)
    ksub = np.empty_like(qsub)
    sel = np.empty((m, kk), np.int32)
    kth = np.empty(m, np.float64)
    scores = np.empty((m, n), np.float64)
    r = _load().vsa_oracle_subblock_select_whole_rows(
        _ptr(q), _ptr(k), h, text_len, video_len, audio_len, frac_as_passed(sparsity), _ptr(flat),
        m, _ptr(qsub), _ptr(ksub), _ptr(sel), _ptr(kth), _ptr(scores), threads or 0)
    if r < 0:
        raise ValueError("bad arguments")
    return {"k": kk, "qsub": qsub, "ksub": ksub, "sel": sel, "kth": kth, "scores": scores}


def fine_lists(q, k, v, lists, rows, threads=None):
    """Rows `rows` of every head, each query tile j attending to the keys of
    its own key tiles lists[h][j] ([H][N][k], global indices); no coarse term,
    no gate.  Returns (bfloat16 bits [n_rows][H][128], float64 [n_rows][H][128])."""
    s, h = q.shape[0], q.shape[1]
    q, k, v = (_check_tensor(x, s, h) for x in (q, k, v))
    lists = np.ascontiguousarray(lists, dtype=np.int32)
    if lists.ndim != 3 or lists.shape[:2] != (h, s // TILE):
        raise ValueError("lists must be [H][N][k]")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out_b = np.empty((len(rows), h, HEAD_DIM), np.uint16)
    out_d = np.empty((len(rows), h, HEAD_DIM), np.float64)
    r = _load().vsa_oracle_fine_lists(_ptr(q), _ptr(k), _ptr(v), h, s, _ptr(lists),
                                      lists.shape[2], _ptr(rows), len(rows), _ptr(out_b),
                                      _ptr(out_d), threads or 0)
    if r < 0:
        raise ValueError("bad arguments")
    return out_b, out_d
