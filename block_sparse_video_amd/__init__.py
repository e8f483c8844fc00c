"""MI355X (gfx950) video sparse attention (VSA) forward.

Python face of ``libvsa.so`` (C ABI in ``include/vsa.h``), with the same entry
point names.  Tensors are torch tensors used as device memory only: q, k, v,
gate and out are bfloat16 ``[S, H, 128]`` contiguous on the current GPU,
selected_tiles is int32 ``[H, n_v, k]``, workspace is a uint8 tensor of at
least ``vsa_workspace_bytes(...)`` bytes.  Every call enqueues on torch's
current stream unless ``stream`` (a raw hipStream_t handle) is given.
"""
from __future__ import annotations

import ctypes

from ._native import LIB_PATH, VsaError, load, status_string  # noqa: F401

HEAD_DIM = 128
TILE = 64

__all__ = ["vsa_topk_count", "vsa_workspace_bytes", "vsa_workspace_layout", "vsa_forward",
           "vsa_pool_pack", "vsa_select_coarse", "vsa_fine_attention", "forward", "VsaError",
           "status_string", "LIB_PATH", "vsa_subblock_count", "vsa_subblock_workspace_bytes",
           "vsa_forward_subblock", "vsa_subblock_select", "forward_subblock",
           "vsa_forward_noalloc", "vsa_subblock_whole_workspace_bytes",
           "vsa_forward_subblock_whole", "vsa_subblock_select_whole", "forward_subblock_whole"]


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise VsaError(status, where)


def _tensor(t, name, dtype, shape=None):
    """Check one tensor argument's type, dtype, shape and layout (None passes
    through).  Every wrapper checks all its arguments this way, then calls
    _on_gpu on them, before anything reaches the library."""
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _on_gpu(**tensors):
    """Every given tensor must be device memory: a host pointer handed to a
    kernel would fault the GPU."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA (HIP) torch tensor")


def _selection(t, num_heads, video_len, k, name="selected_tiles"):
    """selected_tiles is int32 [H][n_v][k].  When k is not a valid count the
    shape is left to the library, which returns the matching status."""
    torch = _torch()
    if k is None or k < 0:
        return _tensor(t, name, torch.int32)
    return _tensor(t, name, torch.int32, (num_heads, video_len // TILE, k))


def vsa_topk_count(video_len: int, topk_frac: float) -> int:
    return int(load().vsa_topk_count(video_len, topk_frac))


def vsa_workspace_bytes(num_heads: int, text_len: int, video_len: int, audio_len: int,
                        topk_frac: float = 0.2) -> int:
    return int(load().vsa_workspace_bytes(num_heads, text_len, video_len, audio_len, topk_frac))


def vsa_workspace_layout(num_heads: int, text_len: int, video_len: int, audio_len: int) -> dict:
    off = (ctypes.c_size_t * 7)()
    _check(load().vsa_workspace_layout(num_heads, text_len, video_len, audio_len, off),
           "vsa_workspace_layout")
    names = ("qbar64", "kbar", "vbar", "coarse", "kpack", "vpack", "total")
    return {n: int(off[i]) for i, n in enumerate(names)}


def _shape_args(q, text_len, video_len, audio_len):
    """Expected [S, H, 128] of the token tensors; H is read from q."""
    torch = _torch()
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a [S, H, 128] tensor")
    s = text_len + video_len + audio_len
    return (s, q.shape[1], HEAD_DIM)


def vsa_forward(q, k, v, gate, text_len, video_len, audio_len, topk_frac, out, selected_tiles,
                workspace=None, stream=None):
    torch = _torch()
    shp = _shape_args(q, text_len, video_len, audio_len)
    q, k, v, out = (_tensor(t, n, torch.bfloat16, shp) for t, n in ((q, "q"), (k, "k"), (v, "v"),
                                                                    (out, "out")))
    gate = _tensor(gate, "gate", torch.bfloat16, shp)
    selected_tiles = _selection(selected_tiles, shp[1], video_len,
                                vsa_topk_count(video_len, topk_frac))
    workspace = _tensor(workspace, "workspace", torch.uint8)
    nbytes = workspace.numel() if workspace is not None else 0
    _on_gpu(q=q, k=k, v=v, gate=gate, out=out, selected_tiles=selected_tiles, workspace=workspace)
    _check(load().vsa_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), shp[1], text_len, video_len,
                              audio_len, topk_frac, _ptr(out), _ptr(selected_tiles), _ptr(workspace),
                              nbytes, _stream(stream)), "vsa_forward")


def vsa_forward_noalloc(q, k, v, gate, text_len, video_len, audio_len, topk_frac, out,
                        selected_tiles, stream=None):
    """vsa_forward with the workspace in the library's fixed device array
    (VSA_NOALLOC_SCRATCH_BYTES per device): allocates nothing.  Calls that
    overlap in time on one device race on that array."""
    torch = _torch()
    shp = _shape_args(q, text_len, video_len, audio_len)
    q, k, v, out = (_tensor(t, n, torch.bfloat16, shp) for t, n in ((q, "q"), (k, "k"), (v, "v"),
                                                                    (out, "out")))
    gate = _tensor(gate, "gate", torch.bfloat16, shp)
    selected_tiles = _selection(selected_tiles, shp[1], video_len,
                                vsa_topk_count(video_len, topk_frac))
    _on_gpu(q=q, k=k, v=v, gate=gate, out=out, selected_tiles=selected_tiles)
    _check(load().vsa_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), shp[1], text_len,
                                      video_len, audio_len, topk_frac, _ptr(out),
                                      _ptr(selected_tiles), _stream(stream)),
           "vsa_forward_noalloc")


def vsa_pool_pack(q, k, v, text_len, video_len, audio_len, workspace, stream=None):
    torch = _torch()
    shp = _shape_args(q, text_len, video_len, audio_len)
    q, k, v = (_tensor(t, n, torch.bfloat16, shp) for t, n in ((q, "q"), (k, "k"), (v, "v")))
    workspace = _tensor(workspace, "workspace", torch.uint8)
    if workspace is None:
        raise ValueError("vsa_pool_pack needs a workspace")
    _on_gpu(q=q, k=k, v=v, workspace=workspace)
    _check(load().vsa_pool_pack(_ptr(q), _ptr(k), _ptr(v), shp[1], text_len, video_len, audio_len,
                                _ptr(workspace), workspace.numel(), _stream(stream)),
           "vsa_pool_pack")


def vsa_select_coarse(num_heads, text_len, video_len, audio_len, topk_frac, selected_tiles,
                      workspace, stream=None):
    torch = _torch()
    selected_tiles = _selection(selected_tiles, num_heads, video_len,
                                vsa_topk_count(video_len, topk_frac))
    workspace = _tensor(workspace, "workspace", torch.uint8)
    if workspace is None:
        raise ValueError("vsa_select_coarse needs a workspace")
    _on_gpu(selected_tiles=selected_tiles, workspace=workspace)
    _check(load().vsa_select_coarse(num_heads, text_len, video_len, audio_len, topk_frac,
                                    _ptr(selected_tiles), _ptr(workspace), workspace.numel(),
                                    _stream(stream)), "vsa_select_coarse")


def vsa_fine_attention(q, gate, text_len, video_len, audio_len, topk_frac, selected_tiles, out,
                       workspace, stream=None):
    torch = _torch()
    shp = _shape_args(q, text_len, video_len, audio_len)
    q, out = (_tensor(t, n, torch.bfloat16, shp) for t, n in ((q, "q"), (out, "out")))
    gate = _tensor(gate, "gate", torch.bfloat16, shp)
    selected_tiles = _selection(selected_tiles, shp[1], video_len,
                                vsa_topk_count(video_len, topk_frac))
    workspace = _tensor(workspace, "workspace", torch.uint8)
    if workspace is None:
        raise ValueError("vsa_fine_attention needs a workspace")
    _on_gpu(q=q, gate=gate, out=out, selected_tiles=selected_tiles, workspace=workspace)
    _check(load().vsa_fine_attention(_ptr(q), _ptr(gate), shp[1], text_len, video_len,
                                     audio_len, topk_frac, _ptr(selected_tiles), _ptr(out),
                                     _ptr(workspace), workspace.numel(), _stream(stream)),
           "vsa_fine_attention")


def alloc_outputs(num_heads, text_len, video_len, audio_len, topk_frac, device=None):
    """Allocate (out, selected_tiles, workspace) torch tensors for one shape."""
    torch = _torch()
    device = device or torch.device("cuda", torch.cuda.current_device())
    s = text_len + video_len + audio_len
    kk = vsa_topk_count(video_len, topk_frac)
    if kk < 0:
        raise ValueError("bad video_len / topk_frac")
    n_v = video_len // TILE
    out = torch.empty((s, num_heads, HEAD_DIM), dtype=torch.bfloat16, device=device)
    sel = torch.empty((num_heads, n_v, kk), dtype=torch.int32, device=device)
    wsb = vsa_workspace_bytes(num_heads, text_len, video_len, audio_len, topk_frac)
    if wsb == 0:
        raise ValueError("bad shape")
    ws = torch.empty(wsb, dtype=torch.uint8, device=device)
    return out, sel, ws


def forward(q, k, v, gate, text_len, video_len, audio_len, topk_frac=0.2, workspace=None,
            stream=None):
    """Convenience wrapper: allocates out / selected_tiles (and the workspace
    if none is given) with torch, then calls vsa_forward."""
    out, sel, ws = alloc_outputs(q.shape[1], text_len, video_len, audio_len, topk_frac, q.device)
    vsa_forward(q, k, v, gate, text_len, video_len, audio_len, topk_frac, out, sel,
                workspace if workspace is not None else ws, stream)
    return out, sel


def vsa_project_qkvg(x, w, num_heads, q, k, v, gate, stream=None):
    """Q/K/V/gate projections: x bf16 [tokens][hidden], w bf16
    [4][num_heads*128][hidden] (q, k, v, gate weights, each out x in); writes
    q, k, v, gate bf16 [tokens][num_heads][128]."""
    torch = _torch()
    x = _tensor(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [tokens][hidden]")
    tokens, hidden = x.shape
    w = _tensor(w, "w", torch.bfloat16, (4, num_heads * HEAD_DIM, hidden))
    outs = [_tensor(t, n, torch.bfloat16, (tokens, num_heads, HEAD_DIM))
            for t, n in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate"))]
    _on_gpu(x=x, w=w, q=outs[0], k=outs[1], v=outs[2], gate=outs[3])
    _check(load().vsa_project_qkvg(_ptr(x), _ptr(w), tokens, hidden, num_heads,
                                   *[_ptr(t) for t in outs], _stream(stream)),
           "vsa_project_qkvg")


def project_qkvg(x, w, num_heads, stream=None):
    """Convenience wrapper: allocates the four outputs with torch and calls
    vsa_project_qkvg."""
    torch = _torch()
    outs = [torch.empty((x.shape[0], num_heads, HEAD_DIM), dtype=torch.bfloat16, device=x.device)
            for _ in range(4)]
    vsa_project_qkvg(x, w, num_heads, *outs, stream=stream)
    return tuple(outs)


def vsa_forward_padded(q, k, v, gate, text_len, video_len, audio_len, valid, topk_frac, out,
                       selected_tiles, workspace, gamma_q=None, gamma_k=None, grid=None,
                       tile=(2, 8, 4), q_out=None, stream=None):
    """vsa_forward on padded segments (valid = (text, video, audio) token
    rows), optionally with Q/K RMSNorm + partial 3D RoPE fused into stage 1
    (gamma_q, gamma_k bf16 [H][128]; grid = latent (T, H, W) of the video
    tokens; q_out receives the preprocessed q)."""
    torch = _torch()
    shp = _shape_args(q, text_len, video_len, audio_len)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _tensor(t, n, torch.bfloat16, shp)
    _tensor(gate, "gate", torch.bfloat16, shp)
    selected_tiles = _selection(selected_tiles, shp[1], video_len,
                                vsa_topk_count(video_len, topk_frac))
    workspace = _tensor(workspace, "workspace", torch.uint8)
    if len(valid) != 3:
        raise ValueError("valid must be (text, video, audio) token rows")
    g6 = None
    if gamma_q is not None or gamma_k is not None:
        _tensor(gamma_q, "gamma_q", torch.bfloat16, (shp[1], HEAD_DIM))
        _tensor(gamma_k, "gamma_k", torch.bfloat16, (shp[1], HEAD_DIM))
        _tensor(q_out, "q_out", torch.bfloat16, shp)
        if gamma_q is None or gamma_k is None or q_out is None or grid is None:
            raise ValueError("gamma_q, gamma_k, q_out and grid go together")
        if len(grid) != 3 or len(tile) != 3:
            raise ValueError("grid and tile are (T, H, W) triples")
        g6 = (ctypes.c_int32 * 6)(*grid, *tile)
    _on_gpu(q=q, k=k, v=v, gate=gate, out=out, selected_tiles=selected_tiles,
            workspace=workspace, gamma_q=gamma_q, gamma_k=gamma_k, q_out=q_out)
    _check(load().vsa_forward_padded(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(gamma_q),
                                     _ptr(gamma_k), g6, shp[1], text_len, video_len, audio_len,
                                     valid[0], valid[1], valid[2], topk_frac, _ptr(q_out),
                                     _ptr(out), _ptr(selected_tiles),
                                     _ptr(workspace) if workspace is not None else None,
                                     workspace.numel() if workspace is not None else 0,
                                     _stream(stream)),
           "vsa_forward_padded")


# ---------------------------------------------------------------------------
# SubBlock router: 16-token sub-block log-sum-exp scores choose the video key
# tiles; no coarse branch, no gate.
# ---------------------------------------------------------------------------

def vsa_subblock_count(video_len: int, sparsity: float) -> int:
    return int(load().vsa_subblock_count(video_len, sparsity))


def vsa_subblock_workspace_bytes(num_heads: int, text_len: int, video_len: int,
                                 audio_len: int) -> int:
    return int(load().vsa_subblock_workspace_bytes(num_heads, text_len, video_len, audio_len))


def vsa_forward_subblock(q, k, v, text_len, video_len, audio_len, sparsity, out, selected_tiles,
                         workspace=None, stream=None):
    torch = _torch()
    shp = _shape_args(q, text_len, video_len, audio_len)
    q, k, v, out = (_tensor(t, n, torch.bfloat16, shp) for t, n in ((q, "q"), (k, "k"), (v, "v"),
                                                                    (out, "out")))
    selected_tiles = _selection(selected_tiles, shp[1], video_len,
                                vsa_subblock_count(video_len, sparsity))
    workspace = _tensor(workspace, "workspace", torch.uint8)
    nbytes = workspace.numel() if workspace is not None else 0
    _on_gpu(q=q, k=k, v=v, out=out, selected_tiles=selected_tiles, workspace=workspace)
    _check(load().vsa_forward_subblock(_ptr(q), _ptr(k), _ptr(v), shp[1], text_len, video_len,
                                       audio_len, sparsity, _ptr(out), _ptr(selected_tiles),
                                       _ptr(workspace), nbytes, _stream(stream)),
           "vsa_forward_subblock")


def vsa_subblock_select(q, k, text_len, video_len, audio_len, sparsity, selected_tiles, workspace,
                        stream=None):
    torch = _torch()
    shp = _shape_args(q, text_len, video_len, audio_len)
    q, k = (_tensor(t, n, torch.bfloat16, shp) for t, n in ((q, "q"), (k, "k")))
    selected_tiles = _selection(selected_tiles, shp[1], video_len,
                                vsa_subblock_count(video_len, sparsity))
    workspace = _tensor(workspace, "workspace", torch.uint8)
    if workspace is None:
        raise ValueError("vsa_subblock_select needs a workspace")
    _on_gpu(q=q, k=k, selected_tiles=selected_tiles, workspace=workspace)
    _check(load().vsa_subblock_select(_ptr(q), _ptr(k), shp[1], text_len, video_len, audio_len,
                                      sparsity, _ptr(selected_tiles), _ptr(workspace),
                                      workspace.numel(), _stream(stream)), "vsa_subblock_select")


def alloc_subblock_outputs(num_heads, text_len, video_len, audio_len, sparsity, device=None):
    """Allocate (out, selected_tiles, workspace) for vsa_forward_subblock."""
    torch = _torch()
    device = device or torch.device("cuda", torch.cuda.current_device())
    s = text_len + video_len + audio_len
    kk = vsa_subblock_count(video_len, sparsity)
    wsb = vsa_subblock_workspace_bytes(num_heads, text_len, video_len, audio_len)
    if kk < 0 or wsb == 0:
        raise ValueError("bad shape or sparsity")
    out = torch.empty((s, num_heads, HEAD_DIM), dtype=torch.bfloat16, device=device)
    sel = torch.empty((num_heads, video_len // TILE, kk), dtype=torch.int32, device=device)
    ws = torch.empty(wsb, dtype=torch.uint8, device=device)
    return out, sel, ws


def forward_subblock(q, k, v, text_len, video_len, audio_len, sparsity=0.75, workspace=None,
                     stream=None):
    """Convenience wrapper of vsa_forward_subblock (allocates with torch)."""
    out, sel, ws = alloc_subblock_outputs(q.shape[1], text_len, video_len, audio_len, sparsity,
                                          q.device)
    vsa_forward_subblock(q, k, v, text_len, video_len, audio_len, sparsity, out, sel,
                         workspace if workspace is not None else ws, stream)
    return out, sel


# ---------------------------------------------------------------------------
# SubBlock router over the whole sequence: every tile a query tile and a
# candidate key tile; selected_tiles is [H][N][k] with global tile indices.
# ---------------------------------------------------------------------------

def vsa_subblock_whole_workspace_bytes(num_heads: int, text_len: int, video_len: int,
                                       audio_len: int) -> int:
    return int(load().vsa_subblock_whole_workspace_bytes(num_heads, text_len, video_len,
                                                         audio_len))


def _whole_k(text_len, video_len, audio_len, sparsity):
    return vsa_subblock_count(text_len + video_len + audio_len, sparsity)


def vsa_forward_subblock_whole(q, k, v, text_len, video_len, audio_len, sparsity, out,
                               selected_tiles, workspace=None, stream=None):
    torch = _torch()
    shp = _shape_args(q, text_len, video_len, audio_len)
    q, k, v, out = (_tensor(t, n, torch.bfloat16, shp) for t, n in ((q, "q"), (k, "k"), (v, "v"),
                                                                    (out, "out")))
    n = shp[0] // TILE
    kk = _whole_k(text_len, video_len, audio_len, sparsity)
    selected_tiles = _tensor(selected_tiles, "selected_tiles", torch.int32,
                             (shp[1], n, kk) if kk >= 0 else None)
    workspace = _tensor(workspace, "workspace", torch.uint8)
    nbytes = workspace.numel() if workspace is not None else 0
    _on_gpu(q=q, k=k, v=v, out=out, selected_tiles=selected_tiles, workspace=workspace)
    _check(load().vsa_forward_subblock_whole(_ptr(q), _ptr(k), _ptr(v), shp[1], text_len,
                                             video_len, audio_len, sparsity, _ptr(out),
                                             _ptr(selected_tiles), _ptr(workspace), nbytes,
                                             _stream(stream)), "vsa_forward_subblock_whole")


def vsa_subblock_select_whole(q, k, text_len, video_len, audio_len, sparsity, selected_tiles,
                              workspace, stream=None):
    torch = _torch()
    shp = _shape_args(q, text_len, video_len, audio_len)
    q, k = (_tensor(t, n, torch.bfloat16, shp) for t, n in ((q, "q"), (k, "k")))
    n = shp[0] // TILE
    kk = _whole_k(text_len, video_len, audio_len, sparsity)
    selected_tiles = _tensor(selected_tiles, "selected_tiles", torch.int32,
                             (shp[1], n, kk) if kk >= 0 else None)
    workspace = _tensor(workspace, "workspace", torch.uint8)
    if workspace is None:
        raise ValueError("vsa_subblock_select_whole needs a workspace")
    _on_gpu(q=q, k=k, selected_tiles=selected_tiles, workspace=workspace)
    _check(load().vsa_subblock_select_whole(_ptr(q), _ptr(k), shp[1], text_len, video_len,
                                            audio_len, sparsity, _ptr(selected_tiles),
                                            _ptr(workspace), workspace.numel(), _stream(stream)),
           "vsa_subblock_select_whole")


def alloc_subblock_whole_outputs(num_heads, text_len, video_len, audio_len, sparsity,
                                 device=None):
    """Allocate (out, selected_tiles, workspace) for vsa_forward_subblock_whole."""
    torch = _torch()
    device = device or torch.device("cuda", torch.cuda.current_device())
    s = text_len + video_len + audio_len
    kk = _whole_k(text_len, video_len, audio_len, sparsity)
    wsb = vsa_subblock_whole_workspace_bytes(num_heads, text_len, video_len, audio_len)
    if kk < 0 or wsb == 0:
        raise ValueError("bad shape or sparsity")
    out = torch.empty((s, num_heads, HEAD_DIM), dtype=torch.bfloat16, device=device)
    sel = torch.empty((num_heads, s // TILE, kk), dtype=torch.int32, device=device)
    ws = torch.empty(wsb, dtype=torch.uint8, device=device)
    return out, sel, ws


def forward_subblock_whole(q, k, v, text_len, video_len, audio_len, sparsity=0.75, workspace=None,
                           stream=None):
    """Convenience wrapper of vsa_forward_subblock_whole (allocates with torch)."""
    out, sel, ws = alloc_subblock_whole_outputs(q.shape[1], text_len, video_len, audio_len,
                                                sparsity, q.device)
    vsa_forward_subblock_whole(q, k, v, text_len, video_len, audio_len, sparsity, out, sel,
                               workspace if workspace is not None else ws, stream)
    return out, sel
