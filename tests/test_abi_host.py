"""Host-side checks of the C ABI (no GPU, no compute call): the library loads,
exports every symbol include/vsa.h declares, and rejects bad arguments with
the documented status codes before touching the GPU."""
import ctypes
import json
import os
import re

import pytest

import block_sparse_video_amd as bsv
from block_sparse_video_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vsa.h")

OK, NULLP, SHAPE, UNALIGNED, TOPK, MISALIGNED, WORKSPACE, DEVICE, HIP, TOO_LARGE = range(10)
FAKE = 0x100000  # 256-byte aligned, never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vsa_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = _native.load()
    names = declared_functions()
    assert {"vsa_forward", "vsa_topk_count", "vsa_workspace_bytes", "vsa_status_string",
            "vsa_pool_pack", "vsa_select_coarse", "vsa_fine_attention",
            "vsa_workspace_layout"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_native.SIGNATURES)


def test_status_strings():
    assert bsv.status_string(0) == "VSA_OK"
    assert bsv.status_string(TOPK) == "VSA_ERR_BAD_TOPK"
    assert bsv.status_string(99) == "VSA_ERR_UNKNOWN"


def test_topk_count_matches_golden_table():
    with open(os.path.join(ROOT, "tests", "golden", "topk_counts.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        assert bsv.vsa_topk_count(64 * c["n_v"], c["frac"]) == c["k"], c
    for bad in g["invalid_fracs"]:
        assert bsv.vsa_topk_count(640, float(bad)) == -1
    assert bsv.vsa_topk_count(65, 0.2) == -1
    assert bsv.vsa_topk_count(-64, 0.2) == -1


def test_workspace_bytes_and_layout():
    n = bsv.vsa_workspace_bytes(56, 1024, 72576, 1024)
    lay = bsv.vsa_workspace_layout(56, 1024, 72576, 1024)
    assert lay["total"] == n
    h, n_v, N = 56, 1134, 1166
    assert lay["kbar"] - lay["qbar64"] >= h * n_v * 128 * 8
    assert lay["total"] - lay["vpack"] >= h * N * 64 * 128 * 2
    assert lay["vpack"] - lay["kpack"] >= h * N * 64 * 128 * 2
    assert all(v % 256 == 0 for v in lay.values())
    assert bsv.vsa_workspace_bytes(0, 64, 64, 64) == 0
    assert bsv.vsa_workspace_bytes(1, 63, 64, 64) == 0
    assert bsv.vsa_workspace_bytes(1, 0, 0, 0) == 0
    assert bsv.vsa_workspace_bytes(1, 0, 64, 0) > 0


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, h=2, t=64, vid=640, au=64, frac=0.2, out=FAKE,
             sel=FAKE, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return _native.load().vsa_forward(a["q"], a["k"], a["v"], a["g"], a["h"], a["t"], a["vid"],
                                      a["au"], a["frac"], a["out"], a["sel"], a["ws"], a["wsb"],
                                      a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULLP), (dict(k=None), NULLP), (dict(v=None), NULLP), (dict(out=None), NULLP),
    (dict(g=None), NULLP), (dict(sel=None), NULLP),
    (dict(h=0), SHAPE), (dict(h=-3), SHAPE), (dict(t=-64), SHAPE), (dict(t=0, vid=0, au=0), SHAPE),
    (dict(t=65), UNALIGNED), (dict(vid=100), UNALIGNED), (dict(au=1), UNALIGNED),
    (dict(frac=0.0), TOPK), (dict(frac=-0.1), TOPK), (dict(frac=1.01), TOPK),
    (dict(frac=float("nan")), TOPK),
    (dict(q=FAKE + 8), MISALIGNED), (dict(out=FAKE + 2), MISALIGNED), (dict(g=FAKE + 4), MISALIGNED),
    (dict(ws=FAKE + 16), MISALIGNED),
    (dict(wsb=1000), WORKSPACE),
    (dict(h=2048), TOO_LARGE), (dict(vid=64 * 20000), TOO_LARGE),
])
def test_forward_validation(kw, code):
    assert fwd(**kw) == code


def test_text_only_allows_null_gate_and_selection_up_to_validation():
    # video_len == 0: gate/selected_tiles may be NULL; the call then fails only
    # on the workspace size (checked before the device), never on NULL pointers.
    assert fwd(vid=0, g=None, sel=None, wsb=10) == WORKSPACE


def test_stage_validation():
    lib = _native.load()
    assert lib.vsa_pool_pack(None, FAKE, FAKE, 2, 64, 640, 64, FAKE, 1 << 40, None) == NULLP
    assert lib.vsa_pool_pack(FAKE, FAKE, FAKE, 2, 64, 640, 64, None, 1 << 40, None) == WORKSPACE
    assert lib.vsa_pool_pack(FAKE, FAKE, FAKE, 2, 64, 640, 64, FAKE, 64, None) == WORKSPACE
    assert lib.vsa_select_coarse(2, 64, 640, 64, 0.2, None, FAKE, 1 << 40, None) == NULLP
    assert lib.vsa_select_coarse(2, 64, 0, 64, 0.2, FAKE, FAKE, 1 << 40, None) == SHAPE
    assert lib.vsa_select_coarse(2, 64, 640, 64, 2.0, FAKE, FAKE, 1 << 40, None) == TOPK
    assert lib.vsa_fine_attention(FAKE, FAKE, 2, 64, 640, 64, 0.2, FAKE, None, FAKE, 1 << 40,
                                  None) == NULLP
    assert lib.vsa_fine_attention(FAKE, FAKE, 2, 64, 640, 64, 0.2, FAKE, FAKE, FAKE, 10,
                                  None) == WORKSPACE


def test_layout_rejects_bad_shape():
    off = (ctypes.c_size_t * 7)()
    assert _native.load().vsa_workspace_layout(1, 64, 65, 0, off) == UNALIGNED
    assert _native.load().vsa_workspace_layout(1, 64, 64, 0, None) == NULLP


def test_project_validation():
    lib = _native.load()
    o = [FAKE] * 4
    assert lib.vsa_project_qkvg(FAKE, FAKE, 4, 96, 2, *o, None) == UNALIGNED   # hidden % 64
    assert lib.vsa_project_qkvg(FAKE, FAKE, 4, 64, 3, *o, None) == UNALIGNED   # odd heads
    assert lib.vsa_project_qkvg(FAKE, FAKE, 0, 64, 2, *o, None) == SHAPE
    assert lib.vsa_project_qkvg(FAKE, FAKE, 4, 32, 2, *o, None) == SHAPE
    assert lib.vsa_project_qkvg(None, FAKE, 4, 64, 2, *o, None) == NULLP
    assert lib.vsa_project_qkvg(FAKE, FAKE, 4, 64, 2, FAKE, FAKE, None, FAKE, None) == NULLP
    assert lib.vsa_project_qkvg(FAKE + 2, FAKE, 4, 64, 2, *o, None) == MISALIGNED
    assert lib.vsa_project_qkvg(FAKE, FAKE, 4, 32768, 2, *o, None) == TOO_LARGE
    assert lib.vsa_project_qkvg(FAKE, FAKE, 4, 64, 2048, *o, None) == TOO_LARGE


def test_subblock_count_matches_oracle():
    import oracle
    for n_v in (0, 1, 5, 7, 8, 9, 15, 16, 17, 100, 640, 1134, 5120):
        for sp in (0.0, 0.1, 0.5, 0.75, 0.8, 0.875, 0.9, 0.95, 0.999):
            assert bsv.vsa_subblock_count(64 * n_v, sp) == oracle.subblock_count(n_v, sp), (n_v, sp)
    assert bsv.vsa_subblock_count(1134 * 64, 0.75) == 280
    for bad in (1.0, -0.01, float("nan"), float("inf")):
        assert bsv.vsa_subblock_count(640, bad) == -1
    assert bsv.vsa_subblock_count(65, 0.5) == -1


def test_subblock_workspace_bytes():
    base = bsv.vsa_workspace_bytes(56, 1024, 72576, 1024)
    n = bsv.vsa_subblock_workspace_bytes(56, 1024, 72576, 1024)
    # Q and K sub-block means, 8 KiB per (head, group of 4 video tiles), 256-byte aligned
    assert n == base + 2 * (56 * 284 * 8192)
    assert bsv.vsa_subblock_workspace_bytes(1, 0, 64 * 5120, 0) > 0
    assert bsv.vsa_subblock_workspace_bytes(1, 0, 64 * 5121, 0) == 0
    assert bsv.vsa_subblock_workspace_bytes(1, 0, 65, 0) == 0


def test_subblock_forward_validation():
    lib = _native.load()
    f = lib.vsa_forward_subblock
    args = dict(q=FAKE, k=FAKE, v=FAKE, h=2, t=64, vid=640, au=64, sp=0.75, out=FAKE, sel=FAKE,
                ws=FAKE, wsb=1 << 40)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["q"], a["k"], a["v"], a["h"], a["t"], a["vid"], a["au"], a["sp"], a["out"],
                 a["sel"], a["ws"], a["wsb"], None)
    assert call(q=None) == NULLP
    assert call(sel=None) == NULLP
    assert call(vid=0, sel=None, wsb=10) == WORKSPACE
    assert call(h=0) == SHAPE
    assert call(vid=100) == UNALIGNED
    assert call(sp=1.0) == TOPK
    assert call(sp=-0.5) == TOPK
    assert call(vid=64 * 5121) == TOO_LARGE
    assert call(out=FAKE + 2) == MISALIGNED
    assert call(sel=FAKE + 4) == MISALIGNED
    assert call(ws=FAKE + 16) == MISALIGNED
    assert call(wsb=bsv.vsa_workspace_bytes(2, 64, 640, 64)) == WORKSPACE


def test_subblock_select_validation():
    f = _native.load().vsa_subblock_select
    assert f(None, FAKE, 2, 64, 640, 64, 0.75, FAKE, FAKE, 1 << 40, None) == NULLP
    assert f(FAKE, FAKE, 2, 64, 640, 64, 0.75, None, FAKE, 1 << 40, None) == NULLP
    assert f(FAKE, FAKE, 2, 64, 0, 64, 0.75, FAKE, FAKE, 1 << 40, None) == SHAPE
    assert f(FAKE, FAKE, 2, 64, 640, 64, 1.5, FAKE, FAKE, 1 << 40, None) == TOPK
    assert f(FAKE, FAKE, 2, 64, 640, 64, 0.75, FAKE, None, 1 << 40, None) == WORKSPACE
    assert f(FAKE, FAKE, 2, 64, 640, 64, 0.75, FAKE, FAKE, 64, None) == WORKSPACE
    assert f(FAKE, FAKE, 2, 64, 64 * 6000, 64, 0.75, FAKE, FAKE, 1 << 40, None) == TOO_LARGE


def padded(**kw):
    """vsa_forward_padded with fake device pointers: every case below fails
    validation before the library touches the GPU."""
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, gq=None, gk=None, grid=None, h=2, t=128, vid=640,
             au=128, tv=100, vv=600, av=65, frac=0.2, qo=None, out=FAKE, sel=FAKE, ws=FAKE,
             wsb=1 << 40)
    a.update(kw)
    grid = None if a["grid"] is None else (ctypes.c_int32 * 6)(*a["grid"])
    return _native.load().vsa_forward_padded(
        a["q"], a["k"], a["v"], a["g"], a["gq"], a["gk"], grid, a["h"], a["t"], a["vid"], a["au"],
        a["tv"], a["vv"], a["av"], a["frac"], a["qo"], a["out"], a["sel"], a["ws"], a["wsb"], None)


PREP = dict(gq=FAKE, gk=FAKE, qo=FAKE, grid=(2, 10, 30, 1, 2, 2))  # 2*10*30 = 600 video tokens


@pytest.mark.parametrize("kw,code", [
    # required pointers
    (dict(q=None), NULLP), (dict(k=None), NULLP), (dict(v=None), NULLP), (dict(out=None), NULLP),
    (dict(g=None), NULLP), (dict(sel=None), NULLP),
    # preprocessing arguments come together: both gammas, q_out and grid
    (dict(PREP, gk=None), NULLP), (dict(PREP, gq=None), NULLP), (dict(PREP, qo=None), NULLP),
    (dict(PREP, grid=None), NULLP),
    # shape
    (dict(h=0), SHAPE), (dict(t=-64), SHAPE), (dict(vid=100), UNALIGNED),
    # valid rows: only a segment's last tile may be padding, and none of an empty segment
    (dict(tv=129), SHAPE), (dict(tv=64), SHAPE), (dict(tv=0), SHAPE),
    (dict(vv=641), SHAPE), (dict(vv=576), SHAPE), (dict(av=-1), SHAPE), (dict(av=64), SHAPE),
    (dict(t=0, tv=1), SHAPE), (dict(au=0, av=5), SHAPE),
    # the latent grid: positive, divisible by the tile, T*H*W = video_valid
    (dict(PREP, grid=(0, 10, 30, 1, 2, 2)), SHAPE), (dict(PREP, grid=(2, 10, 30, 1, 0, 2)), SHAPE),
    (dict(PREP, grid=(2, 10, 30, 1, 3, 2)), SHAPE), (dict(PREP, grid=(2, 10, 30, 2, 2, 4)), SHAPE),
    (dict(PREP, grid=(2, 10, 31, 1, 2, 1)), SHAPE),
    # top-k fraction
    (dict(frac=0.0), TOPK), (dict(frac=1.5), TOPK),
    # alignment of every pointer, gammas and q_out included
    (dict(q=FAKE + 2), MISALIGNED), (dict(out=FAKE + 8), MISALIGNED),
    (dict(sel=FAKE + 4), MISALIGNED), (dict(PREP, qo=FAKE + 2), MISALIGNED),
    (dict(PREP, gq=FAKE + 8), MISALIGNED), (dict(PREP, gk=FAKE + 4), MISALIGNED),
    (dict(ws=FAKE + 16), MISALIGNED),
    # workspace size
    (dict(wsb=1000), WORKSPACE),
    (dict(vid=64 * 20000, vv=64 * 20000), TOO_LARGE),
])
def test_padded_validation(kw, code):
    assert padded(**kw) == code


def test_padded_without_video_allows_null_gate_and_selection():
    assert padded(vid=0, vv=0, g=None, sel=None, wsb=10) == WORKSPACE


def noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, h=2, t=64, vid=640, au=64, frac=0.2, out=FAKE,
             sel=FAKE)
    a.update(kw)
    return _native.load().vsa_forward_noalloc(a["q"], a["k"], a["v"], a["g"], a["h"], a["t"],
                                              a["vid"], a["au"], a["frac"], a["out"], a["sel"],
                                              None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULLP), (dict(out=None), NULLP), (dict(g=None), NULLP), (dict(sel=None), NULLP),
    (dict(h=0), SHAPE), (dict(vid=100), UNALIGNED), (dict(frac=0.0), TOPK),
    (dict(q=FAKE + 2), MISALIGNED), (dict(sel=FAKE + 4), MISALIGNED),
    (dict(h=2048), TOO_LARGE),
    # one head of 16,384 video tiles needs ~0.6 GB of workspace: beyond the array
    (dict(h=1, vid=64 * 16384), TOO_LARGE),
])
def test_noalloc_validation(kw, code):
    assert noalloc(**kw) == code


def test_noalloc_limit_is_one_head_of_workspace():
    cap = 256 << 20
    # the largest video length whose one-head workspace fits is accepted past
    # the size check (it then fails only at the device check on this host)
    n_ok = max(n for n in range(1, 16385, 7)
               if bsv.vsa_workspace_bytes(1, 64, 64 * n, 64) <= cap)
    assert noalloc(h=1, vid=64 * n_ok) not in (TOO_LARGE, SHAPE, UNALIGNED)
    assert noalloc(h=1, vid=64 * (n_ok + 7)) == TOO_LARGE


def test_subblock_whole_validation():
    lib = _native.load()
    f = lib.vsa_forward_subblock_whole
    args = dict(q=FAKE, k=FAKE, v=FAKE, h=2, t=64, vid=640, au=64, sp=0.75, out=FAKE, sel=FAKE,
                ws=FAKE, wsb=1 << 40)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["q"], a["k"], a["v"], a["h"], a["t"], a["vid"], a["au"], a["sp"], a["out"],
                 a["sel"], a["ws"], a["wsb"], None)
    assert call(q=None) == NULLP
    assert call(sel=None) == NULLP
    assert call(h=0) == SHAPE
    assert call(vid=100) == UNALIGNED
    assert call(sp=1.0) == TOPK
    # N counts every tile: 5,119 video + 2 tiles passes the router's 5,120 limit
    assert call(vid=64 * 5119) == TOO_LARGE
    assert call(out=FAKE + 2) == MISALIGNED
    assert call(sel=FAKE + 4) == MISALIGNED
    assert call(wsb=bsv.vsa_subblock_whole_workspace_bytes(2, 64, 640, 64) - 256) == WORKSPACE
    g = lib.vsa_subblock_select_whole
    assert g(FAKE, FAKE, 2, 64, 640, 64, 0.75, FAKE, None, 1 << 40, None) == WORKSPACE
    assert g(FAKE, FAKE, 2, 64, 640, 64, 0.75, None, FAKE, 1 << 40, None) == NULLP


def test_subblock_whole_workspace_and_count():
    # kpack + vpack of every tile, the 1,536 bytes of queue counters (twelve
    # 128-byte lines), then the two piece-mean regions
    h, n = 56, 1166
    n_c = (n + 3) // 4
    total = bsv.vsa_subblock_whole_workspace_bytes(h, 1024, 72576, 1024)
    assert total == 2 * h * n * 16384 + 1536 + 2 * h * n_c * 8192
    assert bsv.vsa_subblock_count(74624, 0.75) == 288   # the whole-sequence kept count
    assert bsv.vsa_subblock_whole_workspace_bytes(1, 64, 64 * 5119, 64) == 0
