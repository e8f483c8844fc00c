"""GPU parity of padded segments and of the fused attention preprocessing
(Q/K RMSNorm + partial 3D RoPE) against the CPU oracle.

Padding: selections bit-exact, outputs within the usual bars, padding rows
exactly zero, and padding contents (even NaN) without any effect.
Preprocessing: each preprocessed Q and K element within one bf16 step of the
oracle's float64 value rounded once (the GPU normalises and rotates in fp32,
so a value next to a rounding boundary may land one step away); the rest of
the path is then checked on the GPU's own preprocessed tensors, as for any
other input.
"""
import numpy as np
import pytest
import torch

import block_sparse_video_amd as bsv
import oracle
import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu
T = 64
D = 128
THREADS = synth.default_threads()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    torch.cuda.set_device(0)
    yield


def announce(msg):
    print(f"[case] {msg}", flush=True)


def run_padded(xd, s_t, s_v, s_a, valid, frac, gq=None, gk=None, grid=None, tile=(2, 8, 4)):
    h = xd["q"].shape[1]
    out, sel, ws = bsv.alloc_outputs(h, s_t, s_v, s_a, frac)
    out.fill_(float("nan"))
    sel.fill_(-7)
    q_out = torch.full_like(xd["q"], float("nan")) if gq is not None else None
    bsv.vsa_forward_padded(xd["q"], xd["k"], xd["v"], xd["gate"], s_t, s_v, s_a, valid, frac, out,
                           sel, ws, gamma_q=gq, gamma_k=gk, grid=grid, tile=tile, q_out=q_out)
    torch.cuda.synchronize()
    return out, sel, ws, q_out


def pad_mask(s_t, s_v, s_a, valid):
    pad = np.ones(s_t + s_v + s_a, bool)
    pad[:valid[0]] = False
    pad[s_t:s_t + valid[1]] = False
    pad[s_t + s_v:s_t + s_v + valid[2]] = False
    return pad


def check_rest(qb, kb, vb, gb, s_t, s_v, s_a, valid, frac, out, sel, rows=None):
    ref = oracle.select_coarse(qb, kb, vb, s_t, s_v, s_a, frac, video_valid=valid[1],
                               threads=THREADS)
    got_sel = sel.cpu().numpy()
    if s_v:
        G.check_selection(got_sel, ref, exempt_ok=False)
    rows = np.arange(s_t + s_v + s_a) if rows is None else rows
    _, ref_out = oracle.fine(qb, kb, vb, gb, s_t, s_v, s_a, got_sel if s_v else None,
                             ref["coarse"], rows, threads=THREADS, valid=valid)
    got = G.from_dev_bits(out)[rows]
    pad = pad_mask(s_t, s_v, s_a, valid)[rows]
    assert not got[pad].any(), "padding rows must be zero"
    return G.assert_outputs_close(got[~pad], ref_out[~pad])


@pytest.mark.parametrize("h,n_t,n_v,n_a,valid,frac,seed", [
    (1, 1, 4, 1, (40, 256, 17), 0.5, 1),      # partial text and audio tiles
    (2, 2, 5, 1, (128, 300, 64), 0.4, 2),     # partial last video tile
    (3, 1, 3, 2, (1, 129, 65), 0.34, 3),      # one text row; audio spills one row
    (2, 0, 6, 0, (0, 321, 0), 1.0, 4),        # video only, dense
    (2, 3, 70, 2, (150, 4470, 70), 0.2, 5),   # several workgroups, ragged everything
])
def test_padded_segments(h, n_t, n_v, n_a, valid, frac, seed):
    announce(f"padded h={h} tiles=({n_t},{n_v},{n_a}) valid={valid}")
    s_t, s_v, s_a = n_t * T, n_v * T, n_a * T
    x = synth.vsa_inputs(seed, h, s_t, s_v, s_a)
    out, sel, _, _ = run_padded(G.inputs_to_dev(x), s_t, s_v, s_a, valid, frac)
    e = check_rest(x["q"], x["k"], x["v"], x["gate"], s_t, s_v, s_a, valid, frac, out, sel)
    print(e)


def test_padding_contents_have_no_effect():
    announce("padding filled with NaN vs zeros")
    h, s_t, s_v, s_a = 2, 128, 64 * 9, 64
    valid = (77, 64 * 8 + 5, 1)
    x = synth.vsa_inputs(6, h, s_t, s_v, s_a)
    pad = pad_mask(s_t, s_v, s_a, valid)
    res = []
    for fill in (0x0000, 0x7FC0):  # zero, quiet NaN
        y = {n: a.copy() for n, a in x.items()}
        for n in y:
            y[n][pad] = fill
        out, sel, _, _ = run_padded(G.inputs_to_dev(y), s_t, s_v, s_a, valid, 0.3)
        res.append((G.from_dev_bits(out), sel.cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
    assert not res[0][0][pad].any()


def _prep_inputs(seed, h, s_t, s_v, s_a):
    x = synth.vsa_inputs(seed, h, s_t, s_v, s_a, std=2.0)
    gq = synth.normal_bf16(seed, 20, (h, D), mean=1.0, std=0.2)
    gk = synth.normal_bf16(seed, 21, (h, D), mean=1.0, std=0.2)
    return x, gq, gk


def prep_bound(ref_bits):
    """Per-element bound for a preprocessed value: one bf16 step of the
    larger of the value and (for rotated dims) the norm of its RoPE pair.
    The normalised value is rounded before the rotation, so a one-step
    difference there reaches the rotated value scaled by the pair's size,
    which can exceed the (cancelled) value itself."""
    r = G.widen(ref_bits)
    pair = np.sqrt(r[..., 0:96:2] ** 2 + r[..., 1:96:2] ** 2)
    scale = np.abs(r).copy()
    scale[..., 0:96:2] = np.maximum(scale[..., 0:96:2], pair)
    scale[..., 1:96:2] = np.maximum(scale[..., 1:96:2], pair)
    return 2.0 ** -7 * scale + 2.0 ** -30


def check_prep(x, gq, gk, s_t, s_v, s_a, valid, grid, tile, q_out, ws):
    h = x["q"].shape[1]
    qo = G.from_dev_bits(q_out)
    ko = G.unpack_k(ws, h, s_t, s_v, s_a)
    pad = pad_mask(s_t, s_v, s_a, valid)
    for got, raw, gam in ((qo, x["q"], gq), (ko, x["k"], gk)):
        ref = oracle.rms_norm_rope(raw, gam, s_t, s_v, s_a, valid, grid, tile)
        g, r = G.widen(got), G.widen(ref)
        assert not got[pad].any()
        err = np.abs(g - r)
        bound = prep_bound(ref)
        assert np.all(err <= bound), float((err / bound).max())
        assert np.mean(got == ref) > 0.99
    return qo, ko


@pytest.mark.parametrize("grid,tile,n_t,n_a,valid_ta,seed", [
    ((2, 8, 8), (2, 8, 4), 1, 1, (40, 17), 1),     # 2 video tiles
    ((4, 16, 8), (2, 8, 4), 2, 1, (100, 64), 2),   # 8 video tiles
    ((2, 8, 12), (2, 8, 4), 0, 2, (0, 77), 3),     # no text
])
def test_preprocessing_small(grid, tile, n_t, n_a, valid_ta, seed):
    s_v = grid[0] * grid[1] * grid[2]
    s_t, s_a = n_t * T, n_a * T
    valid = (valid_ta[0], s_v, valid_ta[1])
    announce(f"prep grid={grid} tiles=({n_t},{s_v // T},{n_a}) valid={valid}")
    h = 3
    x, gq, gk = _prep_inputs(seed, h, s_t, s_v, s_a)
    xd = G.inputs_to_dev(x)
    gqd, gkd = G.to_dev(gq), G.to_dev(gk)
    out, sel, ws, q_out = run_padded(xd, s_t, s_v, s_a, valid, 0.3, gqd, gkd, grid, tile)
    qo, ko = check_prep(x, gq, gk, s_t, s_v, s_a, valid, grid, tile, q_out, ws)
    e = check_rest(qo, ko, x["v"], x["gate"], s_t, s_v, s_a, valid, 0.3, out, sel)
    print(e)


@pytest.mark.slow
def test_pages_request_shape_with_preprocessing():
    """The 10 s request of the pages' workload: 1,000 text, 72,576 video
    (18 x 48 x 84 latent grid) and 810 audio tokens, in 1,024 / 72,576 / 832
    rows; 56 heads; learned-norm and RoPE preprocessing fused in.  All
    selections, coarse, preprocessed Q/K on sampled rows, outputs on
    sampled rows."""
    h, s_t, s_v, s_a = 56, 1024, 72576, 832
    valid = (1000, 72576, 810)
    grid, tile = (18, 48, 84), (2, 8, 4)
    announce(f"pages request: h={h} rows=({s_t},{s_v},{s_a}) valid={valid}")
    x, gq, gk = _prep_inputs(7, h, s_t, s_v, s_a)
    xd = G.inputs_to_dev(x)
    out, sel, ws, q_out = run_padded(xd, s_t, s_v, s_a, valid, 0.2, G.to_dev(gq), G.to_dev(gk),
                                     grid, tile)
    qo = G.from_dev_bits(q_out)
    ko = G.unpack_k(ws, h, s_t, s_v, s_a)
    rows = np.unique(np.concatenate([G.sample_rows(s_t, s_v, s_a, n_video_tiles=3,
                                                   per_tile=(0, 37, 63)),
                                     [999, 1000, 1023, s_t + s_v + 809, s_t + s_v + 810]]))
    # preprocessing on the sampled rows (the oracle works row by row)
    for got, raw, gam in ((qo, x["q"], gq), (ko, x["k"], gk)):
        rb = oracle.rms_norm_rope(raw, gam, s_t, s_v, s_a, valid, grid, tile, rows=rows)
        g, r = G.widen(got[rows]), G.widen(rb)
        assert np.all(np.abs(g - r) <= prep_bound(rb))
    ref = oracle.select_coarse(qo, ko, x["v"], s_t, s_v, s_a, 0.2, video_valid=valid[1],
                               threads=THREADS)
    got_sel = sel.cpu().numpy()
    n_exempt = G.check_selection(got_sel, ref)
    w = G.read_workspace(ws, h, s_t, s_v, s_a)
    np.testing.assert_allclose(w["coarse"], ref["coarse"], rtol=2e-5, atol=2e-7)
    _, ref_out = oracle.fine(qo, ko, x["v"], x["gate"], s_t, s_v, s_a, got_sel, ref["coarse"],
                             rows, threads=THREADS, valid=valid)
    got = G.from_dev_bits(out)[rows]
    pad = pad_mask(s_t, s_v, s_a, valid)[rows]
    assert not got[pad].any()
    e = G.assert_outputs_close(got[~pad], ref_out[~pad])
    print("exempt rows:", n_exempt, e, flush=True)
