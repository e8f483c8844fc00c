"""GPU parity of the projection GEMM (Q/K/V/gate) and of the full layer
(projections, then the VSA forward) against the CPU oracle.

Projection bar: every checked element within 2^-8 of the float64 value
(relative; the bf16 result is that value after fp32 accumulation and one
rounding) plus 1e-5 of the root-sum-square of its products, which absorbs
fp32 accumulation order and nothing else: a wrong row, channel or operand
is off by O(1).
"""
import numpy as np
import pytest
import torch

import block_sparse_video_amd as bsv
import oracle
import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu
THREADS = synth.default_threads()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    torch.cuda.set_device(0)
    yield


def announce(msg):
    print(f"[case] {msg}", flush=True)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_projection(x, w, heads, got, rows):
    """got: the four GPU outputs [tokens][heads][128] (bf16 bits, numpy)."""
    ref = oracle.project_rows(x, w, rows)                       # [4][r][n]
    xf = synth.bf16_bits_to_f32(x[rows]).astype(np.float64)
    wf = synth.bf16_bits_to_f32(w).astype(np.float64)
    scale = np.stack([np.sqrt((xf ** 2) @ (wf[p] ** 2).T) for p in range(4)])
    worst = 0.0
    for p in range(4):
        g = synth.bf16_bits_to_f32(got[p].reshape(got[p].shape[0], -1)[rows]).astype(np.float64)
        err = np.abs(g - ref[p])
        bound = 1.01 * 2.0 ** -8 * np.abs(ref[p]) + 1e-5 * scale[p]
        assert np.all(err <= bound), (p, float((err / bound).max()))
        worst = max(worst, float((err / bound).max()))
    return worst


@pytest.mark.parametrize("tokens,hidden,heads,seed", [
    (1, 64, 2, 1),        # a single token
    (255, 128, 2, 2),     # one token tile, ragged
    (256, 192, 4, 3),     # exact tile
    (300, 64, 2, 4),      # two token tiles, ragged tail
    (777, 320, 6, 5),     # several tiles both ways
])
def test_projection_small_shapes(tokens, hidden, heads, seed):
    announce(f"projection tokens={tokens} hidden={hidden} heads={heads}")
    x = synth.normal_bf16(seed, synth.STREAM_X, (tokens, hidden))
    w = synth.normal_bf16(seed, synth.STREAM_W0, (4, heads * 128, hidden), std=0.05)
    outs = bsv.project_qkvg(_dev(x), _dev(w), heads)
    torch.cuda.synchronize()
    got = [_bits(t) for t in outs]
    worst = check_projection(x, w, heads, got, np.arange(tokens))
    print("worst err/bound", worst)


FULL = dict(text_len=1024, grid=(18, 48, 84), audio_len=1024, hidden=5376, heads=56)


@pytest.mark.slow
def test_full_layer_projection_and_vsa():
    """The full-layer workload: 1,024 text + 72,576 video (smooth fields over
    the 18 x 48 x 84 grid, tile-packed) + 1,024 audio tokens, hidden 5,376,
    56 heads.  Projections on sampled rows; then the VSA forward on the
    projected tensors: every selection row and the coarse branch, outputs on
    sampled rows."""
    announce("full layer: projections + VSA, 56 heads")
    d = synth.full_layer_inputs(0, threads=THREADS, **FULL)
    x, w = d["x"], d["w"]
    s_t, s_a, h = FULL["text_len"], FULL["audio_len"], FULL["heads"]
    s_v = x.shape[0] - s_t - s_a
    xd, wd = _dev(x), _dev(w)
    q, k, v, g = bsv.project_qkvg(xd, wd, h)
    torch.cuda.synchronize()
    del wd
    rows = np.array([0, 1, s_t - 1, s_t, s_t + 4097, s_t + s_v // 2, s_t + s_v - 1,
                     s_t + s_v, x.shape[0] - 1], dtype=np.int64)
    got = [_bits(t) for t in (q, k, v, g)]
    worst = check_projection(x, w, h, got, rows)
    print("projection worst err/bound", worst, flush=True)
    del x, w, d
    out, sel, ws = G.run_forward({"q": q, "k": k, "v": v, "gate": g}, s_t, s_v, s_a, 0.2)
    qb, kb, vb, gb = got
    ref = oracle.select_coarse(qb, kb, vb, s_t, s_v, s_a, 0.2, threads=THREADS)
    got_sel = sel.cpu().numpy()
    n_exempt = G.check_selection(got_sel, ref)
    wsp = G.read_workspace(ws, h, s_t, s_v, s_a)
    np.testing.assert_allclose(wsp["coarse"], ref["coarse"], rtol=2e-5, atol=2e-7)
    # Projected Q/K/V have std ~1.5, so outputs reach several units (iid
    # unit-variance inputs give rms ~0.013): the bf16 rounding of one output
    # element alone is then up to 2^-8 of it, close to 2e-2 by itself.  The
    # max-abs bar therefore applies to the error beyond each element's own
    # output rounding; mean-abs 2e-3 and the relative gate are unchanged.  The
    # summary prints the magnitudes and whether the flat bar held anyway.
    cov = G.full_size_coverage({"q": qb, "k": kb, "v": vb, "gate": gb}, out, got_sel,
                               ref["coarse"], s_t, s_v, s_a, threads=THREADS,
                               rounding_allowance=True, label="full layer")
    orow = G.sample_rows(s_t, s_v, s_a, n_video_tiles=3, per_tile=(0, 37, 63))
    _, ref_out = oracle.fine(qb, kb, vb, gb, s_t, s_v, s_a, got_sel, ref["coarse"], orow,
                             threads=THREADS)
    e = G.assert_outputs_close(G.from_dev_bits(out)[orow], ref_out, rounding_allowance=True)
    e.update(ref_rms=float(np.sqrt((ref_out ** 2).mean())))
    # smooth video fields make neighbouring query tiles choose overlapping key tiles
    s0 = got_sel[0]
    overlap = np.mean([len(np.intersect1d(s0[u], s0[u + 1])) / s0.shape[1] for u in range(0, 1000, 7)])
    print("exempt rows:", n_exempt, "sampled rows:", e, "coverage:", cov,
          "neighbour overlap:", round(float(overlap), 3), flush=True)
