"""CPU checks of the full-layer pieces: the smooth-field input generator
against an independent construction (scipy's Gaussian filter and a numpy
tile packing), and the oracle's projection against brute force and closed
forms."""
import numpy as np
import pytest
from scipy.ndimage import gaussian_filter1d

import oracle
import synth


def _f(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("grid,tile,sigma,channels", [
    ((4, 16, 8), (2, 8, 4), (1.0, 2.0, 2.0), 5),
    ((6, 8, 12), (2, 4, 4), (1.0, 1.0, 2.0), 3),
])
def test_smooth_field_matches_scipy_construction(grid, tile, sigma, channels):
    T, H, W = grid
    got = synth.smooth_field_bf16(3, grid, channels, sigma, tile)
    # white noise: element ((t*H + h)*W + w)*C + c of the field stream
    z = synth.normal_f64(3, synth.STREAM_FIELD, (T, H, W, channels))
    for ax, s in enumerate(sigma):
        z = gaussian_filter1d(z, s, axis=ax, mode="reflect", truncate=3.0)
    z = z / np.sqrt((z ** 2).mean(axis=(0, 1, 2)))
    pt, ph, pw = tile
    packed = z.reshape(T // pt, pt, H // ph, ph, W // pw, pw, channels)
    packed = packed.transpose(0, 2, 4, 1, 3, 5, 6).reshape(T * H * W, channels)
    ref = _f(synth.f32_to_bf16_bits(packed.astype(np.float32)))
    g = _f(got)
    # both sides round the same real number; allow one bf16 step for the rare
    # case where the two float64 summation orders fall on either side of a tie
    assert np.all(np.abs(g - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-30)
    assert np.mean(g == ref) > 0.999


def test_smooth_field_is_smooth_and_unit_rms():
    grid = (8, 16, 16)
    v = _f(synth.smooth_field_bf16(0, grid, 16, (1.0, 2.0, 2.0), (2, 8, 4)))
    assert np.allclose(np.sqrt((v ** 2).mean(0)), 1.0, atol=0.01)
    # inside a tile, raster neighbours along w are strongly correlated
    # (sigma_w = 2 cells), unlike iid noise
    t = v.reshape(-1, 64, 16)  # tiles of 2 x 8 x 4 = 64 points
    a, b = t[:, 0::4, :].ravel(), t[:, 1::4, :].ravel()
    assert np.corrcoef(a, b)[0, 1] > 0.7


def test_full_layer_inputs_layout():
    d = synth.full_layer_inputs(1, 64, (2, 8, 4), 64, hidden=128, heads=2)
    x, w = d["x"], d["w"]
    assert x.shape == (64 + 64 + 64, 128) and w.shape == (4, 256, 128)
    assert np.array_equal(x[:64], synth.normal_bf16(1, synth.STREAM_X, (64, 128)))
    assert np.array_equal(x[128:], synth.normal_bf16(1, synth.STREAM_X, (64, 128), offset=128 * 128))
    assert np.array_equal(x[64:128], synth.smooth_field_bf16(1, (2, 8, 4), 128))
    wf = _f(w)
    assert abs(wf.std() - 0.02) < 0.002


def test_project_rows_brute_force():
    rng = np.random.default_rng(0)
    x = synth.f32_to_bf16_bits(rng.standard_normal((5, 7)).astype(np.float32))
    w = synth.f32_to_bf16_bits(rng.standard_normal((4, 3, 7)).astype(np.float32))
    rows = [4, 0, 2]
    got = oracle.project_rows(x, w, rows)
    xf, wf = _f(x), _f(w)
    for p in range(4):
        for i, r in enumerate(rows):
            for n in range(3):
                s = 0.0
                for c in range(7):
                    s += xf[r, c] * wf[p, n, c]
                assert got[p, i, n] == pytest.approx(s, rel=1e-14, abs=1e-14)


def test_project_rows_identity_and_scaling():
    rng = np.random.default_rng(1)
    x = synth.f32_to_bf16_bits(rng.standard_normal((9, 16)).astype(np.float32))
    eye = synth.f32_to_bf16_bits(np.eye(16, dtype=np.float32))
    w = np.stack([eye, 2 * 0 + eye, eye, eye])
    w[1] = synth.f32_to_bf16_bits(2.0 * np.eye(16, dtype=np.float32))
    w[3] = synth.f32_to_bf16_bits(-np.eye(16, dtype=np.float32)[::-1].copy())
    out = oracle.project_rows(x, w, np.arange(9))
    xf = _f(x)
    assert np.array_equal(out[0], xf) and np.array_equal(out[2], xf)
    assert np.array_equal(out[1], 2 * xf)
    assert np.array_equal(out[3], -xf[:, ::-1])
