"""Pins of the oracle's padded-segment semantics and of its attention
preprocessing (Q/K RMSNorm + partial 3D RoPE), against independent
constructions: the masked dense brute force, closed forms and properties
of rotations.  Pages: "UniServe: serving FastH3 at its fastest", section
"Fused attention preprocessing" (pooling over valid tokens, padding handled
inside the kernel, learned Q/K RMSNorm, partial RoPE), and the SGLang
Diffusion benchmark page (RoPE dimension 96, norm rounded before RoPE)."""
import math

import numpy as np
import pytest

import oracle
import synth
from tests._bruteforce import vsa_dense_masked, widen

T = 64
D = 128


def rand_inputs(seed, h, s_t, s_v, s_a):
    return synth.vsa_inputs(seed, h, s_t, s_v, s_a)


@pytest.mark.parametrize("seed,h,n_t,n_v,n_a,valid,frac", [
    (1, 1, 1, 4, 1, (40, 256, 17), 0.5),     # partial text and audio tiles
    (2, 2, 2, 5, 1, (128, 300, 64), 0.4),    # partial last video tile
    (3, 1, 1, 3, 2, (1, 129, 65), 0.34),     # one valid text row; audio spills one row
    (4, 2, 0, 6, 0, (0, 321, 0), 1.0),       # video only, dense
])
def test_padded_segments_match_masked_bruteforce(seed, h, n_t, n_v, n_a, valid, frac):
    s_t, s_v, s_a = n_t * T, n_v * T, n_a * T
    x = rand_inputs(seed, h, s_t, s_v, s_a)
    sc = oracle.select_coarse(x["q"], x["k"], x["v"], s_t, s_v, s_a, frac, video_valid=valid[1])
    rows = np.arange(s_t + s_v + s_a)
    _, got = oracle.fine(x["q"], x["k"], x["v"], x["gate"], s_t, s_v, s_a, sc["sel"], sc["coarse"],
                         rows, valid=valid)
    ref, sel, coarse, _ = vsa_dense_masked(x["q"], x["k"], x["v"], x["gate"], s_t, s_v, s_a,
                                           sc["k"], valid=valid)
    assert np.array_equal(sc["sel"], sel)
    np.testing.assert_allclose(sc["coarse"], coarse, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_padding_content_is_ignored():
    """Whatever the padding rows hold, valid outputs and selections are the
    same, and padding rows output zeros."""
    h, s_t, s_v, s_a = 2, 64, 64 * 5, 64
    valid = (33, 64 * 4 + 7, 50)
    x = rand_inputs(7, h, s_t, s_v, s_a)
    y = {n: a.copy() for n, a in x.items()}
    pad = np.ones(s_t + s_v + s_a, bool)
    pad[:valid[0]] = False
    pad[s_t:s_t + valid[1]] = False
    pad[s_t + s_v:s_t + s_v + valid[2]] = False
    for n in y:
        y[n][pad] = synth.f32_to_bf16_bits(np.full(y[n][pad].shape, 3.0e4, np.float32))
    rows = np.arange(s_t + s_v + s_a)
    res = []
    for z in (x, y):
        sc = oracle.select_coarse(z["q"], z["k"], z["v"], s_t, s_v, s_a, 0.4, video_valid=valid[1])
        ob, _ = oracle.fine(z["q"], z["k"], z["v"], z["gate"], s_t, s_v, s_a, sc["sel"],
                            sc["coarse"], rows, valid=valid)
        res.append((sc["sel"], ob))
    assert np.array_equal(res[0][0], res[1][0])
    assert np.array_equal(res[0][1], res[1][1])
    assert not res[0][1][pad].any()


def test_pool_over_valid_rows_closed_form():
    # last tile has 5 valid rows with values 1..5 in every dim: mean 3
    x = np.zeros((128, 1, D), np.float32)
    x[:64] = 7.0
    x[64:69] = np.arange(1, 6, dtype=np.float32)[:, None, None]
    x[69:] = 1e6  # padding
    bits = synth.f32_to_bf16_bits(x)
    out = np.empty((1, 2, D), np.float32)
    oracle._load().vsa_oracle_pool_valid(bits.ctypes.data, 1, 0, 2, 69, out.ctypes.data, 1)
    assert np.all(out[0, 0] == 7.0) and np.all(out[0, 1] == 3.0)


def test_bf16_round_vectorised_matches_single_rounding():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))
    x[:100] = 0.0
    x[100:200] = rng.standard_normal(100) * 1e-39      # bfloat16 subnormals
    m, e = rng.integers(0, 128, 500), rng.integers(-20, 20, 500)
    ties = (128.0 + m + 0.5) * 2.0 ** (e - 7.0)         # exactly between two bfloat16 values
    for v in (x, ties):
        ref = np.array([oracle.bf16_from_f64(float(t)) for t in v], np.uint16)
        assert np.array_equal(oracle.bf16_round(v), ref)


# ---------------------------------------------------------------------------
# RMSNorm + partial 3D RoPE
# ---------------------------------------------------------------------------

GRID, TILE = (2, 8, 8), (2, 8, 4)   # 128 video tokens = 2 tiles


def _prep(x, gamma, s_t, s_v, s_a, valid):
    return oracle.rms_norm_rope(x, gamma, s_t, s_v, s_a, valid, GRID, TILE)


def test_video_positions_invert_the_generator_packing():
    pos = oracle.video_positions(GRID, TILE, 128)
    T_, Hh, Ww = GRID
    pt, ph, pw = TILE
    for i, (t, h, w) in enumerate(pos):
        tile = ((t // pt) * (Hh // ph) + h // ph) * (Ww // pw) + w // pw
        row = tile * 64 + ((t % pt) * ph + h % ph) * pw + w % pw
        assert row == i
    assert len({tuple(p) for p in pos}) == 128


def test_rms_norm_closed_form_on_text_rows():
    # text rows are normalised but never rotated
    x = np.zeros((64 + 128, 1, D), np.float32)
    x[:64] = 0.5
    x[3, 0, :64], x[3, 0, 64:] = 2.0, -2.0
    g = np.linspace(0.5, 1.5, D).astype(np.float32)[None]
    gb = synth.f32_to_bf16_bits(g)
    y = widen(_prep(synth.f32_to_bf16_bits(x), gb, 64, 128, 0, (64, 128, 0)))
    gw = widen(gb)[0]
    exp0 = oracle.bf16_round(0.5 / math.sqrt(0.25 + 1e-6) * gw)
    assert np.array_equal(synth.f32_to_bf16_bits(y[0, 0].astype(np.float32)), exp0)
    exp3 = oracle.bf16_round(np.where(np.arange(D) < 64, 1, -1) * 2.0 / math.sqrt(4.0 + 1e-6) * gw)
    assert np.array_equal(synth.f32_to_bf16_bits(y[3, 0].astype(np.float32)), exp3)


def test_rope_hand_computed_angles():
    # video token 0 sits at grid (0,0,0): no rotation.  The token at
    # (t=1, h=0, w=0) turns pair i of axis t by 10000^(-i/16) radians.
    pos = oracle.video_positions(GRID, TILE, 128)
    i1 = int(np.flatnonzero((pos == [1, 0, 0]).all(axis=1))[0])
    rng = np.random.default_rng(3)
    x = synth.f32_to_bf16_bits(rng.standard_normal((128, 1, D)).astype(np.float32))
    g = np.full((1, D), 0x3F80, np.uint16)  # gamma = 1
    y = widen(_prep(x, g, 0, 128, 0, (0, 128, 0)))
    n = widen(oracle.bf16_round(widen(x) / np.sqrt((widen(x) ** 2).mean(axis=2, keepdims=True) + 1e-6)))
    assert np.array_equal(y[0], n[0])
    for i in range(16):
        th = 10000.0 ** (-i / 16)
        a, b = n[i1, 0, 2 * i], n[i1, 0, 2 * i + 1]
        assert y[i1, 0, 2 * i] == widen(oracle.bf16_round(np.array([a * math.cos(th) - b * math.sin(th)])))[0]
        assert y[i1, 0, 2 * i + 1] == widen(oracle.bf16_round(np.array([a * math.sin(th) + b * math.cos(th)])))[0]
    # axes h and w and dims 96.. are untouched at this position
    assert np.array_equal(y[i1, 0, 32:], n[i1, 0, 32:])


def test_rope_preserves_pair_norms_and_relative_positions():
    """Rotations keep |pair| and make q(p).k(p') depend on p - p' only: the
    dot products of one pair of vectors placed at two grid points equal those
    at the two points shifted by the same offset (bfloat16-level agreement)."""
    pos = oracle.video_positions(GRID, TILE, 128)
    rng = np.random.default_rng(4)
    base_q = rng.standard_normal(D).astype(np.float32)
    base_k = rng.standard_normal(D).astype(np.float32)
    x = np.zeros((128, 2, D), np.float32)
    x[:, 0] = base_q
    x[:, 1] = base_k
    g = np.full((2, D), 0x3F80, np.uint16)
    y = widen(_prep(synth.f32_to_bf16_bits(x), g, 0, 128, 0, (0, 128, 0)))
    n = y[np.flatnonzero((pos == [0, 0, 0]).all(axis=1))[0]]  # unrotated reference
    for t in range(128):
        pr = y[t].reshape(2, -1, 2)
        nr = n.reshape(2, -1, 2)
        np.testing.assert_allclose(np.hypot(pr[..., 0], pr[..., 1]), np.hypot(nr[..., 0], nr[..., 1]),
                                   rtol=2 ** -7, atol=2 ** -12)
    def at(p):
        return int(np.flatnonzero((pos == p).all(axis=1))[0])
    pairs = [([0, 1, 2], [1, 3, 5], [0, 2, 1]), ([1, 0, 0], [0, 4, 7], [0, 3, 0])]
    for p1, p2, shift in pairs:
        a = y[at(p1), 0, :96] @ y[at(p2), 1, :96]
        b = y[at(np.add(p1, shift)), 0, :96] @ y[at(np.add(p2, shift)), 1, :96]
        assert abs(a - b) <= 2 ** -6 * max(1.0, abs(a))


def test_padding_rows_become_zero_and_audio_is_not_rotated():
    rng = np.random.default_rng(5)
    x = synth.f32_to_bf16_bits(rng.standard_normal((64 + 128 + 64, 1, D)).astype(np.float32))
    g = np.full((1, D), 0x3F80, np.uint16)
    y = _prep(x, g, 64, 128, 64, (10, 128, 20))
    assert not y[10:64].any() and not y[192 + 20:].any()
    n = oracle.bf16_round(widen(x) / np.sqrt((widen(x) ** 2).mean(axis=2, keepdims=True) + 1e-6))
    assert np.array_equal(y[192:212], n[192:212])
    assert np.array_equal(y[:10], n[:10])
