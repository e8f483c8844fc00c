"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Method: page "UniServe: serving FastH3 at its fastest" -- "The FastH3
workload" (tiles of 64, dense text/audio rows, top 20% video tiles, coarse
branch over mean-pooled tiles), "Fused attention preprocessing" (FP32 pooled
statistics), "Fused output combination" (output = fine + gate * coarse),
"Setup" (exact top-k).  Each test names the mistake it is there to catch.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from tests._bruteforce import vsa_dense_masked, widen

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

HERE = os.path.dirname(os.path.abspath(__file__))
D = 128
T = 64
BF16_NEG_INF = np.uint16(0xFF80)
BF16_POS_INF = np.uint16(0x7F80)


def bits(x) -> np.ndarray:
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def rand_inputs(seed, h, s_t, s_v, s_a):
    return synth.vsa_inputs(seed, h, s_t, s_v, s_a)


# --------------------------------------------------------------------------
# k = number of selected tiles
# --------------------------------------------------------------------------

def test_topk_count_golden(oracle_mod):
    """Catches: banker's rounding, truncation, no clamp to >= 1."""
    with open(os.path.join(HERE, "golden", "topk_counts.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        assert oracle_mod.topk_count(c["n_v"], c["frac"]) == c["k"], c
    for bad in g["invalid_fracs"]:
        assert oracle_mod.topk_count(10, float(bad)) == -1


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def test_bf16_rounding_matches_torch_on_float32_values(oracle_mod):
    """Catches: truncation instead of round-to-nearest-even, wrong subnormal
    quantum, wrong overflow.  torch's float32 -> bfloat16 is the textbook
    round-to-nearest-even conversion."""
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(2000).astype(np.float32),
        (rng.standard_normal(500) * 1e-39).astype(np.float32),   # float32 subnormals
        (rng.standard_normal(500) * 3e38).astype(np.float32),    # near overflow
        np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 1.01171875, 3.3895314e38], np.float32),
    ])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle_mod.bf16_from_f64(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_rounding_single_rounding_from_f64(oracle_mod):
    """1 + 2^-8 + 2^-40 lies just above the midpoint of 1 and 1 + 2^-7: one
    rounding gives 1 + 2^-7; rounding through float32 first would give 1."""
    assert oracle_mod.bf16_from_f64(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert oracle_mod.bf16_from_f64(1.0 + 2.0 ** -8) == 0x3F80          # tie -> even
    assert oracle_mod.bf16_from_f64(1.0 + 3 * 2.0 ** -8) == 0x3F82      # tie -> even (up)
    assert oracle_mod.bf16_from_f64(float("inf")) == 0x7F80
    assert oracle_mod.bf16_from_f64(-float("inf")) == 0xFF80


# --------------------------------------------------------------------------
# pooling
# --------------------------------------------------------------------------

def test_pool_designed_tile_values(oracle_mod):
    """Catches: pooling the wrong rows (missing text offset, wrong tile
    stride) or the wrong head.  Token value = tile index + head/4, so each
    tile mean is known exactly."""
    h, s_t, s_v = 3, 128, 64 * 6
    s = s_t + s_v + 64
    x = np.zeros((s, h, D), np.float32)
    for row in range(s):
        for hh in range(h):
            x[row, hh, :] = (row // T) + hh / 4
    pooled = oracle_mod.pool(bits(x), s_t, s_v // T)
    for hh in range(h):
        for u in range(s_v // T):
            assert np.all(pooled[hh, u] == np.float32(s_t // T + u + hh / 4))


def test_pool_is_rounded_exact_mean(oracle_mod):
    """The pooled statistic is the exact mean rounded once to float32."""
    x = rand_inputs(3, 2, 64, 64 * 4, 0)["k"]
    pooled = oracle_mod.pool(x, 64, 4)
    from fractions import Fraction
    xf = widen(x)
    for hh in range(2):
        for u in range(4):
            for d in (0, 17, 127):
                exact = sum(Fraction(float(t)) for t in xf[64 + 64 * u: 64 + 64 * u + 64, hh, d]) / 64
                assert pooled[hh, u, d] == np.float32(float(exact))


# --------------------------------------------------------------------------
# brute force on tiny inputs
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed,h,n_t,n_v,n_a,frac", [
    (0, 2, 1, 8, 2, 0.2),
    (1, 1, 0, 6, 0, 0.5),
    (2, 2, 2, 5, 0, 0.4),
    (3, 1, 0, 4, 1, 0.2),
    (4, 1, 1, 1, 1, 0.2),
    (5, 2, 1, 0, 1, 0.2),
    (6, 1, 0, 7, 0, 1.0),
])
def test_oracle_matches_masked_dense_bruteforce(oracle_mod, seed, h, n_t, n_v, n_a, frac):
    """Catches: wrong key set (dropped text/audio keys, wrong tile offsets),
    wrong selection, coarse on text/audio rows, several softmaxes instead of
    one, wrong gate."""
    s_t, s_v, s_a = n_t * T, n_v * T, n_a * T
    x = rand_inputs(seed, h, s_t, s_v, s_a)
    r = oracle_mod.forward(x["q"], x["k"], x["v"], x["gate"], s_t, s_v, s_a, frac)
    kk = r["k"]
    ref, sel, coarse, _ = vsa_dense_masked(x["q"], x["k"], x["v"], x["gate"], s_t, s_v, s_a, kk)
    if n_v:
        assert np.array_equal(r["sel"], sel)
        np.testing.assert_allclose(r["coarse"], coarse, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["out_f64"], ref, rtol=1e-11, atol=1e-12)
    # bf16 output is the float64 output rounded once
    again = np.array([oracle_mod.bf16_from_f64(v) for v in r["out_f64"].ravel()[:512]], np.uint16)
    assert np.array_equal(again, r["out"].ravel()[:512])


def test_selection_bruteforce_full_sort(oracle_mod):
    """Selection against an independent full sort of (score, index) pairs,
    with the oracle's own scores, on many rows."""
    s_t, s_v = 64, 64 * 40
    x = rand_inputs(11, 2, s_t, s_v, 0)
    r = oracle_mod.select_coarse(x["q"], x["k"], x["v"], s_t, s_v, 0, 0.2, want_scores=True)
    kk = r["k"]
    assert kk == 8
    for hh in range(2):
        for u in range(40):
            sc = r["scores"][hh, u]
            order = np.lexsort((np.arange(40), -sc))
            assert list(r["sel"][hh, u]) == sorted(order[:kk].tolist())
            assert r["kth"][hh, u] == sc[order[kk - 1]]


# --------------------------------------------------------------------------
# special cases that reduce to a library routine
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n_t,n_v,n_a,h", [(1, 6, 1, 2), (0, 5, 0, 1), (2, 3, 2, 1)])
def test_topk_one_is_dense_attention_sdpa(oracle_mod, n_t, n_v, n_a, h):
    """topk_frac = 1 keeps every tile: the fine branch is plain softmax
    attention with scale 1/sqrt(128).  With the gate at -inf the coarse term
    vanishes, so the output equals torch's scaled_dot_product_attention
    (float64, CPU).  Catches: wrong softmax scale, missing keys."""
    s_t, s_v, s_a = n_t * T, n_v * T, n_a * T
    x = rand_inputs(21 + n_v, h, s_t, s_v, s_a)
    g = np.full_like(x["gate"], BF16_NEG_INF)
    r = oracle_mod.forward(x["q"], x["k"], x["v"], g, s_t, s_v, s_a, 1.0)
    assert r["k"] == n_v
    assert np.array_equal(r["sel"], np.broadcast_to(np.arange(n_v), (h, n_v, n_v)))
    Q, K, V = (torch.from_numpy(widen(x[n]).transpose(1, 0, 2).copy()) for n in ("q", "k", "v"))
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V).numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(r["out_f64"], ref, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_constant_v_closed_form(oracle_mod):
    """V == c everywhere: fine output is c and the coarse output is c, so a
    video row is c * (1 + sigmoid(G)) and a text/audio row is c.  Catches: a
    dropped coarse term, coarse added to text/audio rows, a wrong gate."""
    h, s_t, s_v, s_a = 2, 64, 64 * 5, 64
    x = rand_inputs(7, h, s_t, s_v, s_a)
    c = np.array([0.75, -1.5], np.float32)
    v = bits(np.broadcast_to(c[None, :, None], x["v"].shape))
    r = oracle_mod.forward(x["q"], x["k"], v, x["gate"], s_t, s_v, s_a, 0.4)
    G = widen(x["gate"])
    expect = np.broadcast_to(c[None, :, None].astype(np.float64), G.shape).copy()
    vid = slice(s_t, s_t + s_v)
    expect[vid] = expect[vid] * (1.0 + 1.0 / (1.0 + np.exp(-G[vid])))
    np.testing.assert_allclose(r["out_f64"], expect, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(r["coarse"], np.broadcast_to(c[:, None, None], r["coarse"].shape),
                               rtol=1e-14)


def test_zero_query_closed_form_and_tie_break(oracle_mod):
    """Q == 0: all scores tie, so the selection is tiles {0..k-1} (ties to the
    lower index); the fine output is the plain mean of V over the key set and
    the coarse output is the plain mean of the pooled V."""
    h, s_t, s_v, s_a = 1, 64, 64 * 10, 128
    x = rand_inputs(8, h, s_t, s_v, s_a)
    q = np.zeros_like(x["q"])
    g = np.full_like(x["gate"], BF16_NEG_INF)
    r = oracle_mod.forward(q, x["k"], x["v"], g, s_t, s_v, s_a, 0.3)
    kk = r["k"]
    assert kk == 3
    assert np.array_equal(r["sel"][0], np.broadcast_to(np.arange(kk), (10, kk)))
    V = widen(x["v"])[:, 0, :]
    keys = np.r_[0:s_t, s_t:s_t + kk * T, s_t + s_v:s_t + s_v + s_a]
    np.testing.assert_allclose(r["out_f64"][s_t + 5, 0], V[keys].mean(axis=0), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["out_f64"][0, 0], V.mean(axis=0), rtol=1e-12, atol=1e-14)
    vbar = r["vbar"][0].astype(np.float64)
    np.testing.assert_allclose(r["coarse"][0], np.broadcast_to(vbar.mean(axis=0), (10, D)),
                               rtol=1e-12, atol=1e-14)


def test_single_video_tile_coarse_is_pooled_v(oracle_mod):
    """n_v = 1: the coarse softmax has one entry, so c = vbar_0 exactly."""
    x = rand_inputs(9, 2, 64, 64, 64)
    r = oracle_mod.select_coarse(x["q"], x["k"], x["v"], 64, 64, 64, 0.2)
    assert r["k"] == 1 and np.all(r["sel"] == 0)
    assert np.array_equal(r["coarse"], r["vbar"].astype(np.float64))


def test_two_tile_coarse_logistic(oracle_mod):
    """Two video tiles with pooled keys 0 and b*e0 and pooled query a*e0: the
    coarse weights are the logistic function of a*b/sqrt(128).  Catches a
    wrong or missing scale in the coarse softmax and a swapped weight."""
    h, s_v = 1, 128
    q = np.zeros((s_v, h, D), np.float32)
    k = np.zeros_like(q)
    v = np.zeros_like(q)
    q[:, 0, 0] = 2.0
    k[64:, 0, 0] = 3.0
    v[:64, 0, :] = 1.0
    v[64:, 0, :] = -2.0
    r = oracle_mod.select_coarse(bits(q), bits(k), bits(v), 0, s_v, 0, 0.5)
    w1 = 1.0 / (1.0 + math.exp(-6.0 / math.sqrt(128.0)))
    expect = (1.0 - w1) * 1.0 + w1 * (-2.0)
    np.testing.assert_allclose(r["coarse"][0], expect, rtol=1e-14)
    assert np.array_equal(r["sel"][0], [[1], [1]])  # the tile with the larger score


@pytest.mark.parametrize("gate_bits,sig", [(BF16_NEG_INF, 0.0), (np.uint16(0), 0.5),
                                           (BF16_POS_INF, 1.0)])
def test_gate_extremes(oracle_mod, gate_bits, sig):
    """sigmoid(-inf) = 0, sigmoid(0) = 1/2, sigmoid(+inf) = 1: catches a wrong
    sign in the gate or a gate without the sigmoid."""
    h, s_t, s_v, s_a = 1, 64, 64 * 4, 64
    x = rand_inputs(10, h, s_t, s_v, s_a)
    g = np.full_like(x["gate"], gate_bits)
    g_off = np.full_like(x["gate"], BF16_NEG_INF)
    r = oracle_mod.forward(x["q"], x["k"], x["v"], g, s_t, s_v, s_a, 0.5)
    r0 = oracle_mod.forward(x["q"], x["k"], x["v"], g_off, s_t, s_v, s_a, 0.5)
    vid = slice(s_t, s_t + s_v)
    c_rows = np.repeat(r["coarse"][0], T, axis=0)
    np.testing.assert_allclose(r["out_f64"][vid, 0], r0["out_f64"][vid, 0] + sig * c_rows,
                               rtol=1e-14, atol=1e-15)
    assert np.array_equal(r["out_f64"][:s_t], r0["out_f64"][:s_t])


# --------------------------------------------------------------------------
# designed rankings
# --------------------------------------------------------------------------

@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_designed_ranking(oracle_mod, sign):
    """Pooled key of tile w is (w+1)/16 * e0 and the pooled query is
    sign * e0: the top tiles are the highest indices for sign +1 and the
    lowest for sign -1.  Catches: reversed order, pooled Q and K swapped
    (then every score of a row ties), a text offset missing from pooling."""
    h, s_t, n_v = 1, 64, 15
    s_v = n_v * T
    x = rand_inputs(12, h, s_t, s_v, 64)
    q = np.zeros((s_t + s_v + 64, h, D), np.float32)
    k = np.zeros_like(q)
    q[s_t:s_t + s_v, 0, 0] = sign
    for w in range(n_v):
        k[s_t + w * T: s_t + (w + 1) * T, 0, 0] = (w + 1) / 16
    r = oracle_mod.select_coarse(bits(q), bits(k), x["v"], s_t, s_v, 64, 0.2)
    kk = r["k"]
    assert kk == 3
    want = np.arange(n_v - kk, n_v) if sign > 0 else np.arange(kk)
    assert np.array_equal(r["sel"][0], np.broadcast_to(want, (n_v, kk)))


def test_duplicate_key_tiles_tie_to_lower_index(oracle_mod):
    """Every video key tile identical: all scores of a row tie exactly, so
    every row selects {0..k-1}."""
    h, s_v = 2, 64 * 12
    x = rand_inputs(13, h, 0, s_v, 0)
    k = np.tile(x["k"][:64], (12, 1, 1))
    r = oracle_mod.select_coarse(x["q"], k, x["v"], 0, s_v, 0, 0.25)
    assert np.array_equal(r["sel"], np.broadcast_to(np.arange(3), (h, 12, 3)))


# --------------------------------------------------------------------------
# invariances
# --------------------------------------------------------------------------

def test_heads_are_independent(oracle_mod):
    """The first two heads of a 4-head run equal a 2-head run bitwise."""
    s_t, s_v, s_a = 64, 64 * 6, 64
    x4 = rand_inputs(14, 4, s_t, s_v, s_a)
    x2 = {n: np.ascontiguousarray(a[:, :2]) for n, a in x4.items()}
    r4 = oracle_mod.forward(x4["q"], x4["k"], x4["v"], x4["gate"], s_t, s_v, s_a, 0.34)
    r2 = oracle_mod.forward(x2["q"], x2["k"], x2["v"], x2["gate"], s_t, s_v, s_a, 0.34)
    assert np.array_equal(r4["out"][:, :2], r2["out"])
    assert np.array_equal(r4["sel"][:2], r2["sel"])


def test_permuting_tokens_inside_a_tile(oracle_mod):
    """Permuting the 64 tokens of one video tile (in Q, K, V and gate)
    leaves pooled values, selection and coarse output unchanged and permutes
    the output rows of that tile."""
    h, s_t, s_v, s_a = 1, 64, 64 * 6, 64
    x = rand_inputs(15, h, s_t, s_v, s_a)
    perm = np.random.default_rng(0).permutation(T)
    idx = np.arange(s_t + s_v + s_a)
    tile = 2
    lo = s_t + tile * T
    idx[lo:lo + T] = lo + perm
    xp = {n: a[idx] for n, a in x.items()}
    r = oracle_mod.forward(x["q"], x["k"], x["v"], x["gate"], s_t, s_v, s_a, 0.34)
    rp = oracle_mod.forward(xp["q"], xp["k"], xp["v"], xp["gate"], s_t, s_v, s_a, 0.34)
    assert np.array_equal(r["sel"], rp["sel"])
    assert np.array_equal(r["coarse"], rp["coarse"])
    np.testing.assert_allclose(rp["out_f64"], r["out_f64"][idx], rtol=1e-12, atol=1e-14)


def test_fine_accepts_foreign_selection(oracle_mod):
    """The fine branch honours the selection it is given (used to compare
    another implementation's outputs on that implementation's index sets):
    a different selection changes exactly the video rows."""
    h, s_t, s_v, s_a = 1, 64, 64 * 6, 64
    x = rand_inputs(16, h, s_t, s_v, s_a)
    r = oracle_mod.forward(x["q"], x["k"], x["v"], x["gate"], s_t, s_v, s_a, 0.34)
    other = (r["sel"] + 1) % 6
    other.sort(axis=-1)
    rows = np.arange(s_t + s_v + s_a)
    ob, od = oracle_mod.fine(x["q"], x["k"], x["v"], x["gate"], s_t, s_v, s_a, other,
                             r["coarse"], rows)
    assert np.array_equal(od[:s_t], r["out_f64"][:s_t])
    assert not np.allclose(od[s_t:s_t + s_v], r["out_f64"][s_t:s_t + s_v])
