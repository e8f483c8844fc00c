"""Pins of the oracle's SubBlock router (SGLang Diffusion benchmark page,
section "How SubBlock Sparse Attention Works").  The rule, restated: tiles of
64 tokens are cut into four 16-token pieces on the query and on the key side;
a log-sum-exp over the 16 scaled dot products of piece means scores each
(query tile, key tile) pair as an estimate of the key tile's unnormalised
softmax weight; each query tile keeps its best-scoring key tiles, a whole
multiple of 8 of them.

The pins do not retype the oracle's loops: the score is checked against the
exact softmax mass of token-level inputs whose rows are constant inside each
sub-block (where the estimate is exact up to the factor 16 x 16), against the
already pinned tile-score rule when the four sub-blocks of a tile share one
mean, against a matrix-form statement with scipy's logsumexp, and for ties
and the rounding of the kept count by hand."""
import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from tests import _bruteforce as bf

T, D = 64, 128
ALPHA = 1.0 / np.sqrt(128.0)


def _bits(x):
    """float array -> bfloat16 bits (values chosen exactly representable)."""
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _widen(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("n_v,sp,want", [
    (1134, 0.75, 280),   # 283.5 tiles kept -> 35.44 groups of 8 -> 35 groups
    (1134, 0.80, 224),   # 226.8 -> 28.35 groups -> 28
    (1134, 0.90, 112),   # 113.4 -> 14.2 groups -> 14
    (640, 0.75, 160),    # exactly 20 groups
    (16, 0.75, 8),       # 4 tiles kept -> 0.5 groups -> rounds up to 1
    (16, 0.95, 8),       # 0.8 tiles -> 0 groups -> at least one group
    (5, 0.75, 5),        # fewer tiles than a group: all of them
    (100, 0.0, 100),     # 12.5 -> 13 groups = 104 -> at most n_v
    (0, 0.5, 0),
])
def test_kept_count(n_v, sp, want):
    assert oracle.subblock_count(n_v, sp) == want
    assert want % 8 == 0 or want == n_v


@pytest.mark.parametrize("sp", [1.0, -0.1, float("nan"), 1.5])
def test_kept_count_rejects(sp):
    assert oracle.subblock_count(64, sp) == -1


def _subblock_constant_inputs(rng, h, n_t, n_v, n_a):
    """q, k whose 16 rows inside every 16-token sub-block are equal (random
    bf16 values per sub-block), so every sub-block mean is that row."""
    s = T * (n_t + n_v + n_a)
    out = []
    for _ in range(2):
        sub = rng.standard_normal((s // 16, h, D)).astype(np.float32)
        out.append(_bits(np.repeat(sub, 16, axis=0)))
    return out


def test_score_is_log_softmax_mass_for_constant_subblocks():
    """Rows constant inside each sub-block: the estimate is exact.  The mass
    sum over query rows i of block u and key rows j of block w of
    exp(alpha q_i . k_j) equals 256 * sum over sub-block pairs, so
    score(u, w) = log(mass(u, w)) - log(256), computed here from the tokens."""
    rng = np.random.default_rng(11)
    h, n_t, n_v, n_a = 2, 1, 5, 1
    q, k = _subblock_constant_inputs(rng, h, n_t, n_v, n_a)
    r = oracle.subblock_select(q, k, T * n_t, T * n_v, T * n_a, 0.5, want_scores=True)
    Q, K = _widen(q), _widen(k)
    s_t = T * n_t
    for hh in range(h):
        Qv = Q[s_t:s_t + T * n_v, hh].reshape(n_v, T, D)
        Kv = K[s_t:s_t + T * n_v, hh].reshape(n_v, T, D)
        for u in range(n_v):
            for w in range(n_v):
                mass = np.exp(ALPHA * (Qv[u] @ Kv[w].T)).sum()
                want = np.log(mass) - np.log(256.0)
                got = r["scores"][hh, u, w]
                assert abs(got - want) <= 1e-12 * max(1.0, abs(want)), (hh, u, w, got, want)


def test_equal_subblock_means_reduce_to_tile_score():
    """If the four sub-blocks of every tile have one mean (each sub-block
    holds the same 16 rows, in a different order), all 16 logits of a pair
    equal alpha * (tile mean Q . tile mean K), so score = log 16 + alpha *
    s(u, w) with s the pinned tile score, and the selection is the tile-score
    selection with the same k."""
    rng = np.random.default_rng(12)
    h, n_t, n_v, n_a = 3, 1, 24, 1
    s = T * (n_t + n_v + n_a)
    qk = []
    for _ in range(2):
        base = rng.standard_normal((s // T, 16, h, D)).astype(np.float32)
        blocks = [base[:, rng.permutation(16)] for _ in range(4)]
        qk.append(_bits(np.concatenate(blocks, axis=1).reshape(s, h, D)))
    q, k = qk
    v = q  # the coarse branch is not compared here
    r = oracle.subblock_select(q, k, T * n_t, T * n_v, T * n_a, 0.75, want_scores=True)
    kk = r["k"]
    assert kk == 8
    main = oracle.select_coarse(q, k, v, T * n_t, T * n_v, T * n_a, kk / n_v, want_scores=True)
    assert main["k"] == kk
    np.testing.assert_array_equal(r["sel"], main["sel"])
    want = np.log(16.0) + ALPHA * main["scores"]
    np.testing.assert_allclose(r["scores"], want, rtol=1e-13, atol=1e-13)


def test_matches_matrix_form_on_random_inputs():
    """Random bf16 inputs: sub-block means (numpy, float64 then float32),
    logits as a matrix product, scipy's logsumexp over each 4 x 4 block, and
    the ranking (score desc, index asc) by a plain sort."""
    rng = np.random.default_rng(13)
    h, n_t, n_v, n_a = 2, 2, 37, 1
    s = T * (n_t + n_v + n_a)
    q = _bits(rng.standard_normal((s, h, D)))
    k = _bits(rng.standard_normal((s, h, D)) * 2.0)
    for sp in (0.75, 0.5, 0.9):
        r = oracle.subblock_select(q, k, T * n_t, T * n_v, T * n_a, sp, want_scores=True)
        kk = r["k"]
        s_t = T * n_t
        for hh in range(h):
            subs = []
            for x in (q, k):
                X = _widen(x[s_t:s_t + T * n_v, hh]).reshape(n_v, 4, 16, D)
                subs.append(X.mean(axis=2).astype(np.float32).astype(np.float64))
            qs, ks = subs
            np.testing.assert_array_equal(r["qsub"][hh], qs.astype(np.float32))
            np.testing.assert_array_equal(r["ksub"][hh], ks.astype(np.float32))
            logits = ALPHA * np.einsum("uad,wbd->uwab", qs, ks)
            score = logsumexp(logits.reshape(n_v, n_v, 16), axis=2)
            np.testing.assert_allclose(r["scores"][hh], score, rtol=1e-13, atol=1e-13)
            for u in range(n_v):
                order = sorted(range(n_v), key=lambda w: (-score[u, w], w))
                assert r["sel"][hh, u].tolist() == sorted(order[:kk])
                assert r["kth"][hh, u] == pytest.approx(score[u, order[kk - 1]], rel=1e-13)


def test_dominant_pair_and_subblock_position():
    """One sub-block pair far above the rest dominates the log-sum-exp: q rows
    16a..16a+15 of tile u and k rows 16b..16b+15 of tile w share a direction
    e, every other row is zero.  Then score(u, w) = log(15 + exp(alpha c)),
    with c = |e|^2 (times the key scale), every other pair scores log 16, and
    moving the planted rows to another sub-block moves nothing else."""
    h, n_v = 1, 20
    s = T * n_v
    u, w = 4, 13
    e = np.zeros(D, np.float32)
    e[:16] = 1.0
    for a, b in [(0, 0), (2, 3), (3, 1)]:
        q = np.zeros((s, h, D), np.float32)
        k = np.zeros((s, h, D), np.float32)
        q[T * u + 16 * a: T * u + 16 * a + 16, 0] = e
        k[T * w + 16 * b: T * w + 16 * b + 16, 0] = 4.0 * e
        r = oracle.subblock_select(_bits(q), _bits(k), 0, s, 0, 0.5, want_scores=True)
        assert r["k"] == 8
        sc = r["scores"][0]
        c = 4.0 * 16.0
        assert sc[u, w] == pytest.approx(np.log(15.0 + np.exp(ALPHA * c)), rel=1e-14)
        others = np.ones_like(sc, dtype=bool)
        others[u, w] = False
        np.testing.assert_allclose(sc[others], np.log(16.0), rtol=1e-15)
        # equal scores keep the lowest indices; row u keeps w and tiles 0..6
        assert r["sel"][0, 0].tolist() == list(range(8))
        assert r["sel"][0, u].tolist() == list(range(7)) + [w]


def test_ties_take_lower_index():
    """Key tiles with identical content score identically; at the cut the
    lower index wins.  Tiles 2, 5, 9 of 12 are copies of one tile, k = 8."""
    rng = np.random.default_rng(14)
    h, n_v = 2, 12
    s = T * n_v
    q = _bits(rng.standard_normal((s, h, D)))
    kf = rng.standard_normal((s, h, D)).astype(np.float32)
    for w in (5, 9):
        kf[T * w: T * w + T] = kf[T * 2: T * 2 + T]
    k = _bits(kf)
    r = oracle.subblock_select(q, k, 0, s, 0, 0.3, want_scores=True)
    kk = r["k"]
    assert kk == 8
    for hh in range(h):
        for u in range(n_v):
            sc = r["scores"][hh, u]
            assert sc[2] == sc[5] == sc[9]
            order = sorted(range(n_v), key=lambda x: (-sc[x], x))
            assert r["sel"][hh, u].tolist() == sorted(order[:kk])
            # the copies straddle the cut in some rows: then the lower ones win
            taken = [x for x in (2, 5, 9) if x in r["sel"][hh, u]]
            assert taken == [2, 5, 9][:len(taken)]


def test_fine_with_router_selection_matches_dense_masked():
    """The router's selection fed to the oracle's fine branch with a zero
    coarse term is dense attention over text, audio and the selected video
    tiles (matrix-form statement in tests/_bruteforce.py)."""
    rng = np.random.default_rng(15)
    h, n_t, n_v, n_a = 2, 1, 9, 1
    s_t, s_v, s_a = T * n_t, T * n_v, T * n_a
    s = s_t + s_v + s_a
    q, k, v = (_bits(rng.standard_normal((s, h, D))) for _ in range(3))
    r = oracle.subblock_select(q, k, s_t, s_v, s_a, 0.2)
    assert r["k"] == 8
    zero_gate = np.zeros((s, h, D), np.uint16)
    _, got = oracle.fine(q, k, v, zero_gate, s_t, s_v, s_a, r["sel"],
                         np.zeros((h, n_v, D)), np.arange(s))
    want = bf.dense_masked_given_sel(q, k, v, s_t, s_v, s_a, r["sel"])
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_row_subset_matches_all_rows():
    rng = np.random.default_rng(16)
    h, n_v = 3, 21
    s = T * (n_v + 2)
    q, k = (_bits(rng.standard_normal((s, h, D))) for _ in range(2))
    full = oracle.subblock_select(q, k, T, T * n_v, T, 0.6, want_scores=True)
    rows = [(2, 20), (0, 0), (1, 7), (2, 3)]
    part = oracle.subblock_select_rows(q, k, T, T * n_v, T, 0.6, rows)
    for i, (hh, u) in enumerate(rows):
        np.testing.assert_array_equal(part["sel"][i], full["sel"][hh, u])
        np.testing.assert_array_equal(part["scores"][i], full["scores"][hh, u])
    np.testing.assert_array_equal(part["qsub"], full["qsub"])
