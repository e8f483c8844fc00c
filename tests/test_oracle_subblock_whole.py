"""Pins of the oracle's whole-sequence SubBlock router and of its fine step
over per-tile key lists (SGLang Diffusion benchmark page, section "How
SubBlock Sparse Attention Works": the sequence is cut into 64-token blocks,
every query block ranks the key blocks of its row, and the kept blocks go to
the block-sparse kernel).  Here every tile of [text | video | audio] is a
query tile and a candidate key tile, so text and audio keys compete like any
other; nothing is attended densely.

The pins reach outside the oracle: the exact softmax mass of token-level
inputs whose rows are constant inside each 16-token piece (now over all
blocks, text and audio included), a matrix-form statement with scipy's
logsumexp and a plain sort, agreement with the separately pinned video mode
on video-only sequences, the dense case (sparsity 0) against torch's
scaled_dot_product_attention, and a token-mask brute force for arbitrary
key-tile lists."""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from tests import _bruteforce as bf

T, D = 64, 128
ALPHA = 1.0 / np.sqrt(128.0)


def _bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _widen(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("n,sp,want", [
    (1166, 0.75, 288),   # 291.5 tiles -> 36.44 groups of 8 -> 36 groups
    (1166, 0.80, 232),   # 233.2 -> 29.15 groups -> 29
    (591, 0.75, 144),    # the 5 s shape: 147.75 -> 18.47 groups -> 18
    (20, 0.5, 8),        # 10 tiles -> 1.25 groups -> 1
    (6, 0.5, 6),         # fewer tiles than a group: all of them
])
def test_kept_count_over_all_tiles(n, sp, want):
    assert oracle.subblock_count(n, sp) == want
    q = np.zeros((T * n, 1, D), np.uint16)
    assert oracle.subblock_select_whole(q, q, 0, T * n, 0, sp)["k"] == want


def test_score_is_log_softmax_mass_for_constant_pieces_over_all_blocks():
    """Rows constant inside every 16-token piece of every tile (text, video
    and audio): score(u, w) = log(sum of exp(alpha q_i . k_j) over the 64 x 64
    token pairs of tiles u and w) - log(256), for all N x N tile pairs."""
    rng = np.random.default_rng(21)
    h, n_t, n_v, n_a = 2, 2, 4, 1
    s = T * (n_t + n_v + n_a)
    qk = []
    for _ in range(2):
        piece = rng.standard_normal((s // 16, h, D)).astype(np.float32)
        qk.append(_bits(np.repeat(piece, 16, axis=0)))
    q, k = qk
    r = oracle.subblock_select_whole(q, k, T * n_t, T * n_v, T * n_a, 0.5, want_scores=True)
    n = n_t + n_v + n_a
    Q, K = _widen(q), _widen(k)
    for hh in range(h):
        Qt = Q[:, hh].reshape(n, T, D)
        Kt = K[:, hh].reshape(n, T, D)
        for u in range(n):
            for w in range(n):
                mass = np.exp(ALPHA * (Qt[u] @ Kt[w].T)).sum()
                want = np.log(mass) - np.log(256.0)
                got = r["scores"][hh, u, w]
                assert abs(got - want) <= 1e-12 * max(1.0, abs(want)), (hh, u, w, got, want)


def test_matches_matrix_form_over_the_whole_sequence():
    rng = np.random.default_rng(22)
    h, n_t, n_v, n_a = 2, 3, 19, 2
    s = T * (n_t + n_v + n_a)
    n = s // T
    q = _bits(rng.standard_normal((s, h, D)))
    k = _bits(rng.standard_normal((s, h, D)) * 1.5)
    for sp in (0.75, 0.5):
        r = oracle.subblock_select_whole(q, k, T * n_t, T * n_v, T * n_a, sp, want_scores=True)
        kk = r["k"]
        assert kk == oracle.subblock_count(n, sp)
        for hh in range(h):
            subs = [_widen(x[:, hh]).reshape(n, 4, 16, D).mean(axis=2).astype(np.float32)
                    .astype(np.float64) for x in (q, k)]
            qs, ks = subs
            np.testing.assert_array_equal(r["qsub"][hh], qs.astype(np.float32))
            np.testing.assert_array_equal(r["ksub"][hh], ks.astype(np.float32))
            score = logsumexp((ALPHA * np.einsum("uad,wbd->uwab", qs, ks)).reshape(n, n, 16),
                              axis=2)
            np.testing.assert_allclose(r["scores"][hh], score, rtol=1e-13, atol=1e-13)
            for u in range(n):
                order = sorted(range(n), key=lambda w: (-score[u, w], w))
                assert r["sel"][hh, u].tolist() == sorted(order[:kk])


def test_video_only_sequence_equals_the_video_mode():
    """With no text or audio tiles the two candidate sets coincide: the same
    scores and the same selection as the (separately pinned) video mode."""
    rng = np.random.default_rng(23)
    h, n_v = 3, 30
    s = T * n_v
    q, k = (_bits(rng.standard_normal((s, h, D))) for _ in range(2))
    whole = oracle.subblock_select_whole(q, k, 0, s, 0, 0.7, want_scores=True)
    video = oracle.subblock_select(q, k, 0, s, 0, 0.7, want_scores=True)
    np.testing.assert_array_equal(whole["sel"], video["sel"])
    np.testing.assert_array_equal(whole["scores"], video["scores"])


def test_text_and_audio_tiles_compete():
    """Unlike the video mode, a text or audio key tile is kept only when it
    scores: with k = 8 of 12 tiles, a text key tile made strongly repulsive
    (its keys point against every query) is dropped by every query tile, an
    audio key tile made strongly attractive is kept by every one, and text
    query tiles are routed as well."""
    rng = np.random.default_rng(24)
    h, n_t, n_v, n_a = 1, 2, 9, 1
    s = T * (n_t + n_v + n_a)
    e = np.zeros(D, np.float32)
    e[:8] = 1.0
    qf = rng.standard_normal((s, h, D)).astype(np.float32) * 0.25 + e
    kf = rng.standard_normal((s, h, D)).astype(np.float32) * 0.25
    kf[0:T] -= 6.0 * e            # text tile 0: repulsive
    kf[s - T:s] += 6.0 * e        # audio tile 11: attractive
    q, k = _bits(qf), _bits(kf)
    r = oracle.subblock_select_whole(q, k, T * n_t, T * n_v, T * n_a, 0.4)
    assert r["k"] == 8
    sel = r["sel"][0]
    assert sel.shape == (12, 8)
    assert not np.any(sel == 0) and np.all(np.any(sel == 11, axis=1))
    assert np.all(np.diff(sel, axis=1) > 0)


def test_dense_case_is_softmax_attention():
    """Sparsity 0 keeps every tile: the fine step over the router's lists is
    plain softmax attention, checked against torch's SDPA in float64 on CPU."""
    rng = np.random.default_rng(25)
    h, n = 2, 7
    s = T * n
    q, k, v = (_bits(rng.standard_normal((s, h, D))) for _ in range(3))
    r = oracle.subblock_select_whole(q, k, T, T * 5, T, 0.0)
    assert r["k"] == n
    np.testing.assert_array_equal(r["sel"], np.broadcast_to(np.arange(n), (h, n, n)))
    _, got = oracle.fine_lists(q, k, v, r["sel"], np.arange(s))
    Q, K, V = (torch.from_numpy(_widen(x)).permute(1, 0, 2).unsqueeze(0) for x in (q, k, v))
    want = torch.nn.functional.scaled_dot_product_attention(Q, K, V)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_fine_lists_matches_token_mask_brute_force():
    """Arbitrary distinct key-tile lists per (head, query tile), including
    the router's own: the oracle's fine step equals dense attention under the
    explicit token-level mask of tests/_bruteforce.py."""
    rng = np.random.default_rng(26)
    h, n = 2, 9
    s = T * n
    q, k, v = (_bits(rng.standard_normal((s, h, D))) for _ in range(3))
    lists = np.stack([np.stack([np.sort(rng.choice(n, size=4, replace=False)) for _ in range(n)])
                      for _ in range(h)]).astype(np.int32)
    _, got = oracle.fine_lists(q, k, v, lists, np.arange(s))
    np.testing.assert_allclose(got, bf.dense_masked_lists(q, k, v, lists), rtol=1e-10, atol=1e-12)
    r = oracle.subblock_select_whole(q, k, T, T * 7, T, 0.3)
    _, got = oracle.fine_lists(q, k, v, r["sel"], np.arange(s))
    np.testing.assert_allclose(got, bf.dense_masked_lists(q, k, v, r["sel"]), rtol=1e-10,
                               atol=1e-12)


def test_ties_take_lower_index_across_segments():
    """Copies of one key tile in the text, video and audio segments score
    alike; at the cut the lower global index wins."""
    rng = np.random.default_rng(27)
    h, n_t, n_v, n_a = 2, 2, 8, 2
    s = T * (n_t + n_v + n_a)
    n = s // T
    q = _bits(rng.standard_normal((s, h, D)))
    kf = rng.standard_normal((s, h, D)).astype(np.float32)
    for w in (5, 11):
        kf[T * w: T * w + T] = kf[T * 1: T * 1 + T]
    k = _bits(kf)
    r = oracle.subblock_select_whole(q, k, T * n_t, T * n_v, T * n_a, 0.4, want_scores=True)
    kk = r["k"]
    assert kk == 8
    for hh in range(h):
        for u in range(n):
            sc = r["scores"][hh, u]
            assert sc[1] == sc[5] == sc[11]
            order = sorted(range(n), key=lambda x: (-sc[x], x))
            assert r["sel"][hh, u].tolist() == sorted(order[:kk])
            taken = [x for x in (1, 5, 11) if x in r["sel"][hh, u]]
            assert taken == [1, 5, 11][:len(taken)]


def test_row_subset_matches_all_rows():
    rng = np.random.default_rng(28)
    h, n = 3, 14
    s = T * n
    q, k = (_bits(rng.standard_normal((s, h, D))) for _ in range(2))
    full = oracle.subblock_select_whole(q, k, T, T * 12, T, 0.6, want_scores=True)
    rows = [(2, 13), (0, 0), (1, 7), (2, 3)]
    part = oracle.subblock_select_whole_rows(q, k, T, T * 12, T, 0.6, rows)
    for i, (hh, u) in enumerate(rows):
        np.testing.assert_array_equal(part["sel"][i], full["sel"][hh, u])
        np.testing.assert_array_equal(part["scores"][i], full["scores"][hh, u])
