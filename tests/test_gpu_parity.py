"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Acceptance (per row): selected tiles equal the oracle's except boundary ties
within 1e-6 relative; outputs on identical index sets within max-abs 2e-2
and mean-abs 2e-3 of the oracle (bf16 outputs), plus a stricter internal
relative-RMS gate of 5e-3.  Pooled statistics are compared bit for bit.
"""
import os

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
BF16_NEG_INF = np.uint16(0xFF80)
BF16_POS_INF = np.uint16(0x7F80)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    torch.cuda.set_device(0)
    yield


def announce(msg):
    print(f"[case] {msg}", flush=True)


def full_check(x, s_t, s_v, s_a, frac, rel_rms=G.REL_RMS, exempt_ok=True):
    """Every row against the oracle; returns (ref, errors, gpu arrays)."""
    xd = G.inputs_to_dev(x)
    out, sel, ws = G.run_forward(xd, s_t, s_v, s_a, frac)
    ref = oracle.select_coarse(x["q"], x["k"], x["v"], s_t, s_v, s_a, frac, threads=THREADS)
    got_sel = sel.cpu().numpy()
    if s_v:
        G.check_selection(got_sel, ref, exempt_ok=exempt_ok)
    rows = np.arange(s_t + s_v + s_a)
    _, ref_out = oracle.fine(x["q"], x["k"], x["v"], x["gate"], s_t, s_v, s_a,
                             got_sel if s_v else None, ref["coarse"], rows, threads=THREADS)
    e = G.assert_outputs_close(G.from_dev_bits(out), ref_out, rel_rms=rel_rms)
    return ref, e, out, got_sel, ws


# --------------------------------------------------------------------------
# tiny workload: 1 head, 64 text + 1024 video + 64 audio tokens, k = 3, seed 0
# --------------------------------------------------------------------------

def test_tiny_full_parity_and_stages():
    announce("tiny 1x(64,1024,64) seed 0")
    s_t, s_v, s_a = 64, 1024, 64
    x = synth.vsa_inputs(0, 1, s_t, s_v, s_a)
    ref, e, out, sel, ws = full_check(x, s_t, s_v, s_a, 0.2, exempt_ok=False)
    assert ref["k"] == 3
    w = G.read_workspace(ws, 1, s_t, s_v, s_a)
    # pooled statistics: bitwise equal to the oracle's FP32 means
    assert np.array_equal(w["qbar64"], ref["qbar"].astype(np.float64))
    assert np.array_equal(w["kbar"], ref["kbar"])
    assert np.array_equal(w["vbar"], ref["vbar"])
    np.testing.assert_allclose(w["coarse"], ref["coarse"], rtol=2e-6, atol=1e-7)
    print(e)


@pytest.mark.parametrize("h,n_t,n_v,n_a,frac,seed", [
    (2, 1, 16, 1, 0.2, 1),
    (3, 0, 37, 0, 0.2, 2),     # video only, ragged tile count
    (2, 2, 5, 3, 0.5, 3),
    (1, 1, 1, 1, 0.2, 4),      # a single video tile
    (2, 0, 2, 1, 0.2, 5),      # k clamps to 1
    (4, 3, 70, 2, 0.3, 6),     # several select workgroups per head, ragged tail
    (1, 2, 9, 0, 1.0, 7),      # dense (k = n_v)
])
def test_small_shapes_full_parity(h, n_t, n_v, n_a, frac, seed):
    announce(f"small h={h} tiles=({n_t},{n_v},{n_a}) frac={frac} seed={seed}")
    x = synth.vsa_inputs(seed, h, n_t * T, n_v * T, n_a * T)
    full_check(x, n_t * T, n_v * T, n_a * T, frac, exempt_ok=False)


def test_no_video_tiles_is_dense_attention():
    announce("no video: h=2 tiles=(2,0,1)")
    s_t, s_a = 128, 64
    x = synth.vsa_inputs(8, 2, s_t, 0, s_a)
    xd = G.inputs_to_dev(x)
    out = torch.empty_like(xd["q"])
    ws = torch.empty(bsv.vsa_workspace_bytes(2, s_t, 0, s_a), dtype=torch.uint8, device="cuda")
    bsv.vsa_forward(xd["q"], xd["k"], xd["v"], None, s_t, 0, s_a, 0.2, out, None, ws)
    torch.cuda.synchronize()
    _, ref = oracle.fine(x["q"], x["k"], x["v"], x["gate"], s_t, 0, s_a, None, None,
                         np.arange(s_t + s_a))
    G.assert_outputs_close(G.from_dev_bits(out), ref)


# --------------------------------------------------------------------------
# structured cases
# --------------------------------------------------------------------------

def test_coarse_isolating_case():
    """Gate at +inf (sigmoid = 1) and V carrying a per-tile offset, so the
    coarse term is O(1): a path that dropped or misplaced the coarse branch
    fails by far more than the tolerance."""
    announce("coarse-isolating h=2 tiles=(1,12,1)")
    h, s_t, s_v, s_a = 2, 64, 64 * 12, 64
    x = synth.vsa_inputs(9, h, s_t, s_v, s_a)
    v = G.widen(x["v"]).astype(np.float32) * 0.25
    for u in range(12):
        v[s_t + u * T: s_t + (u + 1) * T] += (u + 1) / 8  # same sign: survives the coarse average
    x["v"] = synth.f32_to_bf16_bits(v)
    x["gate"] = np.full_like(x["gate"], BF16_POS_INF)
    ref, e, *_ = full_check(x, s_t, s_v, s_a, 0.25, exempt_ok=False)
    assert np.abs(ref["coarse"]).mean() > 0.1


def test_constant_v_and_gate_extremes():
    announce("constant V, gates -inf/0/+inf")
    h, s_t, s_v, s_a = 3, 64, 64 * 8, 64
    x = synth.vsa_inputs(10, h, s_t, s_v, s_a)
    c = np.array([0.5, -1.25, 2.0], np.float32)
    x["v"] = synth.f32_to_bf16_bits(np.broadcast_to(c[None, :, None], x["v"].shape))
    g = np.empty_like(x["gate"])
    g[:, 0], g[:, 1], g[:, 2] = BF16_NEG_INF, 0, BF16_POS_INF
    x["gate"] = g
    xd = G.inputs_to_dev(x)
    out, sel, _ = G.run_forward(xd, s_t, s_v, s_a, 0.2)
    o = G.widen(G.from_dev_bits(out))
    vid = slice(s_t, s_t + s_v)
    expect = np.broadcast_to(c[None, :, None].astype(np.float64), o.shape).copy()
    expect[vid, 1] *= 1.5
    expect[vid, 2] *= 2.0
    np.testing.assert_allclose(o, expect, rtol=8e-3, atol=0)


def test_zero_query_ties_and_duplicate_keys():
    announce("Q = 0 and duplicated K tiles: all scores tie")
    h, s_t, s_v, s_a = 2, 64, 64 * 20, 64
    x = synth.vsa_inputs(11, h, s_t, s_v, s_a)
    x0 = dict(x, q=np.zeros_like(x["q"]))
    ref, *_ = full_check(x0, s_t, s_v, s_a, 0.2, exempt_ok=False)
    assert np.array_equal(ref["sel"], np.broadcast_to(np.arange(4), (h, 20, 4)))
    kdup = x["k"].copy()
    kdup[s_t:s_t + s_v] = np.tile(x["k"][s_t:s_t + T], (20, 1, 1))
    full_check(dict(x, k=kdup), s_t, s_v, s_a, 0.2, exempt_ok=False)


def test_paired_key_tiles_tie_at_the_boundary():
    """K tiles equal in pairs: every score is tied with exactly one other, so
    with k odd the k-th and (k+1)-th largest scores tie in every row and the
    lower index must win.  Selection must match the oracle exactly."""
    announce("paired K tiles: h=2 tiles=(1,70,1) frac=0.3 (k=21)")
    h, s_t, n_v, s_a = 2, 64, 70, 64
    s_v = n_v * T
    x = synth.vsa_inputs(16, h, s_t, s_v, s_a)
    kp = x["k"].copy()
    for w in range(0, n_v, 2):
        a = s_t + w * T
        kp[a + T: a + 2 * T] = kp[a: a + T]
    ref, *_ = full_check(dict(x, k=kp), s_t, s_v, s_a, 0.3, exempt_ok=False)
    assert ref["k"] == 21


@pytest.mark.parametrize("log2_w0", [-30, -20, -14, -8])
def test_close_pairs_decided_in_float64(log2_w0):
    """K tiles equal in pairs except for one bf16 step in dimension 0 of one
    row, and every query row weights dimension 0 by w0 = 2^log2_w0: the two
    scores of a pair differ by about w0 * 2^-14 (2^-44 .. 2^-22, from far
    below the float32 resolution of the scores to several of its steps, the
    range in which the kernel's float32 score products can misorder them),
    and with k odd the selection boundary of every row falls inside such a
    pair.  The larger float64 score must win, whichever index it has.
    Selection must match the oracle exactly."""
    announce(f"close pairs 2^{log2_w0}: h=2 tiles=(1,70,1) frac=0.3 (k=21)")
    h, s_t, n_v, s_a = 2, 64, 70, 64
    s_v = n_v * T
    x = synth.vsa_inputs(23, h, s_t, s_v, s_a)
    kp, qp = x["k"].copy(), x["q"].copy()
    qp[..., 0] = synth.f32_to_bf16_bits(np.array(2.0 ** log2_w0, np.float32))
    rng = np.random.default_rng(23)
    for w in range(0, n_v, 2):
        a = s_t + w * T
        kp[a + T: a + 2 * T] = kp[a: a + T]
        bits = kp[a + T, :, 0].astype(np.int32)
        step = 1 if rng.random() < 0.5 else -1  # the next or the previous bf16 value
        step = np.where((bits & 0x7FFF) == 0, 1, step)  # never step below a zero
        kp[a + T, :, 0] = (bits + step).astype(np.uint16)
    assert np.all(np.isfinite(G.widen(kp)))
    ref, *_ = full_check(dict(x, q=qp, k=kp), s_t, s_v, s_a, 0.3, exempt_ok=False)
    assert ref["k"] == 21
    # the construction does what it says: in every row the 21st and 22nd
    # largest float64 scores differ, by less than 2^-16 of the row's largest
    # score magnitude; at the smallest weights they round to the same float32
    tied = close = 0
    for hh in range(h):
        for u in range(n_v):
            s = np.sort(oracle.row_scores(ref["qbar"], ref["kbar"], hh, u))[::-1]
            tied += int(s[20] != s[21] and np.float32(s[20]) == np.float32(s[21]))
            close += int(0 < s[20] - s[21] < 2.0 ** -16 * np.abs(s).max())
    assert close == h * n_v, close
    if log2_w0 <= -20:
        assert tied >= n_v, tied


@pytest.mark.parametrize("log2_scale", [40, 52])
def test_huge_magnitudes_rank_every_key_in_float64(log2_scale):
    """Q and K scaled by 2^40 or 2^52 (exact in bf16).  At 2^40 the float32
    scores and their error bound decide as usual; at 2^52 |Qbar_u|
    max|Kbar_w| exceeds 2^100, where the float32 score products could leave
    their range, so every row is ranked by recomputed float64 scores.
    Selection must match the oracle exactly (the coarse branch is not
    checked: float32 score rows do not hold such magnitudes to its bar)."""
    announce(f"huge magnitudes: h=2 tiles=(1,70,1) frac=0.2, Q and K x 2^{log2_scale}")
    h, s_t, n_v, s_a = 2, 64, 70, 64
    s_v = n_v * T
    x = synth.vsa_inputs(27, h, s_t, s_v, s_a)
    for n in ("q", "k"):
        x[n] = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(x[n]) * np.float32(2.0 ** log2_scale))
    xd = G.inputs_to_dev(x)
    kk = bsv.vsa_topk_count(s_v, 0.2)
    ws = torch.empty(bsv.vsa_workspace_bytes(h, s_t, s_v, s_a, 0.2), dtype=torch.uint8, device="cuda")
    sel = torch.full((h, n_v, kk), -7, dtype=torch.int32, device="cuda")
    bsv.vsa_pool_pack(xd["q"], xd["k"], xd["v"], s_t, s_v, s_a, ws)
    bsv.vsa_select_coarse(h, s_t, s_v, s_a, 0.2, sel, ws)
    torch.cuda.synchronize()
    ref = oracle.select_coarse(x["q"], x["k"], x["v"], s_t, s_v, s_a, 0.2)
    w = G.read_workspace(ws, h, s_t, s_v, s_a)
    qn = np.linalg.norm(w["qbar64"], axis=-1).min()
    kn = np.linalg.norm(w["kbar"].astype(np.float64), axis=-1).max()
    assert (qn * kn > 2.0 ** 100) == (log2_scale == 52), (qn, kn)
    G.check_selection(sel.cpu().numpy(), ref, exempt_ok=False)


def test_longest_rows_of_the_matrix_core_select():
    """n_v = 1,280 video tiles, the most the matrix-core select kernel takes
    (20 keys per lane in its top-k, 82 KiB of float32 score rows, one
    workgroup per CU): every selection row exactly and the coarse branch."""
    h, s_t, s_v, s_a = 2, 64, 64 * 1280, 64
    announce(f"n_v = 1280: h={h} k={bsv.vsa_topk_count(s_v, 0.2)}")
    x = synth.vsa_inputs(24, h, s_t, s_v, s_a, threads=THREADS)
    xd = G.inputs_to_dev(x)
    out, sel, ws = G.run_forward(xd, s_t, s_v, s_a, 0.2)
    ref = oracle.select_coarse(x["q"], x["k"], x["v"], s_t, s_v, s_a, 0.2, threads=THREADS)
    G.check_selection(sel.cpu().numpy(), ref, exempt_ok=False)
    w = G.read_workspace(ws, h, s_t, s_v, s_a)
    np.testing.assert_allclose(w["coarse"], ref["coarse"], rtol=2e-5, atol=2e-7)


@pytest.mark.slow
def test_long_rows_use_the_radix_select():
    """n_v = 1,300 video tiles: rows too long for the register bisection go
    through the LDS radix select.  Every selection row and the coarse branch
    are checked; outputs on sampled rows."""
    h, s_t, s_v, s_a = 2, 64, 64 * 1300, 64
    announce(f"long rows: h={h} ({s_t},{s_v},{s_a}) k={bsv.vsa_topk_count(s_v, 0.2)}")
    x = synth.vsa_inputs(17, h, s_t, s_v, s_a, threads=THREADS)
    xd = G.inputs_to_dev(x)
    out, sel, ws = G.run_forward(xd, s_t, s_v, s_a, 0.2)
    ref = oracle.select_coarse(x["q"], x["k"], x["v"], s_t, s_v, s_a, 0.2, threads=THREADS)
    got_sel = sel.cpu().numpy()
    G.check_selection(got_sel, ref)
    w = G.read_workspace(ws, h, s_t, s_v, s_a)
    np.testing.assert_allclose(w["coarse"], ref["coarse"], rtol=2e-5, atol=2e-7)
    rows = G.sample_rows(s_t, s_v, s_a, n_video_tiles=3, per_tile=(0, 37, 63))
    _, ref_out = oracle.fine(x["q"], x["k"], x["v"], x["gate"], s_t, s_v, s_a, got_sel,
                             ref["coarse"], rows, threads=THREADS)
    G.assert_outputs_close(G.from_dev_bits(out)[rows], ref_out)


@pytest.mark.slow
def test_maximum_video_tiles():
    """The largest video segment the library takes (16,384 tiles, 1,048,576
    video tokens; k = 3,277): the radix select on one-row workgroups, 64-bit
    offsets in every stage.  Every selection row and the coarse branch are
    checked; outputs on sampled rows (a text row attends to all 1,048,704
    keys)."""
    h, s_t, s_v, s_a = 1, 64, 64 * 16384, 64
    announce(f"maximum n_v: h={h} ({s_t},{s_v},{s_a}) k={bsv.vsa_topk_count(s_v, 0.2)}")
    x = synth.vsa_inputs(18, h, s_t, s_v, s_a, threads=THREADS)
    xd = G.inputs_to_dev(x)
    out, sel, ws = G.run_forward(xd, s_t, s_v, s_a, 0.2)
    ref = oracle.select_coarse(x["q"], x["k"], x["v"], s_t, s_v, s_a, 0.2, threads=THREADS)
    got_sel = sel.cpu().numpy()
    assert ref["k"] == 3277
    G.check_selection(got_sel, ref)
    w = G.read_workspace(ws, h, s_t, s_v, s_a)
    np.testing.assert_allclose(w["coarse"], ref["coarse"], rtol=2e-5, atol=2e-7)
    rows = G.sample_rows(s_t, s_v, s_a, n_video_tiles=3, per_tile=(0, 63))
    _, ref_out = oracle.fine(x["q"], x["k"], x["v"], x["gate"], s_t, s_v, s_a, got_sel,
                             ref["coarse"], rows, threads=THREADS)
    G.assert_outputs_close(G.from_dev_bits(out)[rows], ref_out)


def test_designed_ranking():
    announce("designed ranking")
    h, s_t, n_v = 1, 64, 15
    s_v = n_v * T
    x = synth.vsa_inputs(12, h, s_t, s_v, 64)
    q = np.zeros((s_t + s_v + 64, h, D), np.float32)
    k = np.zeros_like(q)
    q[s_t:s_t + s_v, 0, 0] = -1.0
    q[s_t + 7 * T: s_t + 8 * T, 0, 0] = 1.0
    for w in range(n_v):
        k[s_t + w * T: s_t + (w + 1) * T, 0, 0] = (w + 1) / 16
    x["q"], x["k"] = synth.f32_to_bf16_bits(q), synth.f32_to_bf16_bits(k)
    ref, _, _, sel, _ = full_check(x, s_t, s_v, 64, 0.2, exempt_ok=False)
    assert np.array_equal(sel[0, 7], [12, 13, 14])
    assert np.array_equal(sel[0, 0], [0, 1, 2])


def test_late_large_scores_recompute():
    """The fine kernel's softmax reference is the column max of the first
    half-tile it meets; a later key tile scoring far above it makes the
    denominator pass 2^100 and the unit is recomputed with a raised
    reference.  Head 0: the excess is ~110 (log2 units), a finite sum past
    2^100 (one extra pass).  Head 1: ~330, where the first sums overflow
    to inf (two extra passes).  Text keys are 0, so every list starts at
    score 0."""
    announce("late large scores: h=2 tiles=(1,16,1)")
    h, s_t, n_v, s_a = 2, 64, 16, 64
    s_v = n_v * T
    x = synth.vsa_inputs(17, h, s_t, s_v, s_a)
    q = G.widen(x["q"]).astype(np.float32)
    k = G.widen(x["k"]).astype(np.float32)
    w_star = 9
    for hh, c in ((0, 2.6), (1, 4.5)):
        q[:, hh] = c
        k[:s_t, hh] = 0.0
        k[s_t + w_star * T: s_t + (w_star + 1) * T, hh] = c
    x["q"], x["k"] = synth.f32_to_bf16_bits(q), synth.f32_to_bf16_bits(k)
    # the inputs do reach the recompute condition (host arithmetic)
    c2 = np.log2(np.e) / np.sqrt(D)
    qw, kw = G.widen(x["q"]), G.widen(x["k"])
    top = [float(qw[0, hh] @ kw[s_t + w_star * T, hh]) * c2 for hh in range(h)]
    assert 100 < top[0] < 120 and top[1] > 300, top
    ref, e, *_ = full_check(x, s_t, s_v, s_a, 0.2, exempt_ok=False)
    assert np.all(ref["sel"][:, :, -1] >= w_star) and np.all(np.any(ref["sel"] == w_star, axis=-1))
    print(e)


def test_split_dense_units_combine_parts():
    """A text/audio query tile's key list is walked as several parts (here
    6: N = 24 tiles, video lists of 8, parts of about half a list) whose
    outputs are merged with weights 2^(m_p - max m).  Scores grow by ~0.5
    (log2 units) per key tile, so the parts start from references about 2
    apart and all contribute; a merge that ignored the references would be
    far off.  Video query tiles select the last k video tiles (pooled scores
    grow with the tile index)."""
    announce("split dense units: h=1 tiles=(2,20,2)")
    h, s_t, n_v, s_a = 1, 128, 20, 128
    s_v = n_v * T
    x = synth.vsa_inputs(23, h, s_t, s_v, s_a)
    q = np.zeros((s_t + s_v + s_a, h, D), dtype=np.float32)
    q[:, :, 0] = 1.0
    k = G.widen(x["k"]).astype(np.float32) * 0.25
    rows = np.arange(s_t + s_v + s_a)
    k[:, 0, 0] = 4.0 * (rows // T)  # exact in bfloat16
    x["q"], x["k"] = synth.f32_to_bf16_bits(q), synth.f32_to_bf16_bits(k)
    assert bsv.vsa_topk_count(s_v, 0.2) == 4
    ref, e, _, sel, _ = full_check(x, s_t, s_v, s_a, 0.2, exempt_ok=False)
    assert np.array_equal(sel[0, 0], np.arange(n_v - 4, n_v))
    # the dense rows' weights really span the parts: the last key tile
    # carries most of each dense row's softmax mass, the first parts little
    c2 = np.log2(np.e) / np.sqrt(D)
    assert 4.0 * (s_t + s_v + s_a - T) / T * c2 > 10
    print(e)


def test_fine_stage_on_oracle_selection():
    """The fine stage honours the index sets it is given: run it on the
    oracle's own selection (and on a shifted one) and compare."""
    announce("fine stage on given selections")
    h, s_t, s_v, s_a = 2, 64, 64 * 10, 128
    x = synth.vsa_inputs(13, h, s_t, s_v, s_a)
    xd = G.inputs_to_dev(x)
    ref = oracle.select_coarse(x["q"], x["k"], x["v"], s_t, s_v, s_a, 0.3)
    out, sel, ws = bsv.alloc_outputs(h, s_t, s_v, s_a, 0.3)
    bsv.vsa_pool_pack(xd["q"], xd["k"], xd["v"], s_t, s_v, s_a, ws)
    bsv.vsa_select_coarse(h, s_t, s_v, s_a, 0.3, sel, ws)
    rows = np.arange(s_t + s_v + s_a)
    for other in (ref["sel"], np.sort((ref["sel"] + 3) % 10, axis=-1)):
        seld = torch.from_numpy(np.ascontiguousarray(other, dtype=np.int32)).cuda()
        bsv.vsa_fine_attention(xd["q"], xd["gate"], s_t, s_v, s_a, 0.3, seld, out, ws)
        torch.cuda.synchronize()
        _, r = oracle.fine(x["q"], x["k"], x["v"], x["gate"], s_t, s_v, s_a, other, ref["coarse"], rows)
        G.assert_outputs_close(G.from_dev_bits(out), r)


def test_fine_stage_rejects_malformed_rows():
    """vsa_fine_attention checks every caller-supplied selection row on the
    device: a row with an index out of range, a repeated index or indices out
    of order is not attended and its 64 output rows come back as NaN; every
    other row is computed as usual."""
    announce("malformed selection rows: h=2 tiles=(1,12,1) k=4")
    h, s_t, s_v, s_a = 2, 64, 64 * 12, 64
    x = synth.vsa_inputs(27, h, s_t, s_v, s_a)
    xd = G.inputs_to_dev(x)
    ref = oracle.select_coarse(x["q"], x["k"], x["v"], s_t, s_v, s_a, 0.3)
    assert ref["k"] == 4
    out, sel, ws = bsv.alloc_outputs(h, s_t, s_v, s_a, 0.3)
    bsv.vsa_pool_pack(xd["q"], xd["k"], xd["v"], s_t, s_v, s_a, ws)
    bsv.vsa_select_coarse(h, s_t, s_v, s_a, 0.3, sel, ws)
    bad_sel = ref["sel"].copy()
    bad = {(0, 1): [0, 3, 5, 12],     # index == n_v
           (0, 7): [-1, 2, 3, 4],     # negative index
           (1, 0): [2, 2, 5, 6],      # repeated
           (1, 11): [1, 4, 3, 8]}     # out of order
    for (hh, u), row in bad.items():
        bad_sel[hh, u] = row
    seld = torch.from_numpy(np.ascontiguousarray(bad_sel, dtype=np.int32)).cuda()
    out.fill_(0.0)
    bsv.vsa_fine_attention(xd["q"], xd["gate"], s_t, s_v, s_a, 0.3, seld, out, ws)
    torch.cuda.synchronize()
    o = G.widen(G.from_dev_bits(out))
    for hh in range(h):
        for u in range(12):
            rows = slice(s_t + u * T, s_t + (u + 1) * T)
            if (hh, u) in bad:
                assert np.isnan(o[rows, hh]).all(), (hh, u)
            else:
                assert np.isfinite(o[rows, hh]).all(), (hh, u)
    all_rows = np.arange(s_t + s_v + s_a)
    _, r0 = oracle.fine(x["q"], x["k"], x["v"], x["gate"], s_t, s_v, s_a, ref["sel"],
                        ref["coarse"], all_rows)
    got = G.from_dev_bits(out)
    for hh in range(h):
        good = [r for r in all_rows
                if not (s_t <= r < s_t + s_v and (hh, (r - s_t) // T) in bad)]
        G.assert_outputs_close(got[good, hh], r0[good, hh])
    # the fused entry point never validates (its selection is its own) and the
    # same workspace still gives the oracle's result afterwards
    bsv.vsa_fine_attention(xd["q"], xd["gate"], s_t, s_v, s_a, 0.3, sel, out, ws)
    torch.cuda.synchronize()
    _, r1 = oracle.fine(x["q"], x["k"], x["v"], x["gate"], s_t, s_v, s_a, sel.cpu().numpy(),
                        ref["coarse"], np.arange(s_t + s_v + s_a))
    G.assert_outputs_close(G.from_dev_bits(out), r1)


def test_deterministic_and_head_slice():
    announce("determinism + head slice")
    s_t, s_v, s_a = 64, 64 * 24, 64
    x4 = synth.vsa_inputs(14, 4, s_t, s_v, s_a)
    xd4 = G.inputs_to_dev(x4)
    o1, s1, _ = G.run_forward(xd4, s_t, s_v, s_a, 0.2)
    o2, s2, _ = G.run_forward(xd4, s_t, s_v, s_a, 0.2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(s1, s2)
    x2 = {n: np.ascontiguousarray(a[:, :2]) for n, a in x4.items()}
    o3, s3, _ = G.run_forward(G.inputs_to_dev(x2), s_t, s_v, s_a, 0.2)
    assert torch.equal(o1[:, :2].contiguous().view(torch.int16), o3.view(torch.int16))
    assert torch.equal(s1[:2], s3)


def test_library_owned_workspace():
    announce("workspace = NULL")
    s_t, s_v, s_a = 64, 64 * 8, 64
    x = synth.vsa_inputs(15, 2, s_t, s_v, s_a)
    xd = G.inputs_to_dev(x)
    o1, s1, _ = G.run_forward(xd, s_t, s_v, s_a, 0.2)
    out = torch.empty_like(o1)
    sel = torch.empty_like(s1)
    bsv.vsa_forward(xd["q"], xd["k"], xd["v"], xd["gate"], s_t, s_v, s_a, 0.2, out, sel, None)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), out.view(torch.int16)) and torch.equal(s1, sel)


# --------------------------------------------------------------------------
# full-size workloads: every selection row, sampled output rows
# --------------------------------------------------------------------------

BIG = {
    "5s_14h": (14, 1024, 36288, 512),
    "10s_14h": (14, 1024, 72576, 1024),
    "10s_56h": (56, 1024, 72576, 1024),
    # an odd head count: one video queue shared by all eight XCDs (14 heads
    # give two head groups, 56 give four)
    "10s_7h": (7, 1024, 72576, 1024),
}


@pytest.mark.slow
@pytest.mark.parametrize("name,seed", [(n, 0) for n in BIG] + [("10s_56h", 1)])
def test_full_size_selection_and_outputs(name, seed):
    """Every selection row and coarse vector; the whole output finite; all 64
    rows of several tiles of 8 heads and one row of every query tile of the
    first and last head against the oracle (the persistent queues and the
    split dense parts only run at these sizes).  The 56-head shape runs on a
    second seed as well: other near-ties at the selection boundary, and the
    queues hand the units to other slots."""
    h, s_t, s_v, s_a = BIG[name]
    announce(f"full size {name} seed {seed}: h={h} ({s_t},{s_v},{s_a}) "
             f"k={bsv.vsa_topk_count(s_v, 0.2)}")
    x = synth.vsa_inputs(seed, h, s_t, s_v, s_a, threads=THREADS)
    xd = G.inputs_to_dev(x)
    out, sel, ws = G.run_forward(xd, s_t, s_v, s_a, 0.2)
    ref = oracle.select_coarse(x["q"], x["k"], x["v"], s_t, s_v, s_a, 0.2, threads=THREADS)
    got_sel = sel.cpu().numpy()
    n_exempt = G.check_selection(got_sel, ref)
    w = G.read_workspace(ws, h, s_t, s_v, s_a)
    np.testing.assert_allclose(w["coarse"], ref["coarse"], rtol=2e-5, atol=2e-7)
    cov = G.full_size_coverage(x, out, got_sel, ref["coarse"], s_t, s_v, s_a, threads=THREADS,
                               label=name)
    print(name, "exempt rows:", n_exempt, cov, flush=True)
    del xd, out, ws
    torch.cuda.empty_cache()


def test_non_default_stream():
    """The library enqueues on the stream it is given: a forward on a side
    stream equals the default-stream forward bit for bit."""
    announce("side stream: h=2 tiles=(1,20,1)")
    s_t, s_v, s_a = 64, 64 * 20, 64
    x = synth.vsa_inputs(26, 2, s_t, s_v, s_a)
    xd = G.inputs_to_dev(x)
    o1, s1, _ = G.run_forward(xd, s_t, s_v, s_a, 0.2)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out, sel, ws = bsv.alloc_outputs(2, s_t, s_v, s_a, 0.2)
        out.fill_(float("nan"))
        bsv.vsa_forward(xd["q"], xd["k"], xd["v"], xd["gate"], s_t, s_v, s_a, 0.2, out, sel, ws)
    side.synchronize()
    assert torch.equal(o1.view(torch.int16), out.view(torch.int16)) and torch.equal(s1, sel)


def test_graph_capture_replays():
    """vsa_forward with a caller workspace records into a HIP graph (no
    allocation, no memset on the path): every replay, with new input values
    copied into the captured buffers between replays and eager work in
    between, equals an eager forward on the same values bit for bit."""
    announce("graph capture: h=2 tiles=(1,24,1)")
    s_t, s_v, s_a = 64, 64 * 24, 64
    h = 2
    xs = [G.inputs_to_dev(synth.vsa_inputs(30 + i, h, s_t, s_v, s_a)) for i in range(3)]
    static = {n: t.clone() for n, t in xs[0].items()}
    out, sel, ws = bsv.alloc_outputs(h, s_t, s_v, s_a, 0.2)
    args = lambda d, o, s_, w: (d["q"], d["k"], d["v"], d["gate"], s_t, s_v, s_a, 0.2, o, s_, w)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bsv.vsa_forward(*args(static, out, sel, ws))  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        bsv.vsa_forward(*args(static, out, sel, ws))
    torch.cuda.synchronize()
    for rep in range(3):
        for n in static:
            static[n].copy_(xs[rep][n])
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_s = out.clone(), sel.clone()
        e_out, e_sel, e_ws = bsv.alloc_outputs(h, s_t, s_v, s_a, 0.2)
        bsv.vsa_forward(*args(xs[rep], e_out, e_sel, e_ws))
        torch.cuda.synchronize()
        assert torch.equal(got_o.view(torch.int16), e_out.view(torch.int16)), rep
        assert torch.equal(got_s, e_sel), rep
