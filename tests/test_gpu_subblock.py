"""GPU parity of the SubBlock router path (vsa_forward_subblock) against the
oracle: sub-block means bit for bit, selections equal except boundary ties
within 1e-6 relative, outputs on identical index sets within the same bars
as the main path (max-abs 2e-2, mean-abs 2e-3, rel-RMS 5e-3)."""
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


def run_subblock(xd, s_t, s_v, s_a, sp):
    h = xd["q"].shape[1]
    out, sel, ws = bsv.alloc_subblock_outputs(h, s_t, s_v, s_a, sp)
    out.fill_(float("nan"))
    sel.fill_(-7)
    bsv.vsa_forward_subblock(xd["q"], xd["k"], xd["v"], s_t, s_v, s_a, sp, out, sel, ws)
    torch.cuda.synchronize()
    return out, sel, ws


def read_subs(ws, h, s_t, s_v, s_a):
    """Q and K sub-block means from the workspace as float32 [H][n_v][4][128].
    Packed per (head, group c of 4 tiles): [i 8][lane 64][e 4], lane = 16 g +
    j, holding row j (tile 4c + j / 4, sub-block j % 4), dim 32 g + 4 i + e."""
    n_v = s_v // T
    n_c = (n_v + 3) // 4
    base = bsv.vsa_workspace_bytes(h, s_t, s_v, s_a)
    nb = h * n_c * 8192
    out = []
    for off in (base, base + nb):
        raw = ws[off:off + nb].cpu().numpy().view(np.float32)
        a = raw.reshape(h, n_c, 8, 4, 16, 4).transpose(0, 1, 4, 3, 2, 5)  # h c j g i e
        out.append(a.reshape(h, 4 * n_c, 4, D)[:, :n_v].copy())
    return out


def check_rows(gpu_rows, ref_sel, ref_scores, ref_kth, exempt_ok=True):
    """gpu_rows, ref_sel [n][k]: equal, or differing only in tiles whose oracle
    score is within TIE_REL of the row's k-th largest.  Returns #exempted."""
    n_v = ref_scores.shape[-1]
    assert gpu_rows.shape == ref_sel.shape
    assert gpu_rows.min() >= 0 and gpu_rows.max() < n_v
    if gpu_rows.shape[-1] > 1:
        assert np.all(np.diff(gpu_rows, axis=-1) > 0), "rows not strictly ascending"
    bad = np.flatnonzero(np.any(gpu_rows != ref_sel, axis=-1))
    for i in bad:
        assert exempt_ok, f"selection differs at row {i}"
        kth = ref_kth[i]
        for t in set(gpu_rows[i].tolist()) ^ set(ref_sel[i].tolist()):
            assert abs(ref_scores[i, t] - kth) <= G.TIE_REL * abs(kth), (i, t, ref_scores[i, t], kth)
    return len(bad)


def full_check(x, s_t, s_v, s_a, sp, exempt_ok=False):
    h = x["q"].shape[1]
    xd = G.inputs_to_dev({n: x[n] for n in ("q", "k", "v")})
    out, sel, ws = run_subblock(xd, s_t, s_v, s_a, sp)
    n_v = s_v // T
    rows = np.arange(s_t + s_v + s_a)
    got_sel = sel.cpu().numpy()
    if n_v:
        ref = oracle.subblock_select(x["q"], x["k"], s_t, s_v, s_a, sp, want_scores=True,
                                     threads=THREADS)
        assert got_sel.shape == ref["sel"].shape
        qs, ks = read_subs(ws, h, s_t, s_v, s_a)
        assert np.array_equal(qs, ref["qsub"]) and np.array_equal(ks, ref["ksub"])
        check_rows(got_sel.reshape(-1, ref["k"]), ref["sel"].reshape(-1, ref["k"]),
                   ref["scores"].reshape(-1, n_v), ref["kth"].reshape(-1), exempt_ok)
    else:
        ref = None
    zero = np.zeros_like(x["q"])
    _, ref_out = oracle.fine(x["q"], x["k"], x["v"], zero, s_t, s_v, s_a,
                             got_sel if n_v else None, np.zeros((h, n_v, D)), rows,
                             threads=THREADS)
    e = G.assert_outputs_close(G.from_dev_bits(out), ref_out)
    return ref, e, got_sel


@pytest.mark.parametrize("h,n_t,n_v,n_a,sp,seed", [
    (2, 1, 16, 1, 0.75, 1),
    (3, 0, 37, 0, 0.75, 2),     # video only, n_v not a multiple of 4
    (2, 2, 5, 3, 0.5, 3),       # fewer than 8 tiles: all kept
    (1, 1, 1, 1, 0.5, 4),       # a single video tile
    (4, 3, 70, 2, 0.75, 6),     # several workgroups per head, ragged last group
    (1, 2, 23, 0, 0.0, 7),      # no sparsity: every tile
    (2, 1, 130, 1, 0.9, 8),
    (1, 0, 18, 0, 0.6, 9),      # last workgroup holds one group of 2 tiles
])
def test_small_shapes_full_parity(h, n_t, n_v, n_a, sp, seed):
    announce(f"subblock small h={h} tiles=({n_t},{n_v},{n_a}) sparsity={sp} seed={seed}")
    x = synth.vsa_inputs(seed, h, n_t * T, n_v * T, n_a * T)
    ref, e, _ = full_check(x, n_t * T, n_v * T, n_a * T, sp)
    assert ref["k"] == oracle.subblock_count(n_v, sp)
    print(e)


def test_no_video_tiles_is_dense_attention():
    announce("subblock no video: h=2 tiles=(2,0,1)")
    x = synth.vsa_inputs(20, 2, 128, 0, 64)
    full_check(x, 128, 0, 64, 0.75)


def test_subblock_structure_decides():
    """Key tile 9's sub-blocks point +e, -e, +e, -e (tile mean 0, so the
    pooled tile score cannot see it); query tile 3's second sub-block is +e.
    The router must keep tile 9 for query tile 3 and, with every other score
    equal, the lowest indices elsewhere."""
    announce("subblock structure decides: h=1 tiles=(1,24,1)")
    h, s_t, n_v, s_a = 1, 64, 24, 64
    s_v = n_v * T
    s = s_t + s_v + s_a
    x = synth.vsa_inputs(21, h, s_t, s_v, s_a)
    q = np.zeros((s, h, D), np.float32)
    k = np.zeros_like(q)
    e = np.zeros(D, np.float32)
    e[::4] = 0.5
    q[s_t + 3 * T + 16: s_t + 3 * T + 32, 0] = e
    for b in range(4):
        r0 = s_t + 9 * T + 16 * b
        k[r0: r0 + 16, 0] = e if b % 2 == 0 else -e
    x["q"], x["k"] = synth.f32_to_bf16_bits(q), synth.f32_to_bf16_bits(k)
    ref, _, sel = full_check(x, s_t, s_v, s_a, 0.75)
    assert ref["k"] == 8
    assert 9 in sel[0, 3].tolist()
    assert sel[0, 0].tolist() == list(range(8))


def test_copied_key_tiles_tie_exactly():
    """K tiles 2, 5, 9, 14 are copies: their scores tie bit for bit on both
    sides, and at the cut the lower indices win.  Exact match required."""
    announce("subblock copied key tiles: h=2 tiles=(1,24,1)")
    h, s_t, n_v, s_a = 2, 64, 24, 64
    s_v = n_v * T
    x = synth.vsa_inputs(22, h, s_t, s_v, s_a)
    k = x["k"].copy()
    for w in (5, 9, 14):
        k[s_t + w * T: s_t + (w + 1) * T] = k[s_t + 2 * T: s_t + 3 * T]
    x["k"] = k
    full_check(x, s_t, s_v, s_a, 0.7, exempt_ok=False)


def test_near_triples_ranked_in_float64():
    """Key tiles 3i + 1 and 3i + 2 copy tile 3i with one token's dimension 0
    moved by one and two bf16 steps, so the three scores differ by ~1e-9 to
    ~1e-6: inside the band that the router's float32 products and
    log-sum-exp leave undecided, far above float64 rounding.  With k = 8 the
    cut of every row falls inside a triple and is resolved by the recomputed
    float64 scores.  Exact match required."""
    announce("subblock near triples: h=2 tiles=(1,40,1) sp=0.75")
    h, s_t, n_v, s_a = 2, 64, 40, 64
    s_v = n_v * T
    x = synth.vsa_inputs(25, h, s_t, s_v, s_a)
    k = x["k"].copy()
    for w in range(0, n_v - 2, 3):
        a = s_t + w * T
        for j, step in ((1, 1), (2, 2)):
            k[a + j * T: a + (j + 1) * T] = k[a: a + T]
            bits = k[a + j * T + 5, :, 0].astype(np.int32)
            k[a + j * T + 5, :, 0] = (bits + step).astype(np.uint16)
    x["k"] = k
    ref, _, _ = full_check(x, s_t, s_v, s_a, 0.75, exempt_ok=False)
    kk = ref["k"]
    s = -np.sort(-ref["scores"].reshape(-1, n_v), axis=1)
    gap = s[:, kk - 1] - s[:, kk]
    # the construction does what it says: every row is cut inside a triple
    assert np.sum((gap > 0) & (gap < 1e-5)) == h * n_v, np.sort(gap)[-12:]


def test_all_key_tiles_equal():
    """Every key tile a copy of the first and Q nonzero: every score of a row
    is the same value on both sides (a band of all 100 keys, more than a
    wavefront's lanes), and the lowest k indices win.  Exact match
    required."""
    announce("subblock identical key tiles: h=1 tiles=(1,100,1)")
    h, s_t, n_v, s_a = 1, 64, 100, 64
    s_v = n_v * T
    x = synth.vsa_inputs(26, h, s_t, s_v, s_a)
    k = x["k"].copy()
    for w in range(1, n_v):
        k[s_t + w * T: s_t + (w + 1) * T] = k[s_t: s_t + T]
    x["k"] = k
    ref, _, sel = full_check(x, s_t, s_v, s_a, 0.75, exempt_ok=False)
    assert np.array_equal(sel, np.broadcast_to(np.arange(ref["k"]), sel.shape))


@pytest.mark.parametrize("log2_scale", [46, 52])
def test_huge_magnitudes_rank_every_key_in_float64(log2_scale):
    """Q and K scaled by 2^46 or 2^52 (exact in bf16).  At 2^46 the logits
    reach ~2^90 and the float32 scores and their bounds decide as usual (a
    fused x - m in the log-sum-exp overflowed here); at 2^52 the bounds
    exceed 2^100, so every key of every row is in the band and more than 64
    keys are ranked by bisection on their recomputed float64 scores.  Router
    selection must match the oracle exactly."""
    announce(f"subblock huge magnitudes: h=2 tiles=(1,70,1) sp=0.75, Q and K x 2^{log2_scale}")
    h, s_t, n_v, s_a = 2, 64, 70, 64
    s_v = n_v * T
    x = synth.vsa_inputs(28, h, s_t, s_v, s_a)
    for n in ("q", "k"):
        x[n] = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(x[n]) * np.float32(2.0 ** log2_scale))
    xd = G.inputs_to_dev({n: x[n] for n in ("q", "k")})
    kk = bsv.vsa_subblock_count(s_v, 0.75)
    ws = torch.empty(bsv.vsa_subblock_workspace_bytes(h, s_t, s_v, s_a), dtype=torch.uint8,
                     device="cuda")
    sel = torch.full((h, n_v, kk), -7, dtype=torch.int32, device="cuda")
    bsv.vsa_subblock_select(xd["q"], xd["k"], s_t, s_v, s_a, 0.75, sel, ws)
    torch.cuda.synchronize()
    ref = oracle.subblock_select(x["q"], x["k"], s_t, s_v, s_a, 0.75, want_scores=True,
                                 threads=THREADS)
    qs, ks = read_subs(ws, h, s_t, s_v, s_a)
    n2 = np.linalg.norm(qs.astype(np.float64), axis=-1).max() ** 2
    assert n2 > 2.0 ** 90 and (n2 > 2.0 ** 100) == (log2_scale == 52), np.log2(n2)
    check_rows(sel.cpu().numpy().reshape(-1, kk), ref["sel"].reshape(-1, kk),
               ref["scores"].reshape(-1, n_v), ref["kth"].reshape(-1), exempt_ok=False)


def test_zero_queries_take_lowest_indices():
    announce("subblock Q = 0: every score log 16")
    h, s_t, n_v, s_a = 2, 64, 40, 64
    x = synth.vsa_inputs(23, h, s_t, n_v * T, s_a)
    x["q"] = np.zeros_like(x["q"])
    ref, _, sel = full_check(x, s_t, n_v * T, s_a, 0.75)
    assert np.array_equal(sel, np.broadcast_to(np.arange(ref["k"]), sel.shape))


def test_deterministic_and_library_workspace():
    announce("subblock determinism + workspace = NULL")
    s_t, s_v, s_a = 64, 64 * 30, 64
    x = synth.vsa_inputs(24, 3, s_t, s_v, s_a)
    xd = G.inputs_to_dev({n: x[n] for n in ("q", "k", "v")})
    o1, s1, _ = run_subblock(xd, s_t, s_v, s_a, 0.75)
    o2, s2, _ = run_subblock(xd, s_t, s_v, s_a, 0.75)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(s1, s2)
    out, sel = torch.empty_like(o1), torch.empty_like(s1)
    bsv.vsa_forward_subblock(xd["q"], xd["k"], xd["v"], s_t, s_v, s_a, 0.75, out, sel, None)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), out.view(torch.int16)) and torch.equal(s1, sel)
    # the router stage alone selects the same tiles
    _, sel2, ws2 = bsv.alloc_subblock_outputs(3, s_t, s_v, s_a, 0.75)
    sel2.fill_(-1)
    bsv.vsa_subblock_select(xd["q"], xd["k"], s_t, s_v, s_a, 0.75, sel2, ws2)
    torch.cuda.synchronize()
    assert torch.equal(s1, sel2)


@pytest.mark.slow
@pytest.mark.parametrize("n_v", [1280, 1300, 2700])
def test_long_rows(n_v):
    """n_v = 1,280 fills the two-workgroups-per-CU router (8 rows of 1,280
    slots, 80 KiB of LDS each, 20 keys per lane in the top-k); longer rows
    take the 8-row (n_v <= 2,560) and 4-row workgroups, one per CU, with
    longer register rows in the top-k.  Every selection row is checked,
    outputs on sampled rows."""
    h, s_t, s_a = 1, 64, 64
    s_v = n_v * T
    sp = 0.8
    announce(f"subblock long rows h={h} n_v={n_v} k={bsv.vsa_subblock_count(s_v, sp)}")
    x = synth.vsa_inputs(25, h, s_t, s_v, s_a, threads=THREADS)
    xd = G.inputs_to_dev({n: x[n] for n in ("q", "k", "v")})
    out, sel, ws = run_subblock(xd, s_t, s_v, s_a, sp)
    ref = oracle.subblock_select(x["q"], x["k"], s_t, s_v, s_a, sp, want_scores=True,
                                 threads=THREADS)
    got = sel.cpu().numpy()
    check_rows(got.reshape(-1, ref["k"]), ref["sel"].reshape(-1, ref["k"]),
               ref["scores"].reshape(-1, n_v), ref["kth"].reshape(-1))
    rows = G.sample_rows(s_t, s_v, s_a, n_video_tiles=3, per_tile=(0, 37, 63))
    _, ref_out = oracle.fine(x["q"], x["k"], x["v"], np.zeros_like(x["q"]), s_t, s_v, s_a, got,
                             np.zeros((h, n_v, D)), rows, threads=THREADS)
    G.assert_outputs_close(G.from_dev_bits(out)[rows], ref_out)


@pytest.mark.slow
def test_full_size_10s_56h_sampled():
    """The 10 s shape (1,024 text + 72,576 video + 1,024 audio tokens, 56
    heads) at sparsity 0.75 (k = 280): sampled (head, tile) selection rows
    against the oracle's row-wise router, every row checked for validity,
    outputs on sampled rows."""
    h, s_t, s_v, s_a = 56, 1024, 72576, 1024
    sp = 0.75
    announce(f"subblock full size 10s_56h sparsity={sp}")
    x = synth.vsa_inputs(0, h, s_t, s_v, s_a, threads=THREADS)
    xd = G.inputs_to_dev({n: x[n] for n in ("q", "k", "v")})
    out, sel, ws = run_subblock(xd, s_t, s_v, s_a, sp)
    got = sel.cpu().numpy()
    n_v = s_v // T
    assert got.shape == (h, n_v, 280)
    assert got.min() >= 0 and got.max() < n_v and np.all(np.diff(got, axis=-1) > 0)
    rng = np.random.default_rng(5)
    pairs = [(0, 0), (h - 1, n_v - 1), (17, 563)] + \
        [(int(a), int(b)) for a, b in zip(rng.integers(0, h, 40), rng.integers(0, n_v, 40))]
    ref = oracle.subblock_select_rows(x["q"], x["k"], s_t, s_v, s_a, sp, pairs, threads=THREADS)
    gp = np.stack([got[a, b] for a, b in pairs])
    check_rows(gp, ref["sel"], ref["scores"], ref["kth"])
    qs, ks = read_subs(ws, h, s_t, s_v, s_a)
    assert np.array_equal(qs, ref["qsub"]) and np.array_equal(ks, ref["ksub"])
    G.full_size_coverage({n: x[n] for n in ("q", "k", "v")}, out, got, None, s_t, s_v, s_a,
                         threads=THREADS, label="subblock 10s_56h")


def test_subblock_graph_capture_replays():
    """vsa_forward_subblock with a caller workspace records into a HIP graph;
    replays with new inputs match eager calls bit for bit."""
    announce("subblock graph capture: h=2 tiles=(1,30,1)")
    s_t, s_v, s_a = 64, 64 * 30, 64
    h = 2
    xs = [G.inputs_to_dev({n: a for n, a in synth.vsa_inputs(40 + i, h, s_t, s_v, s_a).items()
                           if n != "gate"}) for i in range(2)]
    static = {n: t.clone() for n, t in xs[0].items()}
    out, sel, ws = bsv.alloc_subblock_outputs(h, s_t, s_v, s_a, 0.75)
    call = lambda d, o, s_, w: bsv.vsa_forward_subblock(d["q"], d["k"], d["v"], s_t, s_v, s_a,
                                                        0.75, o, s_, w)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(static, out, sel, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(static, out, sel, ws)
    torch.cuda.synchronize()
    for rep in (0, 1, 0):
        for n in static:
            static[n].copy_(xs[rep][n])
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_s = out.clone(), sel.clone()
        e_out, e_sel, e_ws = bsv.alloc_subblock_outputs(h, s_t, s_v, s_a, 0.75)
        call(xs[rep], e_out, e_sel, e_ws)
        torch.cuda.synchronize()
        assert torch.equal(got_o.view(torch.int16), e_out.view(torch.int16)), rep
        assert torch.equal(got_s, e_sel), rep
