"""GPU parity of the whole-sequence SubBlock router path
(vsa_forward_subblock_whole) against the oracle: every tile of [text | video
| audio] ranks every key tile; piece means bit for bit, selections equal
except boundary ties within 1e-6 relative, outputs on identical index sets
within max-abs 2e-2, mean-abs 2e-3 and rel-RMS 5e-3 of oracle.fine_lists."""
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


def run_whole(xd, s_t, s_v, s_a, sp):
    h = xd["q"].shape[1]
    out, sel, ws = bsv.alloc_subblock_whole_outputs(h, s_t, s_v, s_a, sp)
    out.fill_(float("nan"))
    sel.fill_(-7)
    bsv.vsa_forward_subblock_whole(xd["q"], xd["k"], xd["v"], s_t, s_v, s_a, sp, out, sel, ws)
    torch.cuda.synchronize()
    return out, sel, ws


def check_rows(gpu_rows, ref_sel, ref_scores, ref_kth, n):
    """Rows valid (k distinct ascending indices in [0, n)) and equal to the
    oracle's, except tiles whose oracle score lies within 1e-6 relative of
    the k-th largest score.  Returns the number of exempt rows."""
    assert gpu_rows.min() >= 0 and gpu_rows.max() < n
    if gpu_rows.shape[1] > 1:
        assert np.all(np.diff(gpu_rows, axis=1) > 0)
    bad = np.argwhere(np.any(gpu_rows != ref_sel, axis=1)).ravel()
    for i in bad:
        diff = set(gpu_rows[i].tolist()) ^ set(ref_sel[i].tolist())
        for t in diff:
            assert abs(ref_scores[i, t] - ref_kth[i]) <= G.TIE_REL * abs(ref_kth[i]), (i, t)
    return len(bad)


def read_pieces(ws, h, s_t, s_v, s_a):
    """Q and K piece means [H][N][4][128] from the workspace (the last two
    regions, packed per (head, group of 4 tiles) as [i 8][lane 64][e 4],
    lane = 16 g + j: row j (tile 4c + j / 4, piece j % 4), dim 32 g + 4 i + e)."""
    n = (s_t + s_v + s_a) // T
    n_c = (n + 3) // 4
    nb = h * n_c * 8192
    total = bsv.vsa_subblock_whole_workspace_bytes(h, s_t, s_v, s_a)
    out = []
    for off in (total - 2 * nb, total - nb):
        raw = ws[off:off + nb].cpu().numpy().view(np.float32)
        a = raw.reshape(h, n_c, 8, 4, 16, 4).transpose(0, 1, 4, 3, 2, 5)
        out.append(a.reshape(h, 4 * n_c, 4, D)[:, :n].copy())
    return out


@pytest.mark.parametrize("h,n_t,n_v,n_a,sp,seed", [
    (2, 1, 16, 1, 0.75, 1),
    (3, 2, 37, 1, 0.6, 2),      # ragged groups of 4 tiles
    (1, 0, 12, 0, 0.5, 3),      # video only
    (2, 3, 5, 2, 0.5, 4),       # text and audio a third of the tiles
    (2, 1, 70, 2, 0.9, 5),      # several routing workgroups per head
    (1, 1, 6, 1, 0.0, 6),       # sparsity 0: every tile kept (dense)
])
def test_small_shapes_full_parity(h, n_t, n_v, n_a, sp, seed):
    s_t, s_v, s_a = n_t * T, n_v * T, n_a * T
    announce(f"subblock whole h={h} tiles=({n_t},{n_v},{n_a}) sparsity={sp}")
    x = synth.vsa_inputs(seed, h, s_t, s_v, s_a)
    xd = G.inputs_to_dev({n: x[n] for n in ("q", "k", "v")})
    out, sel, ws = run_whole(xd, s_t, s_v, s_a, sp)
    ref = oracle.subblock_select_whole(x["q"], x["k"], s_t, s_v, s_a, sp, want_scores=True)
    n = n_t + n_v + n_a
    got = sel.cpu().numpy()
    assert got.shape == (h, n, ref["k"])
    ex = check_rows(got.reshape(-1, ref["k"]), ref["sel"].reshape(-1, ref["k"]),
                    ref["scores"].reshape(-1, n), ref["kth"].reshape(-1), n)
    assert ex == 0
    qs, ks = read_pieces(ws, h, s_t, s_v, s_a)
    assert np.array_equal(qs, ref["qsub"]) and np.array_equal(ks, ref["ksub"])
    _, want = oracle.fine_lists(x["q"], x["k"], x["v"], got, np.arange(s_t + s_v + s_a))
    G.assert_outputs_close(G.from_dev_bits(out), want)


def test_text_and_audio_tiles_compete_on_the_gpu():
    """The oracle's planted case: a repulsive text key tile is dropped by
    every query tile and an attractive audio key tile kept by every one."""
    announce("subblock whole planted text/audio tiles")
    rng = np.random.default_rng(24)
    h, n_t, n_v, n_a = 1, 2, 9, 1
    s = T * (n_t + n_v + n_a)
    e = np.zeros(D, np.float32)
    e[:8] = 1.0
    qf = rng.standard_normal((s, h, D)).astype(np.float32) * 0.25 + e
    kf = rng.standard_normal((s, h, D)).astype(np.float32) * 0.25
    kf[0:T] -= 6.0 * e
    kf[s - T:s] += 6.0 * e
    vf = rng.standard_normal((s, h, D)).astype(np.float32)
    x = {"q": synth.f32_to_bf16_bits(qf), "k": synth.f32_to_bf16_bits(kf),
         "v": synth.f32_to_bf16_bits(vf)}
    out, sel, _ = run_whole(G.inputs_to_dev(x), T * n_t, T * n_v, T * n_a, 0.4)
    got = sel.cpu().numpy()[0]
    assert got.shape == (12, 8)
    assert not np.any(got == 0) and np.all(np.any(got == 11, axis=1))
    ref = oracle.subblock_select_whole(x["q"], x["k"], T * n_t, T * n_v, T * n_a, 0.4)
    np.testing.assert_array_equal(got, ref["sel"][0])
    _, want = oracle.fine_lists(x["q"], x["k"], x["v"], ref["sel"], np.arange(s))
    G.assert_outputs_close(G.from_dev_bits(out), want)


def test_router_stage_alone_matches_forward():
    announce("subblock whole router stage h=2 tiles=(1,30,1)")
    h, s_t, s_v, s_a = 2, 64, 64 * 30, 64
    x = synth.vsa_inputs(7, h, s_t, s_v, s_a)
    xd = G.inputs_to_dev({n: x[n] for n in ("q", "k", "v")})
    _, sel_f, _ = run_whole(xd, s_t, s_v, s_a, 0.75)
    _, sel, ws = bsv.alloc_subblock_whole_outputs(h, s_t, s_v, s_a, 0.75)
    bsv.vsa_subblock_select_whole(xd["q"], xd["k"], s_t, s_v, s_a, 0.75, sel, ws)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel_f)


@pytest.mark.slow
def test_full_size_10s_56h():
    """The 10 s shape (1,024 text + 72,576 video + 1,024 audio tokens, 56
    heads, N = 1,166 tiles) at sparsity 0.75 (k = 288): sampled selection
    rows against the oracle's row-wise router, every row checked for
    validity, piece means of every tile bit for bit, and the output coverage
    of the other full-size tests against oracle.fine_lists."""
    h, s_t, s_v, s_a = 56, 1024, 72576, 1024
    sp = 0.75
    announce(f"subblock whole full size 10s_56h sparsity={sp}")
    x = synth.vsa_inputs(0, h, s_t, s_v, s_a, threads=THREADS)
    xd = G.inputs_to_dev({n: x[n] for n in ("q", "k", "v")})
    out, sel, ws = run_whole(xd, s_t, s_v, s_a, sp)
    got = sel.cpu().numpy()
    n = (s_t + s_v + s_a) // T
    assert got.shape == (h, n, 288)
    assert got.min() >= 0 and got.max() < n and np.all(np.diff(got, axis=-1) > 0)
    rng = np.random.default_rng(6)
    pairs = [(0, 0), (h - 1, n - 1), (3, 5), (9, n - 3)] + \
        [(int(a), int(b)) for a, b in zip(rng.integers(0, h, 40), rng.integers(0, n, 40))]
    ref = oracle.subblock_select_whole_rows(x["q"], x["k"], s_t, s_v, s_a, sp, pairs,
                                            threads=THREADS)
    gp = np.stack([got[a, b] for a, b in pairs])
    n_exempt = check_rows(gp, ref["sel"], ref["scores"], ref["kth"], n)
    qs, ks = read_pieces(ws, h, s_t, s_v, s_a)
    assert np.array_equal(qs, ref["qsub"]) and np.array_equal(ks, ref["ksub"])
    del qs, ks
    cov = G.full_size_coverage({n_: x[n_] for n_ in ("q", "k", "v")}, out, got, None, s_t, s_v,
                               s_a, threads=THREADS, label="subblock whole 10s_56h", lists=True)
    print("exempt sampled rows:", n_exempt, cov, flush=True)
