"""vsa_forward_noalloc (workspace in the library's fixed device array) against
vsa_forward (caller workspace), through the C ABI: two calls in a row, the
second on a smaller input, each bit for bit equal to vsa_forward on the same
inputs (same kernels, same per-unit arithmetic; the heads run in groups that
fit the array)."""
import numpy as np
import pytest
import torch

import block_sparse_video_amd as bsv
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


def _both(x, s_t, s_v, s_a, frac):
    xd = G.inputs_to_dev(x)
    ref_out, ref_sel, _ = G.run_forward(xd, s_t, s_v, s_a, frac)
    h = xd["q"].shape[1]
    out = torch.full_like(ref_out, float("nan"))
    kk = bsv.vsa_topk_count(s_v, frac)
    sel = torch.full((h, s_v // 64, kk), -7, dtype=torch.int32, device="cuda")
    bsv.vsa_forward_noalloc(xd["q"], xd["k"], xd["v"], xd["gate"], s_t, s_v, s_a, frac, out, sel)
    torch.cuda.synchronize()
    return ref_out, ref_sel, out, sel


def test_noalloc_matches_forward_twice_second_smaller():
    # first call: 14 heads at the 5 s shape, ~27 MB of workspace per head, so
    # the 256 MiB array takes the heads in two groups (9 + 5)
    h, s_t, s_v, s_a = 14, 1024, 36288, 512
    print(f"[case] noalloc 1: h={h} ({s_t},{s_v},{s_a})", flush=True)
    x = synth.vsa_inputs(0, h, s_t, s_v, s_a, threads=THREADS)
    ref_out, ref_sel, out, sel = _both(x, s_t, s_v, s_a, 0.2)
    assert torch.equal(sel, ref_sel)
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    del ref_out, out
    # second call: a smaller shape (one group), after the array holds the
    # first call's contents
    h, s_t, s_v, s_a = 3, 128, 64 * 40, 64
    print(f"[case] noalloc 2: h={h} ({s_t},{s_v},{s_a})", flush=True)
    x = synth.vsa_inputs(1, h, s_t, s_v, s_a)
    ref_out, ref_sel, out, sel = _both(x, s_t, s_v, s_a, 0.2)
    assert torch.equal(sel, ref_sel)
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    # and the oracle agrees on the second call (the bar of every other test)
    import oracle
    ref = oracle.forward(x["q"], x["k"], x["v"], x["gate"], s_t, s_v, s_a, 0.2)
    assert np.array_equal(sel.cpu().numpy(), ref["sel"])
    G.assert_outputs_close(G.from_dev_bits(out), ref["out_f64"])


def test_noalloc_without_video_tiles():
    h, s_t, s_a = 2, 128, 64
    print(f"[case] noalloc no video: h={h} ({s_t},0,{s_a})", flush=True)
    x = synth.vsa_inputs(2, h, s_t, 0, s_a)
    xd = G.inputs_to_dev(x)
    ref = torch.empty_like(xd["q"])
    ws = torch.empty(bsv.vsa_workspace_bytes(h, s_t, 0, s_a), dtype=torch.uint8, device="cuda")
    bsv.vsa_forward(xd["q"], xd["k"], xd["v"], None, s_t, 0, s_a, 0.2, ref, None, ws)
    out = torch.full_like(ref, float("nan"))
    bsv.vsa_forward_noalloc(xd["q"], xd["k"], xd["v"], None, s_t, 0, s_a, 0.2, out, None)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
