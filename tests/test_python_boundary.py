"""The Python binding rejects malformed arguments before any compute entry
point of the library runs (CPU only): a selected_tiles tensor shaped for a
different k or shape, a workspace of the wrong dtype or in host memory, and
host tensors in general.  The library handle is wrapped so that reaching a
compute entry point fails the test; the host helpers (k, workspace sizes)
still run."""
import pytest
import torch

import block_sparse_video_amd as bsv
from block_sparse_video_amd import _native

H, S_T, S_V, S_A = 2, 64, 640, 64
S = S_T + S_V + S_A
FRAC = 0.2
HOST_ONLY = {"vsa_topk_count", "vsa_subblock_count", "vsa_workspace_bytes",
             "vsa_subblock_workspace_bytes", "vsa_status_string", "vsa_workspace_layout"}


class _HostOnly:
    def __init__(self, lib):
        self._lib = lib

    def __getattr__(self, name):
        if name not in HOST_ONLY:
            raise AssertionError(f"compute entry point {name} reached")
        return getattr(self._lib, name)


@pytest.fixture(autouse=True)
def host_only(monkeypatch):
    lib = _HostOnly(_native.load())
    monkeypatch.setattr(bsv, "load", lambda: lib)


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def tensors(kk=None, n_v=S_V // 64):
    kk = bsv.vsa_topk_count(S_V, FRAC) if kk is None else kk
    return dict(q=bf(S, H, 128), k=bf(S, H, 128), v=bf(S, H, 128), gate=bf(S, H, 128),
                out=bf(S, H, 128), sel=torch.zeros((H, n_v, kk), dtype=torch.int32),
                ws=torch.zeros(1024, dtype=torch.uint8))


def test_k_of_the_test_shape():
    assert bsv.vsa_topk_count(S_V, FRAC) == 2
    assert bsv.vsa_subblock_count(S_V, 0.5) == 8


@pytest.mark.parametrize("bad", [dict(kk=3), dict(kk=1), dict(n_v=9)])
def test_forward_rejects_selection_shape(bad):
    t = tensors(**bad)
    with pytest.raises(ValueError, match="selected_tiles"):
        bsv.vsa_forward(t["q"], t["k"], t["v"], t["gate"], S_T, S_V, S_A, FRAC, t["out"], t["sel"],
                        t["ws"])


def test_stage_calls_reject_selection_shape():
    t = tensors(kk=5)
    with pytest.raises(ValueError, match="selected_tiles"):
        bsv.vsa_select_coarse(H, S_T, S_V, S_A, FRAC, t["sel"], t["ws"])
    with pytest.raises(ValueError, match="selected_tiles"):
        bsv.vsa_fine_attention(t["q"], t["gate"], S_T, S_V, S_A, FRAC, t["sel"], t["out"], t["ws"])


def test_selection_shape_follows_topk_frac():
    # k = 2 at 0.2; the same tensor is wrong for 0.5 (k = 5)
    t = tensors()
    with pytest.raises(ValueError, match="selected_tiles"):
        bsv.vsa_forward(t["q"], t["k"], t["v"], t["gate"], S_T, S_V, S_A, 0.5, t["out"], t["sel"],
                        t["ws"])


def test_padded_rejects_selection_shape_and_workspace():
    t = tensors(kk=4)
    with pytest.raises(ValueError, match="selected_tiles"):
        bsv.vsa_forward_padded(t["q"], t["k"], t["v"], t["gate"], S_T, S_V, S_A, (64, 640, 64),
                               FRAC, t["out"], t["sel"], t["ws"])
    t = tensors()
    with pytest.raises(TypeError, match="workspace"):
        bsv.vsa_forward_padded(t["q"], t["k"], t["v"], t["gate"], S_T, S_V, S_A, (64, 640, 64),
                               FRAC, t["out"], t["sel"], torch.zeros(1024, dtype=torch.float32))
    # right shapes and dtypes, host memory: refused before the call
    with pytest.raises(TypeError, match="CUDA"):
        bsv.vsa_forward_padded(t["q"], t["k"], t["v"], t["gate"], S_T, S_V, S_A, (64, 640, 64),
                               FRAC, t["out"], t["sel"], t["ws"])


def test_padded_preprocessing_arguments_go_together():
    t = tensors()
    g = bf(H, 128)
    with pytest.raises(ValueError, match="together"):
        bsv.vsa_forward_padded(t["q"], t["k"], t["v"], t["gate"], S_T, S_V, S_A, (64, 640, 64),
                               FRAC, t["out"], t["sel"], t["ws"], gamma_q=g, gamma_k=None,
                               grid=(1, 2, 320), q_out=bf(S, H, 128))
    with pytest.raises(ValueError, match="gamma_k"):
        bsv.vsa_forward_padded(t["q"], t["k"], t["v"], t["gate"], S_T, S_V, S_A, (64, 640, 64),
                               FRAC, t["out"], t["sel"], t["ws"], gamma_q=g, gamma_k=bf(H, 64),
                               grid=(1, 2, 320), q_out=bf(S, H, 128))


def test_subblock_rejects_selection_shape():
    t = tensors(kk=2)  # the SubBlock count at sparsity 0.5 is 8
    with pytest.raises(ValueError, match="selected_tiles"):
        bsv.vsa_forward_subblock(t["q"], t["k"], t["v"], S_T, S_V, S_A, 0.5, t["out"], t["sel"],
                                 t["ws"])
    with pytest.raises(ValueError, match="selected_tiles"):
        bsv.vsa_subblock_select(t["q"], t["k"], S_T, S_V, S_A, 0.5, t["sel"], t["ws"])


@pytest.mark.parametrize("call", ["forward", "pool_pack", "select", "fine", "subblock"])
def test_host_tensors_are_refused(call):
    t = tensors()
    with pytest.raises(TypeError, match="CUDA"):
        if call == "forward":
            bsv.vsa_forward(t["q"], t["k"], t["v"], t["gate"], S_T, S_V, S_A, FRAC, t["out"],
                            t["sel"], t["ws"])
        elif call == "pool_pack":
            bsv.vsa_pool_pack(t["q"], t["k"], t["v"], S_T, S_V, S_A, t["ws"])
        elif call == "select":
            bsv.vsa_select_coarse(H, S_T, S_V, S_A, FRAC, t["sel"], t["ws"])
        elif call == "fine":
            bsv.vsa_fine_attention(t["q"], t["gate"], S_T, S_V, S_A, FRAC, t["sel"], t["out"],
                                   t["ws"])
        else:
            sel = torch.zeros((H, S_V // 64, 8), dtype=torch.int32)
            bsv.vsa_forward_subblock(t["q"], t["k"], t["v"], S_T, S_V, S_A, 0.5, t["out"], sel,
                                     t["ws"])


def test_token_tensor_shapes_and_dtypes():
    t = tensors()
    with pytest.raises(ValueError, match="out"):
        bsv.vsa_forward(t["q"], t["k"], t["v"], t["gate"], S_T, S_V, S_A, FRAC, bf(S - 64, H, 128),
                        t["sel"], t["ws"])
    with pytest.raises(TypeError, match="k must be"):
        bsv.vsa_forward(t["q"], t["k"].float(), t["v"], t["gate"], S_T, S_V, S_A, FRAC, t["out"],
                        t["sel"], t["ws"])
    with pytest.raises(ValueError, match="q must be"):
        bsv.vsa_forward(bf(S, H), t["k"], t["v"], t["gate"], S_T, S_V, S_A, FRAC, t["out"],
                        t["sel"], t["ws"])
    with pytest.raises(TypeError, match="workspace"):
        bsv.vsa_forward(t["q"], t["k"], t["v"], t["gate"], S_T, S_V, S_A, FRAC, t["out"],
                        t["sel"], torch.zeros(16, dtype=torch.int32))


def test_stage_calls_need_a_workspace():
    t = tensors()
    with pytest.raises(ValueError, match="workspace"):
        bsv.vsa_pool_pack(t["q"], t["k"], t["v"], S_T, S_V, S_A, None)
    with pytest.raises(ValueError, match="workspace"):
        bsv.vsa_select_coarse(H, S_T, S_V, S_A, FRAC, t["sel"], None)
    with pytest.raises(ValueError, match="workspace"):
        bsv.vsa_fine_attention(t["q"], t["gate"], S_T, S_V, S_A, FRAC, t["sel"], t["out"], None)


def test_workspace_bytes_checks_topk_frac():
    assert bsv.vsa_workspace_bytes(H, S_T, S_V, S_A, FRAC) > 0
    for bad in (0.0, -0.1, 1.5, float("nan")):
        assert bsv.vsa_workspace_bytes(H, S_T, S_V, S_A, bad) == 0
    # no video tiles: any valid fraction gives the dense-only workspace
    assert bsv.vsa_workspace_bytes(H, S_T, 0, S_A, 1.0) > 0
