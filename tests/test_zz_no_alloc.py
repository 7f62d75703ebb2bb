"""fmoe_forward_noalloc (the library's static per-GPU workspace) against fmoe_forward with a
caller workspace: the same kernels and tile plan, so outputs and routing are bit-equal.  Two
calls in a row, the second with a smaller input (the buffer keeps the first call's contents),
then shapes beyond the buffer are rejected before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

import mixture_experts_layer_sigmoid_amd as fm
from mixture_experts_layer_sigmoid_amd import synth
from gpu_common import BF16_TOL, FP8_TOL, Layer, announce, row_rel_err

pytestmark = pytest.mark.gpu


def run_both(L: Layer):
    ws = fm.workspace(L.shape)
    ref, ids_r, wts_r = fm.fmoe_forward(L.shape, L.x_gpu, L.logits_gpu, L.w, ws=ws, return_routing=True)
    out = torch.empty_like(ref)
    ids = torch.empty_like(ids_r)
    wts = torch.empty_like(wts_r)
    fm.fmoe_forward_noalloc(L.shape, L.x_gpu, L.logits_gpu, L.w, out=out, routing_out=(ids, wts))
    torch.cuda.synchronize()
    return ref, ids_r, wts_r, out, ids, wts


@pytest.mark.parametrize("fp8", [False, True])
def test_noalloc_forward_matches_forward_twice_second_smaller(fp8):
    for T in (256, 40):  # the second call is smaller and finds the first one's data in the buffer
        announce(f"noalloc forward T={T} fp8={fp8}")
        L = Layer(config=synth.FP8_LAYER if fp8 else synth.BF16_LAYER, weight_config=synth.BF16_LAYER, T=T, H=2048,
                  I=768, E=128, k=8, fp8=fp8, routing="concentrated" if T == 40 else "uniform")
        ref, ids_r, wts_r, out, ids, wts = run_both(L)
        assert torch.equal(ids, ids_r) and torch.equal(wts, wts_r)
        assert torch.equal(out, ref), "noalloc output differs from fmoe_forward"
        # and against the oracle on a few tokens, to the layer's bar
        ids_o, w_o = L.oracle_routing()
        assert np.array_equal(ids.cpu().numpy(), ids_o)
        tok = np.array([0, T // 2, T - 1], np.int32)
        err = row_rel_err(out.float().cpu().numpy()[tok], L.oracle_tokens(ids_o, w_o, tok))
        assert err <= (FP8_TOL if fp8 else BF16_TOL)


def test_noalloc_forward_rejects_shapes_beyond_its_buffer():
    announce("noalloc forward: shapes beyond the static buffer")
    lib = fm.load_library()
    s = fm.make_shape(4096, 2048, 768, 128, 8)
    assert fm.fmoe_workspace_bytes(s) > fm.NOALLOC_MAX_WORKSPACE
    w = fm.fmoe_weights(0x1000, 0x2000, 0x3000, None, None, None)
    P = ctypes.c_void_p
    assert lib.fmoe_forward_noalloc(ctypes.byref(s), P(0x100), P(0x100), 0, 0, 1, ctypes.byref(w), P(0x300), None,
                                    None, None) == fm.FMOE_ERR_WORKSPACE
    s1024 = fm.make_shape(1024, 2048, 768, 128, 8)
    assert fm.fmoe_workspace_bytes(s1024) <= fm.NOALLOC_MAX_WORKSPACE
