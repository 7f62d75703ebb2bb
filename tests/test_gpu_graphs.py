"""HIP-graph capture of fmoe_forward at padded token buckets, padding rows NaN in x and in the
logits: routing of the real rows bit for bit, their outputs within the layer's bar and finite
(FP8 included: the per-row activation quantizer keeps NaN rows to themselves), replays
interleaved with eager calls, one capture per bucket."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_sigmoid_amd as fm
from mixture_experts_layer_sigmoid_amd.graphs import BucketedForward
from gpu_common import BF16_TOL, FP8_TOL, WEIGHT_TOL, Layer, announce, row_rel_err

pytestmark = pytest.mark.gpu


def check_real_rows(L, out, ids, wts):
    ids_ref, w_ref = L.oracle_routing()
    assert np.array_equal(ids.cpu().numpy(), ids_ref), "routing of the real rows differs from the oracle"
    assert np.abs(wts.cpu().numpy() - w_ref).max() <= WEIGHT_TOL
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all(), "a real row picked up a NaN from the padding"
    ref = L.oracle_tokens(ids_ref, w_ref, np.arange(L.T, dtype=np.int32))
    assert row_rel_err(got, ref) <= (FP8_TOL if L.fp8 else BF16_TOL)


@pytest.mark.parametrize("fp8", [False, True])
def test_bucketed_graphs_with_nan_padding_rows(fp8):
    H, I, E, k = 512, 256, 16, 4
    cases = [(96, 37), (97, 64), (98, 5), (99, 37), (100, 1)]  # (input config, real tokens)
    layers = [Layer(config=c, weight_config=95, T=T, H=H, I=I, E=E, k=k, fp8=fp8) for c, T in cases]
    bf = BucketedForward(H, I, E, k, layers[0].w, fp8=fp8, buckets=(8, 64))
    for L in layers:
        announce(f"graph bucket {bf.bucket(L.T)} with {L.T} real rows, fp8={fp8}")
        out, ids, wts = bf(L.x_gpu, L.logits_gpu, return_routing=True)
        torch.cuda.synchronize()
        check_real_rows(L, out, ids, wts)
        # eager work between replays: the same rows without padding, through the plain call
        eo, eids, ewts = fm.fmoe_forward(L.shape, L.x_gpu, L.logits_gpu, layers[0].w, ws=fm.workspace(L.shape),
                                         return_routing=True)
        torch.cuda.synchronize()
        assert torch.equal(eids, ids)
        check_real_rows(L, eo, eids, ewts)
    assert sorted(bf._entries) == [8, 64]  # one capture per bucket
    with pytest.raises(ValueError):
        bf(torch.zeros((65, H), dtype=torch.bfloat16, device="cuda"),
           torch.zeros((65, E), dtype=torch.bfloat16, device="cuda"))
