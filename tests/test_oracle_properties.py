"""Property tests of the CPU oracle on shapes drawn by hypothesis (T <= 64, E <= 16, k <= E):
the router against NumPy's stable sort of the sanitised logits and the closed-form weights,
the grouping against NumPy's bincount and stable argsort, and the layer against a dense
torch float64 mixture in which every expert sees every token.  CPU only."""
import numpy as np
import pytest
import scipy.special
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

FLT_MAX = np.float32(np.finfo(np.float32).max)
SETTINGS = settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def logit_batches(draw):
    """fp32 logits [T, E] from N(0,1), with some entries NaN or +-inf, some rows all NaN, and
    ties from rounding to a coarse grid (so equal keys are common)."""
    T = draw(st.integers(1, 64))
    E = draw(st.integers(1, 16))
    k = draw(st.integers(1, E))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    g = np.random.default_rng(seed)
    lg = g.standard_normal((T, E)).astype(np.float32)
    if draw(st.booleans()):
        lg = np.round(lg * 2) / 2  # ties
    special = g.random((T, E))
    lg[special < 0.05] = np.nan
    lg[(special >= 0.05) & (special < 0.07)] = np.inf
    lg[(special >= 0.07) & (special < 0.09)] = -np.inf
    if T > 1 and draw(st.booleans()):
        lg[g.integers(0, T)] = np.nan
    return lg, k


def sanitised(lg):
    v = np.where(np.isnan(lg), -FLT_MAX, lg)
    return np.clip(v, -FLT_MAX, FLT_MAX).astype(np.float32)


@SETTINGS
@given(logit_batches(), st.sampled_from(["softmax", "sigmoid"]), st.booleans())
def test_router_is_the_stable_sort_of_sanitised_logits(batch, scoring, renorm):
    lg, k = batch
    ids, w = oracle.router_topk(lg, k, scoring, renorm)
    v = sanitised(lg).astype(np.float64)
    ref = np.argsort(-v, axis=1, kind="stable")[:, :k]
    assert np.array_equal(ids, ref)
    assert all(len(set(r)) == k for r in ids.tolist())
    picked = np.take_along_axis(v, ids, axis=1)
    if scoring == "softmax":
        if renorm:
            ref_w = scipy.special.softmax(picked, axis=1)
        else:
            ref_w = np.take_along_axis(scipy.special.softmax(v, axis=1), ids, axis=1)
    else:
        s = scipy.special.expit(picked)
        if renorm:
            tot = s.sum(axis=1, keepdims=True)
            ref_w = np.where(tot > 0, s / np.where(tot > 0, tot, 1), 1.0 / k)
        else:
            ref_w = s
    assert np.abs(w - ref_w).max() <= 1e-6
    if renorm:
        assert np.abs(w.sum(axis=1) - 1).max() <= 1e-6


@SETTINGS
@given(st.integers(1, 64), st.integers(1, 16), st.data())
def test_grouping_is_bincount_and_stable_argsort(T, E, data):
    k = data.draw(st.integers(1, 8))
    ep_size = data.draw(st.sampled_from([d for d in (1, 2, 4, 8) if E % d == 0]))
    ep_rank = data.draw(st.integers(0, ep_size - 1))
    seed = data.draw(st.integers(0, 2 ** 31 - 1))
    ids = np.random.default_rng(seed).integers(-2, E + 2, (T, k)).astype(np.int32)  # repeats and bad ids
    r = oracle.route_permute(ids, E, ep_size, ep_rank)
    El = E // ep_size
    flat = ids.ravel()
    local = flat - ep_rank * El
    ok = (flat >= 0) & (flat < E) & (local >= 0) & (local < El)
    assert np.array_equal(r["counts"], np.bincount(local[ok], minlength=El))
    assert np.array_equal(r["offsets"], np.concatenate([[0], np.cumsum(r["counts"])]))
    order = np.nonzero(ok)[0]
    order = order[np.argsort(local[ok], kind="stable")]
    assert np.array_equal(r["perm_src"], order)
    inv = np.full(T * k, -1)
    inv[order] = np.arange(len(order))
    assert np.array_equal(r["inv_perm"], inv)
    assert r["dropped"] == int(((flat < 0) | (flat >= E)).sum())


def bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).numpy().view(np.uint16)


@SETTINGS
@given(st.integers(1, 12), st.sampled_from([128, 256]), st.sampled_from([128, 256]), st.integers(1, 8), st.data())
def test_layer_is_the_dense_gated_mixture(T, H, I, E, data):
    k = data.draw(st.integers(1, E))
    scoring = data.draw(st.sampled_from(["softmax", "sigmoid"]))
    seed = data.draw(st.integers(0, 2 ** 31 - 1))
    g = np.random.default_rng(seed)
    x = bf16(g.standard_normal((T, H)))
    wg, wu = bf16(0.05 * g.standard_normal((E, I, H))), bf16(0.05 * g.standard_normal((E, I, H)))
    wd = bf16(0.05 * g.standard_normal((E, H, I)))
    lg = g.standard_normal((T, E)).astype(np.float32)
    ids, w = oracle.router_topk(lg, k, scoring, True)
    out = oracle.moe_tokens(bits(x), ids, w, bits(wg), bits(wu), bits(wd), E=E)
    gate = np.zeros((T, E))
    np.put_along_axis(gate, ids, w, axis=1)
    xd = x.double()
    ys = torch.stack([(torch.nn.functional.silu(xd @ wg[e].double().T) * (xd @ wu[e].double().T)) @ wd[e].double().T
                      for e in range(E)], 1)
    ref = (torch.from_numpy(gate)[:, :, None] * ys).sum(1).numpy()
    assert np.allclose(out, ref, rtol=1e-9, atol=1e-12)


if __name__ == "__main__":
    pytest.main([__file__, "-q"])
