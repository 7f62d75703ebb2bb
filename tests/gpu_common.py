"""Helpers shared by the GPU parity tests: seeded layer cases, the oracle on the same bytes,
and the error measure.

Error measure (the layer's relative-error bars): per output row, max_h |y - y_ref| divided
by max_h |y_ref|, maximised over rows; a row whose reference is exactly zero must be
exactly zero on the GPU too.
"""
from __future__ import annotations

import functools

import numpy as np
import torch

import mixture_experts_layer_sigmoid_amd as fm
import oracle
from mixture_experts_layer_sigmoid_amd import synth

BF16_TOL = 2e-2
FP8_TOL = 6e-2
WEIGHT_TOL = 1e-6


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max(axis=1)
    zero = den == 0
    assert np.all(got[zero] == 0.0), "rows with an all-zero reference must be exactly zero"
    if (~zero).sum() == 0:
        return 0.0
    return float((np.abs(got - ref).max(axis=1)[~zero] / den[~zero]).max())


def announce(msg: str):
    print(f"[case] {msg}", flush=True)


class Layer:
    """A seeded layer case: inputs on the GPU plus their CPU bytes for the oracle."""

    def __init__(self, *, config, T, H, I, E, k, ep_size=1, ep_rank=0, fp8=False, routing="uniform", seed=0,
                 weight_config=None, scoring="softmax", renorm=True):
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.ep_size, self.ep_rank, self.fp8 = ep_size, ep_rank, fp8
        self.scoring, self.renorm = scoring, renorm
        self.El = E // ep_size
        wc = config if weight_config is None else weight_config
        self.x = synth.activations(config, T, H, seed)
        self.logits = synth.routed_logits(config, T, E, k, routing, seed=seed)
        if fp8:
            q = synth.expert_weights_fp8(wc, self.El, H, I, ep_rank * self.El, seed)
            self.w_cpu = q
            gpu = [t.cuda() for t in q]
            self.w = fm.ExpertWeights(*gpu)
        else:
            q = synth.expert_weights_bf16(wc, self.El, H, I, ep_rank * self.El, seed)
            self.w_cpu = q
            self.w = fm.ExpertWeights(*[t.cuda() for t in q])
        self.x_gpu = self.x.cuda()
        self.logits_gpu = self.logits.cuda()
        self.shape = fm.make_shape(T, H, I, E, k, ep_size, ep_rank, fp8)

    plan = None  # an fmoe_plan to force tile choices (None: the library's heuristic)

    def forward(self, ws=None):
        sc = fm.FMOE_SOFTMAX if self.scoring == "softmax" else fm.FMOE_SIGMOID
        return fm.fmoe_forward(self.shape, self.x_gpu, self.logits_gpu, self.w, sc, self.renorm, ws=ws,
                               return_routing=True, plan=self.plan)

    def oracle_routing(self):
        return oracle.router_topk(synth.bf16_bits(self.logits), self.k, self.scoring, self.renorm)

    def oracle_tokens(self, ids, w, tokens):
        if self.fp8:
            qg, qu, qd, sg, su, sd = (t.numpy() for t in self.w_cpu)
            return oracle.moe_tokens(synth.bf16_bits(self.x), ids, w, qg, qu, qd, E=self.E, ep_size=self.ep_size,
                                     ep_rank=self.ep_rank, sg=sg, su=su, sd=sd, tokens=tokens)
        wg, wu, wd = (synth.bf16_bits(t) for t in self.w_cpu)
        return oracle.moe_tokens(synth.bf16_bits(self.x), ids, w, wg, wu, wd, E=self.E, ep_size=self.ep_size,
                                 ep_rank=self.ep_rank, tokens=tokens)


@functools.lru_cache(maxsize=None)
def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    if T <= n:
        return np.arange(T, dtype=np.int32)
    g = np.random.default_rng(seed + T)
    mid = g.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, T - 1], mid])).astype(np.int32)


def check_layer(L: Layer, n_sample: int = 32, tol: float | None = None) -> dict:
    """Run the layer on the GPU, compare routing bit for bit over all tokens and the output on
    a token sample (all tokens when T <= n_sample) against the oracle."""
    out, ids, wts = L.forward()
    torch.cuda.synchronize()
    ids_ref, w_ref = L.oracle_routing()
    ids_g = ids.cpu().numpy()
    assert np.array_equal(ids_g, ids_ref), "top-k ids differ from the oracle"
    werr = float(np.abs(wts.cpu().numpy() - w_ref).max()) if L.T else 0.0
    assert werr <= WEIGHT_TOL, f"routing weights differ by {werr}"
    tok = sample_tokens(L.T, n_sample)
    ref = L.oracle_tokens(ids_ref, w_ref, tok)
    got = out.float().cpu().numpy()[tok]
    err = row_rel_err(got, ref)
    bar = tol if tol is not None else (FP8_TOL if L.fp8 else BF16_TOL)
    assert err <= bar, f"max row relative error {err:.3e} > {bar}"
    return dict(err=err, werr=werr)
