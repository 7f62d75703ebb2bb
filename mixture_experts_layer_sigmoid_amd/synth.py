"""Seeded synthetic inputs for the fused MoE layer.

The pages measured on model traffic and on an unpublished synthetic script, so every
tensor here is a seeded stand-in with the stated shapes and distributions:
  * activations x ~ N(0,1), router logits ~ N(0,1), expert and router weights ~ N(0,0.02),
    all generated in fp32 by NumPy's PCG64 and rounded to bf16 (round to nearest even);
  * the router test batch of 128 tokens x 128 experts carries NaNs in 10% of its entries
    and 4 all-NaN rows (the padding-row failure of "PR #39593 ... CUDA graphs IMA",
    Root cause and Test Plan), plus a row of equal values and a row with exact ties
    straddling the top-k boundary;
  * concentrated routing sends 90% of the assignments to 8 experts by adding 16 to the
    logits of each token's chosen experts, so that the real router reproduces the sets;
  * FP8 expert weights are the bf16 weights scaled per [128,128] block to a maximum
    magnitude of 448 and cast with torch's float8_e4m3fn conversion (an offline weight
    preparation step, not part of the layer).

Every generator draws from its own stream keyed by (config, T, tensor[, expert]) so that
any subset can be regenerated alone.  The GPU path and the oracle receive the same bytes.
This module holds none of the layer's arithmetic.
"""
from __future__ import annotations

import functools
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

# tensor ids inside a config's key
X, LOGITS, WR, WG, WU, WD, ROUTE = range(7)

# config ids
TINY, ROUTER, BF16_LAYER, FP8_LAYER, EP_SHARD = 1, 2, 3, 4, 5


def rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def to_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def normal_bf16(shape, std: float, *key: int) -> torch.Tensor:
    a = rng(*key).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return to_bf16(a)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 numpy view of its bit patterns (CPU copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------- tiny layer

def tiny_layer(T: int = 16, H: int = 256, E: int = 8, I: int = 128, seed: int = 0) -> dict:
    """Tiny layer: bf16 x ~ N(0,1) [T,H]; Wr [E,H], W_gate/W_up [E,I,H], W_down [E,H,I] ~ N(0,0.02)."""
    c = TINY
    return dict(
        x=normal_bf16((T, H), 1.0, c, T, X, seed),
        wr=normal_bf16((E, H), 0.02, c, 0, WR, seed),
        wg=normal_bf16((E, I, H), 0.02, c, 0, WG, seed),
        wu=normal_bf16((E, I, H), 0.02, c, 0, WU, seed),
        wd=normal_bf16((E, H, I), 0.02, c, 0, WD, seed),
    )


# ----------------------------------------------------------------------------- router batch

def router_batch(T: int = 128, E: int = 128, k: int = 8, seed: int = 0) -> torch.Tensor:
    """bf16 logits [T,E] ~ N(0,1); round(10% of T*E) seeded NaN positions; 4 seeded all-NaN
    rows; one row of equal values; one row whose values at ranks k-2..k+1 are exact ties."""
    g = rng(ROUTER, T, LOGITS, seed)
    a = g.standard_normal(size=(T, E), dtype=np.float32)
    flat = a.reshape(-1)
    n_nan = int(round(0.10 * T * E))
    flat[g.choice(T * E, size=n_nan, replace=False)] = np.nan
    special = g.choice(T, size=min(T, 6), replace=False)
    for r in special[:4]:
        a[r, :] = np.nan
    if len(special) > 4:
        a[special[4], :] = np.float32(0.5)
    if len(special) > 5 and E >= k + 2:
        r = special[5]
        a[r, :] = g.standard_normal(size=E, dtype=np.float32)
        order = np.argsort(-a[r], kind="stable")
        tie = np.float32(a[r, order[k - 2]])
        for pos in range(k - 2, min(k + 2, E)):
            a[r, order[pos]] = tie
    return to_bf16(a)


# ----------------------------------------------------------------------------- layer inputs

def activations(config: int, T: int, H: int, seed: int = 0) -> torch.Tensor:
    return normal_bf16((T, H), 1.0, config, T, X, seed)


def routed_logits(config: int, T: int, E: int, k: int, routing: str = "uniform", hot: int = 8,
                  hot_frac: float = 0.9, seed: int = 0) -> torch.Tensor:
    """Router logits [T,E] bf16.

    uniform:      N(0,1).
    concentrated: N(0,1) + 16 on each token's chosen set.  round(hot_frac*T*k) assignments go
                  to the experts 0..hot-1 (hot <= E - k): every token takes floor(hot_total/T) of them and a
                  seeded subset of tokens one more (never more than min(hot,k)); its remaining
                  picks are seeded distinct experts from hot..E-1."""
    base = rng(config, T, LOGITS, seed).standard_normal(size=(T, E), dtype=np.float32)
    if routing == "uniform":
        return to_bf16(base)
    if routing != "concentrated":
        raise ValueError(routing)
    hot = min(hot, E - k)  # leave k cold experts for every token
    if hot < 1:
        raise ValueError("concentrated routing needs E > top_k")
    g = rng(config, T, ROUTE, seed)
    total = int(round(hot_frac * T * k))
    per = np.full(T, total // T, np.int64)
    extra = total - int(per.sum())
    per[g.permutation(T)[:extra]] += 1
    per = np.minimum(per, min(hot, k))
    for t in range(T):
        hot_ids = g.choice(hot, size=int(per[t]), replace=False)
        cold_ids = hot + g.choice(E - hot, size=k - int(per[t]), replace=False)
        base[t, hot_ids] += np.float32(16.0)
        base[t, cold_ids] += np.float32(16.0)
    return to_bf16(base)


@functools.lru_cache(maxsize=4)
def expert_weights_bf16(config: int, E_loc: int, H: int, I: int, first_expert: int = 0, seed: int = 0):
    """bf16 W_gate, W_up [E_loc,I,H] and W_down [E_loc,H,I] ~ N(0,0.02), one stream per
    (tensor, global expert id) so a rank's shard matches the same experts of a full set."""
    out = []
    jobs = []
    for tid, shape in ((WG, (I, H)), (WU, (I, H)), (WD, (H, I))):
        w = torch.empty((E_loc,) + shape, dtype=torch.bfloat16)
        out.append(w)
        jobs += [(w, l, shape, tid) for l in range(E_loc)]

    def fill(job):  # NumPy's generator and torch's cast release the GIL on large arrays
        w, l, shape, tid = job
        w[l] = normal_bf16(shape, 0.02, config, 0, tid, seed, first_expert + l)

    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        list(ex.map(fill, jobs))
    return tuple(out)


def block_quantize_fp8(w: torch.Tensor):
    """Offline FP8 weight preparation: bf16 [E,N,K] -> (e4m3 codes uint8 [E,N,K], fp32 scales
    [E,N/128,K/128]); scale = block max |w| / 448 (1 for an all-zero block), code =
    float8_e4m3fn cast of w/scale clamped to +-448."""
    E, N, K = w.shape
    codes = torch.empty((E, N, K), dtype=torch.uint8)
    scales = torch.empty((E, N // 128, K // 128), dtype=torch.float32)

    def one(e):
        b = w[e].float().reshape(N // 128, 128, K // 128, 128)
        amax = b.abs().amax(dim=(1, 3))
        s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        q = (b / s[:, None, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        codes[e] = q.reshape(N, K).view(torch.uint8)
        scales[e] = s

    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        list(ex.map(one, range(E)))
    return codes, scales


@functools.lru_cache(maxsize=2)
def expert_weights_fp8(config: int, E_loc: int, H: int, I: int, first_expert: int = 0, seed: int = 0):
    """FP8 block-scaled versions of expert_weights_bf16: (qg, qu, qd, sg, su, sd)."""
    wg, wu, wd = expert_weights_bf16(config, E_loc, H, I, first_expert, seed)
    qg, sg = block_quantize_fp8(wg)
    qu, su = block_quantize_fp8(wu)
    qd, sd = block_quantize_fp8(wd)
    return qg, qu, qd, sg, su, sd
