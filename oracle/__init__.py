"""Reference implementation of the fused MoE layer (CPU) -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library never loads it and shares no code with it; the product
path fails when its own HIP library is missing instead of falling back to this code.

The arithmetic lives in ``oracle.c`` (plain C, IEEE double except where fp32 decides an
integer or a stored code); this module only builds it with gcc and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        lib.oracle_bf16_to_f32.restype = ctypes.c_float
        lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_e4m3_decode.restype = ctypes.c_float
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.oracle_router_logits.argtypes = [P, P, i, i, i, P]
        lib.oracle_router_topk.argtypes = [P, i, i, i, i, i, i, P, P]
        lib.oracle_router_topk_grouped.argtypes = [P, i, i, i, i, i, i, i, i, P, P]
        lib.oracle_rows_per_expert_estimate.restype = i
        lib.oracle_rows_per_expert_estimate.argtypes = [ctypes.c_longlong] * 3
        lib.oracle_route_permute.argtypes = [i, i, i, i, i, P, P, P, P, P, P]
        lib.oracle_act_quant.argtypes = [P, i, i, P, P]
        lib.oracle_moe_tokens.argtypes = [i] * 8 + [P] * 9 + [P, i, P]
        lib.oracle_num_threads.restype = i
        lib.oracle_set_num_threads.argtypes = [i]
        lib.oracle_grouped_gemm.restype = i
        lib.oracle_grouped_gemm.argtypes = [i] * 9 + [P, P, P, i, P, P, P, P, P]
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- scalar formats

def bf16_to_f32(b: int) -> float:
    return float(_load().oracle_bf16_to_f32(int(b)))


def e4m3_decode(code: int) -> float:
    return float(_load().oracle_e4m3_decode(int(code)))


def e4m3_encode(x: float) -> int:
    return int(_load().oracle_e4m3_encode(float(x)))


# ---------------------------------------------------------------- router

def router_logits(x_bf16: np.ndarray, wr_bf16: np.ndarray) -> np.ndarray:
    """x [T,H] and Wr [E,H] as uint16 bf16 bit patterns -> fp32 logits [T,E]."""
    x = _c(x_bf16, np.uint16)
    wr = _c(wr_bf16, np.uint16)
    T, H = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), np.float32)
    _load().oracle_router_logits(_p(x), _p(wr), T, H, E, _p(out))
    return out


def router_topk(logits: np.ndarray, k: int, scoring: str = "softmax", renorm: bool = True,
                is_bf16: bool | None = None):
    """logits [T,E] fp32, or uint16 bf16 bit patterns -> (ids int32 [T,k], weights float64 [T,k])."""
    if is_bf16 is None:
        is_bf16 = logits.dtype == np.uint16
    lg = _c(logits, np.uint16 if is_bf16 else np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _load().oracle_router_topk(_p(lg), int(is_bf16), T, E, k, 0 if scoring == "softmax" else 1,
                               int(bool(renorm)), _p(ids), _p(w))
    return ids, w


def router_topk_grouped(logits: np.ndarray, k: int, n_group: int, topk_group: int, scoring: str = "softmax",
                        renorm: bool = True, is_bf16: bool | None = None):
    """Grouped (group-limited) top-k, the definition in oracle.c: keep the topk_group groups
    (of E/n_group consecutive experts) with the largest best logit, then plain top-k among
    their experts.  logits [T,E] fp32 or uint16 bf16 bits -> (ids int32 [T,k], weights float64)."""
    if is_bf16 is None:
        is_bf16 = logits.dtype == np.uint16
    lg = _c(logits, np.uint16 if is_bf16 else np.float32)
    T, E = lg.shape
    if n_group < 1 or E % n_group or not 1 <= topk_group <= n_group or k > topk_group * (E // n_group):
        raise ValueError("need E % n_group == 0, 1 <= topk_group <= n_group, k <= topk_group * E / n_group")
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _load().oracle_router_topk_grouped(_p(lg), int(is_bf16), T, E, k, n_group, topk_group,
                                       0 if scoring == "softmax" else 1, int(bool(renorm)), _p(ids), _p(w))
    return ids, w


def rows_per_expert_estimate(T: int, k: int, E: int) -> int:
    return int(_load().oracle_rows_per_expert_estimate(T, k, E))


# ---------------------------------------------------------------- grouping

def route_permute(ids: np.ndarray, E: int, ep_size: int = 1, ep_rank: int = 0):
    """ids [T,k] int32 -> dict(counts, offsets, perm_src (length R), inv_perm [T*k], dropped)."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    El = E // ep_size
    counts = np.empty(El, np.int32)
    offsets = np.empty(El + 1, np.int32)
    perm_src = np.empty(max(T * k, 1), np.int32)
    inv_perm = np.empty(max(T * k, 1), np.int32)
    dropped = ctypes.c_longlong(0)
    _load().oracle_route_permute(T, k, E, ep_size, ep_rank, _p(ids), _p(counts), _p(offsets),
                                 _p(perm_src), _p(inv_perm), ctypes.byref(dropped))
    R = int(offsets[El])
    return dict(counts=counts, offsets=offsets, perm_src=perm_src[:R].copy(),
                inv_perm=inv_perm[:T * k].copy(), dropped=int(dropped.value))


# ---------------------------------------------------------------- FP8 activation quantisation

def act_quant(x: np.ndarray):
    """x [rows, cols] fp32 (cols a multiple of 128) -> (codes uint8 [rows, cols], scales fp32 [rows, cols/128])."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 128), np.float32)
    _load().oracle_act_quant(_p(x), rows, cols, _p(q), _p(s))
    return q, s


# ---------------------------------------------------------------- layer

def moe_tokens(x_bf16, ids, w, wg, wu, wd, *, E, ep_size=1, ep_rank=0, sg=None, su=None, sd=None,
               tokens=None) -> np.ndarray:
    """Layer output (float64 [len(tokens), H]) for the listed tokens (default: all).

    x_bf16 [T,H] uint16; ids [T,k] int32; w [T,k] routing weights (float64 or fp32);
    wg/wu [E_loc,I,H] and wd [E_loc,H,I] as uint16 (bf16) or uint8 (e4m3 codes, with the
    fp32 block scales sg/su [E_loc,I/128,H/128] and sd [E_loc,H/128,I/128])."""
    x = _c(x_bf16, np.uint16)
    ids = _c(ids, np.int32)
    w = _c(w, np.float64)
    T, H = x.shape
    k = ids.shape[1]
    fp8 = wg.dtype == np.uint8
    wdt = np.uint8 if fp8 else np.uint16
    wg = _c(wg, wdt)
    wu = _c(wu, wdt)
    wd = _c(wd, wdt)
    I = wg.shape[1]
    if fp8:
        sg, su, sd = (_c(s, np.float32) for s in (sg, su, sd))
    else:
        sg = su = sd = np.zeros(1, np.float32)
    tok = np.arange(T, dtype=np.int32) if tokens is None else _c(tokens, np.int32)
    out = np.zeros((len(tok), H), np.float64)
    _load().oracle_moe_tokens(T, H, I, E, k, ep_size, ep_rank, int(fp8), _p(x), _p(ids), _p(w),
                              _p(wg), _p(wu), _p(wd), _p(sg), _p(su), _p(sd), _p(tok), len(tok), _p(out))
    return out


def grouped_gemm(stage: int, ids: np.ndarray, E: int, a, w0, w1=None, *, a_scale=None, s0=None, s1=None,
                 ep_size: int = 1, ep_rank: int = 0) -> np.ndarray:
    """One grouped GEMM stage (oracle.c oracle_grouped_gemm) -> float64 [R, N] in grouped order.

    ids [T,k] int32 (grouped as route_permute does); stage 0: a [T,H] activation rows, w0/w1 gate
    and up [E_loc,I,H]; stage 1: a [T*k,I] grouped rows (first R used), w0 down [E_loc,H,I].
    a: uint16 bf16 bits, or uint8 e4m3 codes with a_scale [rows, K/128]; weights: uint16 bf16 bits,
    or uint8 codes with block scales s0 (and s1 for up)."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    a_fp8 = a.dtype == np.uint8
    a = _c(a, np.uint8 if a_fp8 else np.uint16)
    K = a.shape[1]
    w_fp8 = w0.dtype == np.uint8
    wdt = np.uint8 if w_fp8 else np.uint16
    w0 = _c(w0, wdt)
    N = w0.shape[1]
    w1 = _c(w1, wdt) if stage == 0 else w0
    a_scale = _c(a_scale, np.float32) if a_fp8 else np.zeros(1, np.float32)
    if w_fp8:
        s0 = _c(s0, np.float32)
        s1 = _c(s1, np.float32) if stage == 0 else s0
    else:
        s0 = s1 = np.zeros(1, np.float32)
    out = np.zeros((max(T * k, 1), N), np.float64)
    R = _load().oracle_grouped_gemm(stage, T, k, E, ep_size, ep_rank, N, K, int(a_fp8), _p(ids), _p(a),
                                    _p(a_scale), int(w_fp8), _p(w0), _p(w1), _p(s0), _p(s1), _p(out))
    return out[:R].copy()


def set_num_threads(n: int) -> None:
    """OpenMP threads of the oracle's parallel loops (n <= 0 leaves the setting)."""
    _load().oracle_set_num_threads(int(n))


def num_threads() -> int:
    return int(_load().oracle_num_threads())
