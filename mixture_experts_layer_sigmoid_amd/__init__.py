"""Python binding of libfmoe, the fused mixture-of-experts layer for MI355X (gfx950).

Argument marshalling only: every function here checks tensor devices, dtypes and shapes,
allocates outputs with torch (device memory), and calls the C entry point of the same name
in ``libfmoe.so`` with raw device pointers and torch's current HIP stream.  Every step of
the layer runs in the library's HIP kernels.  There is no fallback: if the library is not
built, or a call fails, these functions raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfmoe.so")

FMOE_OK, FMOE_ERR_ARG, FMOE_ERR_UNSUPPORTED, FMOE_ERR_WORKSPACE, FMOE_ERR_HIP = range(5)
FMOE_BF16, FMOE_FP32, FMOE_FP8_E4M3 = 0, 1, 2
FMOE_SOFTMAX, FMOE_SIGMOID = 0, 1
FMOE_NUM_STAGES = 10
STAGES = ("router", "group", "quant_x", "gemm1", "gemm1_split", "gemm1_heavy", "quant_h", "gemm2", "gemm2_heavy",
          "combine")
EXPORTED = ("fmoe_abi_version", "fmoe_status_string", "fmoe_workspace_bytes", "fmoe_router_logits",
            "fmoe_router_topk", "fmoe_route_permute", "fmoe_experts", "fmoe_forward", "fmoe_forward_profiled",
            "fmoe_forward_planned", "fmoe_router_topk_grouped", "fmoe_read_stats", "fmoe_act_quant",
            "fmoe_workspace_layout", "fmoe_grouped_gemm", "fmoe_forward_noalloc")


class fmoe_shape(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("ep_size", ctypes.c_int32),
                ("ep_rank", ctypes.c_int32), ("weight_dtype", ctypes.c_int32)]


class fmoe_weights(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("gate_scale", ctypes.c_void_p), ("up_scale", ctypes.c_void_p), ("down_scale", ctypes.c_void_p)]


class fmoe_plan(ctypes.Structure):
    """Tile plan overrides (0 keeps the heuristic's choice): tile_rows 16/32, split_gate_up and
    split_down 1 (streaming kernel), 2 or 4 wavefronts per reduction, light_tiles 1 or 8 light
    tiles per expert at most (8: heavy-tile launches left out when no expert can need more),
    heavy_rows 256 or 320 (bf16: experts of 257..320 rows as one heavy tile of five row groups)."""
    _fields_ = [("tile_rows", ctypes.c_int32), ("split_gate_up", ctypes.c_int32), ("split_down", ctypes.c_int32),
                ("light_tiles", ctypes.c_int32), ("heavy_rows", ctypes.c_int32)]


class fmoe_layout(ctypes.Structure):
    """Byte offsets of the intermediate buffers inside a workspace (0: absent for this dtype)."""
    _fields_ = [(n, ctypes.c_size_t) for n in ("x_codes", "x_scales", "h_f32", "h_codes", "h_scales", "h_bf16",
                                               "y", "perm_src", "inv_perm", "total")]


class fmoe_stats(ctypes.Structure):
    _fields_ = [("dropped_ids", ctypes.c_int64), ("local_rows", ctypes.c_int32), ("max_rows", ctypes.c_int32),
                ("empty_experts", ctypes.c_int32), ("m_tiles", ctypes.c_int32), ("rows_estimate", ctypes.c_int32),
                ("tile_rows", ctypes.c_int32), ("heavy_tiles", ctypes.c_int32),
                ("heavy_rows", ctypes.c_int32), ("light_rows", ctypes.c_int32),
                ("split_light_tiles", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.fmoe_abi_version.restype = ctypes.c_int
    lib.fmoe_abi_version.argtypes = []
    lib.fmoe_status_string.restype = ctypes.c_char_p
    lib.fmoe_status_string.argtypes = [ctypes.c_int]
    lib.fmoe_workspace_bytes.argtypes = [ctypes.POINTER(fmoe_shape), ctypes.POINTER(sz)]
    lib.fmoe_router_logits.argtypes = [P, P, i32, i32, i32, P, P]
    lib.fmoe_router_topk.argtypes = [P, i32, i32, i32, i32, i32, i32, P, P, P]
    lib.fmoe_router_topk_grouped.argtypes = [P, i32, i32, i32, i32, i32, i32, i32, i32, P, P, P]
    lib.fmoe_route_permute.argtypes = [ctypes.POINTER(fmoe_shape), P, P, P, P, P, P, sz, P]
    lib.fmoe_experts.argtypes = [ctypes.POINTER(fmoe_shape), P, P, P, ctypes.POINTER(fmoe_weights), P, P, sz, P]
    lib.fmoe_forward.argtypes = [ctypes.POINTER(fmoe_shape), P, P, i32, i32, i32, ctypes.POINTER(fmoe_weights), P,
                                 P, P, P, sz, P]
    lib.fmoe_forward_profiled.argtypes = lib.fmoe_forward.argtypes + [P]
    lib.fmoe_forward_planned.argtypes = lib.fmoe_forward.argtypes + [ctypes.POINTER(fmoe_plan)]
    lib.fmoe_read_stats.argtypes = [P, P, ctypes.POINTER(fmoe_stats)]
    lib.fmoe_act_quant.argtypes = [P, i32, ctypes.c_int64, i32, P, P, P]
    lib.fmoe_forward_noalloc.argtypes = [ctypes.POINTER(fmoe_shape), P, P, i32, i32, i32,
                                         ctypes.POINTER(fmoe_weights), P, P, P, P]
    lib.fmoe_workspace_layout.argtypes = [ctypes.POINTER(fmoe_shape), ctypes.POINTER(fmoe_layout)]
    lib.fmoe_grouped_gemm.argtypes = [ctypes.POINTER(fmoe_shape), ctypes.POINTER(fmoe_plan), i32, P, P, P,
                                      ctypes.POINTER(fmoe_weights), i32, P, P, P, sz, P]
    for name in EXPORTED:
        if name != "fmoe_status_string":
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(name: str, rc: int):
    if rc != FMOE_OK:
        msg = load_library().fmoe_status_string(rc).decode()
        raise RuntimeError(f"{name} failed: {msg} (status {rc})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor, what: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    return t


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FMOE_BF16
    if t.dtype == torch.float32:
        return FMOE_FP32
    raise ValueError(f"unsupported logits dtype {t.dtype}")


# ----------------------------------------------------------------------------- shapes and weights

def make_shape(tokens, hidden, inter, experts, top_k, ep_size=1, ep_rank=0, fp8=False) -> fmoe_shape:
    return fmoe_shape(tokens, hidden, inter, experts, top_k, ep_size, ep_rank, FMOE_FP8_E4M3 if fp8 else FMOE_BF16)


class ExpertWeights:
    """Local expert weights on the GPU: gate, up [E_loc,I,H], down [E_loc,H,I] (bf16, or uint8
    e4m3 codes with fp32 block scales gate_scale, up_scale [E_loc,I/128,H/128], down_scale
    [E_loc,H/128,I/128])."""

    def __init__(self, gate, up, down, gate_scale=None, up_scale=None, down_scale=None):
        self.fp8 = gate.dtype == torch.uint8
        wdt = torch.uint8 if self.fp8 else torch.bfloat16
        self.gate = _dev(gate, "gate", wdt)
        self.up = _dev(up, "up", wdt)
        self.down = _dev(down, "down", wdt)
        if self.fp8:
            self.gate_scale = _dev(gate_scale, "gate_scale", torch.float32)
            self.up_scale = _dev(up_scale, "up_scale", torch.float32)
            self.down_scale = _dev(down_scale, "down_scale", torch.float32)
        else:
            self.gate_scale = self.up_scale = self.down_scale = None
        self.E_loc, self.I, self.H = gate.shape
        if tuple(up.shape) != (self.E_loc, self.I, self.H) or tuple(down.shape) != (self.E_loc, self.H, self.I):
            raise ValueError("gate/up must be [E_loc,I,H] and down [E_loc,H,I]")

    def struct(self) -> fmoe_weights:
        return fmoe_weights(self.gate.data_ptr(), self.up.data_ptr(), self.down.data_ptr(),
                            _ptr(self.gate_scale), _ptr(self.up_scale), _ptr(self.down_scale))


# ----------------------------------------------------------------------------- entry points

def fmoe_abi_version() -> int:
    return int(load_library().fmoe_abi_version())


def fmoe_workspace_bytes(shape: fmoe_shape) -> int:
    n = ctypes.c_size_t(0)
    _check("fmoe_workspace_bytes", load_library().fmoe_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)))
    return int(n.value)


def workspace(shape: fmoe_shape, device="cuda") -> torch.Tensor:
    """A uint8 workspace tensor of fmoe_workspace_bytes(shape) bytes (256-byte aligned by torch)."""
    return torch.empty(max(fmoe_workspace_bytes(shape), 1), dtype=torch.uint8, device=device)


def fmoe_router_logits(x: torch.Tensor, w_r: torch.Tensor) -> torch.Tensor:
    """x [T,H] bf16, w_r [E,H] bf16 -> fp32 logits [T,E]."""
    _dev(x, "x", torch.bfloat16)
    _dev(w_r, "w_r", torch.bfloat16)
    T, H = x.shape
    E = w_r.shape[0]
    if w_r.shape[1] != H:
        raise ValueError("w_r must be [E,H]")
    out = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _check("fmoe_router_logits",
           load_library().fmoe_router_logits(_ptr(x), _ptr(w_r), T, H, E, _ptr(out), _stream(x.device)))
    return out


def fmoe_router_topk(logits: torch.Tensor, k: int, scoring: int = FMOE_SOFTMAX, renormalize: bool = True):
    """logits [T,E] bf16 or fp32 -> (ids int32 [T,k], weights fp32 [T,k])."""
    _dev(logits, "logits")
    T, E = logits.shape
    ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    wts = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check("fmoe_router_topk",
           load_library().fmoe_router_topk(_ptr(logits), _dtype_code(logits), T, E, k, scoring, int(bool(renormalize)),
                                           _ptr(ids), _ptr(wts), _stream(logits.device)))
    return ids, wts


def fmoe_router_topk_grouped(logits: torch.Tensor, k: int, n_group: int, topk_group: int,
                             scoring: int = FMOE_SOFTMAX, renormalize: bool = True):
    """Grouped (group-limited) top-k: logits [T,E] bf16 or fp32 -> (ids int32 [T,k], weights fp32 [T,k])."""
    _dev(logits, "logits")
    T, E = logits.shape
    ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    wts = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check("fmoe_router_topk_grouped",
           load_library().fmoe_router_topk_grouped(_ptr(logits), _dtype_code(logits), T, E, k, n_group, topk_group,
                                                   scoring, int(bool(renormalize)), _ptr(ids), _ptr(wts),
                                                   _stream(logits.device)))
    return ids, wts


def fmoe_route_permute(shape: fmoe_shape, topk_ids: torch.Tensor, ws: torch.Tensor | None = None) -> dict:
    """Grouping of topk_ids [T,k] -> dict(counts [E_loc], offsets [E_loc+1], perm_src [T*k], inv_perm [T*k])."""
    _dev(topk_ids, "topk_ids", torch.int32)
    dev = topk_ids.device
    El = shape.experts // shape.ep_size
    n = shape.tokens * shape.top_k
    if tuple(topk_ids.shape) != (shape.tokens, shape.top_k):
        raise ValueError("topk_ids must be [T,k]")
    ws = workspace(shape, dev) if ws is None else ws
    counts = torch.empty(El, dtype=torch.int32, device=dev)
    offsets = torch.empty(El + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
    inv = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
    _check("fmoe_route_permute",
           load_library().fmoe_route_permute(ctypes.byref(shape), _ptr(topk_ids), _ptr(counts), _ptr(offsets),
                                             _ptr(perm), _ptr(inv), _ptr(ws), ws.numel(), _stream(dev)))
    return dict(counts=counts, offsets=offsets, perm_src=perm[:n], inv_perm=inv[:n], ws=ws)


def fmoe_experts(shape: fmoe_shape, x: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                 w: ExpertWeights, ws: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """Expert computation for given routing -> out [T,H] bf16."""
    _dev(x, "x", torch.bfloat16)
    _dev(topk_ids, "topk_ids", torch.int32)
    _dev(topk_weights, "topk_weights", torch.float32)
    ws = workspace(shape, x.device) if ws is None else ws
    out = torch.empty((shape.tokens, shape.hidden), dtype=torch.bfloat16, device=x.device) if out is None else out
    ws_struct = w.struct()
    _check("fmoe_experts",
           load_library().fmoe_experts(ctypes.byref(shape), _ptr(x), _ptr(topk_ids), _ptr(topk_weights),
                                       ctypes.byref(ws_struct), _ptr(out), _ptr(ws), ws.numel(), _stream(x.device)))
    return out


def fmoe_forward(shape: fmoe_shape, x: torch.Tensor, logits: torch.Tensor, w: ExpertWeights,
                 scoring: int = FMOE_SOFTMAX, renormalize: bool = True, ws: torch.Tensor | None = None,
                 out: torch.Tensor | None = None, return_routing: bool = False, stage_events=None,
                 routing_out: tuple | None = None, plan: fmoe_plan | None = None):
    """Whole layer -> out [T,H] bf16 (and (ids, weights) when return_routing).

    routing_out: optional preallocated (ids [T,k] int32, weights [T,k] fp32) that receive the
    routing (fixed buffers for graph capture); returned when return_routing.
    stage_events: optional list of FMOE_NUM_STAGES+1 entries, each a timing event (an object
    with a `cuda_event` handle, such as torch.cuda.Event(enable_timing=True)) or None; when
    given, fmoe_forward_profiled records the events around the stages (None entries are
    skipped).
    plan: optional fmoe_plan; when given, fmoe_forward_planned replaces the heuristic's tile
    choices with its nonzero fields (not combined with stage_events)."""
    _dev(x, "x", torch.bfloat16)
    _dev(logits, "logits")
    dev = x.device
    ws = workspace(shape, dev) if ws is None else ws
    out = torch.empty((shape.tokens, shape.hidden), dtype=torch.bfloat16, device=dev) if out is None else out
    ids = wts = None
    if routing_out is not None:
        ids, wts = routing_out
        _dev(ids, "routing ids", torch.int32)
        _dev(wts, "routing weights", torch.float32)
        if ids.shape != (shape.tokens, shape.top_k) or wts.shape != (shape.tokens, shape.top_k):
            raise ValueError("routing_out must be ([T, k] int32, [T, k] float32)")
    elif return_routing:
        ids = torch.empty((shape.tokens, shape.top_k), dtype=torch.int32, device=dev)
        wts = torch.empty((shape.tokens, shape.top_k), dtype=torch.float32, device=dev)
    ws_struct = w.struct()
    args = [ctypes.byref(shape), _ptr(x), _ptr(logits), _dtype_code(logits), scoring, int(bool(renormalize)),
            ctypes.byref(ws_struct), _ptr(out), _ptr(ids), _ptr(wts), _ptr(ws), ws.numel(), _stream(dev)]
    lib = load_library()
    if plan is not None:
        if stage_events is not None:
            raise ValueError("plan and stage_events cannot be combined")
        _check("fmoe_forward_planned", lib.fmoe_forward_planned(*args, ctypes.byref(plan)))
    elif stage_events is None:
        _check("fmoe_forward", lib.fmoe_forward(*args))
    else:
        if len(stage_events) != FMOE_NUM_STAGES + 1:
            raise ValueError("stage_events needs FMOE_NUM_STAGES + 1 events")
        for e in stage_events:  # torch creates the underlying hipEvent lazily
            if e is not None and e.cuda_event == 0:
                e.record()
        handles = (ctypes.c_void_p * len(stage_events))(*[e.cuda_event if e is not None else None
                                                          for e in stage_events])
        _check("fmoe_forward_profiled", lib.fmoe_forward_profiled(*args, handles))
    return (out, ids, wts) if return_routing else out


def fmoe_read_stats(ws: torch.Tensor) -> dict:
    """Counters the last call left in ws (synchronises the stream)."""
    st = fmoe_stats()
    _check("fmoe_read_stats", load_library().fmoe_read_stats(_ptr(ws), _stream(ws.device), ctypes.byref(st)))
    return {name: getattr(st, name) for name, _ in fmoe_stats._fields_}


def fmoe_act_quant(x: torch.Tensor):
    """Per-row, per-128-column e4m3 quantisation: x [rows, cols] bf16 or fp32 -> (codes uint8
    [rows, cols], scales fp32 [rows, cols/128])."""
    _dev(x, "x")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    sc = torch.empty((rows, max(cols // 128, 1)), dtype=torch.float32, device=x.device)
    _check("fmoe_act_quant", load_library().fmoe_act_quant(_ptr(x), _dtype_code(x), rows, cols, _ptr(q), _ptr(sc),
                                                           _stream(x.device)))
    return q, sc


def fmoe_workspace_layout(shape: fmoe_shape) -> dict:
    """Byte offsets of the layer's intermediate buffers in a workspace of this shape (0: absent)."""
    lay = fmoe_layout()
    _check("fmoe_workspace_layout", load_library().fmoe_workspace_layout(ctypes.byref(shape), ctypes.byref(lay)))
    return {name: int(getattr(lay, name)) for name, _ in fmoe_layout._fields_}


def ws_view(ws: torch.Tensor, offset: int, dtype, shape) -> torch.Tensor:
    """A typed view of `shape` elements at byte `offset` of a uint8 workspace tensor."""
    n = 1
    for d in shape:
        n *= int(d)
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    return ws[offset:offset + nbytes].view(dtype).view(*shape)


def fmoe_grouped_gemm(shape: fmoe_shape, stage: int, topk_ids: torch.Tensor, a: torch.Tensor, w: ExpertWeights,
                      a_scale: torch.Tensor | None = None, out_dtype: int | None = None,
                      plan: fmoe_plan | None = None, ws: torch.Tensor | None = None):
    """One grouped GEMM stage on given operands (rows in grouped order, T*k of them allocated).
    stage 0 -> out [T*k, I] (bf16 weights: bf16; FP8: fp32, or (codes, scales) for out_dtype
    FMOE_FP8_E4M3); stage 1 -> out [T*k, H] bf16."""
    _dev(topk_ids, "topk_ids", torch.int32)
    _dev(a, "a")
    if a_scale is not None:
        _dev(a_scale, "a_scale", torch.float32)
    dev = a.device
    n = max(shape.tokens * shape.top_k, 1)
    if out_dtype is None:
        out_dtype = FMOE_FP32 if (w.fp8 and stage == 0) else FMOE_BF16
    N = shape.inter if stage == 0 else shape.hidden
    out_scale = None
    if out_dtype == FMOE_FP32:
        out = torch.empty((n, N), dtype=torch.float32, device=dev)
    elif out_dtype == FMOE_FP8_E4M3:
        out = torch.empty((n, N), dtype=torch.uint8, device=dev)
        out_scale = torch.empty((n, N // 128), dtype=torch.float32, device=dev)
    else:
        out = torch.empty((n, N), dtype=torch.bfloat16, device=dev)
    ws = workspace(shape, dev) if ws is None else ws
    ws_struct = w.struct()
    _check("fmoe_grouped_gemm",
           load_library().fmoe_grouped_gemm(ctypes.byref(shape), None if plan is None else ctypes.byref(plan), stage,
                                            _ptr(topk_ids), _ptr(a), _ptr(a_scale), ctypes.byref(ws_struct), out_dtype,
                                            _ptr(out), _ptr(out_scale), _ptr(ws), ws.numel(), _stream(dev)))
    return (out, out_scale) if out_dtype == FMOE_FP8_E4M3 else out


NOALLOC_MAX_WORKSPACE = 64 << 20  # FMOE_NOALLOC_MAX_WORKSPACE


def fmoe_forward_noalloc(shape: fmoe_shape, x: torch.Tensor, logits: torch.Tensor, w: ExpertWeights,
                         scoring: int = FMOE_SOFTMAX, renormalize: bool = True, out: torch.Tensor | None = None,
                         routing_out: tuple | None = None):
    """fmoe_forward on the library's static per-GPU workspace (no workspace argument; the C call
    allocates nothing).  out and routing_out may be preallocated; returns out, or (out, ids,
    weights) when routing_out is given."""
    _dev(x, "x", torch.bfloat16)
    _dev(logits, "logits")
    dev = x.device
    out = torch.empty((shape.tokens, shape.hidden), dtype=torch.bfloat16, device=dev) if out is None else out
    ids = wts = None
    if routing_out is not None:
        ids, wts = routing_out
        _dev(ids, "routing ids", torch.int32)
        _dev(wts, "routing weights", torch.float32)
    ws_struct = w.struct()
    _check("fmoe_forward_noalloc",
           load_library().fmoe_forward_noalloc(ctypes.byref(shape), _ptr(x), _ptr(logits), _dtype_code(logits),
                                               scoring, int(bool(renormalize)), ctypes.byref(ws_struct), _ptr(out),
                                               _ptr(ids), _ptr(wts), _stream(dev)))
    return out if routing_out is None else (out, ids, wts)
