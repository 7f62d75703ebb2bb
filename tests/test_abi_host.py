"""Host-side checks of the C ABI that need no GPU: the library loads, exports every entry
point the header declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_sigmoid_amd as fm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fmoe.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(fmoe_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = fm.load_library()
    names = declared_functions()
    assert len(names) >= 10
    assert set(names) == set(fm.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings():
    lib = fm.load_library()
    assert fm.fmoe_abi_version() == 4
    text = open(HEADER).read()
    assert "#define FMOE_ABI_VERSION 4" in text
    for code, word in [(0, b"ok"), (1, b"invalid"), (2, b"unsupported"), (3, b"workspace"), (4, b"HIP")]:
        assert word in lib.fmoe_status_string(code)


def ws_bytes(**kw):
    base = dict(tokens=16, hidden=256, inter=128, experts=8, top_k=2)
    base.update(kw)
    return fm.fmoe_workspace_bytes(fm.make_shape(**base))


def test_workspace_bytes_worst_case_and_growth():
    small = ws_bytes()
    assert small > 0
    # the Y buffer alone is T*k*H*2 bytes; the workspace holds at least that
    assert ws_bytes(tokens=4096, hidden=2048, inter=768, experts=128, top_k=8) >= 4096 * 8 * 2048 * 2
    assert ws_bytes(tokens=32) > ws_bytes(tokens=16)
    assert ws_bytes(tokens=1 << 22, top_k=2) > 0  # T*k = 2^23, the largest supported
    # fp8 keeps fp32 activations and codes on top of the bf16 layout
    assert ws_bytes(fp8=True) > 0
    # the size does not depend on the expert-parallel rank
    a = ws_bytes(tokens=288, hidden=7168, inter=2048, experts=400, top_k=6, ep_size=8, ep_rank=0, fp8=True)
    b = ws_bytes(tokens=288, hidden=7168, inter=2048, experts=400, top_k=6, ep_size=8, ep_rank=7, fp8=True)
    assert a == b
    assert ws_bytes(tokens=0) > 0


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=200), fm.FMOE_ERR_UNSUPPORTED),      # not a multiple of 128
    (dict(inter=100), fm.FMOE_ERR_UNSUPPORTED),
    (dict(top_k=9), fm.FMOE_ERR_ARG),                 # k > E
    (dict(top_k=0), fm.FMOE_ERR_ARG),
    (dict(tokens=-1), fm.FMOE_ERR_ARG),
    (dict(ep_size=3), fm.FMOE_ERR_ARG),               # does not divide E
    (dict(ep_size=2, ep_rank=2), fm.FMOE_ERR_ARG),
    (dict(experts=2048, top_k=2), fm.FMOE_ERR_UNSUPPORTED),
    (dict(experts=128, top_k=65), fm.FMOE_ERR_UNSUPPORTED),
    (dict(tokens=(1 << 22) + 1, top_k=2), fm.FMOE_ERR_UNSUPPORTED),  # T*k above 2^23
])
def test_workspace_bytes_rejects_bad_shapes(kw, code):
    base = dict(tokens=16, hidden=256, inter=128, experts=8, top_k=2)
    base.update(kw)
    s = fm.make_shape(**base)
    n = ctypes.c_size_t(0)
    assert fm.load_library().fmoe_workspace_bytes(ctypes.byref(s), ctypes.byref(n)) == code


def test_entry_points_reject_bad_arguments_without_a_device():
    lib = fm.load_library()
    s = fm.make_shape(16, 256, 128, 8, 2)
    w = fm.fmoe_weights(0x1000, 0x2000, 0x3000, None, None, None)
    ws_n = fm.fmoe_workspace_bytes(s)
    P = ctypes.c_void_p
    # null x
    assert lib.fmoe_experts(ctypes.byref(s), None, P(0x100), P(0x200), ctypes.byref(w), P(0x300), P(0x400),
                            ws_n, None) == fm.FMOE_ERR_ARG
    # misaligned output
    assert lib.fmoe_experts(ctypes.byref(s), P(0x100), P(0x100), P(0x200), ctypes.byref(w), P(0x308), P(0x400),
                            ws_n, None) == fm.FMOE_ERR_ARG
    # workspace too small
    assert lib.fmoe_experts(ctypes.byref(s), P(0x100), P(0x100), P(0x200), ctypes.byref(w), P(0x300), P(0x400),
                            ws_n - 1, None) == fm.FMOE_ERR_WORKSPACE
    # bf16 weights must not carry scales; fp8 weights must
    w_bad = fm.fmoe_weights(0x1000, 0x2000, 0x3000, 0x4000, None, None)
    assert lib.fmoe_experts(ctypes.byref(s), P(0x100), P(0x100), P(0x200), ctypes.byref(w_bad), P(0x300),
                            P(0x400), ws_n, None) == fm.FMOE_ERR_ARG
    s8 = fm.make_shape(16, 256, 128, 8, 2, fp8=True)
    assert lib.fmoe_experts(ctypes.byref(s8), P(0x100), P(0x100), P(0x200), ctypes.byref(w), P(0x300), P(0x400),
                            fm.fmoe_workspace_bytes(s8), None) == fm.FMOE_ERR_ARG
    # router: k > E, bad dtype, bad scoring
    assert lib.fmoe_router_topk(P(0x100), 0, 4, 8, 9, 0, 1, P(0x200), P(0x300), None) == fm.FMOE_ERR_ARG
    assert lib.fmoe_router_topk(P(0x100), 2, 4, 8, 2, 0, 1, P(0x200), P(0x300), None) == fm.FMOE_ERR_UNSUPPORTED
    assert lib.fmoe_router_topk(P(0x100), 0, 4, 8, 2, 5, 1, P(0x200), P(0x300), None) == fm.FMOE_ERR_ARG
    assert lib.fmoe_router_topk(P(0x100), 0, 4, 2000, 2, 0, 1, P(0x200), P(0x300), None) == fm.FMOE_ERR_UNSUPPORTED
    # forward with unsupported logits dtype
    assert lib.fmoe_forward(ctypes.byref(s), P(0x100), P(0x100), 7, 0, 1, ctypes.byref(w), P(0x300), None, None,
                            P(0x400), ws_n, None) == fm.FMOE_ERR_UNSUPPORTED
    # profiled forward needs its events
    assert lib.fmoe_forward_profiled(ctypes.byref(s), P(0x100), P(0x100), 0, 0, 1, ctypes.byref(w), P(0x300), None,
                                     None, P(0x400), ws_n, None, None) == fm.FMOE_ERR_ARG
    # stats need a workspace
    st = fm.fmoe_stats()
    assert lib.fmoe_read_stats(None, None, ctypes.byref(st)) == fm.FMOE_ERR_ARG


def test_zero_tokens_is_a_no_op():
    lib = fm.load_library()
    s = fm.make_shape(0, 256, 128, 8, 2)
    w = fm.fmoe_weights(0x1000, 0x2000, 0x3000, None, None, None)
    P = ctypes.c_void_p
    assert lib.fmoe_experts(ctypes.byref(s), None, None, None, ctypes.byref(w), None, None, 0, None) == fm.FMOE_OK
    assert lib.fmoe_forward(ctypes.byref(s), None, None, 0, 0, 1, ctypes.byref(w), None, None, None, None, 0,
                            None) == fm.FMOE_OK
    assert lib.fmoe_router_topk(None, 0, 0, 8, 2, 0, 1, None, None, None) == fm.FMOE_OK
    assert lib.fmoe_router_logits(None, None, 0, 256, 8, None, None) == fm.FMOE_OK
    assert lib.fmoe_route_permute(ctypes.byref(s), None, None, None, None, None, None, 0, None) == fm.FMOE_OK


def test_forward_planned_rejects_bad_plans_before_launching():
    lib = fm.load_library()
    P = ctypes.c_void_p
    s = fm.make_shape(16, 256, 128, 8, 2)
    w = fm.fmoe_weights(0x1000, 0x2000, 0x3000, None, None, None)
    ws_n = fm.fmoe_workspace_bytes(s)

    def call(shape, weights, plan):
        return lib.fmoe_forward_planned(ctypes.byref(shape), P(0x100), P(0x100), 0, 0, 1, ctypes.byref(weights),
                                        P(0x300), None, None, P(0x400), fm.fmoe_workspace_bytes(shape), None,
                                        ctypes.byref(plan))
    for bad in (fm.fmoe_plan(24, 0, 0), fm.fmoe_plan(0, 3, 0), fm.fmoe_plan(0, 0, 8), fm.fmoe_plan(-16, 1, 1),
                fm.fmoe_plan(64, 1, 1), fm.fmoe_plan(48, 0, 0), fm.fmoe_plan(0, 0, 0, 2), fm.fmoe_plan(0, 0, 0, -1),
                fm.fmoe_plan(16, 1, 1, 16), fm.fmoe_plan(0, 0, 0, 0, 128), fm.fmoe_plan(0, 0, 0, 0, 512)):
        assert call(s, w, bad) == fm.FMOE_ERR_ARG
    # FP8 with a 65536-deep reduction: 32-row tiles would need 68 KB of activation scales in LDS
    s8 = fm.make_shape(16, 65536, 128, 8, 2, fp8=True)
    w8 = fm.fmoe_weights(0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000)
    assert call(s8, w8, fm.fmoe_plan(32, 0, 0)) == fm.FMOE_ERR_UNSUPPORTED
    # tiles of five row groups are bf16 only (FP8's activation scales take that LDS)
    assert call(fm.make_shape(16, 256, 128, 8, 2, fp8=True), w8, fm.fmoe_plan(0, 0, 0, 0, 320)) == fm.FMOE_ERR_UNSUPPORTED
    # a plan with zero tokens is still a no-op
    s0 = fm.make_shape(0, 256, 128, 8, 2)
    assert lib.fmoe_forward_planned(ctypes.byref(s0), None, None, 0, 0, 1, ctypes.byref(w), None, None, None, None, 0,
                                    None, ctypes.byref(fm.fmoe_plan(16, 4, 2))) == fm.FMOE_OK


def test_grouped_router_rejects_bad_groups_before_launching():
    lib = fm.load_library()
    P = ctypes.c_void_p
    call = lambda E, k, ng, tg: lib.fmoe_router_topk_grouped(P(0x100), 0, 4, E, k, ng, tg, 0, 1, P(0x200),
                                                             P(0x300), None)
    assert call(64, 4, 5, 2) == fm.FMOE_ERR_ARG        # 5 does not divide 64
    assert call(64, 4, 8, 0) == fm.FMOE_ERR_ARG        # no group kept
    assert call(64, 4, 8, 9) == fm.FMOE_ERR_ARG        # more groups kept than exist
    assert call(64, 9, 8, 1) == fm.FMOE_ERR_ARG        # 8 experts in one kept group < k
    assert call(256, 4, 128, 2) == fm.FMOE_ERR_UNSUPPORTED  # more than 64 groups
    assert lib.fmoe_router_topk_grouped(P(0x100), 0, 0, 64, 4, 8, 2, 0, 1, None, None, None) == fm.FMOE_OK  # T = 0


def test_quantisation_and_grouped_gemm_reject_bad_arguments_without_a_device():
    lib = fm.load_library()
    P = ctypes.c_void_p
    # fmoe_act_quant: cols not a multiple of 128, unsupported dtype, null or misaligned buffers
    assert lib.fmoe_act_quant(P(0x100), fm.FMOE_BF16, 4, 200, P(0x200), P(0x300), None) == fm.FMOE_ERR_UNSUPPORTED
    assert lib.fmoe_act_quant(P(0x100), fm.FMOE_FP8_E4M3, 4, 256, P(0x200), P(0x300), None) == fm.FMOE_ERR_UNSUPPORTED
    assert lib.fmoe_act_quant(None, fm.FMOE_BF16, 4, 256, P(0x200), P(0x300), None) == fm.FMOE_ERR_ARG
    assert lib.fmoe_act_quant(P(0x108), fm.FMOE_BF16, 4, 256, P(0x200), P(0x300), None) == fm.FMOE_ERR_ARG
    assert lib.fmoe_act_quant(P(0x100), fm.FMOE_BF16, -1, 256, P(0x200), P(0x300), None) == fm.FMOE_ERR_ARG
    assert lib.fmoe_act_quant(None, fm.FMOE_BF16, 0, 256, None, None, None) == fm.FMOE_OK  # no rows: no-op
    # fmoe_grouped_gemm: bad stage, output dtype that does not fit the weights, missing scales
    s = fm.make_shape(16, 256, 128, 8, 2)
    w = fm.fmoe_weights(0x1000, 0x2000, 0x3000, None, None, None)
    n = fm.fmoe_workspace_bytes(s)

    def gg(shape, weights, stage, out_dtype, a_scale=None, out_scale=None, ws_n=None):
        return lib.fmoe_grouped_gemm(ctypes.byref(shape), None, stage, P(0x100), P(0x200), a_scale,
                                     ctypes.byref(weights), out_dtype, P(0x300), out_scale, P(0x400),
                                     n if ws_n is None else ws_n, None)
    assert gg(s, w, 2, fm.FMOE_BF16) == fm.FMOE_ERR_ARG
    assert gg(s, w, 0, fm.FMOE_FP32) == fm.FMOE_ERR_ARG          # bf16 weights write bf16
    assert gg(s, w, 1, fm.FMOE_FP8_E4M3) == fm.FMOE_ERR_ARG
    assert gg(s, w, 0, fm.FMOE_BF16, ws_n=n - 1) == fm.FMOE_ERR_WORKSPACE
    s8 = fm.make_shape(16, 256, 128, 8, 2, fp8=True)
    w8 = fm.fmoe_weights(0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000)
    n = fm.fmoe_workspace_bytes(s8)
    assert gg(s8, w8, 0, fm.FMOE_BF16, a_scale=P(0x500)) == fm.FMOE_ERR_ARG       # FP8 gate/up: fp32 or e4m3
    assert gg(s8, w8, 0, fm.FMOE_FP32) == fm.FMOE_ERR_ARG                          # activation scales missing
    assert gg(s8, w8, 0, fm.FMOE_FP8_E4M3, a_scale=P(0x500)) == fm.FMOE_ERR_ARG   # code scales missing
    assert gg(s8, w, 0, fm.FMOE_FP32, a_scale=P(0x500)) == fm.FMOE_ERR_ARG        # FP8 needs weight scales
    s0 = fm.make_shape(0, 256, 128, 8, 2)
    assert lib.fmoe_grouped_gemm(ctypes.byref(s0), None, 0, None, None, None, ctypes.byref(w), fm.FMOE_BF16, None,
                                 None, None, 0, None) == fm.FMOE_OK


@pytest.mark.parametrize("fp8", [False, True])
def test_workspace_layout_buffers_fit_and_do_not_overlap(fp8):
    T, H, I, E, k = 300, 2048, 768, 128, 8
    s = fm.make_shape(T, H, I, E, k, fp8=fp8)
    lay = fm.fmoe_workspace_layout(s)
    n = T * k
    sizes = dict(x_codes=T * H, x_scales=T * (H // 128) * 4, h_f32=n * I * 4, h_codes=n * I,
                 h_scales=n * (I // 128) * 4, h_bf16=n * I * 2, y=n * H * 2, perm_src=n * 4, inv_perm=n * 4)
    assert lay["total"] == fm.fmoe_workspace_bytes(s)
    present = {k_: v for k_, v in lay.items() if k_ != "total" and v}
    expect = {"x_codes", "x_scales", "h_f32", "h_codes", "h_scales"} if fp8 else {"h_bf16"}
    assert set(present) == expect | {"y", "perm_src", "inv_perm"}
    spans = sorted((off, off + sizes[name], name) for name, off in present.items())
    for (a0, a1, na), (b0, b1, nb) in zip(spans, spans[1:]):
        assert a1 <= b0, f"{na} overlaps {nb}"
    assert spans[-1][1] <= lay["total"] and all(off % 256 == 0 for off in present.values())
